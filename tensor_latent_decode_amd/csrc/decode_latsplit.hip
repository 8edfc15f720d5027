// Dispatch of the streaming bf16 split-K decode kernels (gfx950): shard
// shapes with block_size % 64 == 0 and d_r = 64, whose 64-token tiles are
// contiguous runs of 64 * (d_s + d_r) * 2 bytes inside one page.
//
//   d_s = 256, heads % 128 == 0   decode_roles.hip, 128-head workgroups
//   d_s = 128, heads % 64 == 0    decode_roles.hip, 64-head workgroups
//   d_s = 512                     decode_mla.hip (plain MLA under tensor
//                                 parallelism, or a one-shard TPLA)
//
// All of them write fp16 split outputs with one float scale per 64 columns
// and the layout the merge reads (merge_item.h).
#include "tpla_internal.h"

namespace tpla {

namespace {
constexpr int kTile = 64;
}  // namespace

int decode_latsplit_max_chunk() { return min(decode_roles_max_tiles() * kTile, decode_mla_max_chunk()); }

int decode_latsplit_partial_block() { return 64; }

bool decode_latsplit_supported(int heads, int d_s, int d_r, int block_size) {
  return decode_mla_supported(heads, d_s, d_r, block_size) ||
         decode_roles_supported(heads, d_s, d_r, block_size);
}

// Workgroups per CU the uniform split plan targets (one: every streaming
// kernel fills a CU's LDS).
int decode_latsplit_groups_per_cu(int heads, int d_s) {
  (void)heads;
  (void)d_s;
  return 1;
}

int decode_latsplit_heads_per_group(int heads, int d_s) {
  if (d_s == 512) return decode_mla_group_heads(heads);
  return decode_roles_heads_per_group(heads, d_s);
}

hipError_t launch_decode_latsplit(const DecodeParams& p, hipStream_t s) {
  if (decode_mla_supported(p.heads, p.d_s, p.d_r, p.block_size)) return launch_decode_mla(p, s);
  if (decode_roles_supported(p.heads, p.d_s, p.d_r, p.block_size)) return launch_decode_roles(p, s);
  return hipErrorNotSupported;
}

}  // namespace tpla
