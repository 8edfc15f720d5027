// Paged append of new latent/rope rows into one shard's cache.
//
// Under MLA only the latent cKV (plus the rope key) is cached, and under
// TPLA each device caches only its latent slice (TPLA abstract; paperbot
// revised abstract).  The cache is paged: logical token p of sequence b
// lives at row (block_table[b][p / block_size] * block_size + p % block_size).
//
// One 64-lane wavefront per appended row; lanes copy the row's d_s + d_r
// elements.  Same-type copies move bits; float32 -> bf16 rounds to nearest
// even.  Rows whose sequence, position or block id is out of range are
// skipped, so no write leaves the cache.
#include "tpla_internal.h"

namespace tpla {
namespace {

template <typename TC, typename TS>
__device__ __forceinline__ TC convert(TS v);
template <> __device__ __forceinline__ uint16_t convert<uint16_t, uint16_t>(uint16_t v) { return v; }
template <> __device__ __forceinline__ float convert<float, float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t convert<uint16_t, float>(float v) { return f32_to_bf16(v); }
template <> __device__ __forceinline__ float convert<float, uint16_t>(uint16_t v) { return bf16_to_f32(v); }

template <typename TC, typename TS>
__global__ __launch_bounds__(256) void append_kernel(
    TC* __restrict__ cache, int num_blocks, int block_size, int d_s, int d_r,
    const int32_t* __restrict__ bt, int max_blocks, int batch,
    const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos, int n_rows,
    const TS* __restrict__ latent, int64_t ls, const TS* __restrict__ rope, int64_t rs) {
  const int lane = threadIdx.x & 63;
  const int t = static_cast<int>((static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6);
  if (t >= n_rows) return;
  const int b = row_seq[t];
  const int p = row_pos[t];
  if (b < 0 || b >= batch || p < 0) return;
  const int lb = p / block_size;
  if (lb >= max_blocks) return;
  const int blk = bt[static_cast<int64_t>(b) * max_blocks + lb];
  if (blk < 0 || blk >= num_blocks) return;
  const int width = d_s + d_r;
  TC* dst = cache + (static_cast<int64_t>(blk) * block_size + p % block_size) * width;
  const TS* src_l = latent + static_cast<int64_t>(t) * ls;
  for (int k = lane; k < d_s; k += 64) dst[k] = convert<TC, TS>(src_l[k]);
  if (d_r > 0) {
    const TS* src_r = rope + static_cast<int64_t>(t) * rs;
    for (int k = lane; k < d_r; k += 64) dst[d_s + k] = convert<TC, TS>(src_r[k]);
  }
}

template <typename TC, typename TS>
hipError_t launch_t(void* cache, int num_blocks, int block_size, int d_s, int d_r,
                    const int32_t* bt, int max_blocks, int batch, const int32_t* row_seq,
                    const int32_t* row_pos, int n_rows, const void* latent, int64_t ls,
                    const void* rope, int64_t rs, hipStream_t s) {
  const int blocks = (n_rows + 3) / 4;
  hipLaunchKernelGGL((append_kernel<TC, TS>), dim3(blocks), dim3(256), 0, s,
                     static_cast<TC*>(cache), num_blocks, block_size, d_s, d_r, bt, max_blocks,
                     batch, row_seq, row_pos, n_rows, static_cast<const TS*>(latent), ls,
                     static_cast<const TS*>(rope), rs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(void* cache, int cache_bf16, int num_blocks, int block_size, int d_s,
                         int d_r, const int32_t* bt, int max_blocks, int batch,
                         const int32_t* row_seq, const int32_t* row_pos, int n_rows,
                         const void* latent, int64_t ls, const void* rope, int64_t rs,
                         int src_bf16, hipStream_t s) {
  if (cache_bf16 && src_bf16)
    return launch_t<uint16_t, uint16_t>(cache, num_blocks, block_size, d_s, d_r, bt, max_blocks,
                                        batch, row_seq, row_pos, n_rows, latent, ls, rope, rs, s);
  if (cache_bf16)
    return launch_t<uint16_t, float>(cache, num_blocks, block_size, d_s, d_r, bt, max_blocks,
                                     batch, row_seq, row_pos, n_rows, latent, ls, rope, rs, s);
  if (src_bf16)
    return launch_t<float, uint16_t>(cache, num_blocks, block_size, d_s, d_r, bt, max_blocks,
                                     batch, row_seq, row_pos, n_rows, latent, ls, rope, rs, s);
  return launch_t<float, float>(cache, num_blocks, block_size, d_s, d_r, bt, max_blocks, batch,
                                row_seq, row_pos, n_rows, latent, ls, rope, rs, s);
}

}  // namespace tpla
