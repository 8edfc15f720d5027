// Internal declarations shared by the libtpla translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpla.h"

namespace tpla {

// ---------------------------------------------------------------------------
// bf16 <-> float32 on the device.  bf16 values travel as uint16_t bit
// patterns; conversions to bf16 round to nearest, ties to even (the
// hardware conversion: no branch per value, a NaN stays a quiet NaN).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));   // v_cvt_pk_bf16_f32: RNE
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};

struct MergeParams {
  int splits, batch, heads, d_s;
  int blk_cols;                 // 0: float32 partials; else fp16 partials, scale per blk_cols
  // Non-null: the split outputs are rows [unit, heads] of `splits` units
  // (batch 1 in the scale offset) and sequence b owns units
  // unit_table[2b] .. unit_table[2b] + unit_table[2b+1] - 1.
  const int32_t* unit_table;
  const float* ws_o;
  const float* ws_lse;
  void* out;
  int out_bf16;
  int64_t out_sb, out_sh;
  float* lse;
};

// ---------------------------------------------------------------------------
// Decode kernel parameters (device pointers and sizes after validation).
// ---------------------------------------------------------------------------
struct DecodeParams {
  int batch, heads, d_s, d_r;
  int block_size, num_blocks, max_blocks;
  int max_seq_len;
  int num_splits, chunk;        // tokens per split, multiple of 64
  float scale_log2;             // scale * log2(e)
  const void* q_latent;
  int64_t qls_b, qls_h;
  const void* q_rope;
  int64_t qrs_b, qrs_h;
  const void* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* ws_o;                  // [splits, batch, heads, d_s]
  float* ws_lse;                // [splits, batch, heads]
  // Kernels that cut the work into units themselves (unit_map.h) ignore
  // num_splits: their split outputs are rows [unit, heads], at most
  // max_units units, and unit_table receives each sequence's units.
  int unit_target;              // > 0: units of one chunk size chosen so about this many exist;
                                // 0: chunk = `chunk`
  int max_units;                // bound on the units of this call (launch size, workspace rows)
  int32_t* unit_table;          // [batch][2]: first unit, unit count
};

// Split outputs are either float32 [splits, batch, heads, d_s] at ws_o, or
// fp16 at the same address with one float scale per (split, b, h, block of
// blk_cols columns) at ws_o + fp16_partials_scale_offset(...) bytes.
__host__ __device__ inline size_t fp16_partials_scale_offset(int splits, int batch, int heads,
                                                              int d_s) {
  const size_t n = static_cast<size_t>(splits) * batch * heads * d_s * 2;
  return (n + 255) & ~static_cast<size_t>(255);
}


constexpr int kMaxTp = 16;
struct PartPtrs {
  const void* p[kMaxTp];
};
struct CachePtrs {
  void* p[kMaxTp];
};

// Rotation of query rows and new latent rows, and the paged append of the
// new rows' shard slices (one launch).
struct RotateAppendParams {
  const void* q;
  int64_t qs;
  void* q_out;
  int64_t qos;
  int64_t q_rows;
  int q_bf16, q_out_bf16;
  int q_vec;                    // rows move in 16-byte pieces (set by the launcher)
  const void* lat;              // new latent rows, n wide, unrotated
  int64_t ls;
  const void* rope;             // same dtype as lat
  int64_t rs;
  void* lat_out;                // optional rotated copy (lat's dtype)
  int64_t los;
  int lat_bf16;
  int lat_vec;                  // as q_vec, for lat and lat_out
  int n_rows;
  const int32_t* row_seq;
  const int32_t* row_pos;
  CachePtrs caches;
  int n_caches, first_shard, cache_bf16;
  int num_blocks, block_size, d_s, d_r, max_blocks, batch;
  const int32_t* bt;
  int norm;                     // TPLA_NORM_* of the rotated latent rows
  float norm_eps;
};

// Value up-projection: y[b, h, v] (+)= sum_k o[b, h, k] * w[h, v, k].
struct UpProjectParams {
  const void* o;
  int64_t o_sb, o_sh;
  const void* w;
  int64_t w_sh, w_sv;
  void* y;
  int64_t y_sb, y_sh;
  int batch, heads, d_s, d_v;
  int accumulate;
};

// MLA-form prefill: causal attention of each prompt over its own latent rows
// kv[b, j] = [latent (512) || rope key (64)], bf16, 16-byte aligned rows.
struct PrefillParams {
  int batch, heads, max_len;
  float scale_log2;             // scale * log2(e)
  const void* q_latent;
  int64_t ql_b, ql_s, ql_h;
  const void* q_rope;
  int64_t qr_b, qr_s, qr_h;
  const void* kv;
  int64_t kv_b, kv_s;
  const int32_t* seq_lens;
  void* out;
  int out_bf16;
  int64_t o_b, o_s, o_h;
  float* lse;                   // [batch, max_len, heads] or null
};

// Launchers (return the launch status; they do not synchronise).
hipError_t launch_mla_prefill(const PrefillParams& p, hipStream_t s);
hipError_t launch_prefill_roles(const PrefillParams& p, hipStream_t s);
bool prefill_roles_supported(int heads, int64_t kv_stride_t);
hipError_t launch_up_project(const UpProjectParams& p, bool o_bf16, bool w_bf16, bool y_bf16,
                             hipStream_t s);
hipError_t launch_hadamard(const void* x, int x_bf16, int64_t xs, void* y, int y_bf16, int64_t ys,
                           int64_t rows, int n, hipStream_t s);
hipError_t launch_rotate_append(const RotateAppendParams& p, int n, hipStream_t s);
hipError_t launch_append(void* cache, int cache_bf16, int num_blocks, int block_size, int d_s,
                         int d_r, const int32_t* bt, int max_blocks, int batch,
                         const int32_t* row_seq, const int32_t* row_pos, int n_rows,
                         const void* latent, int64_t ls, const void* rope, int64_t rs,
                         int src_bf16, hipStream_t s);
// Returns hipErrorNotSupported when no matrix-core instantiation fits.
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s);
bool decode_mfma_supported(int heads, int d_s, int d_r);
int decode_mfma_groups_per_cu(int heads, int d_s, int d_r);
hipError_t launch_decode_latsplit(const DecodeParams& p, hipStream_t s);
bool decode_latsplit_supported(int heads, int d_s, int d_r, int block_size);
int decode_latsplit_groups_per_cu(int heads, int d_s);   // workgroups per CU the split plan targets
int decode_latsplit_heads_per_group(int heads, int d_s);
int decode_latsplit_max_chunk();   // tokens per split the latent-split kernel accepts
int decode_latsplit_partial_block();   // columns per scale of its fp16 split outputs
hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t s);
hipError_t launch_decode_roles(const DecodeParams& p, hipStream_t s);
bool decode_roles_supported(int heads, int d_s, int d_r, int block_size);
int decode_roles_max_tiles();      // 64-token tiles one unit of the roles kernel may hold
int decode_roles_heads_per_group(int heads, int d_s);   // heads of one workgroup (128 or 64)
bool decode_mla_supported(int heads, int d_s, int d_r, int block_size);
int decode_mla_max_chunk();
int decode_mla_group_heads(int heads);   // heads per workgroup of the 512-wide kernel
hipError_t launch_decode_generic(const DecodeParams& p, int is_bf16, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_combine(const PartPtrs& parts, int part_bf16, int tp, int batch, int heads,
                          int d_s, void* out, int out_bf16, int accumulate, hipStream_t s);

}  // namespace tpla
