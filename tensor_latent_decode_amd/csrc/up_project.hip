// Value up-projection of one device's latent-space attention output, and
// the summing all-reduce done on one device by accumulation:
//     y[b, h, v] (+)= sum_k o[b, h, k] * w[h, k, v].
//
// Under TPLA each device's attention covers only its slice of the latent, so
// the head output is the sum over devices of that slice's output times the
// matching rows of the head's W_UV (TPLA abstract: per-shard attention,
// results combined with an all-reduce).  w holds those rows transposed
// (latent index first), rotated like the latent.
//
// Layout: one workgroup per (block of 64 output columns, head).  The 64
// columns are the lanes of each wave; the four waves take a quarter of the
// k range each, so every row of w is read once per workgroup with 64
// consecutive columns per load.  The head's rows of o go to LDS 16 batch
// rows at a time and are read as wave-wide broadcasts; the four partial
// sums meet in LDS and are added in wave order (the same order for every
// output), so results do not depend on scheduling.  The work is bound by
// the reads of w (heads * d_s * d_v elements per call).
#include "tpla_internal.h"

namespace tpla {
namespace {

constexpr int kCols = 64;      // output columns per workgroup
constexpr int kRows = 16;      // batch rows per pass
constexpr int kParts = 4;      // waves, each a quarter of the k range

template <typename TO, typename TW, typename TY>
__global__ __launch_bounds__(256) void up_project_kernel(UpProjectParams p) {
  __shared__ float o_s[kRows][kMaxUpProjectK];
  __shared__ float part[kParts][kRows][kCols];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = blockIdx.x * kCols + lane;
  const int kq = (p.d_s + kParts - 1) / kParts;
  const int k0 = wave * kq;
  const int k1 = min(p.d_s, k0 + kq);
  const TW* wh = static_cast<const TW*>(p.w) + static_cast<int64_t>(h) * p.w_sh;

  for (int b0 = 0; b0 < p.batch; b0 += kRows) {
    const int nb = min(kRows, p.batch - b0);
    for (int i = threadIdx.x; i < kRows * p.d_s; i += blockDim.x) {
      const int j = i / p.d_s, k = i % p.d_s;
      o_s[j][k] = j < nb ? Elem<TO>::load(static_cast<const TO*>(p.o) + (b0 + j) * p.o_sb +
                                          static_cast<int64_t>(h) * p.o_sh + k)
                         : 0.f;
    }
    __syncthreads();
    float acc[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) acc[j] = 0.f;
    if (col < p.d_v) {
#pragma unroll 4
      for (int k = k0; k < k1; ++k) {
        const float wv = Elem<TW>::load(wh + static_cast<int64_t>(k) * p.w_sk + col);
#pragma unroll
        for (int j = 0; j < kRows; ++j) acc[j] = fmaf(o_s[j][k], wv, acc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) part[wave][j][lane] = acc[j];
    __syncthreads();
    for (int i = threadIdx.x; i < kRows * kCols; i += blockDim.x) {
      const int j = i / kCols, c = i % kCols;
      const int v = blockIdx.x * kCols + c;
      if (j < nb && v < p.d_v) {
        float s = part[0][j][c];
#pragma unroll
        for (int q = 1; q < kParts; ++q) s += part[q][j][c];
        TY* dst = static_cast<TY*>(p.y) + (b0 + j) * p.y_sb + static_cast<int64_t>(h) * p.y_sh + v;
        if (p.accumulate) s += Elem<TY>::load(dst);
        Elem<TY>::store(dst, s);
      }
    }
    __syncthreads();   // o_s and part are refilled by the next pass
  }
}

template <typename TO, typename TW>
hipError_t launch_w(const UpProjectParams& p, bool y_bf16, hipStream_t s) {
  const dim3 grid((p.d_v + kCols - 1) / kCols, p.heads), block(256);
  if (y_bf16)
    hipLaunchKernelGGL((up_project_kernel<TO, TW, uint16_t>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((up_project_kernel<TO, TW, float>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename TO>
hipError_t launch_o(const UpProjectParams& p, bool w_bf16, bool y_bf16, hipStream_t s) {
  return w_bf16 ? launch_w<TO, uint16_t>(p, y_bf16, s) : launch_w<TO, float>(p, y_bf16, s);
}

}  // namespace

hipError_t launch_up_project(const UpProjectParams& p, bool o_bf16, bool w_bf16, bool y_bf16,
                             hipStream_t s) {
  if (p.d_s > kMaxUpProjectK || p.heads > 65535) return hipErrorInvalidValue;
  return o_bf16 ? launch_o<uint16_t>(p, w_bf16, y_bf16, s) : launch_o<float>(p, w_bf16, y_bf16, s);
}

}  // namespace tpla
