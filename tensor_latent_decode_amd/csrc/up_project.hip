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
// Layout: one workgroup per (block of 32 output columns, head).  Thread t
// owns 2 consecutive columns (t % 16) and a sixteenth of the k range
// (t / 16); it issues its reads of w 16 rows at a time before using them.
// The head's rows of o go to LDS 16 batch rows at a time; all of a pass's
// reads of o and the first w rows go out before any wait, so a pass takes
// about one memory round trip.  The o rows use d_s * 64 bytes of
// dynamic LDS; the 16 partial sums of each output meet in LDS and are added in
// k-part order (the same order for every output), so results do not
// depend on scheduling.  The work is bound by the reads of w
// (heads * d_s * d_v elements per call).
#include <type_traits>

#include "tpla_internal.h"

namespace tpla {
namespace {

constexpr int kCols = 32;      // output columns per workgroup
constexpr int kRows = 16;      // batch rows per pass
constexpr int kCg = 2;         // columns per thread
constexpr int kParts = 16;     // k parts (256 threads / 16 column groups)
constexpr int kChunk = 16;     // w rows read together

// LDS row stride of the staged o rows (floats): room for a 16-wide read
// starting at any multiple of 4 below d_s, rounded to 4.
__host__ __device__ constexpr int up_project_row_stride(int d_s) { return (d_s + 15 + 3) & ~3; }

template <typename TO, typename TW, typename TY>
__global__ __launch_bounds__(256) void up_project_kernel(UpProjectParams p) {
  extern __shared__ float4 o_s4[];              // [kRows][ds4] floats, sized at launch
  float* o_s = reinterpret_cast<float*>(o_s4);
  // Row stride: the product loop reads 16 k from a multiple-of-4 start below
  // d_s, so up to d_s + 14; the pad is zero.
  const int ds4 = up_project_row_stride(p.d_s);
  __shared__ float part[kParts][kRows][kCols];
  const int h = blockIdx.y;
  const int cg = threadIdx.x % (kCols / kCg);
  const int kp = threadIdx.x / (kCols / kCg);
  const int c0 = blockIdx.x * kCols + cg * kCg;
  const int kq = (((p.d_s + kParts - 1) / kParts) + 3) & ~3;   // a multiple of 4
  const int k0 = kp * kq;
  const int k1 = min(p.d_s, k0 + kq);
  const TW* wh = static_cast<const TW*>(p.w) + static_cast<int64_t>(h) * p.w_sh;

  // w rows [kc, kc + kChunk) of this thread's columns.  The reads are
  // unconditional, from indices clamped into the matrix, so they all go out
  // before any wait; a value read for a row >= k1 is never used (the product
  // loop stops at k1) and one for a column >= d_v only feeds an output that
  // is not stored.
  auto load_w = [&](int kc, float (&wv)[kChunk][kCg]) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
#pragma unroll
      for (int c = 0; c < kCg; ++c)
        wv[u][c] = Elem<TW>::load(wh + static_cast<int64_t>(min(kc + u, p.d_s - 1)) * p.w_sk +
                                  min(c0 + c, p.d_v - 1));
  };

  // The head's o rows of one pass (16 batch rows) into LDS: thread t takes
  // columns t, t + 256, ... of every row.  All of a pass's reads of o
  // (indices clamped into the matrix, so unconditional) and the first w
  // rows' reads go out before any wait; rows past the batch become zeros.
  float wv[kChunk][kCg];
  auto stage = [&](auto per_row, int b0, int nb) {
    constexpr int R = decltype(per_row)::value;     // 256-column rounds per row
    float tmp[kRows][R];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const TO* row = static_cast<const TO*>(p.o) + (b0 + min(j, nb - 1)) * p.o_sb +
                      static_cast<int64_t>(h) * p.o_sh;
#pragma unroll
      for (int r = 0; r < R; ++r) tmp[j][r] = Elem<TO>::load(row + min(static_cast<int>(threadIdx.x) + r * 256, p.d_s - 1));
    }
    load_w(k0, wv);
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int k = static_cast<int>(threadIdx.x) + r * 256;
        if (k < p.d_s) o_s[j * ds4 + k] = j < nb ? tmp[j][r] : 0.f;
      }
    const int pad = ds4 - p.d_s;
    for (int i = threadIdx.x; i < kRows * pad; i += 256) o_s[(i / pad) * ds4 + p.d_s + i % pad] = 0.f;
  };
  const int rounds = (p.d_s + 255) / 256;   // 1 .. 4 (d_s <= 1024)

  for (int b0 = 0; b0 < p.batch; b0 += kRows) {
    const int nb = min(kRows, p.batch - b0);
    if (rounds == 1) stage(std::integral_constant<int, 1>(), b0, nb);
    else if (rounds == 2) stage(std::integral_constant<int, 2>(), b0, nb);
    else if (rounds == 3) stage(std::integral_constant<int, 3>(), b0, nb);
    else stage(std::integral_constant<int, 4>(), b0, nb);
    __syncthreads();
    float acc[kRows][kCg];
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
      for (int c = 0; c < kCg; ++c) acc[j][c] = 0.f;
    for (int kc = k0; kc < k1; kc += kChunk) {
      if (kc != k0) load_w(kc, wv);
      // rows past this thread's part contribute nothing (their o values are
      // another part's); o is read four k at a time
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
#pragma unroll
        for (int c = 0; c < kCg; ++c) wv[u][c] = kc + u < k1 ? wv[u][c] : 0.f;
#pragma unroll
      for (int u4 = 0; u4 < kChunk / 4; ++u4) {
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
          const float4 ov = o_s4[(j * ds4 + kc) / 4 + u4];
          const float o4[4] = {ov.x, ov.y, ov.z, ov.w};
#pragma unroll
          for (int uu = 0; uu < 4; ++uu)
#pragma unroll
            for (int c = 0; c < kCg; ++c) acc[j][c] = fmaf(o4[uu], wv[4 * u4 + uu][c], acc[j][c]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
      for (int c = 0; c < kCg; ++c) part[kp][j][cg * kCg + c] = acc[j][c];
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
  const size_t lds = static_cast<size_t>(kRows) * up_project_row_stride(p.d_s) * sizeof(float);
  const void* fn = y_bf16 ? reinterpret_cast<const void*>(&up_project_kernel<TO, TW, uint16_t>)
                          : reinterpret_cast<const void*>(&up_project_kernel<TO, TW, float>);
  // allow the largest o staging (d_s = kMaxUpProjectK) beyond the default
  // dynamic LDS limit
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(kRows * up_project_row_stride(kMaxUpProjectK) *
                                                      sizeof(float)));
  if (e != hipSuccess) return e;
  if (y_bf16)
    hipLaunchKernelGGL((up_project_kernel<TO, TW, uint16_t>), grid, block, lds, s, p);
  else
    hipLaunchKernelGGL((up_project_kernel<TO, TW, float>), grid, block, lds, s, p);
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
