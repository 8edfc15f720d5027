// Value up-projection of one device's latent-space attention output, and
// the summing all-reduce done on one device by accumulation:
//     y[b, h, v] (+)= sum_k o[b, h, k] * w[h, v, k].
//
// Under TPLA each device's attention covers only its slice of the latent, so
// the head output is the sum over devices of that slice's output times the
// matching columns of the head's W_UV (TPLA abstract: per-shard attention,
// results combined with an all-reduce).  w is W_UV in its own layout
// ([head][v][latent], latent contiguous), restricted to the device's latent
// columns and rotated like the latent.
//
// Per head this is a small dense product, Y^T[v, b] = W[v, :] . O[b, :]^T,
// on v_mfma_f32_32x32x16_bf16: W rows are the A operand and o rows the B
// operand, both with the latent index contiguous, which is the 8-k-per-lane
// fragment layout.  A float32 operand is split into three bf16 terms
// (x = hi + mid + lo exactly: each term holds the next 8 significant bits,
// cut by truncation),
// and every pair of terms gets its own MFMA, so the products are exact and
// only the float32 accumulation rounds.  One workgroup per (head, 32 rows
// of v, 32 batch rows), its waves splitting the k-steps; each wave issues
// its reads for 8 k-steps before the MFMAs that use them.
#include <type_traits>

#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kKS = 8;         // k-steps (of 16) whose reads go out together
constexpr int kWaves = 4;      // waves per workgroup, each a quarter of the k-steps

template <typename T>
constexpr int terms() { return std::is_same<T, float>::value ? 3 : 1; }

// The operand fragment of one lane for one k-step: elements k .. k+7 of a
// row of n, as N bf16x8 terms whose sum is the row's values exactly
// (elements at or past n are zero when `zero_tail`, else unspecified).
// bf16 rows are their own single term; a float32 value x splits by
// truncation: hi = x with the low 16 bits cleared, then the same on
// x - hi and on the rest, each difference exact.
template <typename T, bool kVec>
__device__ __forceinline__ void fragment(const T* p, int k, int n, bool zero_tail,
                                         bf16x8_t (&t)[terms<T>()]) {
  if constexpr (std::is_same<T, uint16_t>::value) {
    uint16_t u[8];
    if constexpr (kVec) {
      const int k0 = min(k, n - 8);
      const uint4 w = *reinterpret_cast<const uint4*>(p + k0);
      const uint16_t r[8] = {static_cast<uint16_t>(w.x), static_cast<uint16_t>(w.x >> 16),
                             static_cast<uint16_t>(w.y), static_cast<uint16_t>(w.y >> 16),
                             static_cast<uint16_t>(w.z), static_cast<uint16_t>(w.z >> 16),
                             static_cast<uint16_t>(w.w), static_cast<uint16_t>(w.w >> 16)};
      const int sh = k - k0;   // > 0 only past the row's last full piece
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t v = 0;
#pragma unroll
        for (int f = 0; f < 8; ++f) v = (f == e + sh) ? r[f] : v;
        u[e] = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = p[min(k + e, n - 1)];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      t[0][e] = __builtin_bit_cast(__bf16, (zero_tail && k + e >= n) ? static_cast<uint16_t>(0) : u[e]);
  } else {
    float x[8];
    if constexpr (kVec) {
      const int k0 = min(k, n - 8);
      const float4 a = *reinterpret_cast<const float4*>(p + k0);
      const float4 b = *reinterpret_cast<const float4*>(p + k0 + 4);
      const float r[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      const int sh = k - k0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = 0.f;
#pragma unroll
        for (int f = 0; f < 8; ++f) v = (f == e + sh) ? r[f] : v;
        x[e] = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p[min(k + e, n - 1)];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float r = (zero_tail && k + e >= n) ? 0.f : x[e];
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const uint32_t hb = __float_as_uint(r) & 0xFFFF0000u;
        t[i][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(hb >> 16));
        r -= __uint_as_float(hb);
      }
    }
  }
}

// One workgroup per (32 rows of v, 32 batch rows, head); its four waves
// take a quarter of the k-steps each and their accumulators are added in
// wave order through LDS.
template <typename TO, typename TW, typename TY, bool kVec>
__global__ __launch_bounds__(256) void up_project_kernel(UpProjectParams p) {
  __shared__ float part[kWaves][16][64];
  const int h = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int v0 = blockIdx.x * 32;
  const int b0 = blockIdx.y * 32;
  // A rows / B columns past the end read the last valid row; their outputs
  // are not stored
  const TW* wrow = static_cast<const TW*>(p.w) + static_cast<int64_t>(h) * p.w_sh +
                   static_cast<int64_t>(min(v0 + l31, p.d_v - 1)) * p.w_sv;
  const TO* orow = static_cast<const TO*>(p.o) + static_cast<int64_t>(min(b0 + l31, p.batch - 1)) * p.o_sb +
                   static_cast<int64_t>(h) * p.o_sh;
  constexpr int NW = terms<TW>(), NO = terms<TO>();
  f32x16_t acc = {};
  const int ksteps = (p.d_s + 15) / 16;
  const int kq = (ksteps + kWaves - 1) / kWaves;
  const int s_lo = wave * kq, s_hi = min(ksteps, s_lo + kq);
  for (int s0 = s_lo; s0 < s_hi; s0 += kKS) {
    bf16x8_t at[kKS][NW], bt[kKS][NO];
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      const int k = min(s0 + s, ksteps - 1) * 16 + 8 * half;
      fragment<TW, kVec>(wrow, k, p.d_s, false, at[s]);
      fragment<TO, kVec>(orow, k, p.d_s, true, bt[s]);
    }
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
      if (s0 + s < s_hi) {
#pragma unroll
        for (int i = 0; i < NW; ++i)
#pragma unroll
          for (int j = 0; j < NO; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at[s][i], bt[s][j], acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) part[wave][r][lane] = acc[r];
  __syncthreads();
  // Thread t writes 4 consecutive v of batch row t / 8, so 8 threads cover
  // 32 consecutive outputs.  Accumulator register r of lane l holds
  // v = 8*(r/4) + 4*(l/32) + r%4, b = l%32.
  {
    const int bl = threadIdx.x >> 3, vg = (threadIdx.x & 7) * 4;
    const int src = bl + 32 * ((vg >> 2) & 1), r0 = 4 * (vg >> 3);
    const int b = b0 + bl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = v0 + vg + i;
      if (b < p.batch && v < p.d_v) {
        float sum = part[0][r0 + i][src];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) sum += part[q][r0 + i][src];
        TY* dst = static_cast<TY*>(p.y) + static_cast<int64_t>(b) * p.y_sb +
                  static_cast<int64_t>(h) * p.y_sh + v;
        if (p.accumulate) sum += Elem<TY>::load(dst);
        Elem<TY>::store(dst, sum);
      }
    }
  }
}

template <typename TO, typename TW, typename TY>
hipError_t launch_y(const UpProjectParams& p, bool vec, hipStream_t s) {
  const dim3 grid((p.d_v + 31) / 32, (p.batch + 31) / 32, p.heads), block(256);
  if (vec)
    hipLaunchKernelGGL((up_project_kernel<TO, TW, TY, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((up_project_kernel<TO, TW, TY, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <typename TO, typename TW>
hipError_t launch_w(const UpProjectParams& p, bool y_bf16, bool vec, hipStream_t s) {
  return y_bf16 ? launch_y<TO, TW, uint16_t>(p, vec, s) : launch_y<TO, TW, float>(p, vec, s);
}

template <typename TO>
hipError_t launch_o(const UpProjectParams& p, bool w_bf16, bool y_bf16, bool vec, hipStream_t s) {
  return w_bf16 ? launch_w<TO, uint16_t>(p, y_bf16, vec, s) : launch_w<TO, float>(p, y_bf16, vec, s);
}

// Rows of n >= 8 elements of `elem` bytes at p + i*s1 + j*s2 can be read in
// 16-byte pieces starting at multiples of 8 elements (and at n - 8).
bool rows_vec(const void* p, int64_t s1, int64_t s2, int n, int elem) {
  const int64_t piece = 16 / elem;
  return reinterpret_cast<uintptr_t>(p) % 16 == 0 && s1 % piece == 0 && s2 % piece == 0 &&
         n >= 8 && n % piece == 0;
}

}  // namespace

hipError_t launch_up_project(const UpProjectParams& p, bool o_bf16, bool w_bf16, bool y_bf16,
                             hipStream_t s) {
  if (p.heads > 65535 || (p.batch + 31) / 32 > 65535) return hipErrorInvalidValue;
  const bool vec = rows_vec(p.o, p.o_sb, p.o_sh, p.d_s, o_bf16 ? 2 : 4) &&
                   rows_vec(p.w, p.w_sh, p.w_sv, p.d_s, w_bf16 ? 2 : 4);
  return o_bf16 ? launch_o<uint16_t>(p, w_bf16, y_bf16, vec, s)
                : launch_o<float>(p, w_bf16, y_bf16, vec, s);
}

}  // namespace tpla
