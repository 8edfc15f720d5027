// Log-sum-exp merge of the token splits, and the on-device shard combine.
//
// Merge: each split s of sequence b produced, for every head, the attention
// output over its own tokens o_s (already divided by its own sum) and
// lse_s = log sum exp(scores).  The split results combine exactly:
//     LSE = log sum_s exp(lse_s),   o = sum_s exp(lse_s - LSE) * o_s.
// Splits without tokens carry lse_s = -inf and are skipped (their o_s is
// never read).
//
// Combine: shard g owns latent columns g*d_s .. (g+1)*d_s, so summing the
// zero-padded shard outputs (the all-reduce of the TPLA abstract) places
// them side by side.
#include "tpla_internal.h"

namespace tpla {
namespace {

// One 64-lane wavefront per (b, h); lanes stride over d_s.
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  if (bh >= static_cast<int64_t>(p.batch) * p.heads) return;
  const int64_t stride_s = static_cast<int64_t>(p.batch) * p.heads;
  float mx = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, p.ws_lse[s * stride_s + bh]);
  const int b = static_cast<int>(bh / p.heads);
  const int h = static_cast<int>(bh % p.heads);
  const int64_t obase = b * p.out_sb + h * p.out_sh;
  if (mx == -INFINITY) {
    for (int k = lane; k < p.d_s; k += 64) {
      if (p.out_bf16) static_cast<uint16_t*>(p.out)[obase + k] = 0;
      else static_cast<float*>(p.out)[obase + k] = 0.f;
    }
    if (p.lse != nullptr && lane == 0) p.lse[bh] = -INFINITY;
    return;
  }
  float tot = 0.f;
  for (int s = 0; s < p.splits; ++s) {
    const float l = p.ws_lse[s * stride_s + bh];
    if (l != -INFINITY) tot += __expf(l - mx);
  }
  const float lse = mx + __logf(tot);
  for (int k = lane; k < p.d_s; k += 64) {
    float acc = 0.f;
    for (int s = 0; s < p.splits; ++s) {
      const float l = p.ws_lse[s * stride_s + bh];
      if (l == -INFINITY) continue;
      acc += __expf(l - lse) * p.ws_o[(s * stride_s + bh) * p.d_s + k];
    }
    if (p.out_bf16) static_cast<uint16_t*>(p.out)[obase + k] = f32_to_bf16(acc);
    else static_cast<float*>(p.out)[obase + k] = acc;
  }
  if (p.lse != nullptr && lane == 0) p.lse[bh] = lse;
}

template <typename TP, typename TO>
__global__ __launch_bounds__(256) void combine_kernel(PartPtrs parts, int tp, int batch,
                                                      int heads, int d_s, TO* __restrict__ out,
                                                      int accumulate) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t d_c = static_cast<int64_t>(tp) * d_s;
  const int64_t total = static_cast<int64_t>(batch) * heads * d_c;
  if (i >= total) return;
  const int64_t bh = i / d_c;
  const int col = static_cast<int>(i % d_c);
  const int g = col / d_s;
  const int k = col % d_s;
  const TP* src = static_cast<const TP*>(parts.p[g]) + bh * d_s + k;
  if (!accumulate) {
    if constexpr (sizeof(TP) == sizeof(TO)) {
      out[i] = *src;                                   // same type: bits
    } else {
      Elem<TO>::store(out + i, Elem<TP>::load(src));
    }
  } else {
    Elem<TO>::store(out + i, Elem<TO>::load(out + i) + Elem<TP>::load(src));
  }
}

template <typename TP, typename TO>
hipError_t launch_c(const PartPtrs& parts, int tp, int batch, int heads, int d_s, void* out,
                    int accumulate, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(batch) * heads * tp * d_s;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((combine_kernel<TP, TO>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     s, parts, tp, batch, heads, d_s, static_cast<TO*>(out), accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  const int64_t waves = static_cast<int64_t>(p.batch) * p.heads;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_combine(const PartPtrs& parts, int part_bf16, int tp, int batch, int heads,
                          int d_s, void* out, int out_bf16, int accumulate, hipStream_t s) {
  if (part_bf16 && out_bf16)
    return launch_c<uint16_t, uint16_t>(parts, tp, batch, heads, d_s, out, accumulate, s);
  if (part_bf16) return launch_c<uint16_t, float>(parts, tp, batch, heads, d_s, out, accumulate, s);
  if (out_bf16) return launch_c<float, uint16_t>(parts, tp, batch, heads, d_s, out, accumulate, s);
  return launch_c<float, float>(parts, tp, batch, heads, d_s, out, accumulate, s);
}

}  // namespace tpla
