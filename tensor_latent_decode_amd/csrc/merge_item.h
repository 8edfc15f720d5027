// The log-sum-exp merge of one (sequence b, head h, 8-column block cb) of
// fp16 split outputs (o_s = scale_s * h_s, one scale per blk_cols columns):
//     LSE = log sum_s exp(lse_s),   o = sum_s exp(lse_s - LSE) * o_s,
// splits without tokens (lse_s = -inf) weighing 0.  Up to 16 splits per
// memory round trip (every load of a chunk is issued before any is used),
// with a running max across chunks.  The splits of an item may be shared by
// G adjacent lanes (lane g takes splits g, g + G, ...), whose partial
// results then combine exactly the same way across the lanes.  Split (or
// unit) u holds [d_s / 8][heads][8] halves, scales [d_s / blk_cols][heads]
// and lse [heads]: u = s * batch + b for uniform splits; kUnits: sequence b
// owns units ut.x .. ut.x + ut.y - 1.
#pragma once

#include "tpla_internal.h"

namespace tpla {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

struct MergePart {
  float m, tot;        // running max and sum of exp(lse_s - m)
  float acc[8];        // sum of exp(lse_s - m) * o_s, 8 columns
};

// kShared: one lane per item (G == 1) and scale blocks of a multiple of 64
// columns, so the wavefront's 8 column blocks of 8 heads share each head's
// lse and scale (see below).
template <bool kUnits, bool kShared>
__device__ inline MergePart merge16_partial(const MergeParams& p, int b, int h, int cb, int2 ut, int g,
                                            int G) {
  const int o8 = p.d_s / 8;
  const int nblk = p.d_s / p.blk_cols;
  const int col = cb * 8;
  const int nsplit = ut.y;
  const uint16_t* wh = reinterpret_cast<const uint16_t*>(p.ws_o);
  const float* wsc = reinterpret_cast<const float*>(
      reinterpret_cast<const char*>(p.ws_o) +
      fp16_partials_scale_offset(p.splits, kUnits ? 1 : p.batch, p.heads, p.d_s));   // scales follow the rows
  constexpr int kC = 16;
  MergePart r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.acc[i] = 0.f;
  r.m = -INFINITY;
  r.tot = 0.f;
  for (int s0 = g; s0 < nsplit; s0 += kC * G) {
    float l[kC], f[kC];
    uint4 v[kC];
    // One lane per item (kShared): the wavefront's 8 column blocks of 8
    // heads share each head's lse and scale, so lane r loads those of splits
    // r/8 and r/8 + 8 for its head (lanes r and r % 8 + 8k hold the same
    // head) and the others come by shuffle: 4 loads instead of 32.
    // Every load of the chunk (lse, scales, split outputs) is issued before
    // any result is used: one memory round trip.
    float la = 0.f, lb = 0.f, fa = 0.f, fb = 0.f;
    const int lane = static_cast<int>(threadIdx.x & 63);
    if constexpr (kShared) {
      const int sa = min(s0 + (lane >> 3), nsplit - 1), sb = min(s0 + (lane >> 3) + 8, nsplit - 1);
      const int64_t ua = kUnits ? static_cast<int64_t>(ut.x) + sa : static_cast<int64_t>(sa) * p.batch + b;
      const int64_t ub = kUnits ? static_cast<int64_t>(ut.x) + sb : static_cast<int64_t>(sb) * p.batch + b;
      la = p.ws_lse[ua * p.heads + h];
      lb = p.ws_lse[ub * p.heads + h];
      fa = wsc[(ua * nblk + col / p.blk_cols) * p.heads + h];
      fb = wsc[(ub * nblk + col / p.blk_cols) * p.heads + h];
    }
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const int s = min(s0 + u * G, nsplit - 1);
      const int64_t unit = kUnits ? static_cast<int64_t>(ut.x) + s : static_cast<int64_t>(s) * p.batch + b;
      if constexpr (!kShared) {
        l[u] = p.ws_lse[unit * p.heads + h];
        f[u] = wsc[(unit * nblk + col / p.blk_cols) * p.heads + h];
      }
      if constexpr (kUnits) {
        // streaming load: each unit output is read once (written as 512-byte
        // runs by streaming stores)
        const u32x4_t x = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(wh + ((unit * o8 + cb) * p.heads + h) * 8));
        v[u] = make_uint4(x[0], x[1], x[2], x[3]);
      } else {
        // split rows of the MLA kernel (plain stores)
        v[u] = *reinterpret_cast<const uint4*>(wh + ((unit * o8 + cb) * p.heads + h) * 8);
      }
    }
    // The results are used only past the test for a chunk without tokens;
    // marking them used here keeps the compiler from sinking their loads
    // below it (after the lse round trip).
#pragma unroll
    for (int u = 0; u < kC; ++u) asm volatile("" : : "v"(v[u].x), "v"(v[u].y), "v"(v[u].z), "v"(v[u].w));
    if constexpr (kShared) {
#pragma unroll
      for (int u = 0; u < kC; ++u) {
        const int src = ((u & 7) << 3) | (lane & 7);
        l[u] = __shfl(u < 8 ? la : lb, src);
        f[u] = __shfl(u < 8 ? fa : fb, src);
      }
    }
    float cm = r.m;
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      if (s0 + u * G >= nsplit) l[u] = -INFINITY;
      cm = fmaxf(cm, l[u]);
    }
    if (cm == -INFINITY) continue;              // no tokens so far
    const float sc = __expf(r.m - cm);          // 0 while m is still -inf
    r.tot *= sc;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.acc[i] *= sc;
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const bool use = l[u] != -INFINITY;       // empty splits: weight 0, o never used
      const float w = use ? __expf(l[u] - cm) : 0.f;
      r.tot += w;
      const float wf = use ? w * f[u] : 0.f;
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float hv = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(wd[i >> 1] >> (16 * (i & 1)))));
        r.acc[i] += use ? wf * hv : 0.f;
      }
    }
    r.m = cm;
  }
  return r;
}

// Combines the partials of G adjacent lanes (G a power of two, the group
// aligned to G); every lane of the group ends with the whole.
__device__ inline void merge_lanes(MergePart& r, int G) {
  for (int off = 1; off < G; off <<= 1) {
    const float m_o = __shfl_xor(r.m, off);
    const float t_o = __shfl_xor(r.tot, off);
    float a_o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a_o[i] = __shfl_xor(r.acc[i], off);
    const float mm = fmaxf(r.m, m_o);
    if (mm == -INFINITY) continue;              // neither has tokens
    const float s1 = __expf(r.m - mm), s2 = __expf(m_o - mm);   // 0 for a side at -inf
    r.tot = r.tot * s1 + t_o * s2;
#pragma unroll
    for (int i = 0; i < 8; ++i) r.acc[i] = r.acc[i] * s1 + a_o[i] * s2;
    r.m = mm;
  }
}

// o = acc / tot and LSE = m + log tot (0 and -inf without tokens).
template <bool kBf16Out>
__device__ inline void merge16_store(const MergeParams& p, int b, int h, int cb, const MergePart& r) {
  const int col = cb * 8;
  float acc[8];
  float lse = -INFINITY;
  const float inv = r.m != -INFINITY ? 1.0f / r.tot : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = r.acc[i] * inv;
  if (r.m != -INFINITY) lse = r.m + __logf(r.tot);
  const int64_t obase = b * p.out_sb + h * p.out_sh + col;
  if constexpr (kBf16Out) {
    uint16_t* o = static_cast<uint16_t*>(p.out) + obase;
    if ((reinterpret_cast<uintptr_t>(o) & 15) == 0) {
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] = static_cast<uint32_t>(f32_to_bf16(acc[2 * k])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * k + 1])) << 16);
      *reinterpret_cast<uint4*>(o) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = f32_to_bf16(acc[i]);
    }
  } else {
    float* o = static_cast<float*>(p.out) + obase;
    if ((reinterpret_cast<uintptr_t>(o) & 15) == 0) {
      reinterpret_cast<float4*>(o)[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
      reinterpret_cast<float4*>(o)[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = acc[i];
    }
  }
  if (p.lse != nullptr && col == 0) p.lse[static_cast<int64_t>(b) * p.heads + h] = lse;
}

}  // namespace tpla
