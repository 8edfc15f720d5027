// Log-sum-exp merge of the token splits, and the on-device shard combine.
//
// Merge: each split s of sequence b produced, for every head, the attention
// output over its own tokens o_s (already divided by its own sum) and
// lse_s = log sum exp(scores).  The split results combine exactly:
//     LSE = log sum_s exp(lse_s),   o = sum_s exp(lse_s - LSE) * o_s.
// Splits without tokens carry lse_s = -inf and get weight 0.  o_s comes as
// float32 (generic kernels), or as fp16 h_s with a float scale per block of
// columns (o_s = scale * h_s; the streaming kernels).
//
// Combine: shard g owns latent columns g*d_s .. (g+1)*d_s, so summing the
// zero-padded shard outputs (the all-reduce of the TPLA abstract) places
// them side by side.
#include <type_traits>

#include "merge_item.h"
#include "tpla_internal.h"

namespace tpla {
namespace {

// Four consecutive columns of split s's float32 output for row bh.
__device__ __forceinline__ float4 load_part(const MergeParams& p, int s, int64_t bh, int col, int ncol,
                                            bool vec, int64_t stride_s) {
  const float* src = p.ws_o + (s * stride_s + bh) * p.d_s + col;
  if (vec) return *reinterpret_cast<const float4*>(src);
  return make_float4(src[0], ncol > 1 ? src[1] : 0.f, ncol > 2 ? src[2] : 0.f,
                     ncol > 3 ? src[3] : 0.f);
}

// One thread per (b, h, 4 consecutive columns); a wavefront covers 256
// columns of one or more (b, h) rows, so the lse reads are broadcasts and the
// partial reads are contiguous runs.  Splits are taken 16 at a time with a
// running max (all of a chunk's loads are in flight together); splits
// without tokens get weight 0 by a select (their workspace rows are read but
// never trusted).  Workgroup n handles items ((n % 8) * per_xcd + n / 8) *
// 256 ..., i.e. sequences are spread over the XCDs in the same order as the
// split-K kernel placed them.
template <bool kBf16Out>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p, int64_t n_items, int per_xcd) {
  const int n = blockIdx.x;
  const int64_t wg = static_cast<int64_t>(n & 7) * per_xcd + (n >> 3);
  const int64_t item = wg * 256 + threadIdx.x;
  if (item >= n_items) return;
  const int q4 = (p.d_s + 3) / 4;
  const int64_t bh = item / q4;
  const int col = static_cast<int>(item % q4) * 4;
  const int ncol = min(4, p.d_s - col);
  const bool vec = (p.d_s & 3) == 0;
  const int64_t stride_s = static_cast<int64_t>(p.batch) * p.heads;
  const float* lse_in = p.ws_lse + bh;
  const int b = static_cast<int>(bh / p.heads);
  const int h = static_cast<int>(bh % p.heads);
  const int64_t obase = b * p.out_sb + h * p.out_sh + col;
  // Online over chunks of 16 splits: every load of a chunk is issued before
  // any is used (one memory round trip for up to 16 splits).
  constexpr int kC = 16;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, tot = 0.f;
  for (int s0 = 0; s0 < p.splits; s0 += kC) {
    float l[kC];
    float4 v[kC];
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const int s = min(s0 + u, p.splits - 1);
      l[u] = lse_in[s * stride_s];
      v[u] = load_part(p, s, bh, col, ncol, vec, stride_s);
    }
    float cm = m;
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      if (s0 + u >= p.splits) l[u] = -INFINITY;
      cm = fmaxf(cm, l[u]);
    }
    if (cm == -INFINITY) continue;              // no tokens so far
    const float r = __expf(m - cm);             // 0 while m is still -inf
    tot *= r;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= r;
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const bool use = l[u] != -INFINITY;       // empty splits: weight 0, o never used
      const float w = use ? __expf(l[u] - cm) : 0.f;
      tot += w;
      acc[0] += use ? w * v[u].x : 0.f;
      acc[1] += use ? w * v[u].y : 0.f;
      acc[2] += use ? w * v[u].z : 0.f;
      acc[3] += use ? w * v[u].w : 0.f;
    }
    m = cm;
  }
  float lse = -INFINITY;
  if (m != -INFINITY) {
    const float inv = 1.0f / tot;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= inv;
    lse = m + __logf(tot);
  }
  const bool out_vec = vec && ((reinterpret_cast<uintptr_t>(static_cast<float*>(p.out) + obase) & 15) == 0);
  if (out_vec && !kBf16Out) {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= ncol) break;
      if (kBf16Out) static_cast<uint16_t*>(p.out)[obase + i] = f32_to_bf16(acc[i]);
      else static_cast<float*>(p.out)[obase + i] = acc[i];
    }
  }
  if (p.lse != nullptr && col == 0) p.lse[bh] = lse;
}

// fp16 split outputs (streaming kernels; d_s a multiple of blk_cols, which
// is a multiple of 8): one thread per (b, h, 8 consecutive columns) with
// 16-byte partial loads, up to 16 splits per memory round trip, as above.
// The split outputs of (split or unit) u hold [d_s / 8][heads][8] halves
// and scales [d_s / blk_cols][heads]; u = s * batch + b for uniform splits,
// or, with a unit table, sequence b owns units first_b .. first_b + n_b - 1.
// A wavefront takes 8 heads x 8 column blocks of one sequence, so it reads
// 128-byte runs (8 heads of one block) and writes runs of 8 blocks of one
// head.
template <bool kBf16Out, bool kUnits, int G, bool kShared>
__global__ __launch_bounds__(256) void merge16_kernel(MergeParams p, int64_t n_items, int per_xcd) {
  const int n = blockIdx.x;
  const int64_t wg = static_cast<int64_t>(n & 7) * per_xcd + (n >> 3);
  const int64_t tid = wg * 256 + threadIdx.x;
  const int64_t item = tid / G;                 // G lanes per item (a power of two dividing 256)
  const int g = static_cast<int>(tid % G);
  if (item >= n_items) return;                  // whole groups leave together
  const int o8 = p.d_s / 8;
  const int64_t per_seq = static_cast<int64_t>(o8) * p.heads;   // a multiple of 64
  // one sequence per wavefront, whose unit range comes by a scalar load
  const int b = __builtin_amdgcn_readfirstlane(static_cast<int>(item / per_seq));
  const int ri = static_cast<int>(item % per_seq);
  const int rest = ri >> 6;
  const int h = (rest % (p.heads / 8)) * 8 + (ri & 7);
  const int cb = (rest / (p.heads / 8)) * 8 + ((ri >> 3) & 7);
  MergePart r;
  if constexpr (kUnits) {
    // The sequence's units come from the unit table by a scalar load; the
    // lse, scale and split-output loads then share one round trip.  (Loading
    // the uniform map's range while the table is on its way gained nothing
    // on equal lengths and, being wasted on ragged ones, doubled the
    // traffic there.)
    typedef __attribute__((address_space(4))) const int32_t const_i32_t;
    const const_i32_t* e = (const const_i32_t*)(p.unit_table + 2 * static_cast<int64_t>(b));
    r = merge16_partial<kUnits, kShared>(p, b, h, cb, make_int2(e[0], e[1]), g, G);
  } else {
    r = merge16_partial<kUnits, kShared>(p, b, h, cb, make_int2(0, p.splits), g, G);
  }
  merge_lanes(r, G);
  if (g == 0) merge16_store<kBf16Out>(p, b, h, cb, r);
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

template <bool kBf16Out>
void launch_m(const MergeParams& p, int64_t n_items, int64_t per_xcd, hipStream_t s) {
  hipLaunchKernelGGL((merge_kernel<kBf16Out>), dim3(static_cast<unsigned>(8 * per_xcd)),
                     dim3(256), 0, s, p, n_items, static_cast<int>(per_xcd));
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  // fp16 split outputs: waves of 8 heads x 8 column blocks of one sequence
  if (p.blk_cols != 0) {
    if (p.blk_cols % 8 != 0 || p.d_s % p.blk_cols != 0 || p.heads % 8 != 0 || (p.d_s / 8) % 8 != 0)
      return hipErrorInvalidValue;
    const int64_t items = static_cast<int64_t>(p.batch) * p.heads * (p.d_s / 8);
    const bool units = p.unit_table != nullptr;
    // lanes per item: past 16 splits (two memory round trips for one lane)
    // about 8 splits per lane, so the item takes one round trip and more
    // waves are in flight.  Unit rows: their count per sequence is known
    // only on the device; the launch's average (max_units / batch) decides,
    // which is exact for uniform lengths and only a rate choice otherwise
    const int per_seq = units ? (p.splits + p.batch - 1) / p.batch : p.splits;
    int G = 1;
    if (per_seq > 16)
      while (G < 8 && G * 8 < per_seq) G *= 2;
    const int64_t per_xcd = ((items * G + 255) / 256 + 7) / 8;
    if (8 * per_xcd > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(8 * per_xcd));
    const int px = static_cast<int>(per_xcd);
    auto go = [&](auto units_c, auto g_c) {
      constexpr bool kU = decltype(units_c)::value;
      constexpr int kG = decltype(g_c)::value;
      if (p.out_bf16) hipLaunchKernelGGL((merge16_kernel<true, kU, kG, false>), grid, dim3(256), 0, s, p, items, px);
      else hipLaunchKernelGGL((merge16_kernel<false, kU, kG, false>), grid, dim3(256), 0, s, p, items, px);
    };
    // one lane per item with 64-column scale blocks: lse and scales shared
    // by shuffle
    auto go_shared = [&](auto units_c) {
      constexpr bool kU = decltype(units_c)::value;
      if (p.out_bf16) hipLaunchKernelGGL((merge16_kernel<true, kU, 1, true>), grid, dim3(256), 0, s, p, items, px);
      else hipLaunchKernelGGL((merge16_kernel<false, kU, 1, true>), grid, dim3(256), 0, s, p, items, px);
    };
    auto go_g = [&](auto units_c) {
      if (G == 1 && p.blk_cols % 64 == 0) go_shared(units_c);
      else if (G == 1) go(units_c, std::integral_constant<int, 1>());
      else if (G == 2) go(units_c, std::integral_constant<int, 2>());
      else if (G == 4) go(units_c, std::integral_constant<int, 4>());
      else go(units_c, std::integral_constant<int, 8>());
    };
    if (units) go_g(std::true_type());
    else go_g(std::false_type());
    return hipGetLastError();
  }
  if (p.unit_table != nullptr) return hipErrorInvalidValue;   // units come as fp16 only
  const int64_t n_items = static_cast<int64_t>(p.batch) * p.heads * ((p.d_s + 3) / 4);
  const int64_t wgs = (n_items + 255) / 256;
  const int64_t per_xcd = (wgs + 7) / 8;
  if (8 * per_xcd > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (p.out_bf16) launch_m<true>(p, n_items, per_xcd, s);
  else launch_m<false>(p, n_items, per_xcd, s);
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
