// Fast Walsh-Hadamard transform of latent rows: y = x . H_n / sqrt(n), and
// the same transform fused with the paged append of the new token's row.
//
// TPLA rotates the absorbed query and the latent with an orthogonal
// transform before slicing them across devices (TPLA abstract; edgentiq
// blog, section "How TPLA Works: Smart Slicing and Reparameterization").
// H_n is Sylvester's matrix in natural order.
//
// Layout: one 64-lane wavefront owns 64/n rows when n < 64 (one element per
// lane) or one row when n >= 64 (E = n/64 contiguous elements per lane).
// Butterflies with stride < E run inside a lane's registers; larger strides
// pair lane l with lane l ^ (stride/E) through cross-lane shuffles.  Every
// row is read once and written once (the op is bandwidth-trivial next to
// the decode; one launch handles every row).
#include <algorithm>

#include "tpla_internal.h"

namespace tpla {
namespace {

// Value of lane (lane ^ M) for the cross-lane butterflies: quad permutes
// (M = 1, 2) and a 16-lane row rotation (M = 8) through DPP, the 32-lane
// swizzle for M = 4.  M = 16 and 32 go through the half-swapping permutes in
// cross_butterfly below.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  if constexpr (M == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(x, 0x1F | (4 << 10)));
  if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));
  return v;
}

// One butterfly stage across lanes l and l ^ M: the lower lane keeps
// a + b, the upper lane b - a (a = own value, b = partner's), written as one
// fma with a sign of +-1 (exactly the rounded sum or difference).
template <int E, int M>
__device__ __forceinline__ void cross_butterfly(float (&v)[E], int lane) {
  const float sgn = (lane & M) ? -1.0f : 1.0f;
  if constexpr (M == 16 || M == 32) {
    // The swap leaves r[0] = the lower partner's value and r[1] = the upper
    // partner's value in both lanes of each pair.
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const uint32_t x = __float_as_uint(v[i]);
      float lo, hi;
      if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
      } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        lo = __uint_as_float(r[0]);
        hi = __uint_as_float(r[1]);
      }
      v[i] = fmaf(sgn, hi, lo);
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = fmaf(sgn, v[i], lane_xor<M>(v[i]));
  }
}

// Butterflies of one row held as E contiguous elements per lane, lanes_per_row
// lanes per row (strides below E inside the lane, larger strides across
// lanes).  Unnormalised; the same stage order everywhere, so every caller
// gets bit-identical results.
template <int E>
__device__ __forceinline__ void fwht_row(float (&v)[E], int lane, int lanes_per_row) {
#pragma unroll
  for (int h = 1; h < E; h <<= 1) {
#pragma unroll
    for (int i = 0; i < E; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  if (lanes_per_row > 1) cross_butterfly<E, 1>(v, lane);
  if (lanes_per_row > 2) cross_butterfly<E, 2>(v, lane);
  if (lanes_per_row > 4) cross_butterfly<E, 4>(v, lane);
  if (lanes_per_row > 8) cross_butterfly<E, 8>(v, lane);
  if (lanes_per_row > 16) cross_butterfly<E, 16>(v, lane);
  if (lanes_per_row > 32) cross_butterfly<E, 32>(v, lane);
}

// E consecutive elements of a row, moved in the widest aligned pieces (the
// caller guarantees alignment to min(16, E * sizeof(T)) bytes).
template <int E>
__device__ __forceinline__ void load_row(const uint16_t* p, float (&v)[E]) {
  if constexpr (E >= 8) {
#pragma unroll
    for (int c = 0; c < E / 8; ++c) {
      const uint4 w = reinterpret_cast<const uint4*>(p)[c];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * c + 2 * j] = __uint_as_float(u[j] << 16);
        v[8 * c + 2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
      }
    }
  } else if constexpr (E == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(w.x << 16);
    v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16);
    v[3] = __uint_as_float(w.y & 0xFFFF0000u);
  } else if constexpr (E == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = __uint_as_float(w << 16);
    v[1] = __uint_as_float(w & 0xFFFF0000u);
  } else {
    v[0] = bf16_to_f32(*p);
  }
}
template <int E>
__device__ __forceinline__ void load_row(const float* p, float (&v)[E]) {
  if constexpr (E >= 4) {
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      const float4 w = reinterpret_cast<const float4*>(p)[c];
      v[4 * c] = w.x;
      v[4 * c + 1] = w.y;
      v[4 * c + 2] = w.z;
      v[4 * c + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = p[i];
  }
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}
template <int E>
__device__ __forceinline__ void store_row(uint16_t* p, const float (&v)[E]) {
  if constexpr (E >= 8) {
#pragma unroll
    for (int c = 0; c < E / 8; ++c)
      reinterpret_cast<uint4*>(p)[c] =
          make_uint4(pack_bf16(v[8 * c], v[8 * c + 1]), pack_bf16(v[8 * c + 2], v[8 * c + 3]),
                     pack_bf16(v[8 * c + 4], v[8 * c + 5]), pack_bf16(v[8 * c + 6], v[8 * c + 7]));
  } else if constexpr (E == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
  } else if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16(v[0], v[1]);
  } else {
    *p = f32_to_bf16(v[0]);
  }
}
template <int E>
__device__ __forceinline__ void store_row(float* p, const float (&v)[E]) {
  if constexpr (E >= 4) {
#pragma unroll
    for (int c = 0; c < E / 4; ++c)
      reinterpret_cast<float4*>(p)[c] = make_float4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]);
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) p[i] = v[i];
  }
}

template <int E, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void hadamard_kernel(const TIn* __restrict__ x, int64_t xs,
                                                       TOut* __restrict__ y, int64_t ys,
                                                       int64_t rows, int n, float norm, bool vec) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int lanes_per_row = n / E;                 // 64 when n >= 64, else n
  const int rows_per_wave = 64 / lanes_per_row;
  const int64_t row = wave * rows_per_wave + lane / lanes_per_row;
  const int e0 = (lane % lanes_per_row) * E;
  const bool active = row < rows;

  float v[E];
  if (vec) {
    if (active) load_row<E>(x + row * xs + e0, v);
    else
#pragma unroll
      for (int i = 0; i < E; ++i) v[i] = 0.f;
  } else {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = active ? Elem<TIn>::load(x + row * xs + e0 + i) : 0.f;
  }
  fwht_row<E>(v, lane, lanes_per_row);
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] *= norm;
  if (active) {
    if (vec) {
      store_row<E>(y + row * ys + e0, v);
    } else {
#pragma unroll
      for (int i = 0; i < E; ++i) Elem<TOut>::store(y + row * ys + e0 + i, v[i]);
    }
  }
}

// Steps a1-a3 of a decode step in one launch (n >= 64: one wave per row).
// Waves [0, q_rows) rotate query rows; the next n_rows waves rotate a new
// token's latent row, optionally RMS-normalise it (whole row, or each d_s
// slice on its own: RMSNorm slicing, edgentiq blog "How TPLA Works"),
// optionally store it, and write its shard slices and its rope into the
// shard caches (paged, same rules as the append kernel).  Dtypes are
// wave-uniform run-time flags.
__device__ __forceinline__ float ld(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void st(void* p, int64_t i, float v, bool bf16) {
  if (bf16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else static_cast<float*>(p)[i] = v;
}

template <int E>
__device__ __forceinline__ void load_any(const void* p, int64_t i, bool bf16, bool vec, float (&v)[E]) {
  if (vec) {
    if (bf16) load_row<E>(static_cast<const uint16_t*>(p) + i, v);
    else load_row<E>(static_cast<const float*>(p) + i, v);
  } else {
#pragma unroll
    for (int k = 0; k < E; ++k) v[k] = ld(p, i + k, bf16);
  }
}
template <int E>
__device__ __forceinline__ void store_any(void* p, int64_t i, bool bf16, bool vec, const float (&v)[E]) {
  if (vec) {
    if (bf16) store_row<E>(static_cast<uint16_t*>(p) + i, v);
    else store_row<E>(static_cast<float*>(p) + i, v);
  } else {
#pragma unroll
    for (int k = 0; k < E; ++k) st(p, i + k, v[k], bf16);
  }
}

template <int E>
__global__ __launch_bounds__(256) void rotate_append_kernel(RotateAppendParams p, float norm) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int e0 = lane * E;
  float v[E];
  // New latent rows first: their page lookup is a chain of dependent loads,
  // which then overlaps the query rows instead of ending the launch.
  if (wave >= p.n_rows) {
    const int64_t qr = wave - p.n_rows;
    if (qr >= p.q_rows) return;
    load_any<E>(p.q, qr * p.qs + e0, p.q_bf16, p.q_vec, v);
    fwht_row<E>(v, lane, 64);
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] *= norm;
    store_any<E>(p.q_out, qr * p.qos + e0, p.q_out_bf16, p.q_vec, v);
    return;
  }
  const int64_t t = wave;
  // The row's page is looked up before the transform, so those dependent
  // loads overlap the row load and the butterflies.  Without caches the
  // row tables and the paging sizes are not given (they may be NULL / 0).
  int b = -1, pos = -1, blk = -1;
  if (p.n_caches > 0) {
    b = p.row_seq[t];
    pos = p.row_pos[t];
    const bool placed = b >= 0 && b < p.batch && pos >= 0 && pos / p.block_size < p.max_blocks;
    blk = placed ? p.bt[static_cast<int64_t>(b) * p.max_blocks + pos / p.block_size] : -1;
  }
  load_any<E>(p.lat, t * p.ls + e0, p.lat_bf16, p.lat_vec, v);
  fwht_row<E>(v, lane, 64);
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] *= norm;
  if (p.norm != TPLA_NORM_NONE) {
    // RMS over the whole row, or over this lane's d_s slice (d_s / E lanes,
    // a power of two): a butterfly sum, bit-identical in every lane.
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) ss = fmaf(v[i], v[i], ss);
    const int group = p.norm == TPLA_NORM_GLOBAL ? 64 : p.d_s / E;
    for (int m = 1; m < group; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / static_cast<float>(group * E) + p.norm_eps);
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] *= r;
  }
  if (p.lat_out != nullptr) store_any<E>(p.lat_out, t * p.los + e0, p.lat_bf16, p.lat_vec, v);
  if (blk < 0 || blk >= p.num_blocks) return;
  const int width = p.d_s + p.d_r;
  const int64_t row = (static_cast<int64_t>(blk) * p.block_size + pos % p.block_size) * width;
  for (int c = 0; c < p.n_caches; ++c) {
    void* cache = p.caches.p[c];
    const int c0 = (p.first_shard + c) * p.d_s;     // this shard's first latent column
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const int col = e0 + i - c0;
      if (col >= 0 && col < p.d_s) st(cache, row + col, v[i], p.cache_bf16);
    }
    for (int k = lane; k < p.d_r; k += 64) {
      if (p.lat_bf16 == p.cache_bf16) {     // same type: bits
        if (p.cache_bf16)
          static_cast<uint16_t*>(cache)[row + p.d_s + k] = static_cast<const uint16_t*>(p.rope)[t * p.rs + k];
        else
          static_cast<float*>(cache)[row + p.d_s + k] = static_cast<const float*>(p.rope)[t * p.rs + k];
      } else {
        st(cache, row + p.d_s + k, ld(p.rope, t * p.rs + k, p.lat_bf16), p.cache_bf16);
      }
    }
  }
}

// True when rows of `elem`-byte elements starting at p with `stride`
// elements between rows can move in pieces of min(16, E * elem) bytes.
inline bool row_aligned(const void* p, int64_t stride, int e, int elem) {
  const int64_t piece = std::min<int64_t>(16, static_cast<int64_t>(e) * elem);
  return reinterpret_cast<uintptr_t>(p) % piece == 0 && (stride * elem) % piece == 0;
}

template <int E, typename TIn, typename TOut>
hipError_t launch_e(const void* x, int64_t xs, void* y, int64_t ys, int64_t rows, int n,
                    hipStream_t s) {
  const int lanes_per_row = n / E;
  const int64_t rows_per_wave = 64 / lanes_per_row;
  const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float norm = 1.0f / sqrtf(static_cast<float>(n));
  const bool vec = row_aligned(x, xs, E, sizeof(TIn)) && row_aligned(y, ys, E, sizeof(TOut));
  hipLaunchKernelGGL((hadamard_kernel<E, TIn, TOut>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, static_cast<const TIn*>(x), xs, static_cast<TOut*>(y), ys,
                     rows, n, norm, vec);
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t dispatch(const void* x, int64_t xs, void* y, int64_t ys, int64_t rows, int n,
                    hipStream_t s) {
  switch (n <= 64 ? 1 : n / 64) {
    case 1: return launch_e<1, TIn, TOut>(x, xs, y, ys, rows, n, s);
    case 2: return launch_e<2, TIn, TOut>(x, xs, y, ys, rows, n, s);
    case 4: return launch_e<4, TIn, TOut>(x, xs, y, ys, rows, n, s);
    case 8: return launch_e<8, TIn, TOut>(x, xs, y, ys, rows, n, s);
    case 16: return launch_e<16, TIn, TOut>(x, xs, y, ys, rows, n, s);
    case 32: return launch_e<32, TIn, TOut>(x, xs, y, ys, rows, n, s);
    case 64: return launch_e<64, TIn, TOut>(x, xs, y, ys, rows, n, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_rotate_append(const RotateAppendParams& params, int n, hipStream_t s) {
  RotateAppendParams p = params;
  const int e = n / 64;
  p.q_vec = p.q_rows > 0 && row_aligned(p.q, p.qs, e, p.q_bf16 ? 2 : 4) &&
            row_aligned(p.q_out, p.qos, e, p.q_out_bf16 ? 2 : 4);
  p.lat_vec = p.n_rows > 0 && row_aligned(p.lat, p.ls, e, p.lat_bf16 ? 2 : 4) &&
              (p.lat_out == nullptr || row_aligned(p.lat_out, p.los, e, p.lat_bf16 ? 2 : 4));
  const int64_t waves = p.q_rows + p.n_rows;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float norm = 1.0f / sqrtf(static_cast<float>(n));
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (n / 64) {
    case 1: hipLaunchKernelGGL(rotate_append_kernel<1>, grid, block, 0, s, p, norm); break;
    case 2: hipLaunchKernelGGL(rotate_append_kernel<2>, grid, block, 0, s, p, norm); break;
    case 4: hipLaunchKernelGGL(rotate_append_kernel<4>, grid, block, 0, s, p, norm); break;
    case 8: hipLaunchKernelGGL(rotate_append_kernel<8>, grid, block, 0, s, p, norm); break;
    case 16: hipLaunchKernelGGL(rotate_append_kernel<16>, grid, block, 0, s, p, norm); break;
    case 32: hipLaunchKernelGGL(rotate_append_kernel<32>, grid, block, 0, s, p, norm); break;
    case 64: hipLaunchKernelGGL(rotate_append_kernel<64>, grid, block, 0, s, p, norm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_hadamard(const void* x, int x_bf16, int64_t xs, void* y, int y_bf16,
                           int64_t ys, int64_t rows, int n, hipStream_t s) {
  if (x_bf16 && y_bf16) return dispatch<uint16_t, uint16_t>(x, xs, y, ys, rows, n, s);
  if (x_bf16) return dispatch<uint16_t, float>(x, xs, y, ys, rows, n, s);
  if (y_bf16) return dispatch<float, uint16_t>(x, xs, y, ys, rows, n, s);
  return dispatch<float, float>(x, xs, y, ys, rows, n, s);
}

}  // namespace tpla
