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
#include "tpla_internal.h"

namespace tpla {
namespace {

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
  for (int m = 1; m < lanes_per_row; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float other = __shfl_xor(v[i], m, 64);
      v[i] = upper ? (other - v[i]) : (v[i] + other);
    }
  }
}

template <int E, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void hadamard_kernel(const TIn* __restrict__ x, int64_t xs,
                                                       TOut* __restrict__ y, int64_t ys,
                                                       int64_t rows, int n, float norm) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int lanes_per_row = n / E;                 // 64 when n >= 64, else n
  const int rows_per_wave = 64 / lanes_per_row;
  const int64_t row = wave * rows_per_wave + lane / lanes_per_row;
  const int e0 = (lane % lanes_per_row) * E;
  const bool active = row < rows;

  float v[E];
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = active ? Elem<TIn>::load(x + row * xs + e0 + i) : 0.f;
  fwht_row<E>(v, lane, lanes_per_row);
  if (active) {
#pragma unroll
    for (int i = 0; i < E; ++i) Elem<TOut>::store(y + row * ys + e0 + i, v[i] * norm);
  }
}

// Steps a1-a3 of a decode step in one launch (n >= 64: one wave per row).
// Waves [0, q_rows) rotate query rows; the next n_rows waves rotate a new
// token's latent row, optionally store it, and write its shard slices and
// its rope into the shard caches (paged, same rules as the append kernel).
// Dtypes are wave-uniform run-time flags.
__device__ __forceinline__ float ld(const void* p, int64_t i, bool bf16) {
  return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void st(void* p, int64_t i, float v, bool bf16) {
  if (bf16) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else static_cast<float*>(p)[i] = v;
}

template <int E>
__global__ __launch_bounds__(256) void rotate_append_kernel(RotateAppendParams p, float norm) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int e0 = lane * E;
  float v[E];
  if (wave < p.q_rows) {
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = ld(p.q, wave * p.qs + e0 + i, p.q_bf16);
    fwht_row<E>(v, lane, 64);
#pragma unroll
    for (int i = 0; i < E; ++i) st(p.q_out, wave * p.qos + e0 + i, v[i] * norm, p.q_out_bf16);
    return;
  }
  const int64_t t = wave - p.q_rows;
  if (t >= p.n_rows) return;
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] = ld(p.lat, t * p.ls + e0 + i, p.lat_bf16);
  fwht_row<E>(v, lane, 64);
#pragma unroll
  for (int i = 0; i < E; ++i) v[i] *= norm;
  if (p.lat_out != nullptr) {
#pragma unroll
    for (int i = 0; i < E; ++i) st(p.lat_out, t * p.los + e0 + i, v[i], p.lat_bf16);
  }
  const int b = p.row_seq[t];
  const int pos = p.row_pos[t];
  if (b < 0 || b >= p.batch || pos < 0) return;
  const int lb = pos / p.block_size;
  if (lb >= p.max_blocks) return;
  const int blk = p.bt[static_cast<int64_t>(b) * p.max_blocks + lb];
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

template <int E, typename TIn, typename TOut>
hipError_t launch_e(const void* x, int64_t xs, void* y, int64_t ys, int64_t rows, int n,
                    hipStream_t s) {
  const int lanes_per_row = n / E;
  const int64_t rows_per_wave = 64 / lanes_per_row;
  const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const float norm = 1.0f / sqrtf(static_cast<float>(n));
  hipLaunchKernelGGL((hadamard_kernel<E, TIn, TOut>), dim3(static_cast<unsigned>(blocks)),
                     dim3(256), 0, s, static_cast<const TIn*>(x), xs, static_cast<TOut*>(y), ys,
                     rows, n, norm);
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

hipError_t launch_rotate_append(const RotateAppendParams& p, int n, hipStream_t s) {
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
