// Fast Walsh-Hadamard transform of latent rows: y = x . H_n / sqrt(n).
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

  // strides inside the lane
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
  // strides across lanes: lane bit m = h / E
  for (int m = 1; m < lanes_per_row; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float other = __shfl_xor(v[i], m, 64);
      v[i] = upper ? (other - v[i]) : (v[i] + other);
    }
  }
  if (active) {
#pragma unroll
    for (int i = 0; i < E; ++i) Elem<TOut>::store(y + row * ys + e0 + i, v[i] * norm);
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

hipError_t launch_hadamard(const void* x, int x_bf16, int64_t xs, void* y, int y_bf16,
                           int64_t ys, int64_t rows, int n, hipStream_t s) {
  if (x_bf16 && y_bf16) return dispatch<uint16_t, uint16_t>(x, xs, y, ys, rows, n, s);
  if (x_bf16) return dispatch<uint16_t, float>(x, xs, y, ys, rows, n, s);
  if (y_bf16) return dispatch<float, uint16_t>(x, xs, y, ys, rows, n, s);
  return dispatch<float, float>(x, xs, y, ys, rows, n, s);
}

}  // namespace tpla
