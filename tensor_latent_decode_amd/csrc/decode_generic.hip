// Plain float32 split-K decode for shapes the matrix-core kernel does not
// cover (float32 caches, head counts or widths that are not multiples of
// 32/16).  Same math as the matrix-core kernel: per-shard scores over the
// latent slice plus the whole rope part, online softmax over 16-token
// tiles, value = the latent slice of the row (TPLA abstract: attention per
// shard on its slice; MLA caches only the latent).
//
// Grid: (split, sequence, head group of 8).  A 256-thread workgroup stages
// 16 cache rows and the group's queries in LDS as float32.
#include "tpla_internal.h"

namespace tpla {
namespace {

constexpr int kTT = 16;       // tokens per tile
constexpr int kHG = 8;        // heads per workgroup
constexpr int kMaxD = 1024;   // d_s + d_r limit

template <typename T>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeParams p) {
  extern __shared__ float smem[];
  const int D = p.d_s + p.d_r;
  float* kt = smem;                       // [kTT][D]
  float* qs = kt + kTT * D;               // [kHG][D]
  float* ob = qs + kHG * D;               // [kHG][d_s] running output
  float* sc = ob + kHG * p.d_s;           // [kHG][kTT] scores -> weights
  float* st = sc + kHG * kTT;             // [kHG][3]   m, l, alpha

  const int split = blockIdx.x, b = blockIdx.y;
  const int h0 = blockIdx.z * kHG;
  const int nh = min(kHG, p.heads - h0);
  const int tid = threadIdx.x;
  const T* cache = static_cast<const T*>(p.cache);
  const T* ql = static_cast<const T*>(p.q_latent);
  const T* qr = static_cast<const T*>(p.q_rope);

  int L = p.seq_lens[b];
  L = max(0, min(L, min(p.max_seq_len, p.max_blocks * p.block_size)));
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);
  const int64_t wbase = (static_cast<int64_t>(split) * p.batch + b) * p.heads;
  if (t0 >= t1) {
    if (tid < nh) p.ws_lse[wbase + h0 + tid] = -INFINITY;
    return;
  }

  for (int i = tid; i < nh * D; i += blockDim.x) {
    const int hh = i / D, k = i % D;
    const int h = h0 + hh;
    qs[i] = (k < p.d_s) ? Elem<T>::load(ql + b * p.qls_b + h * p.qls_h + k)
                        : Elem<T>::load(qr + b * p.qrs_b + h * p.qrs_h + (k - p.d_s));
  }
  for (int i = tid; i < nh * p.d_s; i += blockDim.x) ob[i] = 0.f;
  if (tid < nh) {
    st[tid * 3 + 0] = -INFINITY;
    st[tid * 3 + 1] = 0.f;
  }
  __syncthreads();

  for (int tb = t0; tb < t1; tb += kTT) {
    const int nt = min(kTT, t1 - tb);
    for (int i = tid; i < kTT * D; i += blockDim.x) {
      const int r = i / D, k = i % D;
      float v = 0.f;
      if (r < nt) {
        const int tok = tb + r;
        const int blk = p.block_table[static_cast<int64_t>(b) * p.max_blocks + tok / p.block_size];
        if (blk >= 0 && blk < p.num_blocks)
          v = Elem<T>::load(cache + (static_cast<int64_t>(blk) * p.block_size + tok % p.block_size) * D + k);
      }
      kt[i] = v;
    }
    __syncthreads();
    if (tid < kHG * kTT) {
      const int hh = tid / kTT, r = tid % kTT;
      float s = -INFINITY;
      if (hh < nh && r < nt) {
        float acc = 0.f;
        for (int k = 0; k < D; ++k) acc = fmaf(qs[hh * D + k], kt[r * D + k], acc);
        s = acc * p.scale_log2;
      }
      sc[tid] = s;
    }
    __syncthreads();
    if (tid < nh) {
      float mx = -INFINITY;
      for (int r = 0; r < kTT; ++r) mx = fmaxf(mx, sc[tid * kTT + r]);
      const float m_old = st[tid * 3 + 0];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = exp2f(m_old - m_new);
      float l = st[tid * 3 + 1] * alpha;
      for (int r = 0; r < kTT; ++r) {
        const float w = exp2f(sc[tid * kTT + r] - m_new);
        sc[tid * kTT + r] = w;
        l += w;
      }
      st[tid * 3 + 0] = m_new;
      st[tid * 3 + 1] = l;
      st[tid * 3 + 2] = alpha;
    }
    __syncthreads();
    for (int i = tid; i < nh * p.d_s; i += blockDim.x) {
      const int hh = i / p.d_s, k = i % p.d_s;
      float acc = ob[i] * st[hh * 3 + 2];
      for (int r = 0; r < nt; ++r) acc = fmaf(sc[hh * kTT + r], kt[r * D + k], acc);
      ob[i] = acc;
    }
    __syncthreads();
  }
  for (int i = tid; i < nh * p.d_s; i += blockDim.x) {
    const int hh = i / p.d_s, k = i % p.d_s;
    p.ws_o[(wbase + h0 + hh) * p.d_s + k] = ob[i] / st[hh * 3 + 1];
  }
  if (tid < nh) {
    p.ws_lse[wbase + h0 + tid] = (st[tid * 3 + 0] + log2f(st[tid * 3 + 1])) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_decode_generic(const DecodeParams& p, int is_bf16, hipStream_t s) {
  const int D = p.d_s + p.d_r;
  if (D > kMaxD) return hipErrorNotSupported;
  const size_t smem = sizeof(float) * (kTT * D + kHG * D + kHG * p.d_s + kHG * kTT + kHG * 3);
  dim3 grid(p.num_splits, p.batch, (p.heads + kHG - 1) / kHG);
  if (is_bf16) {
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, grid, dim3(256), smem, s, p);
  } else {
    hipLaunchKernelGGL(decode_generic_kernel<float>, grid, dim3(256), smem, s, p);
  }
  return hipGetLastError();
}

}  // namespace tpla
