// bf16 matrix-core split-K decode of one TPLA shard (gfx950).
//
// What it computes (TPLA abstract; edgentiq blog, "How TPLA Works"): for
// each sequence b and head h, attention of the absorbed query slice plus the
// rope query over every cached row of this shard, value = the row's latent
// slice, with this shard's own softmax.  All heads read the same cache rows
// (MQA-like sharing of the latent), so the per-tile work is two dense
// products that map onto the 32x32x16 bf16 MFMA:
//
//   S^T[token, head] = K_tile[token, 0:D] . Q^T[0:D, head]       (D = d_s + d_r)
//   O^T[lat,  head] += V^T[lat, token]  . P^T[token, head]       (V = K_tile[:, 0:d_s])
//
// Work decomposition: a workgroup owns one (token split, sequence, group of
// 32*NW heads); each of its NW wavefronts owns 32 heads and keeps their
// queries (as MFMA B fragments) and output accumulators in registers for
// the whole split.  Cache tiles of 64 tokens are streamed from HBM with
// 16-byte loads (a 64-row page is one contiguous run), staged through LDS
// (double buffered, one barrier per tile) and read by every wavefront.
//
// Register layouts (v_mfma_f32_32x32x16_bf16): lane l feeds row/column
// l % 32 and k-slots 8*(l/32) .. +8; accumulator register r of lane l holds
// row 8*(r/4) + 4*(l/32) + r%4, column l % 32.  With tokens as the S^T row
// index, lane l holds one head (l % 32) and 32 of the tile's 64 tokens; the
// other 32 are in lane l ^ 32, so the softmax max needs one cross-lane step
// and the row sum stays split until the end.  The probabilities of k-step j
// already sit in registers 8*(j%2) .. +8 of accumulator j/2, which is
// exactly a B fragment if the PV contraction visits the tile's tokens in
// the order {16j + 4*(l/32) + 0..3, 16j + 8 + 4*(l/32) + 0..3}; the V^T A
// fragment is gathered from LDS in that same order.
//
// Online softmax in base 2 (scores pre-multiplied by scale*log2 e).  The
// running max used for the exponentials only moves when a new tile max
// exceeds it by more than kRescale (2^8 headroom); then the accumulators
// are rescaled once.  Probabilities are rounded to bf16 for the PV product
// and the row sum adds the same rounded values.
#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;
constexpr float kRescale = 8.0f;
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ __bf16 bf16_from_bits(uint16_t b) {
  return __builtin_bit_cast(__bf16, b);
}

template <int NW, int DS, int DR>
__global__ __launch_bounds__(NW * 64, 1) void decode_mfma_kernel(DecodeParams p) {
  constexpr int D = DS + DR;
  constexpr int KS = D / 16;              // QK^T k-steps
  constexpr int RS = D + 8;               // LDS row stride (elements): +16 B breaks bank aliasing
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int CHUNKS = kTile * CPR;
  constexpr int CPT = (CHUNKS + NT - 1) / NT;
  constexpr int MT = DS / 32;             // PV output tiles

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][kTile * RS];

  const int split = blockIdx.x, b = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int head = blockIdx.z * (32 * NW) + wave * 32 + (lane & 31);
  const int half = lane >> 5;

  int L = p.seq_lens[b];
  L = max(0, min(L, min(p.max_seq_len, p.max_blocks * p.block_size)));
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);
  const int64_t wrow = (static_cast<int64_t>(split) * p.batch + b) * p.heads + head;
  if (t0 >= t1) {
    if (half == 0) p.ws_lse[wrow] = -INFINITY;
    return;
  }

  // Query fragments: k-slot block ks*16 + 8*half of this lane's head.
  bf16x8_t qf[KS];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.qls_b + head * p.qls_h;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qrs_b + head * p.qrs_h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * half;
      const uint16_t* src = (k < DS) ? (ql + k) : (qr + (k - DS));
      qf[ks] = *reinterpret_cast<const bf16x8_t*>(src);
    }
  }

  const uint16_t* cache = static_cast<const uint16_t*>(p.cache);
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int bs = p.block_size;

  uint4 stage[CPT];
  auto load_tile = [&](int tb) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NT;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (c < CHUNKS) {
        const int r = c / CPR, col = c % CPR;
        const int tok = tb + r;
        if (tok < t1) {
          const int blk = bt_row[tok / bs];
          if (blk >= 0 && blk < p.num_blocks) {
            const int64_t row = static_cast<int64_t>(blk) * bs + tok % bs;
            v = *reinterpret_cast<const uint4*>(cache + row * D + col * 8);
          }
        }
      }
      stage[i] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < CHUNKS) {
        const int r = c / CPR, col = c % CPR;
        *reinterpret_cast<uint4*>(&lds[buf][r * RS + col * 8]) = stage[i];
      }
    }
  };

  f32x16_t oacc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
  float m_run = -INFINITY;
  float l_part = 0.f;

  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  load_tile(t0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int tb = t0 + it * kTile;
    if (it + 1 < ntiles) load_tile(tb + kTile);
    const uint16_t* K = lds[buf];

    // S^T = K_tile . Q^T  (two 32-token row tiles)
    f32x16_t sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &K[(mt * 32 + (lane & 31)) * RS + ks * 16 + 8 * half]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
      }
    }

    // mask + tile max (this lane's 32 tokens, then its partner's)
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = tb + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float v = (tok < t1) ? sacc[mt][r] * p.scale_log2 : -INFINITY;
        sacc[mt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (__ballot(mx > m_run + kRescale) != 0ull) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }

    // P^T fragments (B operand of the PV product), rounded to bf16
    bf16x8_t pf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = exp2f(sacc[j >> 1][8 * (j & 1) + i] - m_run);
        const uint16_t pb = f32_to_bf16(pv);
        l_part += bf16_to_f32(pb);
        pf[j][i] = bf16_from_bits(pb);
      }

    // O^T += V^T . P^T ; V^T fragment gathered in the P token order
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const int col = m * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t a;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int tok = 16 * j + 4 * half + i + ((i >> 2) << 2);
          a[i] = bf16_from_bits(K[tok * RS + col]);
        }
        oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[m], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // finish: total row sum, normalise, write the split's partial result
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = 1.0f / l_tot;
  float* wo = p.ws_o + wrow * DS;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t v;
      v[0] = oacc[m][4 * q + 0] * inv;
      v[1] = oacc[m][4 * q + 1] * inv;
      v[2] = oacc[m][4 * q + 2] * inv;
      v[3] = oacc[m][4 * q + 3] * inv;
      *reinterpret_cast<f32x4_t*>(wo + m * 32 + 8 * q + 4 * half) = v;
    }
  if (half == 0) p.ws_lse[wrow] = (m_run + log2f(l_tot)) * kLn2;
}

template <int NW, int DS, int DR>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.num_splits, p.batch, p.heads / (32 * NW));
  hipLaunchKernelGGL((decode_mfma_kernel<NW, DS, DR>), grid, dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

int waves_for(int heads) {
  if (heads % 128 == 0) return 4;
  if (heads % 64 == 0) return 2;
  return 1;
}

}  // namespace

bool decode_mfma_supported(int heads, int d_s, int d_r) {
  if (heads % 32 != 0) return false;
  return (d_s == 256 && d_r == 64) || (d_s == 128 && d_r == 64) || (d_s == 256 && d_r == 0) ||
         (d_s == 128 && d_r == 0) || (d_s == 64 && d_r == 64) || (d_s == 64 && d_r == 0);
}

int decode_mfma_groups_per_cu(int heads, int d_s, int d_r) {
  (void)d_s;
  (void)d_r;
  const int nw = waves_for(heads);
  return nw == 4 ? 1 : (nw == 2 ? 2 : 4);
}

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t s) {
  const int nw = waves_for(p.heads);
#define TPLA_CASE(DS_, DR_)                                   \
  if (p.d_s == DS_ && p.d_r == DR_) {                         \
    if (nw == 4) return launch_t<4, DS_, DR_>(p, s);          \
    if (nw == 2) return launch_t<2, DS_, DR_>(p, s);          \
    return launch_t<1, DS_, DR_>(p, s);                       \
  }
  TPLA_CASE(256, 64)
  TPLA_CASE(128, 64)
  TPLA_CASE(64, 64)
  TPLA_CASE(256, 0)
  TPLA_CASE(128, 0)
  TPLA_CASE(64, 0)
#undef TPLA_CASE
  return hipErrorNotSupported;
}

}  // namespace tpla
