// Streaming bf16 matrix-core split-K decode of one TPLA shard (gfx950).
//
// Same computation as decode_mfma.hip (per-shard attention of the absorbed
// query slice plus the whole rope query over the shard's cached rows, value
// = the latent slice, the shard's own softmax; TPLA abstract, edgentiq blog
// "How TPLA Works"), organised to stream the cache at HBM speed.  It needs
// block_size % 64 == 0, so every 64-token tile is one contiguous run of
// 64 * (d_s + d_r) * 2 bytes inside a single page.
//
// * Tiles go from HBM straight into LDS with global_load_lds_dwordx4 (no
//   register staging); three LDS stages keep two tiles in flight while the
//   third is consumed.  A wave waits only for its own oldest copies
//   (s_waitcnt vmcnt) and one barrier per tile publishes the tile.
// * LDS layout: 16-byte chunk c of tile row r sits at chunk position
//   (c & ~7) | ((c & 7) ^ swz(r)) of the row (rows unpadded).  With rows of
//   40 (d_s=256, d_r=64) or 24 (d_s=128, d_r=64) chunks this makes both
//   access patterns conflict-free on 32- and 64-bank LDS: the QK^T
//   A-fragment reads (16 rows x one chunk per 16 lanes) and the transposed
//   V reads (4 rows x 4 chunks per 32 lanes).
// * S^T = K . Q^T and O^T += V^T . P^T on v_mfma_f32_32x32x16_bf16 exactly as
//   in decode_mfma.hip; the V^T A-fragment is two ds_read_b64_tr_b16 (each
//   16-lane group reads a 4-token x 16-column block and receives it
//   transposed: lane i gets column i of the 4 rows).
// * Softmax in base 2 with the raw v_exp_f32, lazy rescaling (the running
//   max only moves when a tile max exceeds it by more than 64, so P < 2^64
//   in float32/bf16), P rounded to bf16 by v_cvt_pk_bf16_f32.
// * Work units (sequence, head group, split) are laid out so that the units
//   of one sequence land on one XCD (workgroup n runs on XCD n % 8), which
//   keeps that sequence's split partials in one L2 for the merge.
#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kTile = 64;
constexpr int kStages = 3;
constexpr float kRescale = 64.0f;   // log2 units: P stays below 2^64
constexpr float kLn2 = 0.69314718055994531f;

// XOR pattern of tile row r (only r's low 4 bits matter):
// bit2 = r1, bit1 = r0 ^ r3, bit0 = r2.
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}

// Wait until at most N of this wave's vector-memory operations (the LDS
// copies) are outstanding and all its LDS operations are done.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without a memory fence (the waits above order the LDS
// traffic); the empty asm statements stop the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int NW, int DS, int DR, int OCC>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(OCC, OCC)))
void decode_stream_kernel(DecodeParams p, int n_units, int units_per_xcd) {
  constexpr int D = DS + DR;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int SLOTS = kTile * CPR;        // chunks per tile
  constexpr int NT = NW * 64;
  constexpr int IPT = SLOTS / NT;           // LDS copies per thread per tile
  constexpr int KS = D / 16;
  constexpr int MT = DS / 32;
  static_assert(SLOTS % NT == 0, "tile must split evenly over the workgroup");
  static_assert(CPR % 8 == 0 && DS % 32 == 0 && DR % 16 == 0, "shape");

  __shared__ __attribute__((aligned(1024))) uint4 tiles[kStages][SLOTS];

  // ---- work unit (XCD-aware) ----
  const int n = blockIdx.x;
  const int u = (n & 7) * units_per_xcd + (n >> 3);
  if (u >= n_units) return;
  const int S = p.num_splits;
  const int HG = p.heads / (32 * NW);
  const int split = u % S;
  const int bh = u / S;
  const int hg = bh % HG;
  const int b = bh / HG;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int head = hg * (32 * NW) + wave * 32 + l31;

  int L = p.seq_lens[b];
  L = max(0, min(L, min(p.max_seq_len, p.max_blocks * p.block_size)));
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);
  const int64_t wrow = (static_cast<int64_t>(split) * p.batch + b) * p.heads + head;
  if (t0 >= t1) {
    if (half == 0) p.ws_lse[wrow] = -INFINITY;
    return;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;

  // ---- query fragments (B operand of S^T): head `head`, k-slots ks*16 + 8*half ----
  bf16x8_t qf[KS];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.qls_b + head * p.qls_h;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qrs_b + head * p.qrs_h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * half;
      qf[ks] = *reinterpret_cast<const bf16x8_t*>((k < DS) ? (ql + k) : (qr + (k - DS)));
    }
  }

  // ---- per-lane copy offsets: chunk slot (i*NW + wave)*64 + lane of a tile ----
  int src_off[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int r = slot / CPR;
    const int pc = slot % CPR;
    const int c = (pc & ~7) | ((pc & 7) ^ swz(r));
    src_off[i] = r * D + c * 8;
  }

  const uint16_t* cache = static_cast<const uint16_t*>(p.cache);
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int bs = p.block_size;

  // Every call issues exactly IPT copies per wave (the vmcnt waits count on
  // it).  Rows past the end of the sequence copy the tile's row 0 instead
  // (in bounds and finite; their scores are masked to zero weight).  An
  // out-of-range block id reads the cache's first row: unspecified output,
  // no access outside the cache.
  auto issue = [&](int it, int buf) {
    const int tb = t0 + it * kTile;
    const int nvalid = min(kTile, t1 - tb);
    const int page = bt_row[tb / bs];
    const bool ok = page >= 0 && page < p.num_blocks;
    const uint16_t* base =
        ok ? cache + (static_cast<int64_t>(page) * bs + (tb % bs)) * D : cache;
    if (nvalid == kTile) {
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(base + src_off[i]),
            (lds_void_t*)(&tiles[buf][(i * NW + wave) * 64]), 16, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const int r = src_off[i] / D;
        const int off = (r < nvalid) ? src_off[i] : src_off[i] - r * D;
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(base + off),
            (lds_void_t*)(&tiles[buf][(i * NW + wave) * 64]), 16, 0, 0);
      }
    }
  };

  // ---- per-lane LDS read offsets (bytes) ----
  // QK^T A fragment: row l31 (+32*mt), logical chunk 2*ks + half.
  int qk_off[4];
  {
    const int g = half ^ swz(l31);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) qk_off[k2] = (l31 * CPR + ((2 * k2) ^ g)) * 16;
  }
  // V^T fragments: 16-lane group (cg, h), lane (k, q) of the group.
  int tr_off[2][2];
  {
    const int grp = lane >> 4, i16 = lane & 15;
    const int k = i16 >> 2, q = i16 & 3, cg = grp & 1, h = grp >> 1;
    const int x = 2 * cg + (q >> 1);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int sw = ((k >> 1) << 2) | (((k & 1) ^ s) << 1) | h;
#pragma unroll
      for (int par = 0; par < 2; ++par)
        tr_off[s][par] = ((8 * s + 4 * h + k) * CPR + ((4 * par + x) ^ sw)) * 16 + 8 * (q & 1);
    }
  }

  f32x16_t oacc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
  float m_run = -INFINITY;
  float l_part = 0.f;
  f32x16_t sacc[2];
  float mx = -INFINITY;

  // Stage tile `it` (wait for its copies, publish it, start tile it+2) and
  // compute its scores S^T = K_tile . Q^T into sacc, scaled to base 2 and
  // masked past the sequence end; mx = the tile max of this lane's head.
  auto scores = [&](int it) {
    if (it + 1 < ntiles) wait_vm<IPT>();
    else wait_vm<0>();
    barrier();
    if (it + 2 < ntiles) issue(it + 2, (it + 2) % kStages);
    const char* T = reinterpret_cast<const char*>(&tiles[it % kStages][0]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.f;
    // two independent accumulation chains (row tiles 0 and 1), k-steps in order
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            T + qk_off[ks & 3] + (mt * 32 * CPR + ((2 * ks) & ~7)) * 16);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
      }
    }
    const int tb = t0 + it * kTile;
    mx = -INFINITY;
    if (tb + kTile <= t1) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[mt][r] *= p.scale_log2;
          mx = fmaxf(mx, sacc[mt][r]);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = tb + mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float v = (tok < t1) ? sacc[mt][r] * p.scale_log2 : -INFINITY;
          sacc[mt][r] = v;
          mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  };

  // P = exp2(S - m_run) as bf16 B fragments, then O^T += V^T . P^T.
  auto accumulate = [&](int it) {
    const char* T = reinterpret_cast<const char*>(&tiles[it % kStages][0]);
    bf16x8_t pf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(sacc[j >> 1][8 * (j & 1) + i] - m_run);
        l_part += pv;
        pf[j][i] = static_cast<__bf16>(pv);
      }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cst = (16 * j * CPR + 8 * (m >> 1)) * 16;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(T + tr_off[0][m & 1] + cst));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(T + tr_off[1][m & 1] + cst));
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[m], 0, 0, 0);
      }
    }
  };

  issue(0, 0);
  if (ntiles > 1) issue(1, 1);

  // The running max m_run only moves when a tile max exceeds it by more than
  // kRescale; the rescale of the accumulators is kept out of the steady-state
  // loop (which then holds them in accumulation registers throughout).
  int it = 0;
  while (it < ntiles) {
    scores(it);
    if (__ballot(mx > m_run + kRescale) != 0ull) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][r] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }
    accumulate(it);
    ++it;
    for (; it < ntiles; ++it) {
      scores(it);
      if (__ballot(mx > m_run + kRescale) != 0ull) break;
      accumulate(it);
    }
  }

  // ---- split result: o = U / l, lse = m + log l (natural log) ----
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
  if (half == 0) p.ws_lse[wrow] = (m_run + __log2f(l_tot)) * kLn2;
}

template <int NW, int DS, int DR, int OCC>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  const int HG = p.heads / (32 * NW);
  const int n_units = p.num_splits * p.batch * HG;
  const int per_xcd = (n_units + 7) / 8;
  hipLaunchKernelGGL((decode_stream_kernel<NW, DS, DR, OCC>), dim3(8 * per_xcd), dim3(NW * 64), 0,
                     s, p, n_units, per_xcd);
  return hipGetLastError();
}

}  // namespace

bool decode_stream_supported(int heads, int d_s, int d_r, int block_size) {
  if (block_size % kTile != 0) return false;
  if (heads % 128 == 0) return d_s == 256 && d_r == 64;
  if (heads % 64 == 0) return (d_s == 128 && d_r == 64) || (d_s == 256 && d_r == 64);
  return false;
}

int decode_stream_groups_per_cu(int heads, int d_s, int d_r) {
  (void)d_r;
  if (heads % 128 == 0) return 1;
  return d_s == 128 ? 2 : 1;
}

hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t s) {
  if (p.heads % 128 == 0 && p.d_s == 256 && p.d_r == 64) return launch_t<4, 256, 64, 1>(p, s);
  if (p.heads % 64 == 0 && p.d_s == 128 && p.d_r == 64) return launch_t<2, 128, 64, 2>(p, s);
  if (p.heads % 64 == 0 && p.d_s == 256 && p.d_r == 64) return launch_t<2, 256, 64, 1>(p, s);
  return hipErrorNotSupported;
}

}  // namespace tpla
