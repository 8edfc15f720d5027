// Streaming bf16 matrix-core split-K decode of one TPLA shard (gfx950).
//
// Same computation as decode_mfma.hip (per-shard attention of the absorbed
// query slice plus the whole rope query over the shard's cached rows, value
// = the latent slice, the shard's own softmax; TPLA abstract, edgentiq blog
// "How TPLA Works"), organised to stream the cache at HBM speed.  It needs
// block_size % 64 == 0, so every 64-token tile is one contiguous run of
// 64 * (d_s + d_r) * 2 bytes inside a single page.
//
// Per workgroup: one (token split, sequence, group of 32*NW heads); each of
// the NW wavefronts owns 32 heads.  Per 64-token tile:
//
//   S^T[token, head] = K_tile . Q^T      v_mfma_f32_32x32x16_bf16, A = K rows
//                                        from LDS, B = query kept in AGPRs
//   P = exp2(c*S - m_ref)                raw v_exp_f32, bf16 for the MFMA
//   O^T[lat, head]  += V^T . P^T         A = V^T fragments from LDS
//
// Data movement:
// * Tiles go from HBM straight into LDS with global_load_lds_dwordx4, issued
//   from inline assembly (the compiler would otherwise wait for every copy
//   in flight before each transposed LDS read) and waited for explicitly.
//   Two K buffers: tile i+2 is copied while tiles i and i+1 are in use.
// * K tile layout: 16-byte chunk c of row r sits at chunk position
//   (c & ~7) | ((c & 7) ^ swz(r)) of the row (rows unpadded), conflict-free
//   for the QK^T A-fragment reads (16 rows, one chunk, per 16 lanes) and for
//   the transposed reads (4 rows x 4 chunks per 32 lanes).
// * V^T: the MFMA A operand needs 8 consecutive tokens of one latent column
//   per lane.  Once per tile the workgroup converts the latent part with
//   ds_read_b64_tr_b16 (a 16-lane group reads a 4-token x 16-column block
//   and receives it transposed) and stores ready-made A fragments
//   [m-tile][k-step][lane] back to LDS; every wave then reads its PV
//   fragments with plain 16-byte loads.  Transposed reads run at about a
//   quarter of the 16-byte read rate, so each wave transposing the whole
//   tile would cost as much LDS time as the MFMAs.
// * Inside a step, S_{i+1} and PV_i are independent, so their MFMAs, LDS
//   reads and exponentials interleave within one wave.
// * Softmax against a fixed reference max (the split's first tile max), so
//   the accumulators are only ever touched by MFMAs.  If a later tile max
//   exceeds it by more than 64 (base 2), the split runs again with the
//   raised reference (P stays below 2^64).
// * Work units (sequence, head group, split) are laid out so that the units
//   of one sequence land on one XCD (workgroup n runs on XCD n % 8).
#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

// Scalar (constant address space) read of a wave-uniform int32: as a plain
// load it would be a vector load, and its wait would also wait for every
// tile copy in flight.
__device__ __forceinline__ int scalar_load(const int32_t* p) { return *(const const_i32_t*)p; }

constexpr int kTile = 64;
constexpr float kRescale = 64.0f;   // base-2 headroom of P above the reference
constexpr float kLn2 = 0.69314718055994531f;

// XOR pattern of tile row r (only r's low 4 bits matter):
// bit2 = r1, bit1 = r0 ^ r3, bit0 = r2.
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// One 16-byte global -> LDS copy per lane, to LDS address lds + 16*lane.
// `base` and `lds` are wave-uniform; `voff` is the lane's byte offset.
__device__ __forceinline__ void copy16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory");
}

// Wait until this wave has no tile copy in flight and its LDS operations
// are done.
__device__ __forceinline__ void wait_copies() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));   // vmcnt(0) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
}

// Workgroup barrier (only LDS is shared; the empty asm statements stop the
// compiler from moving memory accesses across it).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
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
  constexpr int IPT = SLOTS / NT;           // copies per thread per tile
  constexpr int KS = D / 16;
  constexpr int MT = DS / 32;               // 32-column latent tiles
  constexpr int MPW = MT / NW;              // latent tiles each wave transposes
  static_assert(SLOTS % NT == 0, "tile must split evenly over the workgroup");
  static_assert(CPR % 8 == 0 && DS % 32 == 0 && DR % 16 == 0, "shape");
  static_assert(MT % NW == 0, "latent tiles must split evenly over the waves");
  static_assert(NW * 4 <= SLOTS * 16, "flag space");

  __shared__ __attribute__((aligned(1024))) uint4 ktile[2][SLOTS];
  __shared__ __attribute__((aligned(1024))) uint4 vtile[2][MT * 4 * 64];

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

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int head = hg * (32 * NW) + wave * 32 + l31;

  int L = scalar_load(p.seq_lens + b);
  L = max(0, min(L, min(p.max_seq_len, p.max_blocks * p.block_size)));
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);
  const int64_t wrow = (static_cast<int64_t>(split) * p.batch + b) * p.heads + head;
  if (t0 >= t1) {
    if (half == 0) p.ws_lse[wrow] = -INFINITY;
    return;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  const int nfull = (t1 - t0) / kTile;

  // ---- query fragments (B operand of S^T), kept in AGPRs ----
  bf16x8_t qf[KS];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.qls_b + head * p.qls_h;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qrs_b + head * p.qrs_h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int k = ks * 16 + 8 * half;
      qf[ks] = *reinterpret_cast<const bf16x8_t*>((k < DS) ? (ql + k) : (qr + (k - DS)));
      asm volatile("" : "+a"(qf[ks]));
    }
  }

  // ---- tile copies: chunk slot (i*NW + wave)*64 + lane of a tile ----
  uint32_t src_off[IPT];   // byte offset of the lane's chunk within the tile
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int r = slot / CPR;
    const int pc = slot % CPR;
    const int c = (pc & ~7) | ((pc & 7) ^ swz(r));
    src_off[i] = static_cast<uint32_t>((r * D + c * 8) * 2);
  }
  const uint16_t* cache = static_cast<const uint16_t*>(p.cache);
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int bs = p.block_size;

  // Copy tile t into K buffer kb.  Rows past the split end copy the same
  // chunk of the tile's row 0 (in bounds and finite; their scores are
  // masked).  An out-of-range block id reads the cache's first rows:
  // unspecified output, no access outside the cache.
  auto copy_tile = [&](int t, int kb) {
    const int tb = t0 + t * kTile;
    const int nvalid = min(kTile, t1 - tb);
    const int page = scalar_load(bt_row + tb / bs);
    const bool ok = page >= 0 && page < p.num_blocks;
    const uint16_t* base = cache + (static_cast<int64_t>(ok ? page : 0) * bs + (tb % bs)) * D;
    const uint32_t lbase = lds_addr(&ktile[kb][0]);
    if (nvalid == kTile) {
#pragma unroll
      for (int i = 0; i < IPT; ++i)
        copy16(base, src_off[i], lbase + static_cast<uint32_t>((i * NW + wave) * 64 * 16));
    } else {
#pragma unroll
      for (int i = 0; i < IPT; ++i) {
        const uint32_t r = src_off[i] / (2 * D);
        const uint32_t off = (r < static_cast<uint32_t>(nvalid)) ? src_off[i] : src_off[i] - r * (2 * D);
        copy16(base, off, lbase + static_cast<uint32_t>((i * NW + wave) * 64 * 16));
      }
    }
  };

  // ---- LDS read offsets (bytes) ----
  // QK^T A fragment: row l31 (+32*mt), logical chunk 2*ks + half.
  int qk_off[4];
  {
    const int g = half ^ swz(l31);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) qk_off[k2] = (l31 * CPR + ((2 * k2) ^ g)) * 16;
  }
  // Transposed reads of the latent part: 16-lane group (cg, h), lane (k, q).
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
  float m_run = -INFINITY;   // reference max of the scaled (base-2) scores
  float l_part = 0.f;        // this lane's share of the row sum
  const float c = p.scale_log2;

  // Raw scores of the tile in K buffer kb: S^T = K . Q^T (two chains).
  auto qk = [&](int kb, f32x16_t (&sc)[2]) {
    const char* T = reinterpret_cast<const char*>(&ktile[kb][0]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[mt][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            T + qk_off[ks & 3] + (mt * 32 * CPR + ((2 * ks) & ~7)) * 16);
        sc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sc[mt], 0, 0, 0);
      }
    }
  };

  // V^T A fragments of the tile in K buffer kb -> V buffer vb.  This wave
  // converts latent tiles wave*MPW .. +MPW for all four k-steps; fragment
  // (m, j) of lane l sits at vtile[vb][(m*4 + j)*64 + l].
  auto transpose = [&](int kb, int vb) {
    const char* T = reinterpret_cast<const char*>(&ktile[kb][0]);
#pragma unroll
    for (int mm = 0; mm < MPW; ++mm) {
      const int m = wave * MPW + mm;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cst = (16 * j * CPR + 8 * (m >> 1)) * 16;
        const int par = mm & 1;   // MPW is even, so m & 1 == mm & 1
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(T + tr_off[0][par] + cst));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(T + tr_off[1][par] + cst));
        vtile[vb][(m * 4 + j) * 64 + lane] = __builtin_bit_cast(
            uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
  };

  // Tokens of a tile past the split end get score -inf (last tile only).
  auto mask = [&](int t, f32x16_t (&sc)[2]) {
    const int lim = t1 - (t0 + t * kTile) - 4 * half;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mt * 32 + 8 * (r >> 2) + (r & 3) >= lim) sc[mt][r] = -INFINITY;
  };

  // Scaled max of this lane's head over the tile (both lanes of the head).
  auto tile_max = [&](const f32x16_t (&sc)[2]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    return mx * c;
  };

  // P = exp2(c*S - m_run) rounded to bf16 (B fragments of the PV product).
  auto probs = [&](const f32x16_t (&sc)[2], bf16x8_t (&pf)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[j >> 1][8 * (j & 1) + i], c, -m_run));
        l_part += pv;
        pf[j][i] = static_cast<__bf16>(pv);
      }
  };

  // O^T += V^T . P^T with the fragments in V buffer vb.
  auto pv = [&](int vb, const bf16x8_t (&pf)[4]) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, vtile[vb][(m * 4 + j) * 64 + lane]);
        oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[j], oacc[m], 0, 0, 0);
      }
    }
  };

  // Pipeline (tile t in K buffer t % 2 and, once transposed, V buffer t % 2):
  //   step i:  barrier (tile i+1 copied, V^T of tile i complete; every wave
  //            is done with tile i-1's buffers)
  //            copy tile i+2 -> K buffer i % 2
  //            phase A: S_{i+1} from K buffer (i+1) % 2, interleaved with
  //                     this wave's share of its V^T -> V buffer (i+1) % 2
  //            phase B: PV_i from V buffer i % 2 with P_i, interleaved with
  //                     P_{i+1} = exp2(c*S_{i+1} - m_run), one score per MFMA
  //            wait for this wave's copies of tile i+2
  // The instruction order is written out and pinned with scheduling fences
  // (one wave per SIMD issues in order, so MFMA, LDS and VALU work only
  // overlap when interleaved in the stream): LDS reads run two to three
  // MFMAs ahead of their use.  Only the last tile can be partial; its step
  // is the one with `masked`.  A wave whose tile max passes the reference by
  // more than kRescale only notes it (m_seen); after the last tile the waves
  // compare notes and, if any overflowed, the split runs again.
  bf16x8_t pf[4];
  float m_seen;               // largest tile max that overflowed
  constexpr int NPV = MT * 4;               // PV MFMAs per tile
  constexpr int VPS = 32 / NPV;             // scores handled per PV MFMA
  static_assert(32 % NPV == 0 && MPW * 4 <= KS, "schedule shape");

  auto rd_k = [&](const char* T, int ks, int mt) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(T + qk_off[ks & 3] + (mt * 32 * CPR + ((2 * ks) & ~7)) * 16);
  };
  auto rd_tr = [&](const char* T, int f, int s) -> s16x4_t {
    const int mm = f >> 2, j = f & 3;
    const int m = wave * MPW + mm;
    const int cst = (16 * j * CPR + 8 * (m >> 1)) * 16;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(T + tr_off[s][mm & 1] + cst));
  };

  auto step = [&](int i, bool masked) {
    barrier();
    if (i + 2 < ntiles) copy_tile(i + 2, i & 1);
    const int nb = (i + 1) & 1;
    const char* T = reinterpret_cast<const char*>(&ktile[nb][0]);

    // ---- phase A: scores of tile i+1, V^T of tile i+1 ----
    // Query fragments and output accumulators stay in AGPRs throughout.
#pragma unroll
    for (int m = 0; m < MT; ++m) asm volatile("" : "+a"(oacc[m]));
    f32x16_t sc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[mt][r] = 0.f;
    bf16x8_t qa[4];
    qa[0] = rd_k(T, 0, 0);
    qa[1] = rd_k(T, 0, 1);
    qa[2] = rd_k(T, 1, 0);
    qa[3] = rd_k(T, 1, 1);
    s16x4_t tlo = rd_tr(T, 0, 0), thi = rd_tr(T, 0, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      sc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[(2 * ks) & 3], qf[ks], sc[0], 0, 0, 0);
      if (ks + 2 < KS) qa[(2 * ks) & 3] = rd_k(T, ks + 2, 0);
      sc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[(2 * ks + 1) & 3], qf[ks], sc[1], 0, 0, 0);
      if (ks + 2 < KS) qa[(2 * ks + 1) & 3] = rd_k(T, ks + 2, 1);
      if (ks < MPW * 4) {
        const int f = ks, m = wave * MPW + (f >> 2), j = f & 3;
        vtile[nb][(m * 4 + j) * 64 + lane] = __builtin_bit_cast(
            uint4, __builtin_shufflevector(tlo, thi, 0, 1, 2, 3, 4, 5, 6, 7));
        if (ks + 1 < MPW * 4) {
          tlo = rd_tr(T, ks + 1, 0);
          thi = rd_tr(T, ks + 1, 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- phase B: PV_i with P_i; P_{i+1} from the new scores ----
    const int vb = i & 1;
    const int lim = t1 - (t0 + (i + 1) * kTile) - 4 * half;
    // PV order: k-step j outermost, so consecutive MFMAs update different
    // accumulators.  Fragment (m, j) sits at vtile[vb][(m*4 + j)*64 + lane].
    auto frag = [&](int idx) -> bf16x8_t {
      const int m = idx % MT, j = idx / MT;
      return __builtin_bit_cast(bf16x8_t, vtile[vb][(m * 4 + j) * 64 + lane]);
    };
    bf16x8_t va[3];
    va[0] = frag(0);
    va[1] = frag(1);
    va[2] = frag(2);
    bf16x8_t pn[4];
    float mx = -INFINITY;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 0; idx < NPV; ++idx) {
      const int m = idx % MT, j = idx / MT;
      oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[idx % 3], pf[j], oacc[m], 0, 0, 0);
      if (idx + 3 < NPV) va[idx % 3] = frag(idx + 3);
#pragma unroll
      for (int e = 0; e < VPS; ++e) {
        const int v = idx * VPS + e;                 // score index: sc[v/16][v%16]
        float sv = sc[v >> 4][v & 15];
        if (masked) {
          const int row = (v >> 4) * 32 + 8 * ((v & 15) >> 2) + (v & 3);
          sv = (row >= lim) ? -INFINITY : sv;
        }
        mx = fmaxf(mx, sv);
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -m_run));
        l_part += pv;
        pn[v >> 3][v & 7] = static_cast<__bf16>(pv);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) pf[j] = pn[j];
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    if (mx > m_run + kRescale) m_seen = fmaxf(m_seen, mx);
    wait_copies();
  };

  bool first = true;
  while (true) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
    l_part = 0.f;
    m_seen = -INFINITY;
    copy_tile(0, 0);
    if (ntiles > 1) copy_tile(1, 1);
    wait_copies();
    barrier();
    {
      f32x16_t sc[2];
      qk(0, sc);
      transpose(0, 0);
      if (nfull == 0) mask(0, sc);
      const float mx0 = tile_max(sc);
      m_run = first ? mx0 : fmaxf(m_run, mx0);
      first = false;
      probs(sc, pf);
    }
    for (int i = 0; i + 1 < nfull; ++i) step(i, false);
    if (nfull >= 1 && nfull < ntiles) step(nfull - 1, true);
    barrier();
    pv((ntiles - 1) & 1, pf);
    // compare notes: one flag per wave in K buffer 0 (idle after the barrier)
    int* flags = reinterpret_cast<int*>(&ktile[0][0]);
    const bool over = __ballot(m_seen != -INFINITY) != 0ull;
    if (lane == 0) flags[wave] = over ? 1 : 0;
    barrier();
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= flags[w];
    if (!any) break;
    m_run = fmaxf(m_run, m_seen);
    barrier();   // every wave has read the flags before the buffers are refilled
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
  if (heads % 64 == 0) return d_s == 128 && d_r == 64;
  return false;
}

int decode_stream_groups_per_cu(int heads, int d_s, int d_r) {
  (void)d_r;
  (void)d_s;
  return heads % 128 == 0 ? 1 : 2;
}

hipError_t launch_decode_stream(const DecodeParams& p, hipStream_t s) {
  if (decode_latsplit_supported(p.heads, p.d_s, p.d_r, p.block_size)) return launch_decode_latsplit(p, s);
  if (p.heads % 128 == 0 && p.d_s == 256 && p.d_r == 64) return launch_t<4, 256, 64, 1>(p, s);
  if (p.heads % 64 == 0 && p.d_s == 128 && p.d_r == 64) return launch_t<2, 128, 64, 2>(p, s);
  return hipErrorNotSupported;
}

}  // namespace tpla
