// Split-K decode of one TPLA shard on the matrix cores with separate score
// and value waves (gfx950): 128-head groups with latent slice d_s = 256, or
// 64-head groups with d_s = 128; rope 64.
//
// Per-shard attention of the absorbed query slice plus the whole rope query
// over the shard's cached rows [latent slice || rope]; the value is the
// latent slice; the softmax is the shard's own (TPLA abstract; edgentiq
// blog, "How TPLA Works: Smart Slicing and Reparameterization").
//
// One workgroup per (work unit, HG heads), one workgroup per CU.  A work
// unit is a token range of one sequence from the unit map of the lengths
// (unit_map.h): about one per CU, equal in tiles whatever the mix of
// lengths.  The waves take two roles:
//
//   score waves 0..NS-1   wave h owns heads 32h .. 32h+31 (NS = HG / 32):
//                         S^T[token, head] = K_tile . Q^T over d_s + d_r,
//                         then P = exp2(c*S - m_ref), stored to LDS as the
//                         B fragments of the value product (P^T)
//   value waves NS..NS+3  wave NS+q owns latent columns d_s/4 * q .. for all
//                         HG heads: O^T[lat, head] += V^T . P^T
//
// all on v_mfma_f32_32x32x16_bf16.  Waves w and w+4 share a SIMD, so with
// 128 heads each SIMD holds one wave of each role: the score wave's
// exponentials and LDS waits overlap the value wave's MFMAs and the other
// way round.  The query (KS fragments) lives only in the score waves and
// the output accumulators only in the value waves, which is what lets two
// waves share a SIMD's register file.
//
// Pipeline (tile t in K buffer t % NB, its P^T in ptile[t % 2]); one
// barrier per step.  Step i:
//   score waves   scores of tile i+1 (K fragments from LDS), exponentials,
//                 P^T of tile i+1 -> ptile[(i+1) % 2]
//   value waves   copy of tile i+NB -> K buffer i % NB (global -> LDS DMA),
//                 values of tile i (V^T fragments read during step i-1,
//                 P^T from ptile[i % 2]), V^T fragments of tile i+1 from
//                 K buffer (i+1) % NB, then wait for tile i+2
// so every copy has NB - 1 steps to land and NB - 2 tiles are in flight
// while one is read (NB = 3 for both shapes: 40 KiB tiles for 128 heads
// over 256 columns, 24 KiB tiles for 64 heads over 128 columns).
//
// * Tile rows in LDS: 16-byte chunk c of row r sits at (c & ~7) |
//   ((c & 7) ^ swz(r)), which keeps the score A-fragment reads (16 rows, one
//   chunk, per 16 lanes), the transposing V^T reads and the P^T reads free
//   of bank conflicts.
// * V^T fragments come straight from the K tile by transposing LDS reads
//   (ds_read_b64_tr_b16): in each group of 16 lanes, lane j receives
//   element j % 4 of the 8 bytes read by lanes 4k + j / 4, so lane 4k + q
//   reading token row t_k, columns 4q .. 4q+3 hands lane j four tokens of
//   column j, half of a value A fragment.  The tokens are taken in the order
//   of the P^T fragments (16j + 8*(e/4) + 4h + e%4 for element e of fragment
//   j in lane half h), so no other reordering is needed.
// * Softmax against a fixed reference (the unit's first tile max), with a
//   rerun if a later tile exceeds it by more than 2^64.
// * Split outputs in fp16 with a float scale per 64 columns.
// * Units are spread so that the pieces of a sequence share an XCD.
#include <type_traits>

#include "tpla_internal.h"
#include "unit_map.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int scalar_load(const int32_t* p) { return *(const const_i32_t*)p; }

using kTrue_t = std::integral_constant<bool, true>;
using kFalse_t = std::integral_constant<bool, false>;
constexpr kTrue_t kTrue{};
constexpr kFalse_t kFalse{};

constexpr int kTile = 64;
constexpr int kMaxTiles = 1024;     // tiles per unit (the LDS tile table; the unit map caps units)
constexpr float kRescaleSum = 0x1p64f;   // row sum that makes a split run again
constexpr float kLn2 = 0.69314718055994531f;

// XOR pattern of tile row r: bit2 = r1, bit1 = r0 ^ r3, bit0 = r2.
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer resource of a byte range starting at base: raw (stride 0), range
// checked per dword against nbytes.  Loads past the range return zeros.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(nbytes);
  r[3] = 0x00020000;
  return r;
}

// One 16-byte buffer -> LDS copy per lane, to LDS address lds + 16*lane
// (issued from inline assembly, so the compiler does not wait for it before
// every LDS read; the kernel counts the copies itself).
__device__ __forceinline__ void copy16(const i32x4_t& rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "memory");
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N tile copies of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ i16x4_t read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)const_cast<char*>(p)));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The other lane of this lane's head (lane l +- 32).
__device__ __forceinline__ float both_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float both_halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copy of one 64-token tile into a K buffer by the four waves of one role:
// 16-byte chunk slot (i*4 + cw)*64 + lane of the tile, chunk c of row r at
// position (c & ~7) | ((c & 7) ^ swz(r)).  The source is a range-checked
// buffer over the tile's valid rows, so rows past the split end (and whole
// tiles past its last one) arrive as zeros without a memory access: their
// scores are masked and their values weigh 0.  Every step issues the same
// number of copies, so the waits are fixed.
struct CopyJob {
  i32x4_t rsrc;
  uint32_t lds;
};

template <int HG, int DS, int DR, int NB, int KPRE, int PPRE, int PRIO_S, int PRIO_V, int kPro, bool kLate>
__global__ __attribute__((amdgpu_flat_work_group_size((HG / 32 + 4) * 64, (HG / 32 + 4) * 64),
                          amdgpu_waves_per_eu(2, 2)))
void decode_roles_kernel(DecodeParams p, int n_units, int units_per_xcd) {
  // HG heads per workgroup; NB K buffers (tile t in buffer t % NB, NB - 2
  // tiles in flight while one is read and one waits)
  constexpr int NS = HG / 32;               // score waves (one 32-head tile each)
  constexpr int NV = 4;                     // value waves
  constexpr int D = DS + DR;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int SLOTS = kTile * CPR;        // chunks per tile
  constexpr int IPT = SLOTS / (4 * 64);     // copies per lane per tile (four copying waves)
  constexpr int KS = D / 16;                // k-steps of the score product
  constexpr int MPW = DS / 32 / NV;         // 32-column latent tiles per value wave
  constexpr int NPF = NS * 4;               // P^T fragments per tile: (head tile, 16 tokens)
  constexpr int HF = NPF / 2;               // ... of tokens 0..31 (the rest: 32..63)
  static_assert((NS == 4 || NS == 2) && NV == 4, "two or four score waves, four value waves");
  static_assert(NB >= 2 && NB <= 6, "K buffers");
  static_assert(SLOTS % (4 * 64) == 0, "tile must split evenly over the copying waves");
  static_assert(CPR % 8 == 0 && DS % 64 == 0 && DR % 16 == 0, "shape");
  static_assert(MPW == 1 || MPW == 2, "value waves own one or two latent tiles");
  static_assert(IPT <= NPF && IPT <= 2 * KS && (NB - 1) * IPT < 64, "copies per step");
  static_assert(kMaxTiles % (NS * 64) == 0, "tile table fill");
  static_assert(KPRE >= 2 && KPRE <= 12 && PPRE >= 2 && PPRE <= HF, "prefetch depths");
  static_assert(kPro >= 1 && kPro <= NB, "tiles copied before the first barrier");
  // The 16 exponentials of one 32-token tile ride on one score chain of KS
  // k-steps: k-step kk takes exponentials exp_lo(kk) .. exp_lo(kk + 1) - 1.
  // The P^T fragments of tokens 32..63 of the previous tile are complete
  // after step kSignal of the tile's MFMA stream.
  auto exp_lo = [](int kk) constexpr { return KS >= 16 ? (kk < 16 ? kk : 16) : (kk * 16) / KS; };
  constexpr int kSignal = KS > 16 ? 16 : KS;

  __shared__ __attribute__((aligned(1024))) uint4 ktile[NB][SLOTS];
  __shared__ __attribute__((aligned(1024))) uint4 ptile[2][NPF * 64];
  __shared__ uint32_t trow[kMaxTiles];   // first cache row of each tile / 64
  __shared__ float lsum[HG];
  __shared__ int flags[NS];
  __shared__ int pcount;                 // tiles whose P^T fragments 2, 3 are in LDS (x NS)
  // with one latent tile per value wave, two waves share a 64-column scale
  // block: their block maxima meet here
  __shared__ float vmax[MPW == 1 ? NV : 1][MPW == 1 ? HG : 1];

  // ---- work unit ----
  // Launch slot n -> unit u (XCD-aware: consecutive units, the head groups
  // and token ranges of one sequence, share an XCD and its L2); u -> head
  // group and sequence unit su; su -> (sequence, tokens) from the unit map
  // of the lengths, which workgroup 0 also writes out for the merge.
  const int n = blockIdx.x;
  const int u = (n & 7) * units_per_xcd + (n >> 3);
  if (u >= n_units) return;
  const int HGS = p.heads / HG;
  const int hg = u % HGS;
  const int su = u / HGS;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int head0 = hg * HG;
  const bool is_score = wave < NS;

  WorkUnit wu;
  if (!find_unit(p, su, kMaxTiles, (n == 0 && wave == NS) ? p.unit_table : nullptr, &wu)) return;
  const int b = wu.b;
  const int t0 = wu.t0;
  const int t1 = wu.t1;                     // t0 < t1: a unit has tokens
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int bs = p.block_size;
  const int64_t row0 = static_cast<int64_t>(su) * p.heads;
  const uint16_t* cache = static_cast<const uint16_t*>(p.cache);

  // The softmax takes a tile's max before scaling, which needs a positive
  // scale: a negative one is carried by the query (its fragments are negated
  // at load, exactly), and a zero one becomes 2^-100, which leaves every
  // score's weight exactly 1 (masked ones stay -inf).
  const float c = p.scale_log2 == 0.f ? 0x1p-100f : fabsf(p.scale_log2);

  // First cache row of tile t, in units of 64 rows; an out-of-range block
  // id reads the cache's first rows (unspecified output, no access outside
  // the cache).
  auto tile_row = [&](int t, int page) -> uint32_t {
    const int tb = t0 + t * kTile;
    const bool ok = page >= 0 && page < p.num_blocks;
    return ok ? static_cast<uint32_t>(page) * static_cast<uint32_t>(bs / kTile) +
                    static_cast<uint32_t>((tb % bs) / kTile)
              : 0u;
  };
  // Source offsets of this lane's chunks when it is copying wave cw.
  auto copy_offsets = [&](int cw, uint32_t (&so)[IPT]) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int slot = (i * 4 + cw) * 64 + lane;
      const int r = slot / CPR;
      const int pc = slot % CPR;
      const int cc = (pc & ~7) | ((pc & 7) ^ swz(r));
      so[i] = static_cast<uint32_t>((r * D + cc * 8) * 2);
    }
  };
  auto make_job = [&](int t, int kb, uint32_t row64, int ntiles, int t1) -> CopyJob {
    CopyJob j;
    j.lds = lds_addr(&ktile[kb][0]);
    const int nvalid = t < ntiles ? min(kTile, t1 - (t0 + t * kTile)) : 0;
    j.rsrc = buffer_rsrc(cache + static_cast<int64_t>(t < ntiles ? row64 : 0u) * (kTile * D),
                         static_cast<uint32_t>(nvalid * 2 * D));
    return j;
  };
  const CopyJob none{buffer_rsrc(cache, 0u), 0u};
  auto copy_chunk = [&](const CopyJob& j, const uint32_t (&so)[IPT], int cw, int ci) {
    copy16(j.rsrc, so[ci], j.lds + static_cast<uint32_t>((ci * 4 + cw) * 64 * 16));
  };

  // ---- split outputs ----
  // fp16 with one float scale per (row, 64-column block): o = scale * h,
  // |h| <= 1, which halves the traffic of the split merge at a rounding
  // error below 2^-11 of the block's largest value.  The unit's rows are
  // laid out as the value waves hold them: [column / 8][head][8 columns],
  // so every store of a value wave writes 512 contiguous bytes straight
  // from its accumulators; scales are [column / 64][head].
  uint16_t* const part_h = reinterpret_cast<uint16_t*>(p.ws_o) + row0 * DS;
  float* const part_sc = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws_o) +
                                                  fp16_partials_scale_offset(p.max_units, 1, p.heads, DS)) +
                         row0 * (DS / 64);

  if (is_score) {
    // =====================================================================
    // Score waves
    // =====================================================================
    if constexpr (PRIO_S > 0) __builtin_amdgcn_s_setprio(PRIO_S);
    const int ht = wave;
    const int head = head0 + ht * 32 + l31;
    // First memory round trip after the unit map: the query fragments (B
    // operand of S^T) and the block ids of the unit's tiles (for the tile
    // table).
    bf16x8_t qf[KS];
    {
      const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.qls_b + head * p.qls_h;
      const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qrs_b + head * p.qrs_h;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int k = kk * 16 + 8 * half;
        qf[kk] = *reinterpret_cast<const bf16x8_t*>((k < DS) ? (ql + k) : (qr + (k - DS)));
      }
    }
    constexpr int kFill = kMaxTiles / (NS * 64);
    int fpg[kFill];
#pragma unroll
    for (int k = 0; k < kFill; ++k) {
      const int t = k * NS * 64 + static_cast<int>(threadIdx.x);
      fpg[k] = t < ntiles ? bt_row[min((t0 + t * kTile) / bs, p.max_blocks - 1)] : 0;
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) asm volatile("" : : "v"(qf[kk]));
#pragma unroll
    for (int k = 0; k < kFill; ++k) asm volatile("" : : "v"(fpg[k]));
    const int nfull = (t1 - t0) / kTile;
    if (p.scale_log2 < 0.f) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        uint4 w = __builtin_bit_cast(uint4, qf[kk]);
        w.x ^= 0x80008000u; w.y ^= 0x80008000u; w.z ^= 0x80008000u; w.w ^= 0x80008000u;
        qf[kk] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
#pragma unroll
    for (int k = 0; k < kFill; ++k) {
      const int t = k * NS * 64 + static_cast<int>(threadIdx.x);
      if (t < ntiles) trow[t] = tile_row(t, fpg[k]);
    }

    // Score A fragment (token rows 32*mt + l31, k-step kk) of the tile at T.
    int qk_off[4];
    {
      const int g = half ^ swz(l31);
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) qk_off[k2] = (l31 * CPR + ((2 * k2) ^ g)) * 16;
    }
    auto rd_k = [&](const char* T, int kk, int mt) -> bf16x8_t {
      return *reinterpret_cast<const bf16x8_t*>(T + qk_off[kk & 3] + mt * 32 * CPR * 16 + (kk >> 2) * 128);
    };

    float m_run = -INFINITY;   // reference max of the scaled (base-2) scores
    float l_part = 0.f;        // this lane's share of its head's row sum
    float m_raw;               // largest unscaled score of a careful pass (unmasked rows)
    f32x16_t sp;               // previous tile's token-tile-1 scores, exponentials pending
    const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    // Score v of a tile (0..31) in this lane: token tile v >> 4, register
    // v & 15, i.e. token row (v >> 4)*32 + 8*((v & 15) >> 2) + 4*half + (v & 3);
    // element v & 7 of P^T fragment v >> 3 (tokens 16j + 8*(e/4) + 4*half + e%4).
    auto row_of = [](int v) { return (v >> 4) * 32 + 8 * ((v & 15) >> 2) + (v & 3); };
    bf16x8_t pn[2];
    // Exponential of score v (value sv) of the tile whose P^T goes to pdst;
    // rows at or past lim are masked.  The row sum adds the bf16 weights the
    // value product uses, two at a time (dot product with (1, 1)).  A careful
    // pass also tracks the largest score.
    auto expo = [&](float sv, int v, uint4* pdst, int lim, auto masked_c, auto careful_c) {
      if (decltype(masked_c)::value) sv = (row_of(v) >= lim) ? -INFINITY : sv;
      if (decltype(careful_c)::value) m_raw = fmaxf(m_raw, sv);
      const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -m_run));
      pn[(v >> 3) & 1][v & 7] = static_cast<__bf16>(pv);
      if ((v & 1) == 1) {
        const bf16x2_t pr = {pn[(v >> 3) & 1][(v & 7) - 1], pn[(v >> 3) & 1][v & 7]};
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_part, false);
      }
      if ((v & 7) == 7) pdst[(ht * 4 + (v >> 3)) * 64 + lane] = __builtin_bit_cast(uint4, pn[(v >> 3) & 1]);
    };
    // P^T fragments 2 and 3 of a tile are in LDS: tell the value waves.
    auto signal = [&]() {
      if (lane == 0) __hip_atomic_fetch_add(&pcount, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    // Scores of tile t (at T) into sc[0], sc[1]: token tiles 0 and 1, one
    // chain each, K fragments read KPRE MFMAs ahead.  Every exponential
    // rides in this wave's own MFMA stream: token tile 1 of the previous
    // tile under chain 0 (then its P^T fragments 2, 3 are signalled), token
    // tile 0 of this tile under chain 1; this tile's token tile 1 stays
    // pending in sp.  The first tile of a pass sets the reference max
    // first.
    auto score_tile = [&](int t, auto first_c, auto masked_c, auto careful_c) {
      constexpr bool first = decltype(first_c)::value;
      constexpr bool masked = decltype(masked_c)::value;
      const char* T = reinterpret_cast<const char*>(&ktile[t % NB][0]);
      uint4* pcur = &ptile[t & 1][0];
      uint4* pprev = &ptile[(t + 1) & 1][0];
      const int lim = t1 - (t0 + t * kTile) - 4 * half;
      f32x16_t sc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[mt][r] = 0.f;
      bf16x8_t ka[KPRE];
#pragma unroll
      for (int s2 = 0; s2 < KPRE; ++s2) ka[s2] = rd_k(T, s2 % KS, s2 / KS);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n2 = 0; n2 < 2 * KS; ++n2) {
        const int mt = n2 / KS, kk = n2 % KS;
        sc[mt] = mfma(ka[n2 % KPRE], qf[kk], sc[mt]);
        if (n2 + KPRE < 2 * KS) ka[n2 % KPRE] = rd_k(T, (n2 + KPRE) % KS, (n2 + KPRE) / KS);
        if (!first && mt == 0) {
#pragma unroll
          for (int e = exp_lo(kk); e < exp_lo(kk + 1); ++e) expo(sp[e], 16 + e, pprev, 0, kFalse, careful_c);
        }
        if (!first && n2 == kSignal) signal();
        if (!first && mt == 1) {
#pragma unroll
          for (int e = exp_lo(kk); e < exp_lo(kk + 1); ++e) expo(sc[0][e], e, pcur, lim, masked_c, careful_c);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (first) {
        // reference: the max of the tile's (unmasked) scores
        float m0 = -INFINITY;
#pragma unroll
        for (int v = 0; v < 32; ++v) {
          float sv = sc[v >> 4][v & 15];
          if (masked) sv = (row_of(v) >= lim) ? -INFINITY : sv;
          m0 = fmaxf(m0, sv);
        }
        m0 = both_halves_max(m0) * c;
        m_run = fmaxf(m_run, m0);
#pragma unroll
        for (int v = 0; v < 16; ++v) expo(sc[0][v], v, pcur, lim, masked_c, careful_c);
      }
      sp = sc[1];
    };
    // Step t-1: score tile t (after barrier B_{t-1}).
    auto sstep = [&](int t, auto masked_c, auto careful_c) {
      barrier();                                  // B_{t-1}
      score_tile(t, kFalse, masked_c, careful_c);
    };
    // One pass over the split's tiles.
    auto pass = [&](auto careful_c) {
      if (nfull == 0) score_tile(0, kTrue, kTrue, careful_c);
      else score_tile(0, kTrue, kFalse, careful_c);
      // steps: tile t = i + 1 is scored after barrier B_i; only the last
      // tile can be partial
      for (int t = 1; t < nfull; ++t) sstep(t, kFalse, careful_c);
      if (nfull >= 1 && nfull < ntiles) sstep(nfull, kTrue, careful_c);
      // token tile 1 of the last tile
      const int t = ntiles - 1;
      const int lim = t1 - (t0 + t * kTile) - 4 * half;
      uint4* pl = &ptile[t & 1][0];
      if (nfull < ntiles) {
#pragma unroll
        for (int v = 16; v < 32; ++v) expo(sp[v - 16], v, pl, lim, kTrue, careful_c);
      } else {
#pragma unroll
        for (int v = 16; v < 32; ++v) expo(sp[v - 16], v, pl, lim, kFalse, careful_c);
      }
    };

    // Passes: a normal one; if a head's row sum passed 2^64 (a later score
    // far above the first tile's max) the split runs again with the
    // reference raised by log2 of that sum, after a careful pass that finds
    // the largest score if the sum overflowed float.
    bool careful = false;
    for (int npass = 0;; ++npass) {
      l_part = 0.f;
      m_raw = -INFINITY;
      if (wave == 0 && lane == 0) pcount = 0;
      barrier();                                  // B_a: tile 0 in, table written
      if (careful) pass(kTrue);
      else pass(kFalse);
      barrier();                                  // B_end
      const float l_tot = both_halves_sum(l_part);
      const bool lane_inf = l_tot == INFINITY;
      const bool lane_over = l_tot > kRescaleSum;   // false for NaN
      int code = __ballot(lane_over) != 0ull ? 1 : 0;
      if (!careful && __ballot(lane_inf) != 0ull) code = 2;
      if (npass >= 3) code = 0;                   // bounded: at most 4 passes
      if (lane == 0) flags[wave] = code;
      barrier();                                  // B_f
      int any = 0;
#pragma unroll
      for (int w = 0; w < NS; ++w) any |= flags[w];
      if (!any) break;
      if (careful) m_run = fmaxf(m_run, both_halves_max(m_raw) * c);
      else if (lane_over && !lane_inf) m_run += __log2f(l_tot);
      careful = !careful && (any & 2) != 0;
      barrier();                                  // B_r
    }
    // split result: lse = m + log l (natural log); l for the value waves
    const float l_tot = both_halves_sum(l_part);
    if (half == 0) {
      lsum[ht * 32 + l31] = l_tot;
      p.ws_lse[row0 + head] = (m_run + __log2f(l_tot)) * kLn2;
    }
    barrier();                                    // B_l
    return;
  }

  // =======================================================================
  // Value waves
  // =======================================================================
  if constexpr (PRIO_V > 0) __builtin_amdgcn_s_setprio(PRIO_V);
  const int lq = wave - NS;
  // block ids of tiles 0..NB-1 (scalar loads; index clamped into the table row)
  int pg[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t)
    pg[t] = scalar_load(bt_row + min((t0 + t * kTile) / bs, p.max_blocks - 1));
#pragma unroll
  for (int t = 0; t < NB; ++t) asm volatile("" : : "s"(pg[t]));
  uint32_t src_off[IPT];
  copy_offsets(lq, src_off);

  // Value A fragment (latent tile MPW*lq + mm, token k-step j) of the tile
  // at T: two transposing reads, token rows 16j + 4h + k and 16j + 8 + 4h + k
  // (the swizzle depends on the row's low four bits only, so j moves the
  // address by whole 16-row strides).  Chunk c of a row (8 columns) sits at
  // (c & ~7) | ((c & 7) ^ swz(row)).
  uint32_t tr_off[2][MPW];
  {
    const int trk = (lane & 15) >> 2, trq = lane & 3, trg = (lane >> 4) & 1;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 8 * rr + 4 * half + trk;
#pragma unroll
      for (int mo = 0; mo < MPW; ++mo) {
        const int cc = 4 * MPW * lq + 4 * mo + 2 * trg + (trq >> 1);
        tr_off[rr][mo] = static_cast<uint32_t>(row * CPR * 16 + ((cc & ~7) | ((cc & 7) ^ swz(row))) * 16 +
                                               8 * (trq & 1));
      }
    }
  }
  auto rd_v = [&](const char* T, int mm, int j) -> bf16x8_t {
    const i16x4_t lo = read_tr(T + tr_off[0][mm] + j * 16 * CPR * 16);
    const i16x4_t hi = read_tr(T + tr_off[1][mm] + j * 16 * CPR * 16);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t oacc[MPW][NS];    // O^T tiles: latent tile MPW*lq + mm, head tile ht
  bf16x8_t vc[MPW][4];       // V^T fragments of the tile whose values are due

  // Value product of the tile whose P^T is in ptile[pb] and V^T in vc.  In
  // a step (kStep) fragment (mm, j) of the next tile's V^T is read from T
  // into vc right after its last MFMA, and (kCopy) the copy cj is spread
  // over the MFMAs.  P^T fragments of tokens 0..31 (j = 0, 1) come first;
  // the score waves write those of tokens 32..63 during the step, so in a
  // step the second half waits until the count reaches target.
  auto values = [&](int pb, const char* T, const CopyJob& cj, int target, auto step_c, auto copy_c) {
    constexpr bool kStep = decltype(step_c)::value;
    constexpr bool kCopy = decltype(copy_c)::value;
    const uint4* P = &ptile[pb][0];
    auto frag = [&](int f) -> bf16x8_t {
      const int ht = f % NS, j = f / NS;
      return __builtin_bit_cast(bf16x8_t, P[(ht * 4 + j) * 64 + lane]);
    };
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (kStep && hf == 1) {
        for (int spin = 0; spin < (1 << 22); ++spin) {
          const int seen = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(&pcount, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
          if (seen >= target) break;
          __builtin_amdgcn_s_sleep(1);
        }
      }
      bf16x8_t pa[PPRE];
#pragma unroll
      for (int f = 0; f < PPRE; ++f) pa[f] = frag(HF * hf + f);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = HF * hf; f < HF * hf + HF; ++f) {
        const int ht = f % NS, j = f / NS;
        const int fl = f - HF * hf;
#pragma unroll
        for (int mm = 0; mm < MPW; ++mm) oacc[mm][ht] = mfma(vc[mm][j], pa[fl % PPRE], oacc[mm][ht]);
        if (fl + PPRE < HF) pa[fl % PPRE] = frag(f + PPRE);
        if (kStep && ht == NS - 1) {
#pragma unroll
          for (int mm = 0; mm < MPW; ++mm) vc[mm][j] = rd_v(T, mm, j);
        }
        if (kCopy) {
#pragma unroll
          for (int ci = 0; ci < IPT; ++ci)
            if ((kLate ? NPF / 2 + (ci * (NPF / 2)) / IPT : (ci * NPF) / IPT) == f) copy_chunk(cj, src_off, lq, ci);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  bool first = true;
  while (true) {
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int ht = 0; ht < NS; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][ht][r] = 0.f;
    // Tiles 0 .. kPro-1 go out before the first barrier, the rest of the
    // first NB after it: every CU starts at once, and the copies the memory
    // system holds when tile 0 is wanted delay it.
    auto copy_tile = [&](int t) {
      const uint32_t row64 = first ? (t < ntiles ? tile_row(t, pg[t]) : 0u)
                                   : __builtin_amdgcn_readfirstlane(trow[min(t, ntiles - 1)]);
      const CopyJob j = make_job(t, t, row64, ntiles, t1);
#pragma unroll
      for (int ci = 0; ci < IPT; ++ci) copy_chunk(j, src_off, lq, ci);
    };
#pragma unroll
    for (int t = 0; t < kPro; ++t) copy_tile(t);
    wait_vm<(kPro - 1) * IPT>();                  // tile 0
    barrier();                                    // B_a
#pragma unroll
    for (int t = kPro; t < NB; ++t) copy_tile(t);
    first = false;
#pragma unroll
    for (int k = 0; k < 4 * MPW; ++k) vc[k >> 2][k & 3] = rd_v(reinterpret_cast<const char*>(&ktile[0][0]), k >> 2, k & 3);
    wait_vm<(NB - 2) * IPT>();                    // tile 1
    for (int i = 0; i + 1 < ntiles; ++i) {
      // step i: values of tile i, V^T of tile i+1; unless the score waves
      // copy, also the copy of tile i+NB into the buffer of tile i.  The
      // tile table read waits for this wave's LDS traffic, as the barrier
      // does anyway.
      const uint32_t row64 = __builtin_amdgcn_readfirstlane(trow[min(i + NB, ntiles - 1)]);
      const CopyJob cj = make_job(i + NB, i % NB, row64, ntiles, t1);
      barrier();                                  // B_i
      const char* T = reinterpret_cast<const char*>(&ktile[(i + 1) % NB][0]);
      values(i & 1, T, cj, NS * (i + 1), kTrue, kTrue);
      wait_vm<(NB - 2) * IPT>();                  // tile i+2
    }
    wait_vm<0>();                                 // trailing copies land
    barrier();                                    // B_end
    {
      values((ntiles - 1) & 1, nullptr, none, 0, kFalse, kFalse);
    }
    barrier();                                    // B_f
    int any = 0;
#pragma unroll
    for (int w = 0; w < NS; ++w) any |= flags[w];
    if (!any) break;
    barrier();                                    // B_r
  }
  // this wave's columns of the split outputs, from the accumulators: fp16
  // of o / (block max) and the block's scale max / l, the row sums l from
  // the score waves after B_l.  A 64-column block is one value wave's
  // columns (MPW = 2) or two waves' (MPW = 1: their maxima meet in LDS
  // first).
  float amax_ht[NS];
  auto block_max = [&](int ht) -> float {
    float amax = 0.f;
#pragma unroll
    for (int mm = 0; mm < MPW; ++mm)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(oacc[mm][ht][r]));
    return both_halves_max(amax);
  };
  auto store_halves = [&](int ht) {
    const float amax = amax_ht[ht];
    const float hs = amax > 0.f ? 1.0f / amax : 0.f;
    const int head = head0 + ht * 32 + l31;
#pragma unroll
    for (int mm = 0; mm < MPW; ++mm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const _Float16 lo = static_cast<_Float16>(oacc[mm][ht][4 * q + 2 * k] * hs);
          const _Float16 hi = static_cast<_Float16>(oacc[mm][ht][4 * q + 2 * k + 1] * hs);
          w[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        // 8-column block of columns 32*MPW*lq + 32mm + 8q ..
        const int cb = 4 * MPW * lq + 4 * mm + q;
        // streaming stores: read once, by the merge, from memory
        const u32x2_t wv = {w[0], w[1]};
        __builtin_nontemporal_store(
            wv, reinterpret_cast<u32x2_t*>(part_h + (static_cast<int64_t>(cb) * p.heads + head) * 8 + 4 * half));
      }
  };
  if constexpr (MPW == 2) {
#pragma unroll
    for (int ht = 0; ht < NS; ++ht) {
      amax_ht[ht] = block_max(ht);
      store_halves(ht);
    }
    barrier();                                    // B_l: row sums in lsum
  } else {
#pragma unroll
    for (int ht = 0; ht < NS; ++ht) {
      amax_ht[ht] = block_max(ht);
      if (half == 0) vmax[lq][ht * 32 + l31] = amax_ht[ht];
    }
    barrier();                                    // B_l: row sums in lsum, block maxima in vmax
#pragma unroll
    for (int ht = 0; ht < NS; ++ht) {
      amax_ht[ht] = fmaxf(amax_ht[ht], vmax[lq ^ 1][ht * 32 + l31]);
      store_halves(ht);
    }
  }
  if (half == 0 && (MPW == 2 || (lq & 1) == 0)) {
#pragma unroll
    for (int ht = 0; ht < NS; ++ht)
      part_sc[(MPW * lq / 2) * p.heads + head0 + ht * 32 + l31] = amax_ht[ht] / lsum[ht * 32 + l31];
  }
}

// Launch of HG heads per workgroup with a d_s-wide latent slice, NB K
// buffers and the tuning T (LDS read distances of the K and P^T fragments,
// wave priorities of the two roles, tiles copied before the first barrier,
// and whether a step's tile copies ride on the second half of its value
// fragments instead of all of them).
template <int KPRE, int PPRE, int PRIO_S, int PRIO_V, int PRO, bool LATE>
struct Tuning {};

template <int HG, int DS, int NB, int KPRE, int PPRE, int PRIO_S, int PRIO_V, int PRO, bool LATE>
hipError_t launch_roles_t(const DecodeParams& p, hipStream_t s, Tuning<KPRE, PPRE, PRIO_S, PRIO_V, PRO, LATE>) {
  const int n_units = p.max_units * (p.heads / HG);
  const int per_xcd = (n_units + 7) / 8;
  hipLaunchKernelGGL((decode_roles_kernel<HG, DS, 64, NB, KPRE, PPRE, PRIO_S, PRIO_V, PRO, LATE>),
                     dim3(8 * per_xcd), dim3((HG / 32 + 4) * 64), 0, s, p, n_units, per_xcd);
  return hipGetLastError();
}

// 128 heads over 256 columns: 40 KiB tiles, three buffers.  Score waves at
// wave priority 1 (A/B on the DeepSeek-V3 shard).
using kTune128 = Tuning<4, 3, 1, 0, 2, false>;
// 64 heads over 128 columns: 24 KiB tiles, three buffers (A/B on the
// Kimi-K2 shard: two, three, four and five buffers 55.2, 46.6, 47.6 and
// 48.5 us per call: more tiles in flight stream slower), a step's copies
// on the second half of its value fragments (-0.5 us there; no gain on the
// 128-head shard, +0.8 us on the ragged one).
using kTune64 = Tuning<4, 3, 1, 0, 2, true>;
constexpr int kNB64 = 3;

}  // namespace

int decode_roles_max_tiles() { return kMaxTiles; }

bool decode_roles_supported(int heads, int d_s, int d_r, int block_size) {
  if (d_r != 64 || block_size % kTile != 0) return false;
  return (d_s == 256 && heads % 128 == 0) || (d_s == 128 && heads % 64 == 0);
}

int decode_roles_heads_per_group(int heads, int d_s) {
  (void)heads;
  return d_s == 256 ? 128 : 64;
}

hipError_t launch_decode_roles(const DecodeParams& p, hipStream_t s) {
  if (!decode_roles_supported(p.heads, p.d_s, p.d_r, p.block_size)) return hipErrorNotSupported;
  if (p.chunk > kMaxTiles * kTile || p.chunk % kTile != 0 || p.max_units < 1 ||
      (p.unit_target == 0 && p.chunk < kTile) || p.unit_table == nullptr)
    return hipErrorInvalidValue;
  if (p.d_s == 256) return launch_roles_t<128, 256, 3>(p, s, kTune128{});
  return launch_roles_t<64, 128, kNB64>(p, s, kTune64{});
}

}  // namespace tpla
