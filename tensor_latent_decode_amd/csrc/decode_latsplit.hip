// Streaming bf16 matrix-core split-K decode of one TPLA shard (gfx950).
//
// Per-shard attention of the absorbed query slice plus the whole rope query
// over the shard's cached rows [latent slice || rope]; the value is the
// latent slice; the softmax is the shard's own (TPLA abstract; edgentiq
// blog, "How TPLA Works: Smart Slicing and Reparameterization").  Needs
// block_size % 64 == 0, so a 64-token tile is one contiguous run of
// 64 * (d_s + d_r) * 2 bytes inside one page.
//
// One workgroup of NW waves per (token split, sequence, group of 32*NW
// heads).  Per 64-token tile the work is divided two ways:
//
//   scores   wave w owns heads 32w .. 32w+31 of the group:
//            S^T[token, head] = K_tile . Q^T, then P = exp2(c*S - m_ref)
//   values   wave w owns latent columns 32*MPW*w .. +32*MPW, for every head
//            of the group: O^T[lat, head] += V^T . P^T
//
// all on v_mfma_f32_32x32x16_bf16.  The matrix cores wait on operand loads
// (about 30 cycles per KiB a wave moves from LDS into registers while MFMAs
// run), so the split is about moving few bytes per MFMA:
// * P^T fragments are exchanged through LDS (each wave writes its 32 heads,
//   4 KiB per tile) and each fragment feeds MPW value MFMAs.
// * V^T fragments come straight from the K tile by transposing LDS reads
//   (ds_read_b64_tr_b16).  In each group of 16 lanes, lane j receives
//   element j % 4 of the 8 bytes read by lanes 4k + j / 4, k = 0..3; lane
//   4k + q reads token row t_k, latent columns 4q .. 4q+3 of the group's 16,
//   so lane j gets four tokens of latent column j: half of a value A
//   fragment (row = latent column, k = 8 tokens).  The tokens are taken in
//   the order of the P^T fragments (16j + 8*(e/4) + 4h + e%4 for element e
//   of fragment j in lane half h), so no other reordering is needed.  Each
//   wave reads the fragments of its own MPW latent tiles while it scores the
//   tile and keeps them for the next step's values.
// * Tiles go from HBM straight into LDS (global_load_lds_dwordx4 from
//   inline assembly, waited for explicitly: the compiler would otherwise
//   wait for every copy in flight before each LDS read).  16-byte chunk c of
//   tile row r sits at chunk position (c & ~7) | ((c & 7) ^ swz(r)) of the
//   row, which keeps the score A-fragment reads (16 rows, one chunk, per 16
//   lanes) free of bank conflicts.  With three K buffers tile i+3 is copied
//   while tiles i+1 and i+2 are in use (a copy has a whole step to land);
//   with two, tile i+2 is copied during step i.  The copy instructions ride
//   on the score MFMAs: issued back to back they hold the wave for about as
//   long as the vector memory unit takes to accept them.
// * The block ids of the split's tiles go to an LDS table once; their loads
//   share the kernel's first memory round trip with the query and the
//   sequence length.
// * The P^T fragments are stored as soon as each is complete, and the
//   cross-half max uses v_permlane32_swap, so no LDS wait ends a step.
// * Softmax against a fixed reference max (the split's first tile max); a
//   later tile max more than 64 (base 2) above it makes the split run again
//   with the raised reference.  Accumulators are touched only by MFMAs.
// * Work units are spread so that the splits of a sequence share an XCD
//   (workgroup n runs on XCD n % 8).
#include <type_traits>

#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

// Scalar (constant address space) read of a wave-uniform int32.
__device__ __forceinline__ int scalar_load(const int32_t* p) { return *(const const_i32_t*)p; }

constexpr int kTile = 64;
constexpr int kMaxTiles = 1024;     // tiles per split (the host plans splits to fit)
constexpr float kRescale = 64.0f;
constexpr float kLn2 = 0.69314718055994531f;

// XOR pattern of tile row r: bit2 = r1, bit1 = r0 ^ r3, bit0 = r2.
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// One 16-byte global -> LDS copy per lane, to LDS address lds + 16*lane.
__device__ __forceinline__ void copy16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory");
}

__device__ __forceinline__ void wait_copies() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));   // vmcnt(0) lgkmcnt(0)
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposing LDS read (lane layout in the header).
__device__ __forceinline__ i16x4_t read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)const_cast<char*>(p)));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int NW, int DS, int DR, int NB>
__global__ __attribute__((amdgpu_flat_work_group_size(NW * 64, NW * 64),
                          amdgpu_waves_per_eu(1, 1)))
void decode_latsplit_kernel(DecodeParams p, int n_units, int units_per_xcd) {
  constexpr int D = DS + DR;
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int SLOTS = kTile * CPR;        // chunks per tile
  constexpr int NT = NW * 64;
  constexpr int IPT = SLOTS / NT;           // copies per thread per tile
  constexpr int KS = D / 16;                // k-steps of the score product
  constexpr int KL = DS / 16;               // ... of which latent
  constexpr int MT = DS / 32;               // 32-column latent tiles
  constexpr int MPW = MT / NW;              // latent tiles per wave (value product)
  constexpr int NPF = NW * 4;               // P^T fragments per tile: (head tile, k-step)
  constexpr int NPV = NPF * MPW;            // value MFMAs per wave per tile
  // The 32 exponentials of a lane are spread over the first kExpSlots value
  // MFMAs (slot s handles scores exp_lo(s) .. exp_lo(s+1)-1), so the last
  // P^T fragment is stored well before the step's barrier.
  constexpr int kExpSlots = NPV;
  auto exp_lo = [](int s) constexpr { return s >= kExpSlots ? 32 : (s * 32) / kExpSlots; };
  static_assert(SLOTS % NT == 0, "tile must split evenly over the workgroup");
  static_assert(CPR % 8 == 0 && DS % 64 == 0 && DR % 16 == 0, "shape");
  static_assert(MT % NW == 0 && MPW % 2 == 0, "latent tiles per wave");
  static_assert(((KL / 4) & (KL / 4 - 1)) == 0, "latent k-step groups must be a power of two");
  static_assert(NPV <= 32 && kExpSlots <= NPV && KS >= 4 * MPW, "schedule shape");
  // Tile copies: the first kCopyS ride on the score k-steps (one every
  // kCopyEveryS), any rest on the value MFMAs (one every kCopyEveryV).
  // Measured on the DeepSeek-V3 shard: all ten on the score k-steps is ~1-2%
  // faster than half and half.
  constexpr int kCopyS = IPT;
  constexpr int kCopyEveryS = KS / kCopyS;
  constexpr int kCopyEveryV = (IPT - kCopyS) > 0 ? NPF / (IPT - kCopyS) : NPF;
  static_assert(kCopyS * kCopyEveryS <= KS && (IPT - kCopyS) * kCopyEveryV <= NPF && IPT < 32,
                "copies per tile must fit the step");
  static_assert(kMaxTiles % NT == 0, "tile table fill");

  static_assert(NB == 2 || NB == 3, "K buffers");
  __shared__ __attribute__((aligned(1024))) uint4 ktile[NB][SLOTS];
  __shared__ __attribute__((aligned(1024))) uint4 ptile[2][NPF * 64];
  __shared__ uint32_t trow[kMaxTiles];   // first cache row of each tile / 64

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
  const int head0 = hg * (32 * NW);              // first head of the group
  const int head = head0 + wave * 32 + l31;      // this lane's score head

  // ---- k-step order: latent k-steps rotated so this wave's own latent
  // tiles (k-steps 2*MPW*wave ..) come first, then the rope k-steps ----
  const int rot4 = (MPW / 2) * wave;             // rotation in groups of 4 k-steps
  auto phys_ks = [&](int kk) -> int {
    return kk < KL ? (((kk >> 2) + rot4) & (KL / 4 - 1)) * 4 + (kk & 3) : kk;
  };

  // The first memory round trip carries everything that does not depend on
  // the sequence length: the block ids of the split's first two tiles
  // (index clamped into the table row; unused if the tile does not exist)
  // and the query fragments (B operand of S^T, in rotated k-step order).
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int bs = p.block_size;
  int pg[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
    pg[t] = scalar_load(bt_row + min((split * p.chunk + t * kTile) / bs, p.max_blocks - 1));
  bf16x8_t qf[KS];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.qls_b + head * p.qls_h;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qrs_b + head * p.qrs_h;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k = phys_ks(kk) * 16 + 8 * half;
      qf[kk] = *reinterpret_cast<const bf16x8_t*>((k < DS) ? (ql + k) : (qr + (k - DS)));
    }
  }
  // ... and the block ids of every tile the split may cover (one per
  // thread and pass), for the tile table the steps read.
  constexpr int kFill = kMaxTiles / NT;
  const int ctiles = p.chunk / kTile;
  int fpg[kFill];
#pragma unroll
  for (int k = 0; k < kFill; ++k) {
    const int t = k * NT + static_cast<int>(threadIdx.x);
    fpg[k] = t < ctiles ? bt_row[min((split * p.chunk + t * kTile) / bs, p.max_blocks - 1)] : 0;
  }
  int L = scalar_load(p.seq_lens + b);
  // One wait for all of it, before the branch on L, so the loads above are
  // issued together instead of after the length check.
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) asm volatile("" : : "v"(qf[kk]));
  if (p.scale_log2 < 0.f) {     // scores of -q with |scale| are the scores of q with scale
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      uint4 w = __builtin_bit_cast(uint4, qf[kk]);
      w.x ^= 0x80008000u; w.y ^= 0x80008000u; w.z ^= 0x80008000u; w.w ^= 0x80008000u;
      qf[kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
#pragma unroll
  for (int k = 0; k < kFill; ++k) asm volatile("" : : "v"(fpg[k]));
  asm volatile("" : : "s"(pg[0]), "s"(pg[1]), "s"(L));
  L = max(0, min(L, min(p.max_seq_len, p.max_blocks * p.block_size)));
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);
  const int64_t row0 = (static_cast<int64_t>(split) * p.batch + b) * p.heads;
  if (t0 >= t1) {
    if (half == 0) p.ws_lse[row0 + head] = -INFINITY;
    return;
  }
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  const int nfull = (t1 - t0) / kTile;

  // ---- tile copies: chunk slot (i*NW + wave)*64 + lane of a tile ----
  uint32_t src_off[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;
    const int r = slot / CPR;
    const int pc = slot % CPR;
    const int c = (pc & ~7) | ((pc & 7) ^ swz(r));
    src_off[i] = static_cast<uint32_t>((r * D + c * 8) * 2);
  }
  const uint16_t* cache = static_cast<const uint16_t*>(p.cache);
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

  // Copy of tile t into K buffer kb, issued one 16-byte chunk per lane at a
  // time.  Rows past the split end copy the same chunk of the tile's row 0
  // (finite; their scores are masked).  A tile past the split's last one
  // becomes a harmless re-read of the cache's first row (every copy slot
  // issues the same number of instructions, so the wait counts are fixed).
  struct CopyJob {
    const uint16_t* base;
    uint32_t lim;      // bytes of valid rows
    uint32_t lds;
  };
  auto make_job = [&](int t, int kb, uint32_t row64) -> CopyJob {
    CopyJob j;
    j.lds = lds_addr(&ktile[kb][0]);
    if (t < ntiles) {
      const int nvalid = min(kTile, t1 - (t0 + t * kTile));
      j.base = cache + static_cast<int64_t>(row64) * (kTile * D);
      j.lim = static_cast<uint32_t>(nvalid * 2 * D);
    } else {
      j.base = cache;
      j.lim = 0;
    }
    return j;
  };
  auto copy_chunk = [&](const CopyJob& j, int ci) {
    const uint32_t off = src_off[ci] < j.lim ? src_off[ci] : src_off[ci] % (2 * D);
    copy16(j.base, off, j.lds + static_cast<uint32_t>((ci * NW + wave) * 64 * 16));
  };
  auto copy_all = [&](const CopyJob& j) {
#pragma unroll
    for (int ci = 0; ci < IPT; ++ci) copy_chunk(j, ci);
  };
  // Wait until at most n tile copies of this wave are in flight.
  auto wait_vm = [&](auto n) {
    constexpr int N = decltype(n)::value;
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (7 << 4) | (0xF << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
  };

  // Score A fragment (rows 32*mt + l31, k-step phys_ks(kk)) of the tile at T.
  int qk_off[4];
  {
    const int g = half ^ swz(l31);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) qk_off[k2] = (l31 * CPR + ((2 * k2) ^ g)) * 16;
  }
  auto rd_k = [&](const char* T, int kk, int mt) -> bf16x8_t {
    const int grp = phys_ks(kk) >> 2;   // wave-uniform
    return *reinterpret_cast<const bf16x8_t*>(T + qk_off[kk & 3] + mt * 32 * CPR * 16 + grp * 128);
  };

  // Value A fragment (latent tile MPW*wave + mm, token k-step j) of the
  // tile at T: two transposing reads, token rows 16j + 4h + k and
  // 16j + 8 + 4h + k.  Byte offsets per (j, second read, latent tile odd).
  uint32_t tr_off[4][2][2];
  {
    const int trk = (lane & 15) >> 2, trq = lane & 3, trg = (lane >> 4) & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const int row = 16 * j + 8 * rr + 4 * half + trk;
#pragma unroll
        for (int mo = 0; mo < 2; ++mo)
          tr_off[j][rr][mo] = static_cast<uint32_t>(
              row * CPR * 16 + ((4 * mo + 2 * trg + (trq >> 1)) ^ swz(row)) * 16 + 8 * (trq & 1));
      }
  }
  auto rd_v = [&](const char* T, int mm, int j) -> bf16x8_t {
    const char* b = T + 128 * ((MPW / 2) * wave + (mm >> 1));
    const i16x4_t lo = read_tr(b + tr_off[j][0][mm & 1]);
    const i16x4_t hi = read_tr(b + tr_off[j][1][mm & 1]);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t oacc[MPW][NW];    // O^T tiles: latent tile MPW*wave + mm, head tile ht
  bf16x8_t vc[MPW][4];       // V^T fragments of the tile whose values are due
  float m_run = -INFINITY;   // reference max of the scaled (base-2) scores
  float l_part = 0.f;        // this lane's share of its head's row sum
  float m_seen;              // largest tile max that overflowed
  // The softmax below takes a tile's max before scaling, which needs a
  // positive scale: a negative one is carried by the query instead (its
  // fragments were negated at load, exactly), and a zero one becomes 2^-100,
  // which leaves every score's weight exactly 1 (masked ones stay -inf).
  const float c = p.scale_log2 == 0.f ? 0x1p-100f : fabsf(p.scale_log2);

  // Scores of the tile at T and the V^T fragments of this wave's latent
  // tiles; k-steps in rotated order with the A reads two k-steps ahead.
  auto scores = [&](const char* T, f32x16_t (&sc)[2], bf16x8_t (&vt)[MPW][4], const CopyJob* cj) {
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int ht = 0; ht < NW; ++ht) asm volatile("" : "+a"(oacc[m][ht]));
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[mt][r] = 0.f;
    bf16x8_t qa[4];
    qa[0] = rd_k(T, 0, 0);
    qa[1] = rd_k(T, 0, 1);
    qa[2] = rd_k(T, 1, 0);
    qa[3] = rd_k(T, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      sc[0] = mfma(qa[(2 * kk) & 3], qf[kk], sc[0]);
      if (kk + 2 < KS) qa[(2 * kk) & 3] = rd_k(T, kk + 2, 0);
      sc[1] = mfma(qa[(2 * kk + 1) & 3], qf[kk], sc[1]);
      if (kk + 2 < KS) qa[(2 * kk + 1) & 3] = rd_k(T, kk + 2, 1);
      if (kk < 4 * MPW) vt[kk >> 2][kk & 3] = rd_v(T, kk >> 2, kk & 3);
      if (cj != nullptr && kk % kCopyEveryS == 0 && kk / kCopyEveryS < kCopyS)
        copy_chunk(*cj, kk / kCopyEveryS);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // The other lane of this lane's head (lane l +- 32): one of the two swap
  // results is the lane's own value, the other its partner's.
  auto both_halves_max = [](float v) -> float {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto both_halves_sum = [](float v) -> float {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  // Scaled max of this lane's head over the tile (both lanes of the head).
  auto tile_max = [&](const f32x16_t (&sc)[2]) -> float {
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mt][r]);
    return both_halves_max(mx) * c;
  };

  // Score v of this lane (0..31): token row of the tile and its P^T slot.
  //   sc[v >> 4][v & 15] is row (v >> 4)*32 + 8*((v & 15) >> 2) + 4*half + (v & 3),
  //   and P^T fragment j = v >> 3, element v & 7.
  auto put_p = [&](uint4* dst, const bf16x8_t (&pn)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[(wave * 4 + j) * 64 + lane] = __builtin_bit_cast(uint4, pn[j]);
  };

  // Value product of the tile whose P^T is in ptile[pb] and V^T in vc,
  // with the exponentials of the next tile's scores sc interleaved (masked
  // rows >= lim get P = 0); the new P^T goes to pn.
  auto values = [&](int pb, const f32x16_t (&sc)[2], int lim, bool masked, uint4* pdst,
                    float& mx, const CopyJob& cj) {
    const uint4* P = &ptile[pb][0];
    bf16x8_t pn[4];
    auto frag = [&](int f) -> bf16x8_t {
      const int ht = f % NW, j = f / NW;
      return __builtin_bit_cast(bf16x8_t, P[(ht * 4 + j) * 64 + lane]);
    };
    bf16x8_t pa[3];
    pa[0] = frag(0);
    pa[1] = frag(1);
    pa[2] = frag(2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < NPF; ++f) {
      const int ht = f % NW, j = f / NW;
#pragma unroll
      for (int mm = 0; mm < MPW; ++mm) {
        oacc[mm][ht] = mfma(vc[mm][j], pa[f % 3], oacc[mm][ht]);
        const int slot = f * MPW + mm;
#pragma unroll
        for (int v = exp_lo(slot); v < exp_lo(slot + 1); ++v) {
          float sv = sc[v >> 4][v & 15];
          if (masked) {
            const int row = (v >> 4) * 32 + 8 * ((v & 15) >> 2) + (v & 3);
            sv = (row >= lim) ? -INFINITY : sv;
          }
          mx = fmaxf(mx, sv);
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -m_run));
          l_part += pv;
          pn[v >> 3][v & 7] = static_cast<__bf16>(pv);
          if ((v & 7) == 7) pdst[(wave * 4 + (v >> 3)) * 64 + lane] = __builtin_bit_cast(uint4, pn[v >> 3]);
        }
      }
      if (f + 3 < NPF) pa[f % 3] = frag(f + 3);
      if (f % kCopyEveryV == 1 && kCopyS + f / kCopyEveryV < IPT) copy_chunk(cj, kCopyS + f / kCopyEveryV);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Value product only (after the last tile).
  auto values_last = [&](int pb) {
    const uint4* P = &ptile[pb][0];
#pragma unroll
    for (int f = 0; f < NPF; ++f) {
      const int ht = f % NW, j = f / NW;
      const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, P[(ht * 4 + j) * 64 + lane]);
#pragma unroll
      for (int mm = 0; mm < MPW; ++mm) oacc[mm][ht] = mfma(vc[mm][j], pa, oacc[mm][ht]);
    }
  };

  // Pipeline (tile t in K buffer t % 3, its P^T in ptile[t % 2]):
  //   step i:  barrier (tile i+1 copied, P^T of tile i written by every
  //            wave; every wave is done with tile i's K buffer and with
  //            ptile[(i+1) % 2])
  //            scores of tile i+1 and its V^T (this wave's latent tiles),
  //            with the copy of tile i+3 -> K buffer i % 3 spread over it
  //            values of tile i, interleaved with P of tile i+1, whose
  //            fragments go to ptile[(i+1) % 2] as they complete
  //            wait for this wave's copies of tile i+2
  auto step = [&](int i, bool masked) {
    // The tile table read waits for this wave's LDS traffic, as the
    // barrier does anyway.
    const uint32_t row64 = __builtin_amdgcn_readfirstlane(trow[min(i + NB, ntiles - 1)]);
    const CopyJob cj = make_job(i + NB, i % NB, row64);
    barrier();
    const char* T = reinterpret_cast<const char*>(&ktile[(i + 1) % NB][0]);
    f32x16_t sc[2];
    bf16x8_t vn[MPW][4];
    scores(T, sc, vn, &cj);
    const int lim = t1 - (t0 + (i + 1) * kTile) - 4 * half;
    float mx = -INFINITY;
    values(i & 1, sc, lim, masked, &ptile[(i + 1) & 1][0], mx, cj);
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) vc[m][j] = vn[m][j];
    mx = both_halves_max(mx) * c;
    if (mx > m_run + kRescale) m_seen = fmaxf(m_seen, mx);
    // NB == 3: tile i+2 (copied during step i-1) must be in; NB == 2: tile
    // i+2, copied during this step.
    wait_vm(std::integral_constant<int, NB == 3 ? IPT : 0>());
  };

  // ---- prologue ----
  // The query has arrived (waited for above, before any tile copy was out,
  // so that wait covered nothing else).  Tiles 0 and 1 go out back to back;
  // tile 2's copies are spread over the first score product, which waits
  // for tile 0 only.  (Issuing more at once only holds the wave: every CU
  // starts at the same time and the copies queue behind each other.)
#pragma unroll
  for (int t = 0; t < 2; ++t) copy_all(make_job(t, t, t < ntiles ? tile_row(t, pg[t]) : 0u));
  // Table of tile rows for the steps.
#pragma unroll
  for (int k = 0; k < kFill; ++k) {
    const int t = k * NT + static_cast<int>(threadIdx.x);
    if (t < ntiles) trow[t] = tile_row(t, fpg[k]);
  }

  bool first = true;
  while (true) {
#pragma unroll
    for (int m = 0; m < MPW; ++m)
#pragma unroll
      for (int ht = 0; ht < NW; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[m][ht][r] = 0.f;
    l_part = 0.f;
    m_seen = -INFINITY;
    if (!first) {
#pragma unroll
      for (int t = 0; t < 2; ++t) copy_all(make_job(t, t, __builtin_amdgcn_readfirstlane(trow[min(t, ntiles - 1)])));
    }
    wait_vm(std::integral_constant<int, IPT>());       // tile 0
    barrier();
    {
      f32x16_t sc[2];
      if constexpr (NB == 3) {
        const CopyJob cj2 = make_job(2, 2, __builtin_amdgcn_readfirstlane(trow[min(2, ntiles - 1)]));
        scores(reinterpret_cast<const char*>(&ktile[0][0]), sc, vc, &cj2);
#pragma unroll
        for (int ci = kCopyS; ci < IPT; ++ci) copy_chunk(cj2, ci);
      } else {
        scores(reinterpret_cast<const char*>(&ktile[0][0]), sc, vc, nullptr);
      }
      if (nfull == 0) {
        const int lim = t1 - t0 - 4 * half;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (mt * 32 + 8 * (r >> 2) + (r & 3) >= lim) sc[mt][r] = -INFINITY;
      }
      const float mx0 = tile_max(sc);
      m_run = first ? mx0 : fmaxf(m_run, mx0);
      first = false;
      bf16x8_t pn[4];
#pragma unroll
      for (int v = 0; v < 32; ++v) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[v >> 4][v & 15], c, -m_run));
        l_part += pv;
        pn[v >> 3][v & 7] = static_cast<__bf16>(pv);
      }
      put_p(&ptile[0][0], pn);
    }
    wait_vm(std::integral_constant<int, NB == 3 ? IPT : 0>());   // tile 1 (step 0's barrier shares it)

    for (int i = 0; i + 1 < nfull; ++i) step(i, false);
    if (nfull >= 1 && nfull < ntiles) step(nfull - 1, true);
    wait_copies();   // the trailing re-reads land before any K buffer is reused
    barrier();
    values_last((ntiles - 1) & 1);
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
  // Row sums go through K buffer 1 (idle): the value tiles of a head live
  // in every wave, its sum in the wave that scored it.
  const float l_tot = both_halves_sum(l_part);
  float* lsum = reinterpret_cast<float*>(&ktile[1][0]);
  if (half == 0) {
    lsum[wave * 32 + l31] = l_tot;
    p.ws_lse[row0 + head] = (m_run + __log2f(l_tot)) * kLn2;
  }
  barrier();
  // Split outputs leave as fp16 with one float scale per (row, wave block
  // of 32*MPW columns): o = scale * h, |h| <= 1.  That halves the partial
  // traffic of the split merge at a rounding error below 2^-11 of the
  // block's largest value.  Split u = split * batch + b holds [DS / 8][heads]
  // [8] halves (one store instruction writes 8-byte halves of 16-byte
  // pieces of 32 consecutive heads: 512 contiguous bytes) and scales
  // [DS / (32*MPW)][heads].
  uint16_t* wh = reinterpret_cast<uint16_t*>(p.ws_o);
  float* wsc = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws_o) +
                                        fp16_partials_scale_offset(p.num_splits, p.batch, p.heads, DS));
#pragma unroll
  for (int ht = 0; ht < NW; ++ht) {
    const float inv_l = 1.0f / lsum[ht * 32 + l31];
    float amax = 0.f;
#pragma unroll
    for (int mm = 0; mm < MPW; ++mm)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(oacc[mm][ht][r]));
    amax = both_halves_max(amax);
    const float hs = amax > 0.f ? 1.0f / amax : 0.f;
    const int hh = head0 + ht * 32 + l31;
    const int64_t u = row0 / p.heads;           // split * batch + b
    uint16_t* dst = wh + (u * (DS / 8) + 4 * MPW * wave) * p.heads * 8 + static_cast<int64_t>(hh) * 8 + 4 * half;
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
        *reinterpret_cast<uint2*>(dst + static_cast<int64_t>(4 * mm + q) * p.heads * 8) = make_uint2(w[0], w[1]);
      }
    if (half == 0) wsc[(u * NW + wave) * p.heads + hh] = amax * inv_l;
  }
}

template <int NW, int DS, int DR, int NB>
hipError_t launch_t(const DecodeParams& p, hipStream_t s) {
  if (p.chunk > kMaxTiles * kTile) return hipErrorInvalidValue;
  const int HG = p.heads / (32 * NW);
  const int n_units = p.num_splits * p.batch * HG;
  const int per_xcd = (n_units + 7) / 8;
  hipLaunchKernelGGL((decode_latsplit_kernel<NW, DS, DR, NB>), dim3(8 * per_xcd), dim3(NW * 64), 0, s,
                     p, n_units, per_xcd);
  return hipGetLastError();
}

}  // namespace

int decode_latsplit_max_chunk() { return min(kMaxTiles * kTile, decode_mla_max_chunk()); }

int decode_latsplit_partial_block() { return 64; }

// Instantiated for 64-head groups with d_s = 128, d_r = 64 (two waves, two
// K buffers, two workgroups per CU).  128-head groups with d_s = 256 go to
// the kernel with separate score and value waves in decode_roles.hip.
// The 512-wide latent (plain MLA under tensor parallelism, or a one-shard
// TPLA) goes to the kernel in decode_mla.hip, which keeps the same split
// output format.
bool decode_latsplit_supported(int heads, int d_s, int d_r, int block_size) {
  if (decode_mla_supported(heads, d_s, d_r, block_size)) return true;
  if (block_size % kTile != 0 || d_r != 64) return false;
  if (heads % 128 == 0 && d_s == 256) return true;
  return heads % 64 == 0 && d_s == 128;
}

int decode_latsplit_groups_per_cu(int heads, int d_s) {
  return ((heads % 128 == 0 && d_s == 256) || d_s == 512) ? 1 : 2;
}

int decode_latsplit_heads_per_group(int heads, int d_s) {
  if (d_s == 512) return decode_mla_group_heads(heads);
  return (heads % 128 == 0 && d_s == 256) ? 128 : 64;
}

hipError_t launch_decode_latsplit(const DecodeParams& p, hipStream_t s) {
  if (!decode_latsplit_supported(p.heads, p.d_s, p.d_r, p.block_size)) return hipErrorNotSupported;
  if (decode_mla_supported(p.heads, p.d_s, p.d_r, p.block_size)) return launch_decode_mla(p, s);
  if (decode_roles_supported(p.heads, p.d_s, p.d_r, p.block_size)) return launch_decode_roles(p, s);
  return launch_t<2, 128, 64, 2>(p, s);
}

}  // namespace tpla
