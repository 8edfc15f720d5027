// Streaming bf16 matrix-core split-K decode over a 512-wide latent with a
// 64-wide rope (gfx950): the shape of plain MLA under tensor parallelism,
// where every device keeps the whole latent for its share of the heads
// (TPLA abstract: plain MLA split by heads streams the entire latent cache
// on each device, the baseline TPLA is compared with).  It is also a TPLA
// "shard" at T = 1.
//
// One workgroup of four waves per (token split, sequence, group of 64, 32
// or 16 heads).  Tiles of 32 tokens (one contiguous run of 32 * 576 * 2
// bytes inside a page) go from HBM straight into LDS, three buffers deep.
// The group's NH head tiles of 32 (two for 64 heads, else one; a 16-head
// group fills half a tile) and KP = 4 / NH parts of the latent give the
// four waves: wave w takes head tile w % NH and latent part w / NH (512/KP
// columns and 64/KP of the rope columns):
//
//   scores   a partial S^T[token, head] over the wave's k-steps; the waves
//            of the other parts (same heads) add their partials through
//            LDS in a fixed butterfly order, so all of them hold the same
//            full scores and take the same softmax decisions
//   values   O^T[lat, head] += V^T . P^T for the wave's latent columns and
//            heads, V^T fragments straight from the K tile by transposing
//            LDS reads (ds_read_b64_tr_b16, lane layout below)
//
// all on v_mfma_f32_32x32x16_bf16; P^T never leaves the registers and one
// barrier per tile suffices.  The softmax runs against a fixed reference
// (the split's first tile max); a later tile max more than 64 (base 2)
// above it makes the split run again with the raised reference.  Split
// outputs leave as fp16 with one float scale per (row, 64 columns), the
// format the split merge reads.
#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;

constexpr int kT = 32;                 // tokens per tile
constexpr int kDS = 512, kDR = 64, kD = kDS + kDR;
constexpr int kCPR = kD / 8;           // 16-byte chunks per row (72)
constexpr int kSlots = kT * kCPR;      // chunks per tile (2304)
constexpr int kNT = 256;
constexpr int kIPT = kSlots / kNT;     // copies per thread per tile (9)
constexpr int kNB = 3;                 // K buffers
constexpr int kMaxTiles = 2048;        // tiles per split (the host plans splits to fit)
constexpr float kRescale = 64.0f;
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kSlots % kNT == 0, "tile must split evenly over the workgroup");

__device__ __forceinline__ int scalar_load(const int32_t* p) { return *(const const_i32_t*)p; }

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

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N tile copies of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (7 << 4) | (0xF << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// Transposing LDS read (lane layout described at its use).
__device__ __forceinline__ i16x4_t read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)const_cast<char*>(p)));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The other lane of this lane's head (lane l +- 32): one of the two swap
// results is the lane's own value, the other its partner's.
__device__ __forceinline__ float both_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float both_halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// NH head tiles of 32 per workgroup (1 or 2); the latent is cut into
// KP = 4 / NH parts, wave w = kp * NH + ht taking head tile ht and part kp.
// hv: heads of a group that exist (16 for a 16-head group: lanes 16..31 of
// the head tile repeat heads 0..15 and store nothing).
template <int NH>
__global__ __attribute__((amdgpu_flat_work_group_size(kNT, kNT), amdgpu_waves_per_eu(1, 1)))
void decode_mla_kernel(DecodeParams p, int n_units, int units_per_xcd, int hv) {
  constexpr int KP = 4 / NH;           // latent parts
  constexpr int LK = 32 / KP;          // latent k-steps per part
  constexpr int RK = 4 / KP;           // rope k-steps per part
  constexpr int kKW = LK + RK;         // score k-steps per wave
  constexpr int MTW = LK / 2;          // 32-column latent tiles per wave
  static_assert(NH == 1 || NH == 2, "head tiles per group");
  __shared__ __attribute__((aligned(1024))) uint4 ktile[kNB][kSlots];
  __shared__ __attribute__((aligned(16))) float4 part[2][4][4][64];   // [tile & 1][wave][r/4][lane]
  __shared__ uint32_t trow[kMaxTiles];   // first cache row of each tile / 32
  __shared__ int over_flag[4];

  // ---- work unit (XCD-aware: the splits of a sequence share an XCD) ----
  const int n = blockIdx.x;
  const int u = (n & 7) * units_per_xcd + (n >> 3);
  if (u >= n_units) return;
  const int S = p.num_splits;
  const int HG = p.heads / hv;
  const int split = u % S;
  const int bh = u / S;
  const int hg = bh % HG;
  const int b = bh / HG;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int ht = wave % NH;     // head tile: heads head0 + 32*ht ..
  const int kh = wave / NH;     // latent part: columns 32*MTW*kh .. ; rope k-steps RK*kh ..
  const int head0 = hg * hv;
  const bool real = 32 * ht + l31 < hv;          // this lane's head exists
  const int hd = head0 + (32 * ht + l31) % hv;

  auto ks_of = [&](int j) -> int { return j < LK ? LK * kh + j : 32 + RK * kh + (j - LK); };

  // First round trip: the block ids of the split's first two tiles, the
  // query fragments (B operand of S^T), the block ids of every tile for the
  // table, the sequence length; one wait for all.
  const int32_t* bt_row = p.block_table + static_cast<int64_t>(b) * p.max_blocks;
  const int bs = p.block_size;
  int pg[kNB];
#pragma unroll
  for (int t = 0; t < kNB; ++t)
    pg[t] = scalar_load(bt_row + min((split * p.chunk + t * kT) / bs, p.max_blocks - 1));
  bf16x8_t qf[kKW];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.qls_b + hd * p.qls_h;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qrs_b + hd * p.qrs_h;
#pragma unroll
    for (int j = 0; j < kKW; ++j) {
      const int k = ks_of(j) * 16 + 8 * half;
      qf[j] = *reinterpret_cast<const bf16x8_t*>((k < kDS) ? (ql + k) : (qr + (k - kDS)));
    }
  }
  constexpr int kFill = kMaxTiles / kNT;
  const int ctiles = p.chunk / kT;
  int fpg[kFill];
#pragma unroll
  for (int k = 0; k < kFill; ++k) {
    const int t = k * kNT + static_cast<int>(threadIdx.x);
    fpg[k] = t < ctiles ? bt_row[min((split * p.chunk + t * kT) / bs, p.max_blocks - 1)] : 0;
  }
  int L = scalar_load(p.seq_lens + b);
#pragma unroll
  for (int j = 0; j < kKW; ++j) asm volatile("" : : "v"(qf[j]));
#pragma unroll
  for (int k = 0; k < kFill; ++k) asm volatile("" : : "v"(fpg[k]));
  asm volatile("" : : "s"(pg[0]), "s"(pg[1]), "s"(pg[2]), "s"(L));
  L = max(0, min(L, min(p.max_seq_len, p.max_blocks * p.block_size)));
  const int t0 = split * p.chunk;
  const int t1 = min(L, t0 + p.chunk);
  const int64_t row0 = (static_cast<int64_t>(split) * p.batch + b) * p.heads;
  if (t0 >= t1) {
    if (kh == 0 && half == 0 && real) p.ws_lse[row0 + hd] = -INFINITY;
    return;
  }
  const int ntiles = (t1 - t0 + kT - 1) / kT;

  // ---- tile copies: chunk slot (i*4 + wave)*64 + lane of a tile ----
  uint32_t src_off[kIPT];
#pragma unroll
  for (int i = 0; i < kIPT; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int r = slot / kCPR;
    const int pc = slot % kCPR;
    const int c = (pc & ~7) | ((pc & 7) ^ swz(r));
    src_off[i] = static_cast<uint32_t>((r * kD + c * 8) * 2);
  }
  const uint16_t* cache = static_cast<const uint16_t*>(p.cache);
  // First cache row of tile t in units of 32 rows; an out-of-range block id
  // reads the cache's first rows (unspecified output, no access outside).
  auto tile_row = [&](int t, int page) -> uint32_t {
    const int tb = t0 + t * kT;
    const bool ok = page >= 0 && page < p.num_blocks;
    return ok ? static_cast<uint32_t>(page) * static_cast<uint32_t>(bs / kT) +
                    static_cast<uint32_t>((tb % bs) / kT)
              : 0u;
  };
  struct CopyJob {
    const uint16_t* base;
    uint32_t lim;      // bytes of valid rows
    uint32_t lds;
  };
  // Rows past the split end copy the same chunk of the tile's row 0 (finite;
  // masked).
  auto make_job = [&](int t, int kb, uint32_t row32) -> CopyJob {
    CopyJob j;
    j.lds = lds_addr(&ktile[kb][0]);
    j.base = cache + static_cast<int64_t>(row32) * (kT * kD);
    j.lim = static_cast<uint32_t>(min(kT, t1 - (t0 + t * kT)) * 2 * kD);
    return j;
  };
  auto copy_chunk = [&](const CopyJob& j, int ci) {
    const uint32_t off = src_off[ci] < j.lim ? src_off[ci] : src_off[ci] % (2 * kD);
    copy16(j.base, off, j.lds + static_cast<uint32_t>((ci * 4 + wave) * 64 * 16));
  };

  // Score A fragment (token row l31, k-step ks) of the tile at T.
  const int g = half ^ swz(l31);
  auto rd_k = [&](const char* T, int ks) -> bf16x8_t {
    const int grp = ks >> 2;
    return *reinterpret_cast<const bf16x8_t*>(T + (l31 * kCPR + grp * 8 + ((2 * (ks & 3)) ^ g)) * 16);
  };

  // V^T fragments come straight from the K tile by transposing LDS reads
  // (ds_read_b64_tr_b16): in each group of 16 lanes, lane j receives element
  // j % 4 of the 8 bytes read by lanes 4k + j / 4, k = 0..3.  Lane 4k + q
  // reads token row t_k, latent columns 4q .. 4q+3 of the group's 16, so
  // lane j gets column j of rows t_0..t_3: four tokens of one latent column,
  // half of an A fragment (row = latent column, k = 8 tokens).  Fragment
  // (m, jj) holds, for lane half h, tokens 16jj + 4h + (0..3) in elements
  // 0..3 and 16jj + 8 + 4h + (0..3) in elements 4..7: the token order of
  // the P^T fragments (S^T register r of lane half h is token
  // 8*(r/4) + 4h + r%4).  Byte offsets per (jj, second read, m odd):
  const int trk = (lane & 15) >> 2, trq = lane & 3, trg = (lane >> 4) & 1;
  uint32_t tr_off[2][2][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 16 * jj + 8 * rr + 4 * half + trk;
#pragma unroll
      for (int mo = 0; mo < 2; ++mo)
        tr_off[jj][rr][mo] = static_cast<uint32_t>(
            row * kCPR * 16 + ((4 * mo + 2 * trg + (trq >> 1)) ^ swz(row)) * 16 + 8 * (trq & 1));
    }
  // fragment (m, jj) of latent tile MTW*kh + m of the tile at T
  auto rd_v = [&](const char* T, int m, int jj) -> bf16x8_t {
    const char* b = T + 128 * ((MTW / 2) * kh + (m >> 1));
    const i16x4_t lo = read_tr(b + tr_off[jj][0][m & 1]);
    const i16x4_t hi = read_tr(b + tr_off[jj][1][m & 1]);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t oacc[MTW];    // O^T tiles: latent tile MTW*kh + m, this wave's heads
  float m_run = -INFINITY;   // reference max of this lane's head (scaled, base 2)
  float l_part;          // this lane's share of its head's row sum
  float m_seen;
  const float c = p.scale_log2;

  // One tile: partial scores over this wave's k-steps and V^T of its latent
  // half; the exchange with the wave of the other half (same heads); P^T
  // and the values.  `first`: the tile that sets the reference max.
  auto tile = [&](int i, bool first) {
    const char* T = reinterpret_cast<const char*>(&ktile[i % kNB][0]);
    f32x16_t sp = {};
    bf16x8_t vf[MTW][2];
    bf16x8_t kf[3];
    kf[0] = rd_k(T, ks_of(0));
    kf[1] = rd_k(T, ks_of(1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kKW; ++j) {
      const bf16x8_t a = kf[j % 3];
      if (j + 2 < kKW) kf[(j + 2) % 3] = rd_k(T, ks_of(j + 2));
      if (j < LK) vf[j >> 1][j & 1] = rd_v(T, j >> 1, j & 1);
      sp = mfma(a, qf[j], sp);
      __builtin_amdgcn_sched_barrier(0);
    }
    // tile i+3's block, for its copies after the barrier
    const uint32_t r32 = __builtin_amdgcn_readfirstlane(trow[min(i + kNB, ntiles - 1)]);
    float4* mine = &part[i & 1][wave][0][0];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      mine[r4 * 64 + lane] = make_float4(sp[4 * r4], sp[4 * r4 + 1], sp[4 * r4 + 2], sp[4 * r4 + 3]);
    // this wave's copies of tile i+1 are in (tile i+2's may be in flight)
    if (i + 2 < ntiles) wait_vm<kIPT>(); else wait_vm<0>();
    barrier();           // partial scores visible; tile i+1 in for every wave; tile i's buffer free
    if (i + kNB < ntiles) {
      const CopyJob cj = make_job(i + kNB, i % kNB, r32);
#pragma unroll
      for (int ci = 0; ci < kIPT; ++ci) copy_chunk(cj, ci);
    }
    // full scores: the KP partials of this head tile, added as a butterfly
    // (own + part kh^1, then + (part kh^2 + part kh^3)); every term pair is
    // commutative, so every wave of the head tile gets the same bits
    auto other = [&](int q, int r4) -> float4 { return part[i & 1][q * NH + ht][r4][lane]; };
    float s[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float4 v = other(kh ^ 1, r4);
      if constexpr (KP == 4) {
        const float4 a = other(kh ^ 2, r4), b2 = other(kh ^ 3, r4);
        const float4 x = make_float4(sp[4 * r4] + v.x, sp[4 * r4 + 1] + v.y, sp[4 * r4 + 2] + v.z,
                                     sp[4 * r4 + 3] + v.w);
        v = make_float4(a.x + b2.x, a.y + b2.y, a.z + b2.z, a.w + b2.w);
        s[4 * r4] = x.x + v.x;
        s[4 * r4 + 1] = x.y + v.y;
        s[4 * r4 + 2] = x.z + v.z;
        s[4 * r4 + 3] = x.w + v.w;
      } else {
        s[4 * r4] = sp[4 * r4] + v.x;
        s[4 * r4 + 1] = sp[4 * r4 + 1] + v.y;
        s[4 * r4 + 2] = sp[4 * r4 + 2] + v.z;
        s[4 * r4 + 3] = sp[4 * r4 + 3] + v.w;
      }
    }
    // scaled scores (base 2; any finite scale, zero and negative included);
    // register r holds token 8*(r/4) + 4*half + r%4 of the tile
    // (rows past the split end, only in its last tile, get -inf; branch-free)
    const int lim = t1 - (t0 + i * kT) - 4 * half;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] *= c;
      asm volatile("" : "+v"(s[r]));   // computed for every row, then selected (no branch)
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) < lim) ? s[r] : -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = both_halves_max(mx);
    m_run = first ? fmaxf(m_run, mx) : m_run;
    m_seen = (!first && mx > m_run + kRescale) ? fmaxf(m_seen, mx) : m_seen;
    // P^T fragments (k-step jj = tokens of registers 8jj .. 8jj+7) and values
    bf16x8_t pn[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pv = __builtin_amdgcn_exp2f(s[r] - m_run);
      l_part += pv;
      pn[r >> 3][r & 7] = static_cast<__bf16>(pv);
    }
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) oacc[m] = mfma(vf[m][jj], pn[jj], oacc[m]);
  };

  // Table of tile rows.
#pragma unroll
  for (int k = 0; k < kFill; ++k) {
    const int t = k * kNT + static_cast<int>(threadIdx.x);
    if (t < ntiles) trow[t] = tile_row(t, fpg[k]);
  }

  // Pipeline: tile i in K buffer i % 3, copied right after the barrier of
  // step i-3 (which frees that buffer), so every tile has two steps to
  // arrive.  Step i: scores of tile i; wait for this wave's copies of tile
  // i+1; barrier; copies of tile i+3; softmax and values of tile i.  No copy
  // goes past the split's last tile.
  bool first_pass = true;
  while (true) {
#pragma unroll
    for (int m = 0; m < MTW; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
    l_part = 0.f;
    m_seen = -INFINITY;
#pragma unroll
    for (int t = 0; t < kNB; ++t) {
      if (t < ntiles) {
        const uint32_t r32 = first_pass ? tile_row(t, pg[t]) : __builtin_amdgcn_readfirstlane(trow[t]);
        const CopyJob j = make_job(t, t, r32);
#pragma unroll
        for (int ci = 0; ci < kIPT; ++ci) copy_chunk(j, ci);
      }
    }
    // tile 0 in (tiles 1 and 2 may be in flight)
    if (ntiles >= 3) wait_vm<2 * kIPT>(); else if (ntiles == 2) wait_vm<kIPT>(); else wait_vm<0>();
    barrier();           // tile 0 and the table visible
#pragma nounroll
    for (int i = 0; i < ntiles; ++i) tile(i, first_pass && i == 0);
    // run again if a head of either tile went over its reference (every
    // wave takes the same decision)
    const bool over = __ballot(m_seen != -INFINITY) != 0ull;
    if (lane == 0) over_flag[wave] = over ? 1 : 0;
    barrier();
    const bool again = (over_flag[0] | over_flag[1] | over_flag[2] | over_flag[3]) != 0;
    if (!again) break;
    m_run = fmaxf(m_run, m_seen);
    first_pass = false;
    barrier();           // every wave has read the flags before they are written again
  }

  // ---- split result: o = U / l, lse = m + log l (natural log) ----
  uint16_t* wh = reinterpret_cast<uint16_t*>(p.ws_o);
  float* wsc = reinterpret_cast<float*>(reinterpret_cast<char*>(p.ws_o) +
                                        fp16_partials_scale_offset(p.num_splits, p.batch, p.heads, kDS));
  const float l_tot = both_halves_sum(l_part);
  const int64_t row = row0 + hd;
  const int64_t su = row0 / p.heads;              // split * batch + b
  if (kh == 0 && half == 0 && real) p.ws_lse[row] = (m_run + __log2f(l_tot)) * kLn2;
  const float inv_l = 1.0f / l_tot;
#pragma unroll
  for (int blk = 0; blk < MTW / 2; ++blk) {   // 64-column blocks of this wave
    float amax = 0.f;
#pragma unroll
    for (int m = 2 * blk; m < 2 * blk + 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(oacc[m][r]));
    amax = both_halves_max(amax);
    const float hs = amax > 0.f ? 1.0f / amax : 0.f;
#pragma unroll
    for (int m = 2 * blk; m < 2 * blk + 2; ++m) {
      // split u holds [kDS / 8][heads][8] halves: one store instruction
      // writes 16-byte pieces of 32 consecutive heads
      uint16_t* dst = wh + (su * (kDS / 8) + 4 * (MTW * kh + m)) * p.heads * 8 + static_cast<int64_t>(hd) * 8 +
                      4 * half;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const _Float16 lo = static_cast<_Float16>(oacc[m][4 * q + 2 * k] * hs);
          const _Float16 hi = static_cast<_Float16>(oacc[m][4 * q + 2 * k + 1] * hs);
          w[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, lo)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        if (real) *reinterpret_cast<uint2*>(dst + static_cast<int64_t>(q) * p.heads * 8) = make_uint2(w[0], w[1]);
      }
    }
    if (half == 0 && real) wsc[(su * (kDS / 64) + (MTW / 2) * kh + blk) * p.heads + hd] = amax * inv_l;
  }
}

}  // namespace

// Groups of 64 heads where the head count allows, else 32, else 16.
int decode_mla_group_heads(int heads) { return heads % 64 == 0 ? 64 : (heads % 32 == 0 ? 32 : 16); }

bool decode_mla_supported(int heads, int d_s, int d_r, int block_size) {
  return heads % 16 == 0 && d_s == kDS && d_r == kDR && block_size % kT == 0;
}

int decode_mla_max_chunk() { return kMaxTiles * kT; }

hipError_t launch_decode_mla(const DecodeParams& p, hipStream_t s) {
  if (!decode_mla_supported(p.heads, p.d_s, p.d_r, p.block_size)) return hipErrorNotSupported;
  if (p.chunk > kMaxTiles * kT || p.chunk % kT != 0) return hipErrorInvalidValue;
  const int hv = decode_mla_group_heads(p.heads);
  const int n_units = p.num_splits * p.batch * (p.heads / hv);
  const int per_xcd = (n_units + 7) / 8;
  if (hv == 64)
    hipLaunchKernelGGL(decode_mla_kernel<2>, dim3(8 * per_xcd), dim3(kNT), 0, s, p, n_units, per_xcd, hv);
  else
    hipLaunchKernelGGL(decode_mla_kernel<1>, dim3(8 * per_xcd), dim3(kNT), 0, s, p, n_units, per_xcd, hv);
  return hipGetLastError();
}

}  // namespace tpla
