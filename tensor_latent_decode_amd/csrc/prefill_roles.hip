// MLA-form prefill on the matrix cores with separate score and value waves
// (gfx950): one workgroup per (sequence, position, group of 64 heads).
//
//   o[b, t, h] = sum_{j <= t} softmax_j(scale * (q_lat[b,t,h] . c[b,j] +
//                q_rope[b,t,h] . k_rope[b,j])) * c[b, j]
//
// with rows kv[b, j] = [c (512) || k_rope (64)] (paperbot revised abstract:
// MLA is kept for prefill; edgentiq blog, "Prefill-Decode Separation for
// Optimal Performance").  Every head of a position attends to the same keys
// 0..t, so a workgroup is a decode of its 64 heads over t + 1 contiguous
// rows: the causal mask is a length.
//
// Eight waves, two per SIMD, in two roles:
//   score waves 0..3  wave (ht, tt) = (w & 1, w >> 1): heads 32ht .. 32ht+31
//                     against keys 32tt .. 32tt+31 of the tile,
//                     S^T[key, head] over 576 (36 k-steps), then
//                     P = exp2(c*S - m_ref) as the value product's B
//                     fragments (P^T) in LDS
//   value waves 4..7  wave 4+q owns latent columns 128q .. 128q+127 for the
//                     64 heads: O^T[lat, head] += V^T . P^T
// all on v_mfma_f32_32x32x16_bf16, one barrier per 64-key tile.  A key tile
// is 64 x 576 x 2 = 73,728 bytes, so LDS holds two (and two P^T buffers):
// the value waves hold the V^T fragments of the tile whose values are due in
// registers (read during the step before, right after each fragment's last
// use), which frees that tile's buffer at the start of its step for the copy
// of the tile after next.  Step i:
//   score waves   scores of tile i+1 (buffer (i+1) % 2), P^T -> ptile[(i+1) % 2]
//   value waves   copy of tile i+2 -> buffer i % 2, values of tile i, V^T of
//                 tile i+1 from buffer (i+1) % 2, then wait for tile i+2.
// The softmax reference is the first tile's max (the two score waves of a
// head tile exchange theirs once), with a rerun if a head's row sum passes
// 2^64, as in the decode kernels.  Row sums of the two key halves meet in
// LDS at the end; the value waves write o = U / l and the score waves lse.
#include <type_traits>

#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int scalar_load(const int32_t* p) { return *(const const_i32_t*)p; }

constexpr int kTile = 64;                   // keys per tile
constexpr int kDS = 512, kDR = 64, kD = kDS + kDR;
constexpr int kCPR = kD / 8;                // 16-byte chunks per row (72)
constexpr int kSlots = kTile * kCPR;        // chunks per tile (4608)
constexpr int kIPT = kSlots / (4 * 64);     // copies per lane per tile (18, four copying waves)
constexpr int kKS = kD / 16;                // score k-steps (36)
constexpr int kHG = 64;                     // heads per workgroup
constexpr int kMPW = kDS / 32 / 4;          // 32-column latent tiles per value wave (4)
constexpr int kKPre = 4, kPPre = 2;         // LDS read prefetch depths (score K, value P^T)
constexpr float kRescaleSum = 0x1p64f;
constexpr float kLn2 = 0.69314718055994531f;
static_assert(kSlots % (4 * 64) == 0 && kCPR % 8 == 0, "tile shape");

// XOR pattern of tile row r: bit2 = r1, bit1 = r0 ^ r3, bit0 = r2.
__device__ __forceinline__ int swz(int r) {
  return (((r >> 1) & 1) << 2) | (((r ^ (r >> 3)) & 1) << 1) | ((r >> 2) & 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void_t*)p));
}

// Buffer resource of a byte range starting at base: raw, range checked per
// dword against nbytes (loads past it return zeros).
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = static_cast<int>(static_cast<uint32_t>(a));
  r[1] = static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu);
  r[2] = static_cast<int>(nbytes);
  r[3] = 0x00020000;
  return r;
}

// One 16-byte buffer -> LDS copy per lane, to LDS address lds + 16*lane.
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

__device__ __forceinline__ float both_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float both_halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats to packed bf16 (round to nearest even) in one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

using kTrue_t = std::integral_constant<bool, true>;
using kFalse_t = std::integral_constant<bool, false>;
constexpr kTrue_t kTrue{};
constexpr kFalse_t kFalse{};

template <bool kOutBf16>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void prefill_roles_kernel(PrefillParams p, int n_units) {
  __shared__ __attribute__((aligned(1024))) uint4 ktile[2][kSlots];
  __shared__ __attribute__((aligned(1024))) uint4 ptile[2][8 * 64];   // [ht*4 + k-step][lane]
  // Small exchanges alias buffers that are idle at that moment: the first
  // tile's maxima go to ptile[1] (P^T of tile 1 is written later), the end
  // of a pass uses K buffer 0 (every copy has landed and been read).
  float* const xmax = reinterpret_cast<float*>(&ptile[1][0]);          // [ht][tt][32]
  float* const xsum = reinterpret_cast<float*>(&ktile[0][0]);          // [ht][tt][32] row sums
  float* const xraw = xsum + 128;                                      // [ht][tt][32] raw maxima
  int* const xflag = reinterpret_cast<int*>(xsum + 256);               // [4]
  float* const lsum = xsum + 384;                                      // [64] final row sums

  // ---- work unit: positions late-first; (sequence, head group) fastest ----
  const int u = static_cast<int>(blockIdx.x);
  if (u >= n_units) return;
  const int hgs = p.heads / kHG;
  const int bg = u % (p.batch * hgs);
  const int b = bg / hgs;
  const int hg = bg % hgs;
  const int t = p.max_len - 1 - u / (p.batch * hgs);
  const int L = max(0, min(scalar_load(p.seq_lens + b), p.max_len));
  if (t >= L) return;                         // past the prompt: left as it was
  const int nkeys = t + 1;
  const int ntiles = (nkeys + kTile - 1) / kTile;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int head0 = hg * kHG;
  const bool is_score = wave < 4;
  const uint16_t* kvb = static_cast<const uint16_t*>(p.kv) + b * p.kv_b;

  // zero scale: every weight exactly 1 (masked keys stay 0); a negative
  // scale is carried by the query (negated exactly at load)
  const float c = p.scale_log2 == 0.f ? 0x1p-100f : fabsf(p.scale_log2);

  if (is_score) {
    // the score waves set each step's length (the value waves wait for
    // them at the barrier): their instructions go first on a shared SIMD
    __builtin_amdgcn_s_setprio(1);
    // =====================================================================
    // Score waves
    // =====================================================================
    const int ht = wave & 1, tt = wave >> 1;
    const int head = head0 + ht * 32 + l31;
    bf16x8_t qf[kKS];
    {
      const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.ql_b +
                           static_cast<int64_t>(t) * p.ql_s + static_cast<int64_t>(head) * p.ql_h;
      const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qr_b +
                           static_cast<int64_t>(t) * p.qr_s + static_cast<int64_t>(head) * p.qr_h;
      // one base per part; k-steps are immediate offsets from it
      const bf16x8_t* qlv = reinterpret_cast<const bf16x8_t*>(ql + 8 * half);
      const bf16x8_t* qrv = reinterpret_cast<const bf16x8_t*>(qr + 8 * half);
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) qf[kk] = kk * 16 < kDS ? qlv[2 * kk] : qrv[2 * (kk - kDS / 16)];
    }
    if (p.scale_log2 < 0.f) {
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        uint4 w = __builtin_bit_cast(uint4, qf[kk]);
        w.x ^= 0x80008000u; w.y ^= 0x80008000u; w.z ^= 0x80008000u; w.w ^= 0x80008000u;
        qf[kk] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // Score A fragment (key row 32tt + l31, k-step kk) of the tile at T.
    int qk_off[4];
    {
      const int g = half ^ swz(l31);
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) qk_off[k2] = ((32 * tt + l31) * kCPR + ((2 * k2) ^ g)) * 16;
    }
    auto rd_k = [&](const char* T, int kk) -> bf16x8_t {
      return *reinterpret_cast<const bf16x8_t*>(T + qk_off[kk & 3] + (kk >> 2) * 128);
    };
    const bf16x2_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float m_run = -INFINITY, l_part = 0.f, m_raw = -INFINITY;
    // key of register r of this lane in the tile: 32tt + 8(r/4) + 4half + r%4
    auto key_of = [&](int r) { return 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3); };

    // Scores of tile i (keys i*64 ..) into sc.
    auto scores = [&](int i) -> f32x16_t {
      const char* T = reinterpret_cast<const char*>(&ktile[i & 1][0]);
      f32x16_t sc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = 0.f;
      bf16x8_t ka[kKPre];
#pragma unroll
      for (int s2 = 0; s2 < kKPre; ++s2) ka[s2] = rd_k(T, s2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        sc = mfma(ka[kk % kKPre], qf[kk], sc);
        if (kk + kKPre < kKS) ka[kk % kKPre] = rd_k(T, kk + kKPre);
        __builtin_amdgcn_sched_barrier(0);
      }
      // keys past the position (last tile only) do not count
      const int lim = nkeys - i * kTile;
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = key_of(r) < lim ? sc[r] : -INFINITY;
      return sc;
    };
    // P^T of tile i from its scores (fragments k-step 2tt, 2tt+1 of this
    // head tile); the row sum adds the bf16 weights the product uses.
    auto weights = [&](const f32x16_t& sc, int i, auto careful_c) {
      uint4* pdst = &ptile[i & 1][0];
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        bf16x8_t pn;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = sc[8 * f + e];
          if (decltype(careful_c)::value) m_raw = fmaxf(m_raw, sv);
          pn[e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sv, c, -m_run)));
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2_t pr = {pn[e], pn[e + 1]};
          l_part = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_part, false);
        }
        pdst[(ht * 4 + 2 * tt + f) * 64 + lane] = __builtin_bit_cast(uint4, pn);
      }
    };

    bool careful = false;
    for (int npass = 0;; ++npass) {
      l_part = 0.f;
      m_raw = -INFINITY;
      barrier();                                  // B_a: tile 0 in
      {
        // first tile: the reference is the max over both key halves
        const f32x16_t sc = scores(0);
        if (npass == 0) {
          float m0 = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) m0 = fmaxf(m0, sc[r]);
          m0 = both_halves_max(m0) * c;
          if (half == 0) xmax[(ht * 2 + tt) * 32 + l31] = m0;
        }
        barrier();                                // B_x
        if (npass == 0) m_run = fmaxf(xmax[(ht * 2) * 32 + l31], xmax[(ht * 2 + 1) * 32 + l31]);
        if (careful) weights(sc, 0, kTrue);
        else weights(sc, 0, kFalse);
      }
      for (int i = 0; i + 1 < ntiles; ++i) {
        barrier();                                // B_i
        const f32x16_t sc = scores(i + 1);
        if (careful) weights(sc, i + 1, kTrue);
        else weights(sc, i + 1, kFalse);
      }
      barrier();                                  // B_end: the last values may start
      barrier();                                  // B_f: every buffer idle
      {
        const float ls = both_halves_sum(l_part), mr = both_halves_max(m_raw);
        if (half == 0) {
          xsum[(ht * 2 + tt) * 32 + l31] = ls;
          xraw[(ht * 2 + tt) * 32 + l31] = mr;
        }
      }
      barrier();                                  // B_s: both key halves' sums in
      const float l_tot = xsum[(ht * 2) * 32 + l31] + xsum[(ht * 2 + 1) * 32 + l31];
      const bool lane_inf = l_tot == INFINITY;
      const bool lane_over = l_tot > kRescaleSum;
      int code = __ballot(lane_over) != 0ull ? 1 : 0;
      if (!careful && __ballot(lane_inf) != 0ull) code = 2;
      if (npass >= 3) code = 0;                   // bounded: at most 4 passes
      if (lane == 0) xflag[wave] = code;
      barrier();                                  // B_c
      const int any = xflag[0] | xflag[1] | xflag[2] | xflag[3];
      if (!any) {
        if (tt == 0 && half == 0) {
          lsum[ht * 32 + l31] = l_tot;
          if (p.lse != nullptr)
            p.lse[(static_cast<int64_t>(b) * p.max_len + t) * p.heads + head] = (m_run + __log2f(l_tot)) * kLn2;
        }
        barrier();                                // B_l: row sums for the value waves
        return;
      }
      if (careful) m_run = fmaxf(m_run, fmaxf(xraw[(ht * 2) * 32 + l31], xraw[(ht * 2 + 1) * 32 + l31]) * c);
      else if (lane_over && !lane_inf) m_run += __log2f(l_tot);
      careful = !careful && (any & 2) != 0;
      barrier();                                  // B_r: flags read before the next pass
    }
  }

  // =======================================================================
  // Value waves
  // =======================================================================
  const int lq = wave - 4;
  // this lane's source chunks: (row, swizzled chunk) of copy k, 16 bits
  // each, two copies per register
  uint32_t src_rc[(kIPT + 1) / 2];
#pragma unroll
  for (int k = 0; k < kIPT; ++k) {
    const int slot = (k * 4 + lq) * 64 + lane;
    const int r = slot / kCPR;
    const int pc = slot % kCPR;
    const uint32_t rc = static_cast<uint32_t>(r << 7 | ((pc & ~7) | ((pc & 7) ^ swz(r))));
    if (k % 2 == 0) src_rc[k / 2] = rc;
    else src_rc[k / 2] |= rc << 16;
  }
  const uint32_t row_bytes = static_cast<uint32_t>(p.kv_s) * 2u;
  // copy of tile i into buffer i % 2, rows past the position zero-filled
  auto copy_chunk = [&](int i, int k) {
    const int nvalid = min(kTile, nkeys - i * kTile);
    const i32x4_t rs = buffer_rsrc(kvb + static_cast<int64_t>(i) * kTile * p.kv_s,
                                   static_cast<uint32_t>(nvalid) * row_bytes);
    const uint32_t rc = (src_rc[k / 2] >> (16 * (k % 2))) & 0xffffu;
    copy16(rs, (rc >> 7) * row_bytes + (rc & 127u) * 16u,
           lds_addr(&ktile[i & 1][0]) + static_cast<uint32_t>((k * 4 + lq) * 64 * 16));
  };
  // V^T fragment (latent tile 4lq + mm, key k-step j) of the tile at T: two
  // transposing reads in the key order of the P^T fragments.
  uint32_t tr_off[2][2];
  {
    const int trk = (lane & 15) >> 2, trq = lane & 3, trg = (lane >> 4) & 1;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = 8 * rr + 4 * half + trk;
#pragma unroll
      for (int mo = 0; mo < 2; ++mo)
        tr_off[rr][mo] = static_cast<uint32_t>(row * kCPR * 16 + ((4 * mo + 2 * trg + (trq >> 1)) ^ swz(row)) * 16 +
                                               8 * (trq & 1));
    }
  }
  auto rd_v = [&](const char* T, int mm, int j) -> bf16x8_t {
    const char* bb = T + 128 * (2 * lq + (mm >> 1)) + j * 16 * kCPR * 16;
    const i16x4_t lo = read_tr(bb + tr_off[0][mm & 1]);
    const i16x4_t hi = read_tr(bb + tr_off[1][mm & 1]);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t oacc[kMPW][2];      // O^T tiles: latent tile 4lq + mm, head tile ht
  bf16x8_t vc[kMPW][4];        // V^T fragments of the tile whose values are due

  // Values of tile i (V^T in vc, P^T in ptile[i % 2]); with kNext, V^T of
  // tile i+1 is read into vc right after each fragment's last use, and the
  // copy of tile i+2 (when there is one) is issued first.
  auto values = [&](int i, auto next_c) {
    constexpr bool kNext = decltype(next_c)::value;
    const bool do_copy = kNext && i + 2 < ntiles;
    const uint4* P = &ptile[i & 1][0];
    const char* Tn = reinterpret_cast<const char*>(&ktile[(i + 1) & 1][0]);
    auto frag = [&](int f) -> bf16x8_t {      // f = j * 2 + ht
      return __builtin_bit_cast(bf16x8_t, P[((f & 1) * 4 + (f >> 1)) * 64 + lane]);
    };
    // the copy goes out first: a whole step to land (the tile is mostly
    // in the L2, where spreading the copies over the MFMAs only delays them)
    if (do_copy) {
#pragma unroll
      for (int k = 0; k < kIPT; ++k) copy_chunk(i + 2, k);
    }
    bf16x8_t pa[kPPre];
#pragma unroll
    for (int f = 0; f < kPPre; ++f) pa[f] = frag(f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int j = f >> 1, ht = f & 1;
#pragma unroll
      for (int mm = 0; mm < kMPW; ++mm) oacc[mm][ht] = mfma(vc[mm][j], pa[f % kPPre], oacc[mm][ht]);
      if (f + kPPre < 8) pa[f % kPPre] = frag(f + kPPre);
      if (kNext && ht == 1) {
#pragma unroll
        for (int mm = 0; mm < kMPW; ++mm) vc[mm][j] = rd_v(Tn, mm, j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  while (true) {
#pragma unroll
    for (int mm = 0; mm < kMPW; ++mm)
#pragma unroll
      for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[mm][ht][r] = 0.f;
#pragma unroll
    for (int k = 0; k < kIPT; ++k) copy_chunk(0, k);
    if (ntiles > 1) {
#pragma unroll
      for (int k = 0; k < kIPT; ++k) copy_chunk(1, k);
      wait_vm<kIPT>();                            // tile 0
    } else {
      wait_vm<0>();
    }
    barrier();                                    // B_a
    {
      const char* T0 = reinterpret_cast<const char*>(&ktile[0][0]);
#pragma unroll
      for (int k = 0; k < 4 * kMPW; ++k) vc[k >> 2][k & 3] = rd_v(T0, k >> 2, k & 3);
    }
    wait_vm<0>();                                 // tile 1
    barrier();                                    // B_x
    for (int i = 0; i + 1 < ntiles; ++i) {
      barrier();                                  // B_i
      values(i, kTrue);
      wait_vm<0>();                               // tile i+2
    }
    barrier();                                    // B_end
    values(ntiles - 1, kFalse);
    barrier();                                    // B_f
    barrier();                                    // B_s
    barrier();                                    // B_c
    const int any = xflag[0] | xflag[1] | xflag[2] | xflag[3];
    if (!any) break;
    barrier();                                    // B_r
  }
  barrier();                                      // B_l: row sums in lsum

  // o = U / l: register r of latent tile 4lq + mm holds column
  // 32(4lq + mm) + 8(r/4) + 4half + r%4 of head 32ht + l31, so a lane owns
  // 8- or 16-byte pieces of 32 different rows.  Stored as they are, every
  // store instruction touches 32 rows; instead each head tile goes through
  // LDS (K buffer 1, idle once the last values are done; wave lq owns 32
  // rows x 128 columns of it, 16-byte chunk c of row r at chunk c ^ (r & 15),
  // which keeps both the writes and the reads free of bank conflicts) and
  // comes back as whole 16-byte chunks: one store instruction then writes
  // 4 (bf16) or 2 (float) contiguous 256- or 512-byte row pieces.  Rows that
  // are not 16-byte aligned take the direct stores.
  constexpr int kEs = kOutBf16 ? 2 : 4;      // output element bytes
  constexpr int kRB = 128 * kEs;             // bytes of a wave's piece of one row
  constexpr int kNC = kRB / 16;              // its 16-byte chunks
  auto row_ptr = [&](int head) -> char* {
    return static_cast<char*>(p.out) +
           (b * p.o_b + static_cast<int64_t>(t) * p.o_s + static_cast<int64_t>(head) * p.o_h) * kEs;
  };
  const bool staged =
      ((reinterpret_cast<uintptr_t>(p.out) | static_cast<uint64_t>(p.o_b | p.o_s | p.o_h) * kEs) & 15) == 0;
  char* const stage = reinterpret_cast<char*>(&ktile[1][0]) + lq * 32 * kRB;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const float inv_l = 1.0f / lsum[ht * 32 + l31];
    if (staged) {
#pragma unroll
      for (int mm = 0; mm < kMPW; ++mm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float v0 = oacc[mm][ht][4 * q4] * inv_l, v1 = oacc[mm][ht][4 * q4 + 1] * inv_l;
          const float v2 = oacc[mm][ht][4 * q4 + 2] * inv_l, v3 = oacc[mm][ht][4 * q4 + 3] * inv_l;
          const int cbyte = (32 * mm + 8 * q4 + 4 * half) * kEs;   // byte of the wave's row piece
          char* dst = stage + l31 * kRB + (((cbyte >> 4) ^ (l31 & 15)) << 4) + (cbyte & 15);
          if constexpr (kOutBf16) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          } else {
            *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
          }
        }
#pragma unroll
      for (int k = 0; k < 32 * kNC / 64; ++k) {
        const int idx = k * 64 + lane;
        const int r = idx / kNC, cc = idx % kNC;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + r * kRB + ((cc ^ (r & 15)) << 4));
        *reinterpret_cast<uint4*>(row_ptr(head0 + ht * 32 + r) + lq * kRB + cc * 16) = v;
      }
    } else {
      char* const orow = row_ptr(head0 + ht * 32 + l31);
#pragma unroll
      for (int mm = 0; mm < kMPW; ++mm)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = 32 * (kMPW * lq + mm) + 8 * q4 + 4 * half;
          const float v0 = oacc[mm][ht][4 * q4] * inv_l, v1 = oacc[mm][ht][4 * q4 + 1] * inv_l;
          const float v2 = oacc[mm][ht][4 * q4 + 2] * inv_l, v3 = oacc[mm][ht][4 * q4 + 3] * inv_l;
          if constexpr (kOutBf16) {
            *reinterpret_cast<uint2*>(orow + col * 2) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          } else {
            *reinterpret_cast<float4*>(orow + col * 4) = make_float4(v0, v1, v2, v3);
          }
        }
    }
  }
}

}  // namespace

// 64-head groups; a tile's byte range (64 rows of kv) must fit the 32-bit
// range of a buffer resource.
bool prefill_roles_supported(int heads, int64_t kv_stride_t) {
  return heads % kHG == 0 && kv_stride_t >= kD && kv_stride_t < (int64_t{1} << 25);
}

hipError_t launch_prefill_roles(const PrefillParams& p, hipStream_t s) {
  if (!prefill_roles_supported(p.heads, p.kv_s)) return hipErrorNotSupported;
  const int64_t units = static_cast<int64_t>(p.batch) * (p.heads / kHG) * p.max_len;
  if (units == 0) return hipSuccess;
  if (units > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (p.out_bf16)
    hipLaunchKernelGGL(prefill_roles_kernel<true>, dim3(static_cast<uint32_t>(units)), dim3(512), 0, s, p,
                       static_cast<int>(units));
  else
    hipLaunchKernelGGL(prefill_roles_kernel<false>, dim3(static_cast<uint32_t>(units)), dim3(512), 0, s, p,
                       static_cast<int>(units));
  return hipGetLastError();
}

}  // namespace tpla
