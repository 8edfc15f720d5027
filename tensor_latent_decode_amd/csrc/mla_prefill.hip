// MLA-form prefill attention (gfx950): causal attention of a prompt over its
// own latent rows, unsliced and unrotated.  Prefill keeps the MLA form and
// only decode switches to TPLA (paperbot revised abstract; edgentiq blog,
// "Prefill-Decode Separation for Optimal Performance"); the prompt's rows
// reach the shard caches through the rotate-and-append of decode.
//
//   o[b, t, h] = sum_{j <= t} softmax_j(scale * (q_lat[b,t,h] . c[b,j] +
//                q_rope[b,t,h] . k_rope[b,j])) * c[b, j]
//
// with rows kv[b, j] = [c (512) || k_rope (64)].  Every head of every
// position attends to the same keys (one latent row per position), so the
// (position, head) pairs are the rows of one causal attention with 576-wide
// keys and 512-wide values.
//
// One workgroup of four waves per (sequence, block of 64 rows), rows taken
// position-major (row r = position r / H, head r % H).  Key tiles of 32
// positions (32 contiguous rows of kv) go from memory straight into LDS,
// three buffers deep; the workgroup reads the tiles up to its last
// position.  The rows form two tiles of 32; wave w takes row tile w & 1 and
// latent half w >> 1 (256 columns and 32 of the rope columns):
//
//   scores   a partial S^T[key, row] over the wave's 18 k-steps; the wave of
//            the other half adds its partial through LDS (both hold the
//            same bits: a + b == b + a), then the causal mask of each row
//   softmax  against a fixed reference (the first tile's max, where every
//            row sees key 0); a later tile max more than 64 (base 2) above
//            it makes the block run again with the raised reference
//   values   O^T[lat, row] += V^T . P^T for the wave's 256 latent columns,
//            V^T from the K tile by transposing LDS reads (ds_read_b64_tr_b16:
//            in each group of 16 lanes, lane j receives element j % 4 of the
//            8 bytes read by lanes 4k + j / 4; lanes reading 4 columns of 4
//            key rows hand each lane 4 keys of one column, in the order of
//            the P^T fragments)
//
// all on v_mfma_f32_32x32x16_bf16, one barrier per tile.  No token split:
// each block writes its rows' outputs (o = U / l) and log-sum-exps itself.
// Blocks of late positions (the most tiles) are launched first.
#include "tpla_internal.h"

namespace tpla {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

constexpr int kT = 32;                 // keys per tile
constexpr int kDS = 512, kDR = 64, kD = kDS + kDR;
constexpr int kCPR = kD / 8;           // 16-byte chunks per row (72)
constexpr int kSlots = kT * kCPR;      // chunks per tile (2304)
constexpr int kNT = 256;
constexpr int kIPT = kSlots / kNT;     // copies per thread per tile (9)
constexpr int kNB = 3;                 // K buffers
constexpr int kRows = 64;              // (position, head) rows per workgroup
constexpr int kKW = 18;                // score k-steps per wave: 16 latent + 2 rope
constexpr int kMTW = 8;                // 32-column latent tiles per wave
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

__device__ __forceinline__ i16x4_t read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)((lds_char_t*)const_cast<char*>(p)));
}

__device__ __forceinline__ f32x16_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The other lane of this lane's row (lane l +- 32).
__device__ __forceinline__ float both_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float both_halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <bool kOutBf16>
__global__ __attribute__((amdgpu_flat_work_group_size(kNT, kNT), amdgpu_waves_per_eu(1, 1)))
void mla_prefill_kernel(PrefillParams p, int n_rb) {
  __shared__ __attribute__((aligned(1024))) uint4 ktile[kNB][kSlots];
  __shared__ __attribute__((aligned(16))) float4 part[2][4][4][64];   // [tile & 1][wave][r/4][lane]
  __shared__ int over_flag[4];

  // ---- work unit: sequence b, row block rb (late positions first) ----
  const int b = blockIdx.x % p.batch;
  const int rb = n_rb - 1 - static_cast<int>(blockIdx.x / p.batch);
  int L = scalar_load(p.seq_lens + b);
  L = max(0, min(L, p.max_len));
  const int64_t rows = static_cast<int64_t>(L) * p.heads;
  const int64_t r0 = static_cast<int64_t>(rb) * kRows;
  if (r0 >= rows) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int l31 = lane & 31, half = lane >> 5;
  const int ht = wave & 1;      // row tile: rows r0 + 32*ht ..
  const int kh = wave >> 1;     // latent half: columns 256*kh .. ; rope k-steps 2*kh, 2*kh+1
  const int64_t r = r0 + 32 * ht + l31;
  const bool real = r < rows;   // rows past the sequence repeat its last row, store nothing
  const int64_t rr = real ? r : rows - 1;
  const int pos = static_cast<int>(rr / p.heads);
  const int hd = static_cast<int>(rr % p.heads);
  const int last = static_cast<int>(min(r0 + kRows - 1, rows - 1) / p.heads);   // last position
  const int ntiles = last / kT + 1;

  auto ks_of = [&](int j) -> int { return j < 16 ? 16 * kh + j : 32 + 2 * kh + (j - 16); };

  // query fragments (B operand of S^T): this lane's row, the wave's k-steps
  bf16x8_t qf[kKW];
  {
    const uint16_t* ql = static_cast<const uint16_t*>(p.q_latent) + b * p.ql_b + pos * p.ql_s + hd * p.ql_h;
    const uint16_t* qr = static_cast<const uint16_t*>(p.q_rope) + b * p.qr_b + pos * p.qr_s + hd * p.qr_h;
#pragma unroll
    for (int j = 0; j < kKW; ++j) {
      const int k = ks_of(j) * 16 + 8 * half;
      qf[j] = *reinterpret_cast<const bf16x8_t*>((k < kDS) ? (ql + k) : (qr + (k - kDS)));
    }
  }

  // ---- tile copies: chunk slot (i*4 + wave)*64 + lane of a tile ----
  int src_row[kIPT];
  uint32_t src_c16[kIPT];
#pragma unroll
  for (int i = 0; i < kIPT; ++i) {
    const int slot = (i * 4 + wave) * 64 + lane;
    const int rw = slot / kCPR;
    const int pc = slot % kCPR;
    src_row[i] = rw;
    src_c16[i] = static_cast<uint32_t>(((pc & ~7) | ((pc & 7) ^ swz(rw))) * 16);
  }
  const uint16_t* kvb = static_cast<const uint16_t*>(p.kv) + b * p.kv_b;
  // Rows past the sequence end read the tile's row 0 (never attended: a key
  // past the end is past every row's position).
  auto copy_tile = [&](int t, int kb) {
    const uint16_t* base = kvb + static_cast<int64_t>(t) * kT * p.kv_s;
    const int nvalid = min(kT, L - t * kT);
    const uint32_t lds = lds_addr(&ktile[kb][0]);
#pragma unroll
    for (int ci = 0; ci < kIPT; ++ci) {
      const uint32_t off =
          (src_row[ci] < nvalid ? static_cast<uint32_t>(src_row[ci] * p.kv_s * 2) : 0u) + src_c16[ci];
      copy16(base, off, lds + static_cast<uint32_t>((ci * 4 + wave) * 64 * 16));
    }
  };

  // Score A fragment (key row l31, k-step ks) of the tile at T.
  const int g = half ^ swz(l31);
  auto rd_k = [&](const char* T, int ks) -> bf16x8_t {
    return *reinterpret_cast<const bf16x8_t*>(T + (l31 * kCPR + (ks >> 2) * 8 + ((2 * (ks & 3)) ^ g)) * 16);
  };
  // Value A fragment (latent tile 8*kh + m, key k-step jj): two transposing
  // reads, key rows 16jj + 4h + k and 16jj + 8 + 4h + k.  Byte offsets per
  // (jj, second read, m odd).
  const int trk = (lane & 15) >> 2, trq = lane & 3, trg = (lane >> 4) & 1;
  uint32_t tr_off[2][2][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int row = 16 * jj + 8 * rd + 4 * half + trk;
#pragma unroll
      for (int mo = 0; mo < 2; ++mo)
        tr_off[jj][rd][mo] = static_cast<uint32_t>(
            row * kCPR * 16 + ((4 * mo + 2 * trg + (trq >> 1)) ^ swz(row)) * 16 + 8 * (trq & 1));
    }
  auto rd_v = [&](const char* T, int m, int jj) -> bf16x8_t {
    const char* bb = T + 128 * (4 * kh + (m >> 1));
    const i16x4_t lo = read_tr(bb + tr_off[jj][0][m & 1]);
    const i16x4_t hi = read_tr(bb + tr_off[jj][1][m & 1]);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t oacc[kMTW];   // O^T tiles: latent tile 8*kh + m, this wave's rows
  float m_run = -INFINITY;   // reference max of this lane's row (scaled, base 2)
  float l_part;          // this lane's share of its row sum
  float m_seen;
  const float c = p.scale_log2;

  // Step i: scores of tile i; wait for this wave's copies of tile i+1;
  // barrier; copies of tile i+3 into tile i's buffer; softmax and values.
  auto tile = [&](int i, bool first) {
    const char* T = reinterpret_cast<const char*>(&ktile[i % kNB][0]);
    f32x16_t sp = {};
    bf16x8_t vf[kMTW][2];
    bf16x8_t kf[3];
    kf[0] = rd_k(T, ks_of(0));
    kf[1] = rd_k(T, ks_of(1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kKW; ++j) {
      const bf16x8_t a = kf[j % 3];
      if (j + 2 < kKW) kf[(j + 2) % 3] = rd_k(T, ks_of(j + 2));
      if (j < 16) vf[j >> 1][j & 1] = rd_v(T, j >> 1, j & 1);
      sp = mfma(a, qf[j], sp);
      __builtin_amdgcn_sched_barrier(0);
    }
    float4* mine = &part[i & 1][wave][0][0];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      mine[r4 * 64 + lane] = make_float4(sp[4 * r4], sp[4 * r4 + 1], sp[4 * r4 + 2], sp[4 * r4 + 3]);
    if (i + 2 < ntiles) wait_vm<kIPT>(); else wait_vm<0>();
    barrier();           // partials visible; tile i+1 in for every wave; tile i's buffer free
    if (i + kNB < ntiles) copy_tile(i + kNB, i % kNB);
    const float4* other = &part[i & 1][wave ^ 2][0][0];
    float s[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 v = other[r4 * 64 + lane];
      s[4 * r4] = sp[4 * r4] + v.x;
      s[4 * r4 + 1] = sp[4 * r4 + 1] + v.y;
      s[4 * r4 + 2] = sp[4 * r4 + 2] + v.z;
      s[4 * r4 + 3] = sp[4 * r4 + 3] + v.w;
    }
    // scaled scores; register r holds key 32i + 8*(r/4) + 4*half + r%4,
    // visible to this row while it is <= pos (computed, then selected)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      s[q] *= c;
      asm volatile("" : "+v"(s[q]));
    }
    const int lim = pos + 1 - i * kT - 4 * half;
#pragma unroll
    for (int q = 0; q < 16; ++q) s[q] = (8 * (q >> 2) + (q & 3) < lim) ? s[q] : -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, s[q]);
    mx = both_halves_max(mx);
    m_run = first ? fmaxf(m_run, mx) : m_run;
    m_seen = (!first && mx > m_run + kRescale) ? fmaxf(m_seen, mx) : m_seen;
    bf16x8_t pn[2];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float pv = __builtin_amdgcn_exp2f(s[q] - m_run);
      l_part += pv;
      pn[q >> 3][q & 7] = static_cast<__bf16>(pv);
    }
#pragma unroll
    for (int m = 0; m < kMTW; ++m)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) oacc[m] = mfma(vf[m][jj], pn[jj], oacc[m]);
  };

  bool first_pass = true;
  while (true) {
#pragma unroll
    for (int m = 0; m < kMTW; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) oacc[m][q] = 0.f;
    l_part = 0.f;
    m_seen = -INFINITY;
#pragma unroll
    for (int t = 0; t < kNB; ++t)
      if (t < ntiles) copy_tile(t, t);
    // tile 0 in (tiles 1 and 2 may be in flight)
    if (ntiles >= 3) wait_vm<2 * kIPT>(); else if (ntiles == 2) wait_vm<kIPT>(); else wait_vm<0>();
    barrier();
#pragma nounroll
    for (int i = 0; i < ntiles; ++i) tile(i, first_pass && i == 0);
    const bool over = __ballot(m_seen != -INFINITY) != 0ull;
    if (lane == 0) over_flag[wave] = over ? 1 : 0;
    barrier();           // also: every wave is done with every K buffer
    const bool again = (over_flag[0] | over_flag[1] | over_flag[2] | over_flag[3]) != 0;
    if (!again) break;
    m_run = fmaxf(m_run, m_seen);
    first_pass = false;
    barrier();           // every wave has read the flags before they are written again
  }

  // ---- this block's rows: o = U / l, lse = m + log l (natural log) ----
  const float l_tot = both_halves_sum(l_part);
  if (!real) return;
  if (p.lse != nullptr && kh == 0 && half == 0)
    p.lse[(static_cast<int64_t>(b) * p.max_len + pos) * p.heads + hd] = (m_run + __log2f(l_tot)) * kLn2;
  const float inv_l = 1.0f / l_tot;
  char* orow = static_cast<char*>(p.out) +
               (b * p.o_b + static_cast<int64_t>(pos) * p.o_s + static_cast<int64_t>(hd) * p.o_h) *
                   (kOutBf16 ? 2 : 4);
  // register q of latent tile m holds column 32*(8kh + m) + 8*(q/4) + 4*half + q%4
#pragma unroll
  for (int m = 0; m < kMTW; ++m)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int col = 32 * (kMTW * kh + m) + 8 * q4 + 4 * half;
      const float v0 = oacc[m][4 * q4] * inv_l, v1 = oacc[m][4 * q4 + 1] * inv_l;
      const float v2 = oacc[m][4 * q4 + 2] * inv_l, v3 = oacc[m][4 * q4 + 3] * inv_l;
      if constexpr (kOutBf16) {
        const uint32_t w0 = static_cast<uint32_t>(f32_to_bf16(v0)) | (static_cast<uint32_t>(f32_to_bf16(v1)) << 16);
        const uint32_t w1 = static_cast<uint32_t>(f32_to_bf16(v2)) | (static_cast<uint32_t>(f32_to_bf16(v3)) << 16);
        *reinterpret_cast<uint2*>(orow + col * 2) = make_uint2(w0, w1);
      } else {
        *reinterpret_cast<float4*>(orow + col * 4) = make_float4(v0, v1, v2, v3);
      }
    }
}

}  // namespace

hipError_t launch_mla_prefill(const PrefillParams& p, hipStream_t s) {
  const int64_t n_rb = (static_cast<int64_t>(p.max_len) * p.heads + kRows - 1) / kRows;
  const int64_t grid = n_rb * p.batch;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (p.out_bf16)
    hipLaunchKernelGGL(mla_prefill_kernel<true>, dim3(static_cast<uint32_t>(grid)), dim3(kNT), 0, s, p,
                       static_cast<int>(n_rb));
  else
    hipLaunchKernelGGL(mla_prefill_kernel<false>, dim3(static_cast<uint32_t>(grid)), dim3(kNT), 0, s, p,
                       static_cast<int>(n_rb));
  return hipGetLastError();
}

}  // namespace tpla
