// Work units of a split-K decode launch, derived on the device from the
// sequence lengths: every workgroup derives the same map, so no planning
// launch and no host copy of the lengths is needed.
//
// Sequence b has T_b = ceil(L_b / 64) tiles of 64 tokens (L_b clamped as
// the kernels clamp it).  It is cut into n_b = ceil(T_b / c) units of c
// tiles (the last one shorter), numbered sequence by sequence, so sequence
// b owns units first_b .. first_b + n_b - 1 with first_b = sum_{b' < b} n_b'.
// Sequences without tokens own none.
//
// With a target N (about one unit per CU) the chunk c is the smallest for
// which sum_b n_b <= N: every unit then holds at most c tiles, and in a
// ragged batch short sequences no longer get the long sequences' chunk nor
// long ones a few oversized splits, so the CUs finish at about the same
// time.  c = ceil(sum T / (N - #non-empty)) always fits (each n_b is below
// T_b / c + 1), which bounds the search.  Without a target, c is the host's
// chunk: uniform splits, minus the units on tokens a sequence does not have.
// Either way c is capped at the kernel's largest unit, which may leave more
// than N units; the host sizes the launch for that bound.
#pragma once

#include "tpla_internal.h"

namespace tpla {

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active): DPP
// shifts within rows of 16 lanes, then each row's total broadcast into the
// rows above it.
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);    // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);    // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);    // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);    // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_scan_incl(v), 63);
}

struct WorkUnit {
  int b;        // sequence
  int t0, t1;   // its tokens [t0, t1)
};

// Clamped length of sequence b0 + lane (0 past the batch).
__device__ __forceinline__ int unit_len(const DecodeParams& p, int b0) {
  const int cap = max(0, min(p.max_seq_len, p.max_blocks * p.block_size));
  const int b = b0 + static_cast<int>(threadIdx.x & 63);
  return b < p.batch ? max(0, min(p.seq_lens[b], cap)) : 0;
}

// The chunk c of the map, in tiles (wave-uniform; len_of(b0) gives the
// lengths of sequences b0 + lane).
template <typename LenOf>
__device__ inline int unit_chunk(const DecodeParams& p, int max_tiles, LenOf len_of) {
  int c;
  if (p.unit_target > 0) {
    const int n_target = p.unit_target;
    int total = 0, nonempty = 0;
    for (int b0 = 0; b0 < p.batch; b0 += 64) {
      const int t = (len_of(b0) + 63) >> 6;
      total += wave_sum(t);
      nonempty += __popcll(__ballot(t > 0));
    }
    if (total == 0) {
      c = 1;
    } else if (nonempty >= n_target) {
      c = max_tiles;                          // one unit per sequence (or per max_tiles)
    } else {
      int hi = min(max_tiles, (total + (n_target - nonempty) - 1) / (n_target - nonempty));
      int lo = min(hi, max(1, (total + n_target - 1) / n_target));
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        int units = 0;
        for (int b0 = 0; b0 < p.batch; b0 += 64) units += wave_sum((((len_of(b0) + 63) >> 6) + mid - 1) / mid);
        if (units <= n_target) hi = mid;
        else lo = mid + 1;
      }
      c = lo;
    }
  } else {
    c = max(1, p.chunk >> 6);
  }
  return min(c, max_tiles);
}

// Unit su of the map (call with the whole wave active; every argument
// wave-uniform).  Returns false when su is past the last unit.  With
// table != nullptr the wave also writes table[2b] = first_b and
// table[2b + 1] = n_b for every sequence.
__device__ inline bool find_unit(const DecodeParams& p, int su, int max_tiles, int32_t* table,
                                 WorkUnit* w) {
  const int lane = static_cast<int>(threadIdx.x & 63);
  const int len0 = unit_len(p, 0);            // the first 64 sequences stay in a register
  auto len_of = [&](int b0) -> int { return b0 == 0 ? len0 : unit_len(p, b0); };
  const int c = unit_chunk(p, max_tiles, len_of);

  bool found = false;
  WorkUnit r{0, 0, 0};
  int base = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int len = len_of(b0);
    const int n = (((len + 63) >> 6) + c - 1) / c;
    const int incl = wave_scan_incl(n);
    const int first = base + incl - n;
    if (table != nullptr && b0 + lane < p.batch)
      reinterpret_cast<int2*>(table)[b0 + lane] = make_int2(first, n);
    const uint64_t hit = __ballot(n > 0 && su >= first && su < first + n);
    if (!found && hit != 0ull) {
      const int l = __builtin_ctzll(hit);
      const int f = __builtin_amdgcn_readlane(first, l);
      r.b = b0 + l;
      r.t0 = (su - f) * c * 64;
      r.t1 = min(__builtin_amdgcn_readlane(len, l), r.t0 + c * 64);
      found = true;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  *w = r;
  return found;
}

}  // namespace tpla
