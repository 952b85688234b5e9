// Split-K inside one launch: the partitions of a group of rows each store a
// partial result (normalised output and natural-log log-sum-exp, keyed on
// the ragged row, as the split-K combine takes them), and the group's last
// partition merges them -- no separate combine launch ("msa" page,
// speculative route: partials keyed on the ragged row, one reduce writes the
// ragged output).
//
// Placement.  The chip's 8 XCDs each have their own L2, and those caches
// are not coherent with each other.  The hardware runs workgroup i on XCD
// i mod 8, so the partitions of a group are given indices congruent modulo
// 8 (splitk_slot), which puts the whole exchange on one XCD and lets its L2
// be the point where the partitions meet: partials are ordinary stores (the
// vector L1 writes through to L2) whose completion a wave waits for before
// it raises its flag; flags are set and polled with atomics, which execute
// at L2; the merger reads the partial outputs with ordinary loads, which
// its L1 cannot serve from a stale line because no workgroup reads a
// partial output before its merger does (a column's 512 bytes share no
// cache line with another column), and the log-sum-exps, which do share
// lines between groups, with L2-coherent loads.  (A device-scope fence would instead write back and
// invalidate the whole L2 of the XCD; coherent cross-XCD stores and loads
// would go to memory behind the kernel's own streaming traffic.)
//
// Flags.  A partition's flag holds the call's epoch (never 0, new for every
// call), so whatever a workspace held before never reads as ready; the
// merger clears the flags it read, so a replay of a captured call (same
// epoch) does not find them set either.  The merger is the group's last
// partition, which only waits for workgroups of lower index on its own XCD,
// dispatched before it, so the wait ends; it is also bounded (about a
// second), after which the merged output is NaN rather than the kernel
// never ending.
#pragma once

#include "msa_common.h"

namespace msa {

constexpr int kXcdCount = 8;   // XCDs of the chip; workgroup i runs on XCD i mod 8

// Workgroup index -> (partition, group).  One partition: the identity.
// Several: groups go round the XCDs (group q on XCD q mod 8) and a group's
// partitions sit np * 8 indices apart, all on the group's XCD.  A launch
// with np > 1 has splitk_workgroups(groups, np) workgroups; indices whose
// group is >= groups are padding of the last round and do nothing.
__device__ __forceinline__ void splitk_slot(int idx, int np, int* pi, int* grp) {
  if (np == 1) {
    *pi = 0;
    *grp = idx;
    return;
  }
  const int xcd = idx % kXcdCount, s = idx / kXcdCount;
  *pi = s % np;
  *grp = (s / np) * kXcdCount + xcd;
}

inline size_t splitk_workgroups(size_t groups, int np) {
  return np == 1 ? groups : (groups + kXcdCount - 1) / kXcdCount * kXcdCount * (size_t)np;
}

// Called by every thread of the workgroup once its partial stores are
// issued.  The partitions that only contribute raise their flag and get
// false (they may exit); the merger gets true and waits in splitk_merge.
__device__ __forceinline__ bool splitk_arrive(uint64_t* flags, int pi, int np, uint64_t epoch) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete
  __syncthreads();                 // ... and every wave's
  if (pi != np - 1) {
    if (threadIdx.x == 0)
      __hip_atomic_exchange(flags + pi, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  return true;
}

// The merger's view of the other partitions' flags (wave 0: lane k watches
// partition k, np <= 64), shared through LDS: with wait set, spins until
// every flag is up and clears them (bounded: sh[2] is then set instead of
// the wait never ending); else one look.  Bit k of the result: partition k
// is done (the merger's own bit and bits >= np are set).  Every thread
// calls it.
__device__ __forceinline__ uint64_t splitk_flags(uint64_t* flags, int np, uint64_t epoch, bool wait,
                                                 int* sh) {
  if (threadIdx.x < 64) {
    const bool mine = (int)threadIdx.x < np - 1;
    uint64_t done = 0ull;
    bool late = wait;
    for (int spin = 0; spin < (wait ? (1 << 20) : 1); ++spin) {
      const uint64_t f = mine ? __hip_atomic_fetch_or(flags + threadIdx.x, 0ull, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                              : epoch;
      done = __builtin_amdgcn_ballot_w64(f == epoch);
      if (wait && done == ~0ull) {
        late = false;
        break;
      }
      if (wait) __builtin_amdgcn_s_sleep(2);
    }
    if (wait && mine) __hip_atomic_exchange(flags + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
      sh[0] = (int)(uint32_t)done;
      sh[1] = (int)(uint32_t)(done >> 32);
      sh[2] = late;
    }
  }
  __syncthreads();
  const uint64_t done = ((uint64_t)(uint32_t)sh[1] << 32) | (uint32_t)sh[0];
  __syncthreads();   // sh may be written again by the next call
  return done;
}

// The merger's half: out = sum_pi exp(lse_pi - M) o_pi / sum_pi exp(lse_pi -
// M) over the np partitions, in partition order (deterministic whichever
// partition merges); lse = -inf carries no weight.  The group's nc columns
// (row col_row(c), head col_head(c)) are spread over the nthreads threads:
// 32 / CH threads per column, each taking CH chunks of 4 consecutive dims.
// Partitions are read KB = 32 / CH at a time, every load of a batch in
// flight together, with a running maximum (the sums so far are rescaled
// when a batch raises it).  With np <= KB (one batch) the partials of the
// partitions already done when the merger arrives are requested before it
// waits for the others, so that their loads overlap the wait and only the
// late partitions' reads follow it.  Every thread of the workgroup calls
// this (it synchronises); sh: three ints of LDS.
// part_o [np][rcap][H][128], part_lse [np][rcap][H], out bf16 [rows][H][128].
template <int CH, class ColRow, class ColHead>
__device__ void splitk_merge(uint64_t* flags, uint64_t epoch, int* sh, const float* part_o,
                             const float* part_lse, uint16_t* out, int H, int rcap, int np, int nc,
                             ColRow col_row, ColHead col_head, int tid) {
  constexpr int L = 32 / CH;          // threads per column
  constexpr int KB = 32 / CH;         // partitions per batch: 32 loads of 16 bytes
  const int c = tid / L;
  const bool act = c < nc;
  const int d0 = (tid % L) * 4 * CH;
  const size_t col = act ? (size_t)col_row(c) * H + col_head(c) : 0;
  const size_t pstride = (size_t)rcap * H;
  f32x4 acc[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f, M = neg_inf();
  float lk[KB];
  f32x4 v[KB][CH];
  auto load = [&](int q, int k) {
    // the log-sum-exps of several groups' columns share cache lines, which
    // another merger on this CU may have brought into its L1 before this
    // group's partition wrote its value: read them at L2
    lk[q] = __hip_atomic_load(const_cast<float*>(part_lse) + (size_t)k * pstride + col,
                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float* po = part_o + ((size_t)k * pstride + col) * kDim + d0;
#pragma unroll
    for (int j = 0; j < CH; ++j) v[q][j] = *reinterpret_cast<const f32x4*>(po + 4 * j);
  };
  auto fold = [&](int k0) {
    float mb = M;
#pragma unroll
    for (int q = 0; q < KB; ++q)
      if (k0 + q < np) mb = fmaxf(mb, lk[q]);
    if (mb != M) {
      const float r = M == neg_inf() ? 0.f : __expf(M - mb);
      den *= r;
#pragma unroll
      for (int j = 0; j < CH; ++j) acc[j] *= r;
      M = mb;
    }
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      const float w = (k0 + q < np && lk[q] != neg_inf()) ? __expf(lk[q] - M) : 0.f;
      if (w != 0.f) {
        den += w;
#pragma unroll
        for (int j = 0; j < CH; ++j) acc[j] += w * v[q][j];
      }
    }
  };
  bool poisoned;
  if (np <= KB) {
    const uint64_t early = splitk_flags(flags, np, epoch, false, sh);
#pragma unroll
    for (int q = 0; q < KB; ++q)
      if (act && q < np && ((early >> q) & 1ull)) load(q, q);
    splitk_flags(flags, np, epoch, true, sh);
    poisoned = sh[2] != 0;   // (read before any later write: the next call of
                             //  splitk_flags is in another launch)
    if (!act) return;
#pragma unroll
    for (int q = 0; q < KB; ++q)
      if (q < np && !((early >> q) & 1ull)) load(q, q);
    fold(0);
  } else {
    splitk_flags(flags, np, epoch, true, sh);
    poisoned = sh[2] != 0;
    if (!act) return;
    for (int k0 = 0; k0 < np; k0 += KB) {
#pragma unroll
      for (int q = 0; q < KB; ++q) load(q, min(k0 + q, np - 1));   // past np: re-read the last one, weight 0
      fold(k0);
    }
  }
  const float dinv = poisoned ? __builtin_nanf("") : den > 0.f ? 1.f / den : 0.f;
  uint16_t* op = out + col * kDim + d0;
#pragma unroll
  for (int j = 0; j < CH; ++j)
    *reinterpret_cast<u32x2*>(op + 4 * j) =
        u32x2{pack_bf16(acc[j][0] * dinv, acc[j][1] * dinv), pack_bf16(acc[j][2] * dinv, acc[j][3] * dinv)};
}

}  // namespace msa
