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
// at L2; the merger reads the partials with ordinary loads, which its L1
// cannot serve from a stale line because no workgroup reads a partial before
// its merger does.  (A device-scope fence would instead write back and
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
// issued.  Returns false on the partitions that only contribute (they have
// raised their flag and may exit), true on the merger once every other
// partition's flag is up; *poisoned is then true if the wait gave up.
// timed_out: one LDS int the caller no longer uses (written after the first
// barrier here).
__device__ __forceinline__ bool splitk_arrive(uint64_t* flags, int pi, int np, uint64_t epoch,
                                              bool* poisoned, int* timed_out) {
  __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores are complete
  __syncthreads();                 // ... and every wave's
  if (pi != np - 1) {
    if (threadIdx.x == 0)
      __hip_atomic_exchange(flags + pi, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return false;
  }
  if (threadIdx.x < 64) {
    // wave 0: lane k watches partition k's flag (np <= 64)
    const bool mine = (int)threadIdx.x < np - 1;
    bool late = true;
    for (int spin = 0; spin < (1 << 20); ++spin) {
      const uint64_t f = mine ? __hip_atomic_fetch_or(flags + threadIdx.x, 0ull, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                              : epoch;
      if (__builtin_amdgcn_ballot_w64(f != epoch) == 0) {
        late = false;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (mine) __hip_atomic_exchange(flags + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) *timed_out = late;
  }
  __syncthreads();
  *poisoned = *timed_out != 0;
  return true;
}

// Merge of a group's split-K partials: out = sum_pi exp(lse_pi - M) o_pi /
// sum_pi exp(lse_pi - M) over the np partitions, in partition order
// (deterministic whichever partition merges); lse = -inf carries no weight.
// The group's nc columns (row col_row(c), head col_head(c)) are spread
// over the nthreads threads: 32 / CH threads per column, each taking CH
// chunks of 4 consecutive dims.  Partitions are read KB = 32 / CH at a
// time, every load of a batch in flight together, with a running maximum
// (the sums so far are rescaled when a batch raises it).
// part_o [np][rcap][H][128], part_lse [np][rcap][H], out bf16 [rows][H][128].
template <int CH, class ColRow, class ColHead>
__device__ void splitk_merge(const float* part_o, const float* part_lse, uint16_t* out, int H,
                             int rcap, int np, int nc, ColRow col_row, ColHead col_head, int tid,
                             bool poisoned) {
  constexpr int L = 32 / CH;          // threads per column
  constexpr int KB = 32 / CH;         // partitions per batch: 32 loads of 16 bytes
  const int c = tid / L;
  if (c >= nc) return;
  const int d0 = (tid % L) * 4 * CH;
  const size_t col = (size_t)col_row(c) * H + col_head(c);
  const size_t pstride = (size_t)rcap * H;
  f32x4 acc[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float den = 0.f, M = neg_inf();
  for (int k0 = 0; k0 < np; k0 += KB) {
    float lk[KB];
    f32x4 v[KB][CH];
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      const int k = min(k0 + q, np - 1);   // past np: re-read the last one, weight 0
      lk[q] = part_lse[(size_t)k * pstride + col];
      const float* po = part_o + ((size_t)k * pstride + col) * kDim + d0;
#pragma unroll
      for (int j = 0; j < CH; ++j) v[q][j] = *reinterpret_cast<const f32x4*>(po + 4 * j);
    }
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
  }
  const float dinv = poisoned ? __builtin_nanf("") : den > 0.f ? 1.f / den : 0.f;
  uint16_t* op = out + col * kDim + d0;
#pragma unroll
  for (int j = 0; j < CH; ++j)
    *reinterpret_cast<u32x2*>(op + 4 * j) =
        u32x2{pack_bf16(acc[j][0] * dinv, acc[j][1] * dinv), pack_bf16(acc[j][2] * dinv, acc[j][3] * dinv)};
}

}  // namespace msa
