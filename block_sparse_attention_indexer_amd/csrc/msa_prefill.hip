// Prefill-route kernels (more than 8 new tokens in some sequence):
//
//   * indexer_score_prefill_kernel -- block-max scoring as a tiled GEMM,
//     [tokens x index heads] . [positions x 128]^T on MFMA, with each K tile
//     staged once per workgroup in LDS and reused by 256 columns, and a
//     max-over-128-positions epilogue.
//   * prefill_plan_kernel -- the device-built sparse structure ("msa" page
//     of the MAX Mojo docs, prefill route: the run goes over a device CSR
//     that the host only sizes): for every (sequence, tile of tokens, KV
//     head) the ascending union of the blocks the tile's tokens selected,
//     the page of each, and a bit mask of which tokens selected it.
//   * attn_prefill3_kernel -- MFMA attention over each tile's union blocks;
//     K and V tiles are DMA'd into LDS once per workgroup and shared by its
//     sixteen waves, each wave skipping blocks none of its tokens selected.
//
// The indexer's K tile in LDS is 128 rows of 256 bytes; 16-byte column c of
// row pos is stored at column c ^ (pos & 15), so the 16 rows an MFMA
// A-operand read touches fall in distinct bank groups.  Both the indexer and
// the attention kernel fetch tiles by global->LDS DMA into a ring of stages,
// several blocks ahead of the one being computed.
#include <algorithm>

#include "msa_common.h"
#include "msa_kernels.h"
#include "msa_lds.h"

namespace msa {

__device__ __forceinline__ int k_off(int pos, int c16) { return pos * 256 + ((c16 ^ (pos & 15)) << 4); }

__device__ __forceinline__ u32x4 lds16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}

// ---------------------------------------------------------------------------
// Work lists.  The prefill grids would otherwise be over-launched from host
// bounds (every sequence padded to the longest), leaving long periodic runs
// of empty workgroups between the working ones, which the hardware places
// poorly.  Instead one workgroup lists the non-empty tiles heaviest first
// (counting sort on an integer cost) and a fixed number of persistent
// workgroups take tiles from the list with an atomic counter.  The list and
// the counter live in the caller's workspace; the scheduler resets the
// counter, so no memset is needed.
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;

// cost(i) > 0 for items to run; maxcost bounds every cost.  hist: LDS of
// maxcost + 1 ints.
template <class Cost>
__device__ void schedule_by_cost(int nitems, int maxcost, Cost cost, int32_t* list, int32_t* sched,
                                 int* hist) {
  __shared__ int wsum[kSchedThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = maxcost + 1;
  for (int i = tid; i < m; i += kSchedThreads) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < nitems; i += kSchedThreads) {
    const int c = min(cost(i), maxcost);
    if (c > 0) atomicAdd(&hist[maxcost - c], 1);      // index 0 = heaviest
  }
  __syncthreads();
  // exclusive scan of hist (in place), each thread owning a contiguous run
  const int per = (m + kSchedThreads - 1) / kSchedThreads;
  int local = 0;
  for (int j = 0; j < per; ++j) {
    const int idx = tid * per + j;
    if (idx < m) local += hist[idx];
  }
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  int run = base + incl - local;
  for (int j = 0; j < per; ++j) {
    const int idx = tid * per + j;
    if (idx < m) {
      const int h = hist[idx];
      hist[idx] = run;
      run += h;
    }
  }
  __syncthreads();
  for (int i = tid; i < nitems; i += kSchedThreads) {
    const int c = min(cost(i), maxcost);
    if (c > 0) list[atomicAdd(&hist[maxcost - c], 1)] = i;
  }
  if (tid == kSchedThreads - 1) {
    int total = 0;
    for (int w = 0; w < kSchedThreads / 64; ++w) total += wsum[w];
    sched[0] = total;
    sched[1] = 0;
  }
}

// ---------------------------------------------------------------------------
// XCD-clustered work lists.  The chip's 256 CUs sit in 8 XCDs, each with
// its own L2; a prefill tile streams the blocks of one (sequence, KV head),
// and tiles of the same (sequence, head) stream mostly the same blocks in the
// same ascending order.  The slots are therefore taken in head-major order
// ((head, sequence, tile)), cut into kXcds runs of equal total cost, and run
// i is listed for XCD i (heaviest first inside each list), so that the CUs of
// one XCD work on tiles of the same head and sequence at the same time and
// their block streams meet in that XCD's L2 instead of each coming from the
// last-level cache.  A workgroup takes from its own XCD's list first, then
// from the others' once its own is exhausted.  sched: [0, 8) items per list,
// [8, 16) next item to take, [16, 24) first list entry of each list.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kXcdBuckets = 1024;   // cost buckets per XCD list

// XCD of the calling workgroup, from the hardware register (HW_REG_XCC_ID).
__device__ __forceinline__ int xcd_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) & (kXcds - 1);
}

// Slot i = ((b * ntiles + tile) * H + h), nslots = nbt * H with nbt =
// batch * ntiles; cost(i) > 0 for slots to run, cost <= maxcost.  hist: LDS
// of kXcds * kXcdBuckets ints.
template <class Cost>
__device__ void schedule_by_xcd(int nbt, int H, int maxcost, Cost cost, int32_t* list,
                                int32_t* sched, int* hist) {
  __shared__ int wsum[kSchedThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nslots = nbt * H;
  int shift = 0;
  while ((maxcost >> shift) >= kXcdBuckets) ++shift;
  for (int i = tid; i < kXcds * kXcdBuckets; i += kSchedThreads) hist[i] = 0;
  // each thread owns a contiguous run of the head-major order
  const int per = (nslots + kSchedThreads - 1) / kSchedThreads;
  const int k0 = min(nslots, tid * per), k1 = min(nslots, k0 + per);
  auto slot_of = [&](int k) { return (k % nbt) * H + k / nbt; };
  long long local = 0;
  for (int k = k0; k < k1; ++k) local += max(0, cost(slot_of(k)));
  // exclusive scan of the runs' costs (64-bit: a wave sums into 32 bits, the
  // waves' totals into 64)
  long long incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const long long y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __shared__ long long wsum64[kSchedThreads / 64];
  if (lane == 63) wsum64[wave] = incl;
  __syncthreads();
  long long base = 0, total = 0;
  for (int w = 0; w < kSchedThreads / 64; ++w) {
    if (w < wave) base += wsum64[w];
    total += wsum64[w];
  }
  base += incl - local;
  const long long tot = max(1LL, total);
  auto bin_of = [&](long long prefix, int c) {
    // the run an item's midpoint falls in; 2 (prefix) + c < 2^63 always
    const int x = (int)((2 * prefix + c) * kXcds / (2 * tot));
    const int bucket = min(kXcdBuckets - 1, min(c, maxcost) >> shift);
    return min(x, kXcds - 1) * kXcdBuckets + (kXcdBuckets - 1 - bucket);   // heaviest first
  };
  {
    long long run = base;
    for (int k = k0; k < k1; ++k) {
      const int c = cost(slot_of(k));
      if (c > 0) atomicAdd(&hist[bin_of(run, c)], 1);
      run += max(0, c);
    }
  }
  __syncthreads();
  // exclusive scan of the histogram in place; list starts per XCD
  const int m = kXcds * kXcdBuckets;
  const int hper = m / kSchedThreads;                 // 8 entries per thread
  int hl = 0;
  for (int j = 0; j < hper; ++j) hl += hist[tid * hper + j];
  int hi = hl;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(hi, off);
    if (lane >= off) hi += y;
  }
  if (lane == 63) wsum[wave] = hi;
  __syncthreads();
  int hb = 0;
  for (int w = 0; w < wave; ++w) hb += wsum[w];
  int hrun = hb + hi - hl;
  for (int j = 0; j < hper; ++j) {
    const int idx = tid * hper + j;
    if (idx % kXcdBuckets == 0) sched[16 + idx / kXcdBuckets] = hrun;
    const int h = hist[idx];
    hist[idx] = hrun;
    hrun += h;
  }
  __syncthreads();
  {
    long long run = base;
    for (int k = k0; k < k1; ++k) {
      const int i = slot_of(k);
      const int c = cost(i);
      if (c > 0) list[atomicAdd(&hist[bin_of(run, c)], 1)] = i;
      run += max(0, c);
    }
  }
  __syncthreads();
  if (tid < kXcds) {
    // after the fill, hist[x * kXcdBuckets + last] holds the end of list x
    sched[tid] = hist[tid * kXcdBuckets + kXcdBuckets - 1] - sched[16 + tid];
    sched[8 + tid] = 0;
  }
}

// Persistent loop helper for XCD-clustered lists: the next slot for this
// workgroup (its own XCD's list first), or -1 when every list is exhausted
// (uniform across the workgroup).
__device__ __forceinline__ int take_slot_xcd(int32_t* sched, const int32_t* list, int xcd,
                                             int* item_s) {
  if (threadIdx.x == 0) {
    int got = -1;
    for (int j = 0; j < kXcds && got < 0; ++j) {
      const int x = (xcd + j) & (kXcds - 1);
      const int n = __atomic_load_n(&sched[x], __ATOMIC_RELAXED);
      if (__atomic_load_n(&sched[8 + x], __ATOMIC_RELAXED) >= n) continue;
      const int k = atomicAdd(&sched[8 + x], 1);
      if (k < n) got = list[sched[16 + x] + k];
    }
    *item_s = got;
  }
  __syncthreads();
  const int v = *item_s;
  __syncthreads();
  return v;
}

// Persistent loop helper: returns the next item index, or -1 when the list
// is exhausted (uniform across the workgroup).
__device__ __forceinline__ int take_item(int32_t* sched, int* item_s) {
  if (threadIdx.x == 0) {
    const int k = atomicAdd(&sched[1], 1);
    *item_s = k < sched[0] ? k : -1;
  }
  __syncthreads();
  const int k = *item_s;
  __syncthreads();
  return k;
}

// ---------------------------------------------------------------------------
// Prefill indexer: a tile item is (sequence, tile of tq tokens, index-K head
// hk); its workgroup of 4 waves x 64 columns scores it, a column being a
// (token, KV head) pair.  Block maxima are collected over 16-block windows
// (lane group g keeps blocks 4g..4g+3 of the window) and written as 16-byte
// pieces into rows padded to a multiple of 16 blocks.
// ---------------------------------------------------------------------------
struct IdxTile {
  int b, tile, hk, r0, n, c, t0, ntok, blk_lo, blk_hi;
};

__device__ __forceinline__ IdxTile idx_tile_of(const IndexerParams& p, int item) {
  IdxTile t;
  t.hk = item % p.H_ik;
  const int bt = item / p.H_ik;
  t.tile = bt % p.ntiles;
  t.b = bt / p.ntiles;
  t.r0 = p.rg.offs[t.b];
  t.n = min(p.rg.offs[t.b + 1] - t.r0, p.rg.max_seq);
  t.c = p.rg.clen[t.b];
  t.t0 = t.tile * p.tq;
  t.ntok = min(p.tq, t.n - t.t0);
  const int nb_last = t.ntok > 0 ? (t.c + t.t0 + t.ntok - 1) / kBlock + 1 : 0;
  t.blk_lo = p.init;
  t.blk_hi = nb_last > p.top_k ? min(nb_last - p.local, p.nbmax) : 0;
  return t;
}

__global__ __launch_bounds__(kSchedThreads) void indexer_schedule_kernel(IndexerParams p) {
  extern __shared__ int hist[];
  const int nitems = p.rg.batch * p.ntiles * p.H_ik;
  schedule_by_cost(nitems, p.nbmax,
                   [&](int i) {
                     const IdxTile t = idx_tile_of(p, i);
                     return t.ntok > 0 ? max(0, t.blk_hi - t.blk_lo) : 0;
                   },
                   p.worklist, p.sched, hist);
}

constexpr int kIdxTileBytes = kBlock * 256;   // one BF16 index-K tile
// One FP8 index-K stage: 16 fragments of 1 KiB (fragment 2 pt + h: lane
// (l16, g) holds row 16 pt + l16, code bytes 16 g + 64 h .. + 15, i.e. the
// k-steps 2h and 2h + 1), then the tile's 128 float32 scales.
constexpr int kIdxStageFp8 = kBlock * 128 + kBlock * 4;

template <int NST, bool FP8>
__device__ void indexer_prefill_tile(const IndexerParams& p, const IdxTile& T, char* ring,
                                     int32_t* pages_lds) {
  constexpr int STAGE = FP8 ? kIdxStageFp8 : kIdxTileBytes;
  constexpr int ESZ = FP8 ? 1 : 2;                  // bytes per index-K element
  constexpr int kDmaPerBlock = FP8 ? 5 : 8;         // DMA instructions per wave per tile
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform((int)(tid >> 6));
  const int l16 = lane & 15, g = lane >> 4;
  const int hpi = p.H_kv / p.H_ik;
  const int blk_lo = T.blk_lo, blk_hi = T.blk_hi;
  const int nblk = blk_hi - blk_lo;

  u32x4 qf[4][4];
  int plim[4], orow[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int cc = wave * 64 + ct * 16 + l16;
    const int t = cc / hpi;
    const int h = T.hk + p.H_ik * (cc % hpi);
    const bool ok = t < T.ntok;
    plim[ct] = ok ? T.c + T.t0 + t : -1;
    orow[ct] = ok ? (T.r0 + T.t0 + t) * p.H_kv + h : 0;
    const uint16_t* qp = p.q_idx + (size_t)orow[ct] * kDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // contraction dims of k-step s for lane group g: BF16 32s + 8g + j;
      // FP8 (fragment order) 16g + 64 (s / 2) + 8 (s % 2) + j
      const int d0 = FP8 ? 16 * g + 64 * (s >> 1) + 8 * (s & 1) : 32 * s + 8 * g;
      qf[ct][s] = ok ? ld16(qp + d0) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int p_first = T.c + T.t0;

  const char* pool = static_cast<const char*>(p.ik.data);
  const uint32_t ts = (uint32_t)p.ik.token_stride * ESZ;
  const size_t head_bytes = (size_t)T.hk * p.ik.head_stride * ESZ;
  const size_t page_bytes = (size_t)p.ik.page_stride * ESZ;
  const int32_t* trow = p.rg.table + (size_t)T.b * p.rg.stride;
  const int npages = p.ik.num_pages;
  // The page ids of the whole block range go to LDS first, so the loop
  // never waits on a global load to learn where its next tile is.
  for (int i = tid; i < nblk; i += 256) pages_lds[i] = trow[blk_lo + i];
  __syncthreads();

  // DMA.  BF16: instruction i of this wave fills tile rows 32 wave + 4i ..
  // + 3; a lane lands in row + lane / 16 at physical column lane % 16 and
  // fetches the logical column that the swizzle puts there.  FP8: the wave
  // fills fragments 4 wave + i (i < 4), and its lanes 0..7 fetch scales
  // 32 wave .. + 31.
  constexpr int kDmaK = FP8 ? 4 : 8;
  uint32_t doff[kDmaK];
#pragma unroll
  for (int i = 0; i < kDmaK; ++i) {
    if constexpr (FP8) {
      const int f = 4 * wave + i;
      doff[i] = (16 * (f >> 1) + l16) * ts + 16 * g + 64 * (f & 1);
    } else {
      const int row = 32 * wave + 4 * i + (lane >> 4);
      doff[i] = row * ts + ((((lane & 15) ^ (row & 15))) << 4);
    }
  }
  auto stage = [&](int rel, int buf) {
    int pg = pages_lds[rel];
    if ((unsigned)pg >= (unsigned)npages) {
      pg = 0;
      if (lane == 0) report_error(p.err, kErrPage);
    }
    const char* kb = pool + (size_t)pg * page_bytes + head_bytes;
    char* st = ring + buf * STAGE;
#pragma unroll
    for (int i = 0; i < kDmaK; ++i)
      dma16(kb + doff[i], st + (FP8 ? (4 * wave + i) * 1024 : (32 * wave + 4 * i) * 256));
    if constexpr (FP8) {
      const float* sb = p.ik.scale + (size_t)pg * p.ik.scale_page_stride +
                        (size_t)T.hk * p.ik.scale_head_stride + 32 * wave;
      if (lane < 8) dma16(reinterpret_cast<const char*>(sb + 4 * lane), st + kBlock * 128 + 128 * wave);
    }
  };
#pragma unroll
  for (int j = 0; j < NST - 1; ++j)
    if (j < nblk) stage(j, j);

  float win[4][4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) win[ct][j] = 0.f;

  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const int e = blk - blk_lo;
    const int buf = e % NST;
    // this wave's DMA of block e has landed (the 8 DMA instructions of each
    // younger block may still be in flight), then everyone's has
    if (NST > 2 && e + NST - 2 < nblk) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerBlock * (NST - 2)));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    if (e + NST - 1 < nblk) stage(e + NST - 1, (e + NST - 1) % NST);
    const char* kt = ring + buf * STAGE;
    const bool clip = blk * kBlock + kBlock - 1 > p_first;
    float mx[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) mx[ct] = neg_inf();
#pragma unroll 2
    for (int pt = 0; pt < 8; ++pt) {
      f32x4 acc[4];
      u32x4 w8 = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 a;
        if constexpr (FP8) {
          if ((s & 1) == 0) w8 = lds16(kt, (2 * pt + (s >> 1)) * 1024 + 16 * lane);
          a = fp8x8_to_bf16x8((s & 1) ? u32x2{w8.z, w8.w} : u32x2{w8.x, w8.y});
        } else {
          a = lds16(kt, k_off(16 * pt + l16, 4 * s + g));
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[ct] = mfma_bf16(a, qf[ct][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[ct]);
      }
      if constexpr (FP8) {
        // rows 4g .. 4g + 3 of this C tile are positions 16 pt + 4g + i:
        // value = code * scale, so each row's dot product takes its scale
        const f32x4 sc = *reinterpret_cast<const f32x4*>(kt + kBlock * 128 + (16 * pt + 4 * g) * 4);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = acc[ct] * sc;
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        if (clip) {
          const int lim = plim[ct] - (blk * kBlock + 16 * pt + 4 * g);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i > lim) acc[ct][i] = neg_inf();
        }
        mx[ct] = fmaxf(mx[ct], fmaxf(fmaxf(acc[ct][0], acc[ct][1]), fmaxf(acc[ct][2], acc[ct][3])));
      }
    }
    const int w = blk & 15;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const float m = colgroup_max(mx[ct]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (g == (w >> 2) && (w & 3) == j) win[ct][j] = m;
    }
    if (w == 15 || blk + 1 == blk_hi) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (plim[ct] >= 0)
          *reinterpret_cast<f32x4*>(p.scores + (size_t)orow[ct] * p.score_stride + (blk & ~15) + 4 * g) =
              f32x4{win[ct][0], win[ct][1], win[ct][2], win[ct][3]};
    }
  }
  // every wave is done with the ring before the next tile's DMAs start
  __syncthreads();
}

template <int NST, bool FP8>
__global__ __launch_bounds__(256) void indexer_score_prefill_kernel(IndexerParams p) {
  __shared__ __attribute__((aligned(16))) char ring[NST * (FP8 ? kIdxStageFp8 : kIdxTileBytes)];
  __shared__ int item_s;
  extern __shared__ int32_t pages_lds[];   // page ids of the tile's block range
  for (;;) {
    const int k = take_item(p.sched, &item_s);
    if (k < 0) break;
    const IdxTile T = idx_tile_of(p, p.worklist[k]);
    indexer_prefill_tile<NST, FP8>(p, T, ring, pages_lds);
  }
}

int prefill_indexer_tile(int H_kv, int H_ik) { return 256 / (H_kv / H_ik); }

hipError_t launch_indexer_prefill(const IndexerParams& p, int num_cus, hipStream_t s) {
  hipLaunchKernelGGL(indexer_schedule_kernel, dim3(1), dim3(kSchedThreads),
                     (size_t)(p.nbmax + 1) * sizeof(int), s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Two workgroups per CU when their rings fit in 160 KiB of LDS (two waves
  // per SIMD hide each other's LDS and MFMA latencies), the deeper ring
  // first; otherwise one workgroup per CU with as deep a ring as fits.
  const size_t pages = (size_t)p.nbmax * sizeof(int32_t);
  const size_t lds_cu = 160 * 1024;
  const size_t stage = p.ik_fp8 ? kIdxStageFp8 : kIdxTileBytes;
  auto fits = [&](int nst, int per_cu) { return per_cu * (nst * stage + pages + 64) <= lds_cu; };
  const dim3 block(256);
#define MSA_IDX_LAUNCH(NST, PER_CU)                                                                 \
  do {                                                                                            \
    if (p.ik_fp8)                                                                                 \
      hipLaunchKernelGGL((indexer_score_prefill_kernel<NST, true>), dim3((PER_CU) * num_cus), block, \
                         pages, s, p);                                                            \
    else                                                                                          \
      hipLaunchKernelGGL((indexer_score_prefill_kernel<NST, false>), dim3((PER_CU) * num_cus), block, \
                         pages, s, p);                                                            \
  } while (0)
  if (fits(4, 2)) MSA_IDX_LAUNCH(4, 2);
  else if (fits(2, 2)) MSA_IDX_LAUNCH(2, 2);
  else if (fits(4, 1)) MSA_IDX_LAUNCH(4, 1);
  else MSA_IDX_LAUNCH(3, 1);
#undef MSA_IDX_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill plan of one (sequence, tile, KV head) slot, built by the calling
// workgroup (any number of waves): the ascending union of the blocks the
// tile's tokens selected, each block's page and the mask of the tokens that
// chose it.  member: LDS of nbmax words (an LDS-space pointer, so that no
// generic-pointer conversion is involved).
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ void build_plan(const AttnParams& p, int b, int tile, int h, lds_u32* member) {
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t slot = ((size_t)b * p.ntiles + tile) * p.H_kv + h;
  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  const int t0 = tile * p.tq;
  if (t0 >= n) {
    if (tid == 0) p.plan_cnt[slot] = 0;
    return;
  }
  const int c = p.rg.clen[b];
  const int ntok = min(p.tq, n - t0);
  const int nb_last = min((c + t0 + ntok - 1) / kBlock + 1, p.nbmax);
  // more new tokens than the host bound, or blocks past the table (clipped)
  if (tid == 0 && h == 0 &&
      ((tile == 0 && p.rg.offs[b + 1] - r0 > p.rg.max_seq) || (c + t0 + ntok - 1) / kBlock >= p.nbmax))
    report_error(p.err, kErrLength);
  for (int i = tid; i < nb_last; i += blockDim.x) member[i] = 0u;
  __syncthreads();
  for (int k = tid; k < ntok * p.top_k; k += blockDim.x) {
    const int tl = k / p.top_k;
    const int nbt = min((c + t0 + tl) / kBlock + 1, p.nbmax);
    const int id = p.d_indices[((size_t)(r0 + t0 + tl) * p.H_kv + h) * p.top_k + k % p.top_k];
    if (id >= 0 && id < nbt)
      __hip_atomic_fetch_or(member + id, 1u << tl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  if (tid < 64) {   // the first wave compacts the union
    int32_t* ids = p.plan_ids + slot * p.nbmax;
    int32_t* pgs = p.plan_pages + slot * p.nbmax;
    uint32_t* msk = p.plan_mask + slot * p.nbmax;
    const int32_t* trow = p.rg.table + (size_t)b * p.rg.stride;
    int cnt = 0;
    // dense-causal: every token chose every block it sees (block i is seen
    // by tokens c + t0 + tl >= 128 i of the tile)
    const uint32_t all_tok = ntok >= 32 ? ~0u : (1u << ntok) - 1u;
    bool dense = true;
    for (int base = 0; base < nb_last; base += 64) {
      const int i = base + lane;
      const uint32_t m = i < nb_last ? member[i] : 0u;
      const int lo = min(31, max(0, i * kBlock - (c + t0)));
      const uint32_t seen = i < nb_last ? all_tok & ~((1u << lo) - 1u) : 0u;
      dense = dense && ballot(m != seen) == 0;
      const uint64_t bal = ballot(m != 0u);
      if (m) {
        const int pos = cnt + mask_rank(bal);
        const int pg = trow[i];
        ids[pos] = i;
        pgs[pos] = (unsigned)pg < (unsigned)p.k.num_pages ? pg : -1;
        if ((unsigned)pg >= (unsigned)p.k.num_pages) report_error(p.err, kErrPage);
        msk[pos] = m;
      }
      cnt += __popcll(bal);
    }
    if (lane == 0) p.plan_cnt[slot] = cnt | (dense && cnt > 0 ? kPlanDense : 0);
    if (cnt == 0) {
      // No token of the tile has a visible block: the work list holds
      // non-empty slots only, so the tile's rows of this head group get
      // their result, 0, here.  256-byte rows, written as 16-byte pieces.
      const int pieces = ntok * p.G * (kDim * 2 / 16);
      for (int i = lane; i < pieces; i += 64) {
        const int row = i / (p.G * 16), head = (i / 16) % p.G, col = i % 16;
        uint16_t* op = p.out + ((size_t)(r0 + t0 + row) * p.H_q + h * p.G + head) * kDim + 8 * col;
        *reinterpret_cast<u32x4*>(op) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
}

// Prefill plan launch: one wave per (sequence, tile, KV head).
__global__ __launch_bounds__(64) void prefill_plan_kernel(AttnParams p) {
  extern __shared__ uint32_t member[];   // [nbmax] token mask per block
  int x = blockIdx.x;
  const int h = x % p.H_kv;
  x /= p.H_kv;
  const int tile = x % p.ntiles;
  const int b = x / p.ntiles;
  build_plan(p, b, tile, h, (lds_u32*)member);
}

constexpr int kRingHalf = 256;   // plan entries per half of the LDS ring

// One work list, or (dense_list set; two workgroups) one for the
// dense-causal slots, built by workgroup 1, and one for the rest.
__global__ __launch_bounds__(kSchedThreads) void attn_schedule_kernel(AttnParams p) {
  __shared__ int hist[kXcds * kXcdBuckets];
  const int nbt = p.rg.batch * p.ntiles;
  if (p.dense_list) {
    if (blockIdx.x == 1)
      schedule_by_xcd(nbt, p.H_kv, p.nbmax,
                      [&](int i) { const int c = p.plan_cnt[i]; return (c & kPlanDense) ? c & (kPlanDense - 1) : 0; },
                      p.dense_list, p.dense_sched, hist);
    else
      schedule_by_xcd(nbt, p.H_kv, p.nbmax,
                      [&](int i) { const int c = p.plan_cnt[i]; return (c & kPlanDense) ? 0 : c; },
                      p.worklist, p.sched, hist);
  } else {
    schedule_by_xcd(nbt, p.H_kv, p.nbmax, [&](int i) { return p.plan_cnt[i] & (kPlanDense - 1); },
                    p.worklist, p.sched, hist);
  }
}

// ---------------------------------------------------------------------------
// Prefill attention with direct global->LDS tile loads, BF16 or FP8 KV.
//
// Workgroup = W waves (16 on the prefill route, four per SIMD; 8 of two
// column tiles each for the prefill route's dense-causal slots, two per
// SIMD; 4 for the speculative rows of msa_attention_paged_shared),
// persistent over the slot work list;
// wave w owns columns [w cpw, (w + 1) cpw) of the tile's tq * G (token,
// query head) columns, as 16 * NCT MFMA columns.  K and V tiles are DMA'd
// straight into LDS, row-major (256-byte rows for BF16, 128-byte rows for
// FP8), with an XOR swizzle of 16-byte columns; each lane of a DMA
// instruction picks its source so that its fixed LDS slot receives the right
// swizzled piece.
//
// BF16: K column c of row pos is stored at c ^ (pos & 15), V column c at
// c ^ ((pos & 7) << 1).  The PV A-operand
// (V^T) comes from two ds_read_b64_tr_b16 per fragment: within each 16-lane
// group, output lane i, element k is element i % 4 of source lane i / 4 +
// 4k, so source lane j reads row 16r + 4g + j / 4 at dims 16dt + 4(j % 4),
// which yields for lane (m, g) the positions 16r + 4g + k of dim 16dt + m --
// exactly the P^T B-operand layout.
//
// FP8 (e4m3, widened to BF16 in registers as operands are read): K is kept
// in MFMA fragment order (each operand read is 16 consecutive bytes per
// lane), V column c of row pos at c ^ fv(pos) built from bits 1, 4 and 2 of
// pos, which keeps the rows of a transposed V read in distinct bank groups
// (both layouts measured conflict-free with the LDS bank-conflict counter).
// V^T comes
// from one ds_read_b64_tr_b8 per fragment: within each 16-lane group, output
// lane i, element k is byte i % 8 of source lane i / 8 + 2k, so source lanes
// 2k and 2k + 1 read the row holding P^T position k at dims 16dt and
// 16dt + 8, and lane (m, g) receives the 8 positions of dim 16dt + m.
// ---------------------------------------------------------------------------
constexpr float kLazy = 8.f;   // log2 headroom before the running max moves

// Tile ring: 64 KiB each for K and V, i.e. two BF16 stages or four FP8
// stages of one 128-position block.
constexpr int kRingBytes = 2 * kBlock * 256;
struct PrefillLds3 {
  char k[kRingBytes];
  char v[kRingBytes];
  int32_t ring_blk[2 * kRingHalf], ring_pg[2 * kRingHalf];
  uint32_t ring_msk[2 * kRingHalf];
};


// W waves share each staged block: 16 on the prefill route, 4 for the
// speculative rows of one sequence (see launch_attention_prefill).
template <bool FP8, int NCT, int W>
__device__ void attn_prefill3_tile(const AttnParams& p, int slot, PrefillLds3& L) {
  constexpr int kP3Waves = W;
  constexpr int RB = FP8 ? 128 : 256;       // bytes per LDS tile row
  constexpr int ESZ = FP8 ? 1 : 2;          // bytes per cache element
  constexpr int TILE = kBlock * RB;         // bytes of one K (or V) tile
  constexpr int NST = kRingBytes / TILE;    // ring stages: 2 (BF16), 4 (FP8)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform((int)(tid >> 6));
  const int l16 = lane & 15, g = lane >> 4;
  const int h = slot % p.H_kv;
  const int tile = (slot / p.H_kv) % p.ntiles;
  const int b = slot / p.H_kv / p.ntiles;
  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  const int t0 = tile * p.tq;
  if (t0 >= n) return;
  const int c = p.rg.clen[b];
  const int ntok = min(p.tq, n - t0);
  const int p_tile_max = c + t0 + ntok - 1;
  const int cnt = p.plan_cnt[slot] & (kPlanDense - 1);
  const int32_t* ids = p.plan_ids + (size_t)slot * p.nbmax;
  const int32_t* pgs = p.plan_pages + (size_t)slot * p.nbmax;
  const uint32_t* msks = p.plan_mask + (size_t)slot * p.nbmax;

  // ---- columns of this wave ---------------------------------------------
  const int cpw = p.tq * p.G / kP3Waves;            // columns per wave (<= 16 * NCT)
  const int tok_lo = wave * cpw / p.G;
  const int tok_n = max(1, cpw / p.G);
  uint32_t wave_bits = 0u;
  for (int t = tok_lo; t < tok_lo + tok_n && t < ntok; ++t) wave_bits |= 1u << t;
  int plim_col[NCT], tl_col[NCT];
  u32x4 qf[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int cw = ct * 16 + l16;
    const int cg = wave * cpw + cw;
    tl_col[ct] = cg / p.G;
    const bool ok = cw < cpw && tl_col[ct] < ntok;
    plim_col[ct] = ok ? c + t0 + tl_col[ct] : -1;
    const uint16_t* qp = p.q + ((size_t)(r0 + t0 + tl_col[ct]) * p.H_q + h * p.G + cg % p.G) * kDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // contraction dims of k-step s for lane group g: BF16 32s + 8g + j;
      // FP8 (K in fragment order, s = 2h + t) 16g + 64h + 8t + j
      const int d0 = FP8 ? 16 * g + 64 * (s >> 1) + 8 * (s & 1) : 32 * s + 8 * g;
      qf[ct][s] = ok ? ld16(qp + d0) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int p_wave_min = c + t0 + tok_lo;

  f32x4 O[8][NCT];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[NCT], l_run[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m_run[ct] = neg_inf();
    l_run[ct] = 0.f;
  }
  const float sc = p.scale_log2;

  // ---- lane-constant LDS addresses ---------------------------------------
  // BF16 K A-operand: row 16pt + l16 (+ 64hb), logical column 4s + g
  //   = l16 * 256 + ((4s + g) ^ l16) * 16 = kq ^ (s << 6), kq for s = 0
  // FP8 K is stored in fragment order: fragment f = 2 * (row tile) + h is
  //   1 KiB where lane (l16, g) holds row 16 * tile + l16, bytes 16g + 64h
  //   .. + 15 (k-steps 2h and 2h + 1), so an operand read is at f * 1024 +
  //   16 * lane: linear, hence free of bank conflicts
  const int kq = FP8 ? 16 * lane : l16 * 256 + ((g ^ l16) << 4);
  // BF16 V^T A-operand (transpose read r of chunk ch, dim tile dt): row
  //   32ch + 16r + q with q = 4g + l16 / 4, dims 16dt + 4(l16 % 4); V column
  //   c of row pos is stored at c ^ ((pos & 7) << 1), which puts the 8 rows
  //   one 32-lane half of a transpose read touches in distinct bank groups
  //   = (32ch + 16r) * 256 + (vq ^ (dt << 5))
  // FP8 V^T A-operand (one transpose read of chunk ch, dim tile dt): source
  //   lane l16 reads P^T position k = l16 / 2, i.e. row
  //   32ch + 16(k / 4) + 4g + k % 4, at dims 16dt + 8 (l16 % 2)
  //   = 32ch * 128 + (vq ^ (dt << 4))
  int vq;
  if constexpr (FP8) {
    const int k = l16 >> 1;
    const int vrow = 16 * (k >> 2) + 4 * g + (k & 3);
    vq = vrow * 128 + (fp8_vswz(vrow) << 4) + 8 * (l16 & 1);
  } else {
    const int vq_row = 4 * g + (l16 >> 2);
    vq = vq_row * 256 + (((((l16 & 3) >> 1)) ^ ((vq_row & 7) << 1)) << 4) + 8 * (l16 & 1);
  }
  // DMA.  Row-major tiles: instruction i of this wave covers kRowsPerDma
  // rows from kRowsPerWave * wave + kRowsPerDma * i; a lane lands in row
  // + lane / (RB / 16) at physical column lane % (RB / 16).  FP8 K: one
  // fragment (1 KiB) per instruction, 16 / kP3Waves of them per wave.
  constexpr int kCols = RB / 16;                      // 16-byte columns per row
  constexpr int kRowsPerDma = 64 / kCols;
  constexpr int kRowsPerWave = kBlock / kP3Waves;     // tile rows each wave fetches
  constexpr int kDmaPerWave = kRowsPerWave / kRowsPerDma;
  static_assert(!FP8 || 16 % kP3Waves == 0, "FP8 K fragments split evenly over the waves");
  constexpr int kDmaK = FP8 ? 16 / kP3Waves : kDmaPerWave;
  constexpr int kDmaV = kDmaPerWave;
  const int dr = lane / kCols, dc = lane % kCols;
  const char* kpool = static_cast<const char*>(p.k.data);
  const char* vpool = static_cast<const char*>(p.v.data);
  const uint32_t kts = (uint32_t)p.k.token_stride * ESZ, vts = (uint32_t)p.v.token_stride * ESZ;
  const size_t khead = (size_t)h * p.k.head_stride * ESZ, vhead = (size_t)h * p.v.head_stride * ESZ;
  const size_t kps = (size_t)p.k.page_stride * ESZ, vps = (size_t)p.v.page_stride * ESZ;
  // byte offsets (within a page's tile) of the pieces this lane fetches, and
  // the LDS offsets (within a stage) of the wave's DMA instructions
  uint32_t koff[kDmaK], voff[kDmaV];
  int kdst[kDmaK], vdst[kDmaV];
#pragma unroll
  for (int i = 0; i < kDmaK; ++i) {
    if constexpr (FP8) {
      const int f = wave * kDmaK + i;
      koff[i] = (16 * (f >> 1) + l16) * kts + 16 * g + 64 * (f & 1);
      kdst[i] = f * 1024;
    } else {
      const int row = kRowsPerWave * wave + kRowsPerDma * i + dr;
      koff[i] = row * kts + ((dc ^ (row & 15)) << 4);
      kdst[i] = (kRowsPerWave * wave + kRowsPerDma * i) * RB;
    }
  }
#pragma unroll
  for (int i = 0; i < kDmaV; ++i) {
    const int row = kRowsPerWave * wave + kRowsPerDma * i + dr;
    const uint32_t vcol = (FP8 ? dc ^ fp8_vswz(row) : dc ^ ((row & 7) << 1)) << 4;
    voff[i] = row * vts + vcol;
    vdst[i] = (kRowsPerWave * wave + kRowsPerDma * i) * RB;
  }

  auto stage = [&](int pg, int buf) {
    if (pg < 0) pg = 0;
    const char* kb = kpool + (size_t)pg * kps + khead;
    const char* vb = vpool + (size_t)pg * vps + vhead;
#pragma unroll
    for (int i = 0; i < kDmaK; ++i) dma16(kb + koff[i], L.k + buf * TILE + kdst[i]);
#pragma unroll
    for (int i = 0; i < kDmaV; ++i) dma16(vb + voff[i], L.v + buf * TILE + vdst[i]);
  };

  auto ring_fill = [&](int first) {
    if (tid < kRingHalf) {
      const int i = first + tid;
      if (i < cnt) {
        const int si = i & (2 * kRingHalf - 1);
        L.ring_blk[si] = ids[i];
        L.ring_pg[si] = pgs[i];
        L.ring_msk[si] = msks[i];
      }
    }
  };
  ring_fill(0);
  ring_fill(kRingHalf);
  __syncthreads();
  // Blocks go through the ring in groups of SYNC = NST / 2 (one group of
  // stages being computed while the next is in flight).  The first NST -
  // SYNC blocks are requested up front.  At the start of each group every
  // wave waits for its own DMAs, then all meet at a barrier; the group's
  // blocks are then computed with no barrier between them (waves drift
  // apart by up to a group, which evens out which SIMDs have work), and the
  // blocks NST - SYNC ahead are requested into the stages the previous group
  // released.
  constexpr int SYNC = NST / 2;
#pragma unroll
  for (int j = 0; j < NST - SYNC; ++j)
    if (j < cnt) stage(L.ring_pg[j], j);

  for (int e = 0; e < cnt; ++e) {
    const int buf = e % NST;
    if (e % SYNC == 0) {
      // every DMA this wave issued is for blocks e .. e + NST - SYNC - 1; the
      // group's own blocks are the oldest SYNC of them and the rest
      // (NST - 2 SYNC blocks) may stay in flight
      constexpr int kYounger = (kDmaK + kDmaV) * (NST - 2 * SYNC);
      static_assert(kYounger < 16, "vmcnt immediate holds 4 bits here");
      if (kYounger > 0 && e + NST - SYNC <= cnt) __builtin_amdgcn_s_waitcnt(0xF70 | kYounger);
      else __builtin_amdgcn_s_waitcnt(0xF70);
      // ... and every other wave's.  A bare barrier: a fenced one would also
      // wait for the younger DMAs still in flight.  Nothing before it needs
      // ordering: LDS traffic of earlier blocks was consumed by this wave's
      // MFMAs, and the ring and zeroing writes have barriers of their own.
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_s_barrier();
      if (e >= kRingHalf && (e & (kRingHalf - 1)) == 0) ring_fill(e + kRingHalf);
      // V rows past every token of the tile hold no data: zero them (only
      // the tile's last block can have such rows) so that a zero
      // probability never meets a NaN
      bool zeroed = false;
#pragma unroll
      for (int j = 0; j < SYNC; ++j) {
        if (e + j >= cnt) break;
        const int bj = uniform(L.ring_blk[(e + j) & (2 * kRingHalf - 1)]);
        if (bj * kBlock + kBlock - 1 > p_tile_max) {
          for (int i = tid; i < kBlock * kCols; i += kP3Waves * 64) {
            const int row = i / kCols;
            if (bj * kBlock + row > p_tile_max)
              *reinterpret_cast<u32x4*>(L.v + ((e + j) % NST) * TILE + row * RB + (i % kCols) * 16) =
                  u32x4{0u, 0u, 0u, 0u};
          }
          zeroed = true;
        }
      }
      if (zeroed) __syncthreads();
#pragma unroll
      for (int j = 0; j < SYNC; ++j) {
        const int ej = e + NST - SYNC + j;
        if (ej < cnt) stage(L.ring_pg[ej & (2 * kRingHalf - 1)], ej % NST);
      }
    }
    const int rc = e & (2 * kRingHalf - 1);
    const int blk = uniform(L.ring_blk[rc]);
    const uint32_t msk = uniform(L.ring_msk[rc]);
    if (!(msk & wave_bits)) continue;

    const bool diag = blk * kBlock + kBlock - 1 > p_wave_min;
    bool live[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) live[ct] = plim_col[ct] >= 0 && ((msk >> tl_col[ct]) & 1u);
    const char* kt = L.k + buf * TILE;
    const char* vtl = L.v + buf * TILE;

    // S^T for the block: with few columns both halves are computed up front
    // so that the second half's MFMAs can overlap the first half's softmax;
    // with 64 columns one half at a time fits the register file.
    constexpr int kHalves = kP3Waves >= 16 ? 1 : (NCT <= 1 ? 2 : 1);
    f32x4 S[kHalves][4][NCT];
    auto qk_half = [&](int hb, f32x4 (&Sh)[4][NCT]) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        u32x4 w8 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          u32x4 a;
          if constexpr (FP8) {
            if ((s & 1) == 0)
              w8 = *reinterpret_cast<const u32x4*>(kt + (2 * (4 * hb + pt) + (s >> 1)) * 1024 + kq);
            a = fp8x8_to_bf16x8((s & 1) ? u32x2{w8.z, w8.w} : u32x2{w8.x, w8.y});
          } else {
            a = *reinterpret_cast<const u32x4*>(kt + (64 * hb + 16 * pt) * RB + (kq ^ (s << 6)));
          }
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
            Sh[pt][ct] = mfma_bf16(a, qf[ct][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : Sh[pt][ct]);
        }
      }
    };
    if constexpr (kHalves == 2) {
      qk_half(0, S[0]);
      qk_half(1, S[1]);
    }

#pragma unroll(kHalves)
    for (int hb = 0; hb < 2; ++hb) {
      const int sh = kHalves == 2 ? hb : 0;
      if constexpr (kHalves == 1) qk_half(hb, S[0]);
      bool rescale = false;
      float alpha[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (diag) {
          const int lim = (live[ct] ? plim_col[ct] : -1) - (blk * kBlock + 64 * hb + 4 * g);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * pt + i > lim) S[sh][pt][ct][i] = neg_inf();
        }
        float hmax = neg_inf();
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          hmax = fmaxf(hmax, fmaxf(fmaxf(S[sh][pt][ct][0], S[sh][pt][ct][1]),
                                   fmaxf(S[sh][pt][ct][2], S[sh][pt][ct][3])));
        hmax = colgroup_max(hmax) * sc;
        // lazy rescaling: the reference max only moves when a score would
        // exceed it by more than 2^kLazy, so probabilities stay <= 2^kLazy
        // and O (held in accumulator registers) is rarely rescaled
        const bool move = live[ct] && hmax > m_run[ct] + kLazy;
        const float m_new = move ? hmax : m_run[ct];
        const float m_use = m_new == neg_inf() ? 0.f : m_new;
        const float off = live[ct] ? m_use : __builtin_inff();
        alpha[ct] = move ? fast_exp2(m_run[ct] - m_use) : 1.f;
        rescale |= move;
        float lsum = 0.f;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e2 = fast_exp2(__builtin_fmaf(S[sh][pt][ct][i], sc, -off));
            S[sh][pt][ct][i] = e2;
            lsum += e2;
          }
        l_run[ct] = l_run[ct] * alpha[ct] + lsum;
        m_run[ct] = m_new;
      }
      if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) O[dt][ct] *= alpha[ct];
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        u32x4 bp[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const f32x4 s0 = S[sh][2 * cc][ct], s1 = S[sh][2 * cc + 1][ct];
          bp[ct] = u32x4{pack_bf16(s0[0], s0[1]), pack_bf16(s0[2], s0[3]), pack_bf16(s1[0], s1[1]),
                         pack_bf16(s1[2], s1[3])};
        }
        const int chunk = 2 * hb + cc;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          u32x4 a;
          if constexpr (FP8) {
            a = fp8x8_to_bf16x8(lds_tr_b8(vtl + (32 * chunk) * RB + (vq ^ (dt << 4))));
          } else {
            const char* base = vtl + (32 * chunk) * RB + (vq ^ (dt << 5));
            const u32x2 lo = lds_tr_b16(base);
            const u32x2 hi = lds_tr_b16(base + 16 * RB);
            a = u32x4{lo.x, lo.y, hi.x, hi.y};
          }
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) O[dt][ct] = mfma_bf16(a, bp[ct], O[dt][ct]);
        }
      }
    }
  }

  // ---- epilogue ------------------------------------------------------------
  // O^T tile dt, row m = 4g + i of the C layout is dim 16dt + 4g + i
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const float l_tot = colgroup_sum(l_run[ct]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (plim_col[ct] < 0) continue;
    const int cg = wave * cpw + ct * 16 + l16;
    uint16_t* op = p.out + ((size_t)(r0 + t0 + tl_col[ct]) * p.H_q + h * p.G + cg % p.G) * kDim + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const f32x4 o = O[dt][ct];
      *reinterpret_cast<u32x2*>(op + 16 * dt) = u32x2{pack_bf16(o[0] * inv, o[1] * inv),
                                                     pack_bf16(o[2] * inv, o[3] * inv)};
    }
  }
}

// INLINE: one workgroup per slot, which first builds the slot's plan itself
// (in the K ring, free until the tile's first DMA; nbmax words fit in it).
// Otherwise persistent workgroups over the work list.  (Two instantiations
// rather than a run-time choice: with both paths in one kernel the compiler
// emits an invalid instruction.)
template <bool FP8, int NCT, int W, bool INLINE>
__global__ __launch_bounds__(64 * W) void attn_prefill3_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) PrefillLds3 lds;
  if constexpr (INLINE) {
    const int slot = (int)blockIdx.x;
    int x = slot;
    const int h = x % p.H_kv;
    x /= p.H_kv;
    const int tile = x % p.ntiles;
    build_plan(p, x / p.ntiles, tile, h, (lds_u32*)lds.k);
    __syncthreads();
    attn_prefill3_tile<FP8, NCT, W>(p, slot, lds);
  } else {
    __shared__ int item_s;
    const int xcd = xcd_id();
    for (;;) {
      const int slot = take_slot_xcd(p.sched, p.worklist, xcd, &item_s);
      if (slot < 0) break;
      attn_prefill3_tile<FP8, NCT, W>(p, slot, lds);
    }
  }
}

void prefill_tiling(int G, bool /*fp8*/, int waves, int* tq, int* nct) {
  // `waves` waves of at most 16 columns (one MFMA column tile), both KV
  // types.  Two column tiles per wave do not fit the 128 VGPRs a wave of a
  // 16-wave workgroup has: they spill inside the block loop (measured at
  // group size 16: 32.6 ms against 11.3 ms with 16-token tiles).  The
  // dense-causal kernel (8 waves of two column tiles) takes the same tiles:
  // 8 * 32 / G tokens = 256 / G.
  *tq = std::min(32, waves * 16 / G);
  *nct = 1;
}

hipError_t launch_attention_prefill(const AttnParams& p, bool fp8, int waves, hipStream_t s) {
  const size_t slots = (size_t)p.rg.batch * p.ntiles * p.H_kv;
  if (!p.inline_plan) {
    hipLaunchKernelGGL(prefill_plan_kernel, dim3((unsigned)slots), dim3(64),
                       (size_t)p.nbmax * sizeof(uint32_t), s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(p.dense_list ? 2 : 1), dim3(kSchedThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.dense_list) {
    // the dense-causal slots first, by their own kernel and work list
    AttnParams pd = p;
    pd.worklist = p.dense_list;
    pd.sched = p.dense_sched;
    const dim3 dgrid((unsigned)p.nwg), dblock(64 * kUnionWavesDense);
    if (fp8) hipLaunchKernelGGL((attn_prefill3_kernel<true, 2, kUnionWavesDense, false>), dgrid, dblock, 0, s, pd);
    else hipLaunchKernelGGL((attn_prefill3_kernel<false, 2, kUnionWavesDense, false>), dgrid, dblock, 0, s, pd);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(p.inline_plan ? slots : (size_t)p.nwg)), block(64 * waves);
  if (p.inline_plan) {   // the speculative rows' workgroups of kUnionWavesShared waves
    if (fp8) hipLaunchKernelGGL((attn_prefill3_kernel<true, 1, kUnionWavesShared, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_prefill3_kernel<false, 1, kUnionWavesShared, true>), grid, block, 0, s, p);
  } else {
    if (fp8) hipLaunchKernelGGL((attn_prefill3_kernel<true, 1, kUnionWavesPrefill, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_prefill3_kernel<false, 1, kUnionWavesPrefill, false>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace msa
