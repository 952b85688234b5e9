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
//   * attn_prefill_kernel -- MFMA attention over each tile's union blocks;
//     K and V tiles are staged in LDS once per workgroup and shared by its
//     eight waves, each wave skipping blocks none of its tokens selected.
//
// The indexer's K tile in LDS is 128 rows of 256 bytes; 16-byte column c of
// row pos is stored at column c ^ (pos & 15), so the 16 rows an MFMA
// A-operand read touches fall in distinct bank groups.
//
// Both kernels double-buffer the tiles: the global loads of block e + 1 are
// issued before block e is computed and written to LDS after it, with the
// raw bits held in registers in between (any conversion happens at the LDS
// store so that the loads stay in flight during the compute).
#include <algorithm>

#include "msa_common.h"
#include "msa_kernels.h"

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

__device__ void indexer_prefill_tile(const IndexerParams& p, const IdxTile& T, char (*lds)[kBlock * 256],
                                     int32_t* pages_lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int hpi = p.H_kv / p.H_ik;
  const int blk_lo = T.blk_lo, blk_hi = T.blk_hi;

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
    for (int s = 0; s < 4; ++s) qf[ct][s] = ok ? ld16(qp + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
  }
  const int p_first = T.c + T.t0;

  const char* pool = static_cast<const char*>(p.ik.data);
  const size_t ts = (size_t)p.ik.token_stride * 2;
  const size_t head_off = (size_t)T.hk * p.ik.head_stride;
  const int32_t* trow = p.rg.table + (size_t)T.b * p.rg.stride;
  const int npages = p.ik.num_pages;
  // The page ids of the whole block range go to LDS first, so the loop
  // never waits on a global load to learn where its next tile is.
  for (int i = tid; i < blk_hi - blk_lo; i += 256) pages_lds[i] = trow[blk_lo + i];
  __syncthreads();

  u32x4 stage[8];
  auto tile_base = [&](int pg) -> const char* {
    if ((unsigned)pg >= (unsigned)npages) pg = 0;
    return pool + ((size_t)pg * p.ik.page_stride + head_off) * 2;
  };
  {
    const char* kb = tile_base(pages_lds[0]);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int cidx = tid + 256 * k;
      stage[k] = ld16(kb + (cidx >> 4) * ts + (cidx & 15) * 16);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int cidx = tid + 256 * k;
      *reinterpret_cast<u32x4*>(lds[0] + k_off(cidx >> 4, cidx & 15)) = stage[k];
    }
  }
  float win[4][4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) win[ct][j] = 0.f;

  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const int buf = (blk - blk_lo) & 1;
    __syncthreads();
    const bool more = blk + 1 < blk_hi;
    if (more) {
      const char* kb = tile_base(pages_lds[blk + 1 - blk_lo]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cidx = tid + 256 * k;
        stage[k] = ld16(kb + (cidx >> 4) * ts + (cidx & 15) * 16);
      }
    }
    const char* kt = lds[buf];
    const bool clip = blk * kBlock + kBlock - 1 > p_first;
    float mx[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) mx[ct] = neg_inf();
#pragma unroll 2
    for (int pt = 0; pt < 8; ++pt) {
      f32x4 acc[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 a = lds16(kt, k_off(16 * pt + l16, 4 * s + g));
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
          acc[ct] = mfma_bf16(a, qf[ct][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[ct]);
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
    if (more) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int cidx = tid + 256 * k;
        *reinterpret_cast<u32x4*>(lds[buf ^ 1] + k_off(cidx >> 4, cidx & 15)) = stage[k];
      }
    }
  }
}

__global__ __launch_bounds__(256) void indexer_score_prefill_kernel(IndexerParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2][kBlock * 256];
  __shared__ int item_s;
  extern __shared__ int32_t pages_lds[];   // page ids of the tile's block range
  for (;;) {
    const int k = take_item(p.sched, &item_s);
    if (k < 0) break;
    const IdxTile T = idx_tile_of(p, p.worklist[k]);
    indexer_prefill_tile(p, T, lds, pages_lds);
  }
}

int prefill_indexer_tile(int H_kv, int H_ik) { return 256 / (H_kv / H_ik); }

hipError_t launch_indexer_prefill(const IndexerParams& p, int num_cus, hipStream_t s) {
  hipLaunchKernelGGL(indexer_schedule_kernel, dim3(1), dim3(kSchedThreads),
                     (size_t)(p.nbmax + 1) * sizeof(int), s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // two 64 KiB workgroups fit in a CU's LDS
  hipLaunchKernelGGL(indexer_score_prefill_kernel, dim3(2 * num_cus), dim3(256),
                     (size_t)p.nbmax * sizeof(int32_t), s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill plan: one wave per (sequence, tile, KV head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void prefill_plan_kernel(AttnParams p) {
  extern __shared__ uint32_t member[];   // [nbmax] token mask per block
  const int lane = threadIdx.x;
  int x = blockIdx.x;
  const int h = x % p.H_kv;
  x /= p.H_kv;
  const int tile = x % p.ntiles;
  const int b = x / p.ntiles;
  const size_t slot = ((size_t)b * p.ntiles + tile) * p.H_kv + h;
  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  const int t0 = tile * p.tq;
  if (t0 >= n) {
    if (lane == 0) p.plan_cnt[slot] = 0;
    return;
  }
  const int c = p.rg.clen[b];
  const int ntok = min(p.tq, n - t0);
  const int nb_last = min((c + t0 + ntok - 1) / kBlock + 1, p.nbmax);
  for (int i = lane; i < nb_last; i += 64) member[i] = 0u;
  __syncthreads();
  for (int tl = 0; tl < ntok; ++tl) {
    const int nbt = min((c + t0 + tl) / kBlock + 1, p.nbmax);
    const int32_t* lst = p.d_indices + ((size_t)(r0 + t0 + tl) * p.H_kv + h) * p.top_k;
    for (int i = lane; i < p.top_k; i += 64) {
      const int id = lst[i];
      if (id >= 0 && id < nbt) atomicOr(&member[id], 1u << tl);
    }
  }
  __syncthreads();
  int32_t* ids = p.plan_ids + slot * p.nbmax;
  int32_t* pgs = p.plan_pages + slot * p.nbmax;
  uint32_t* msk = p.plan_mask + slot * p.nbmax;
  const int32_t* trow = p.rg.table + (size_t)b * p.rg.stride;
  int cnt = 0;
  for (int base = 0; base < nb_last; base += 64) {
    const int i = base + lane;
    const uint32_t m = i < nb_last ? member[i] : 0u;
    const uint64_t bal = ballot(m != 0u);
    if (m) {
      const int pos = cnt + mask_rank(bal);
      const int pg = trow[i];
      ids[pos] = i;
      pgs[pos] = (unsigned)pg < (unsigned)p.k.num_pages ? pg : -1;
      msk[pos] = m;
    }
    cnt += __popcll(bal);
  }
  if (lane == 0) p.plan_cnt[slot] = cnt;
}

// ---------------------------------------------------------------------------
// Prefill attention: workgroup = 8 waves over one (sequence, tile of tq
// tokens, KV head).  Wave w owns columns [w * cpw, (w + 1) * cpw) of the
// tile's tq * G (token, query head) columns, as 16 * NCT MFMA columns.
//
// LDS rows are padded to 272 bytes (the 16 rows one MFMA operand read
// touches then start in distinct bank groups), which keeps every operand
// address a per-lane base plus a compile-time offset.
// ---------------------------------------------------------------------------
constexpr int kPrefillWaves = 8;
constexpr int kRingHalf = 256;
constexpr int kPitch = 272;                  // bytes per padded LDS row
constexpr int kTileBytes = kBlock * kPitch;  // 34 KiB

template <bool FP8>
struct TileRegs;
template <>
struct TileRegs<false> {     // BF16: 4 K chunks and 4 V row slices of 16 B
  u32x4 k[4];
  u32x4 v[4];
};
template <>
struct TileRegs<true> {      // FP8: 2 K chunks of 16 B and 4 V row slices of 8 B
  u32x4 k[2];
  u32x2 v[4];
};

// LDS of one prefill attention workgroup.  K tile: row = position.  V^T
// tile: row = head dim d, with positions permuted inside each 32-position
// chunk (32ch + 16a + 4g + i -> 32ch + 8g + 4a + i) so one 16-byte read
// returns exactly the 8 positions of a lane's P^T B-operand.  Plan entries
// pass through a ring of 2 * kRingHalf entries refilled half a ring at a
// time, far ahead of use.
struct PrefillLds {
  char ks[2][kTileBytes];
  char vt[2][kTileBytes];
  int32_t ring_blk[2 * kRingHalf], ring_pg[2 * kRingHalf];
  uint32_t ring_msk[2 * kRingHalf];
};

__global__ __launch_bounds__(kSchedThreads) void attn_schedule_kernel(AttnParams p) {
  extern __shared__ int hist[];
  const int nslots = p.rg.batch * p.ntiles * p.H_kv;
  schedule_by_cost(nslots, p.nbmax, [&](int i) { return p.plan_cnt[i]; }, p.worklist, p.sched, hist);
}

template <bool FP8, int NCT>
__device__ void attn_prefill_tile(const AttnParams& p, int slot, PrefillLds& L) {
  auto& ks = L.ks;
  auto& vt = L.vt;
  auto& ring_blk = L.ring_blk;
  auto& ring_pg = L.ring_pg;
  auto& ring_msk = L.ring_msk;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const int cnt = p.plan_cnt[slot];
  const int32_t* ids = p.plan_ids + (size_t)slot * p.nbmax;
  const int32_t* pgs = p.plan_pages + (size_t)slot * p.nbmax;
  const uint32_t* msks = p.plan_mask + (size_t)slot * p.nbmax;

  // ---- columns of this wave ---------------------------------------------
  const int cpw = p.tq * p.G / kPrefillWaves;       // columns per wave (<= 16 * NCT)
  const int tok_lo = wave * cpw / p.G;               // first token of the wave
  const int tok_n = cpw / p.G;
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
    for (int s = 0; s < 4; ++s) qf[ct][s] = ok ? ld16(qp + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
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
  // operand read bases: K row 16pt + l16 at 16-byte column 4s + g, V^T row
  // 16dt + l16 at column 4ch + g; (pt, s, dt, ch) only add constants
  const int rd_base = l16 * kPitch + 16 * g;

  // ---- staging: K rows and V transposed --------------------------------
  const int esz = FP8 ? 1 : 2;
  const char* kpool = static_cast<const char*>(p.k.data);
  const char* vpool = static_cast<const char*>(p.v.data);
  const size_t kts = (size_t)p.k.token_stride * esz, vts = (size_t)p.v.token_stride * esz;
  const size_t khead = (size_t)h * p.k.head_stride * esz, vhead = (size_t)h * p.v.head_stride * esz;
  const size_t kps = (size_t)p.k.page_stride * esz, vps = (size_t)p.v.page_stride * esz;
  // V sub-block of this thread: rows 32ch + 16a + 4gq + i (i = 0..3), dims 8dg..8dg+7
  const int v_dg = tid & 15, v_gq = (tid >> 4) & 3, v_a = (tid >> 6) & 1, v_ch = tid >> 7;
  const int v_row0 = 32 * v_ch + 16 * v_a + 4 * v_gq;
  const int vt_wr = (8 * v_dg) * kPitch + (4 * v_ch + v_gq) * 16 + 8 * v_a;
  TileRegs<FP8> st;

  auto stage_load = [&](int pg) {
    if (pg < 0) pg = 0;
    const char* kb = kpool + (size_t)pg * kps + khead;
    const char* vb = vpool + (size_t)pg * vps + vhead;
    if constexpr (FP8) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int cidx = tid + 512 * k;     // 16 e4m3 values: position cidx >> 3, dims 16 * (cidx & 7)
        st.k[k] = ld16(kb + (cidx >> 3) * kts + (cidx & 7) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) st.v[i] = ld8(vb + (v_row0 + i) * vts + 8 * v_dg);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int cidx = tid + 512 * k;     // 8 bf16 values: position cidx >> 4, dims 8 * (cidx & 15)
        st.k[k] = ld16(kb + (cidx >> 4) * kts + (cidx & 15) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) st.v[i] = ld16(vb + (v_row0 + i) * vts + 16 * v_dg);
    }
  };
  auto stage_store = [&](int buf, int blk) {
    u32x4 vr[4];
    if constexpr (FP8) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int cidx = tid + 512 * k;
        char* dst = ks[buf] + (cidx >> 3) * kPitch + (cidx & 7) * 32;
        *reinterpret_cast<u32x4*>(dst) = fp8x8_to_bf16x8(u32x2{st.k[k].x, st.k[k].y});
        *reinterpret_cast<u32x4*>(dst + 16) = fp8x8_to_bf16x8(u32x2{st.k[k].z, st.k[k].w});
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = fp8x8_to_bf16x8(st.v[i]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int cidx = tid + 512 * k;
        *reinterpret_cast<u32x4*>(ks[buf] + (cidx >> 4) * kPitch + (cidx & 15) * 16) = st.k[k];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = st.v[i];
    }
    // rows past every token of the tile hold no data: zero them so that a
    // zero probability never meets a NaN
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (blk * kBlock + v_row0 + i > p_tile_max) vr[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const u32x2 w = {pick_halves(vr[0][e >> 1], vr[1][e >> 1], e & 1),
                       pick_halves(vr[2][e >> 1], vr[3][e >> 1], e & 1)};
      *reinterpret_cast<u32x2*>(vt[buf] + vt_wr + e * kPitch) = w;
    }
  };

  auto ring_fill = [&](int first) {   // entries first .. first + kRingHalf - 1
    if (tid < kRingHalf) {
      const int i = first + tid;
      if (i < cnt) {
        const int slot_i = i & (2 * kRingHalf - 1);
        ring_blk[slot_i] = ids[i];
        ring_pg[slot_i] = pgs[i];
        ring_msk[slot_i] = msks[i];
      }
    }
  };
  ring_fill(0);
  ring_fill(kRingHalf);
  __syncthreads();
  if (cnt > 0) {
    stage_load(ring_pg[0]);
    stage_store(0, ring_blk[0]);
  }
  for (int e = 0; e < cnt; ++e) {
    const int buf = e & 1;
    __syncthreads();
    // entries e - kRingHalf .. e - 1 are consumed: reuse their slots
    if (e >= kRingHalf && (e & (kRingHalf - 1)) == 0) ring_fill(e + kRingHalf);
    const bool more = e + 1 < cnt;
    const int rn = (e + 1) & (2 * kRingHalf - 1);
    if (more) stage_load(ring_pg[rn]);
    const int rc = e & (2 * kRingHalf - 1);
    const int blk = uniform(ring_blk[rc]);
    const uint32_t msk = uniform(ring_msk[rc]);
    if (msk & wave_bits) {
      // causal clip needed only where the block reaches past the wave's
      // first token; elsewhere a column either reads the whole block or none
      const bool diag = blk * kBlock + kBlock - 1 > p_wave_min;
      bool live[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) live[ct] = plim_col[ct] >= 0 && ((msk >> tl_col[ct]) & 1u);
      const char* kt = ks[buf] + rd_base;
      const char* vtt = vt[buf] + rd_base;
#pragma unroll 1
      for (int hb = 0; hb < 2; ++hb) {
        const char* kth = kt + 64 * hb * kPitch;
        f32x4 S[4][NCT];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(kth + 16 * pt * kPitch + 64 * s);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
              S[pt][ct] = mfma_bf16(a, qf[ct][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[pt][ct]);
          }
        }
        // online softmax per column, running max in scaled log2 units; a
        // column that does not read this block keeps its state (its
        // probabilities come out as exp2(-inf) = 0)
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
                if (16 * pt + i > lim) S[pt][ct][i] = neg_inf();
          }
          float hmax = neg_inf();
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
            hmax = fmaxf(hmax, fmaxf(fmaxf(S[pt][ct][0], S[pt][ct][1]), fmaxf(S[pt][ct][2], S[pt][ct][3])));
          hmax = colgroup_max(hmax) * sc;
          const float m_new = live[ct] ? fmaxf(m_run[ct], hmax) : m_run[ct];
          const float m_use = m_new == neg_inf() ? 0.f : m_new;
          const float off = live[ct] ? m_use : __builtin_inff();
          alpha[ct] = live[ct] ? fast_exp2(m_run[ct] - m_use) : 1.f;
          rescale |= alpha[ct] != 1.f;
          float lsum = 0.f;
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e2 = fast_exp2(__builtin_fmaf(S[pt][ct][i], sc, -off));
              S[pt][ct][i] = e2;
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
        // O^T += V^T P^T over the two 32-position chunks of this half
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          u32x4 bp[NCT];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const f32x4 s0 = S[2 * cc][ct], s1 = S[2 * cc + 1][ct];
            bp[ct] = u32x4{pack_bf16(s0[0], s0[1]), pack_bf16(s0[2], s0[3]), pack_bf16(s1[0], s1[1]),
                           pack_bf16(s1[2], s1[3])};
          }
          const char* vtc = vtt + 64 * (2 * hb + cc);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(vtc + 16 * dt * kPitch);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) O[dt][ct] = mfma_bf16(a, bp[ct], O[dt][ct]);
          }
        }
      }
    }
    if (more) stage_store(buf ^ 1, uniform(ring_blk[rn]));
  }

  // ---- epilogue ------------------------------------------------------------
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

template <bool FP8, int NCT>
__global__ __launch_bounds__(512) void attn_prefill_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) PrefillLds lds;
  __shared__ int item_s;
  for (;;) {
    const int k = take_item(p.sched, &item_s);
    if (k < 0) break;
    attn_prefill_tile<FP8, NCT>(p, p.worklist[k], lds);
  }
}

// ---------------------------------------------------------------------------
// BF16 prefill attention with direct global->LDS tile loads.
//
// Workgroup = 8 waves (two per SIMD) of 16 * NCT columns each.  K and V tiles are DMA'd
// straight into LDS, row-major, 256-byte rows with 16-byte column c of row
// pos stored at column c ^ (pos & 15); each lane of a DMA instruction picks
// its source so that its fixed LDS slot receives the right swizzled piece.
// The PV A-operand (V^T) comes from two ds_read_b64_tr_b16 per fragment:
// within each 16-lane group, output lane i, element k is element i % 4 of
// source lane i / 4 + 4k, so source lane j reads row 16r + 4g + j / 4 at
// dims 16dt + 4(j % 4), which yields for lane (m, g) the positions
// 16r + 4g + k of dim 16dt + m -- exactly the P^T B-operand layout.
// ---------------------------------------------------------------------------
constexpr int kP3Waves = 16;
constexpr float kLazy = 8.f;   // log2 headroom before the running max moves

struct PrefillLds3 {
  char k[2][kBlock * 256];
  char v[2][kBlock * 256];
  int32_t ring_blk[2 * kRingHalf], ring_pg[2 * kRingHalf];
  uint32_t ring_msk[2 * kRingHalf];
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ u32x2 lds_tr8(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void dma16(const char* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_char*)lds_dst, 16, 0, 0);
}

template <int NCT>
__device__ void attn_prefill3_tile(const AttnParams& p, int slot, PrefillLds3& L) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
  const int cnt = p.plan_cnt[slot];
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
    for (int s = 0; s < 4; ++s) qf[ct][s] = ok ? ld16(qp + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
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
  // K A-operand: row 16pt + l16 (+ 64hb), logical column 4s + g
  //   = l16 * 256 + ((4s + g) ^ l16) * 16 = kq ^ (s << 6), kq for s = 0
  const int kq = l16 * 256 + ((g ^ l16) << 4);
  // V^T A-operand (transpose read r of chunk ch, dim tile dt): row
  // 32ch + 16r + q with q = 4g + l16 / 4, dims 16dt + 4(l16 % 4)
  //   = (32ch + 16r) * 256 + (vq ^ (dt << 5))
  const int vq_row = 4 * g + (l16 >> 2);
  const int vq = vq_row * 256 + (((((l16 & 3) >> 1)) ^ vq_row) << 4) + 8 * (l16 & 1);
  // DMA: instruction i of this wave covers rows 16 wave + 4i .. + 3; lane
  // lands in row 16 wave + 4i + lane / 16 at physical column lane % 16
  const int dr = lane >> 4, dc = lane & 15;
  const char* kpool = static_cast<const char*>(p.k.data);
  const char* vpool = static_cast<const char*>(p.v.data);
  const uint32_t kts = (uint32_t)p.k.token_stride * 2, vts = (uint32_t)p.v.token_stride * 2;
  const size_t khead = (size_t)h * p.k.head_stride * 2, vhead = (size_t)h * p.v.head_stride * 2;
  const size_t kps = (size_t)p.k.page_stride * 2, vps = (size_t)p.v.page_stride * 2;
  // byte offsets (within a tile) of the pieces this lane fetches
  constexpr int kRowsPerWave = kBlock / kP3Waves;      // tile rows each wave fetches
  constexpr int kDmaPerWave = kRowsPerWave / 4;         // 4 rows per DMA instruction
  uint32_t koff[kDmaPerWave], voff[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int row = kRowsPerWave * wave + 4 * i + dr;
    const uint32_t col = (dc ^ (row & 15)) << 4;
    koff[i] = row * kts + col;
    voff[i] = row * vts + col;
  }

  auto stage = [&](int pg, int buf) {
    if (pg < 0) pg = 0;
    const char* kb = kpool + (size_t)pg * kps + khead;
    const char* vb = vpool + (size_t)pg * vps + vhead;
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      dma16(kb + koff[i], L.k[buf] + (kRowsPerWave * wave + 4 * i) * 256);
      dma16(vb + voff[i], L.v[buf] + (kRowsPerWave * wave + 4 * i) * 256);
    }
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
  if (cnt > 0) stage(L.ring_pg[0], 0);

  for (int e = 0; e < cnt; ++e) {
    const int buf = e & 1;
    __builtin_amdgcn_s_waitcnt(0);     // this wave's DMA into buf has landed
    __syncthreads();                   // ... and every other wave's
    if (e >= kRingHalf && (e & (kRingHalf - 1)) == 0) ring_fill(e + kRingHalf);
    const int rc = e & (2 * kRingHalf - 1);
    const int blk = uniform(L.ring_blk[rc]);
    const uint32_t msk = uniform(L.ring_msk[rc]);
    // V rows past every token of the tile hold no data: zero them (only the
    // tile's last block can have such rows) so that a zero probability never
    // meets a NaN
    if (blk * kBlock + kBlock - 1 > p_tile_max) {
      for (int i = tid; i < kBlock * 16; i += kP3Waves * 64) {
        const int row = i >> 4;
        if (blk * kBlock + row > p_tile_max)
          *reinterpret_cast<u32x4*>(L.v[buf] + row * 256 + (i & 15) * 16) = u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();
    }
    if (e + 1 < cnt) stage(L.ring_pg[(e + 1) & (2 * kRingHalf - 1)], buf ^ 1);
    if (!(msk & wave_bits)) continue;

    const bool diag = blk * kBlock + kBlock - 1 > p_wave_min;
    bool live[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) live[ct] = plim_col[ct] >= 0 && ((msk >> tl_col[ct]) & 1u);
    const char* kt = L.k[buf];
    const char* vtl = L.v[buf];

    // S^T for the block: with few columns both halves are computed up front
    // so that the second half's MFMAs can overlap the first half's softmax;
    // with 64 columns one half at a time fits the register file.
    constexpr int kHalves = kP3Waves >= 16 ? 1 : (NCT <= 1 ? 2 : 1);
    f32x4 S[kHalves][4][NCT];
    auto qk_half = [&](int hb, f32x4 (&Sh)[4][NCT]) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(kt + (64 * hb + 16 * pt) * 256 + (kq ^ (s << 6)));
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct)
            Sh[pt][ct] = mfma_bf16(a, qf[ct][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : Sh[pt][ct]);
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
          const char* base = vtl + (32 * chunk) * 256 + (vq ^ (dt << 5));
          const u32x2 lo = lds_tr8(base);
          const u32x2 hi = lds_tr8(base + 16 * 256);
          const u32x4 a = {lo.x, lo.y, hi.x, hi.y};
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

template <int NCT>
__global__ __launch_bounds__(64 * kP3Waves) void attn_prefill3_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) PrefillLds3 lds;
  __shared__ int item_s;
  for (;;) {
    const int k = take_item(p.sched, &item_s);
    if (k < 0) break;
    attn_prefill3_tile<NCT>(p, p.worklist[k], lds);
  }
}

void prefill_tiling(int G, bool fp8, int* tq, int* nct) {
  if (fp8) {   // staged kernel: 8 waves, 16 * nct columns each
    *tq = G >= 16 ? 16 : 32;
    *nct = *tq * G / kPrefillWaves > 16 ? 2 : 1;
  } else {     // direct-load kernel: kP3Waves waves of at most 32 columns
    *tq = std::min(32, kP3Waves * 32 / G);
    const int cpw = *tq * G / kP3Waves;
    *nct = cpw > 16 ? 2 : 1;
  }
}

hipError_t launch_attention_prefill(const AttnParams& p, bool fp8, hipStream_t s) {
  const size_t slots = (size_t)p.rg.batch * p.ntiles * p.H_kv;
  hipLaunchKernelGGL(prefill_plan_kernel, dim3((unsigned)slots), dim3(64),
                     (size_t)p.nbmax * sizeof(uint32_t), s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_schedule_kernel, dim3(1), dim3(kSchedThreads), (size_t)(p.nbmax + 1) * sizeof(int), s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int tq, nct;
  prefill_tiling(p.G, fp8, &tq, &nct);
  const dim3 grid((unsigned)p.nwg);
  if (fp8) {
    const dim3 block(64 * kPrefillWaves);
    if (nct == 2) hipLaunchKernelGGL((attn_prefill_kernel<true, 2>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_prefill_kernel<true, 1>), grid, block, 0, s, p);
  } else {
    const dim3 block(64 * kP3Waves);
    if (nct == 2) hipLaunchKernelGGL((attn_prefill3_kernel<2>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_prefill3_kernel<1>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace msa
