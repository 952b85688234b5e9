// Indexer kernels: per-block max score and top-k block selection.
//
// Semantics ("ferrox_core::block_sparse" page, section "Four rules"): a
// block's score for one (token, KV head) is the maximum over the block's
// positions j <= p of the raw dot product q_idx . k_idx (no softmax scale);
// each KV head selects on its own; the first init and newest local blocks
// are always taken; the remaining top_k - |forced| slots go to the highest
// scores, equal scores to the lower block id.
#include "msa_common.h"
#include "msa_kernels.h"

namespace msa {

// ---------------------------------------------------------------------------
// Block-max scorer for the decode and speculative routes, streaming index-K
// pages from HBM.
//
// Work unit = one 128 x 128 index-K tile scored against one column group: up
// to 16 * NCT columns, a column being one (token, KV head) pair of a sequence
// whose KV head reads index-K head hk (one shared head, or one per KV head).
// Units are ordered (sequence, hk, column group, block) and split into equal
// contiguous shares, one per wave of a grid sized to be resident at once, so
// that every wave streams the same number of bytes whatever the mix of
// context lengths.  Each workgroup recomputes the per-sequence unit counts
// from the ragged metadata (a prefix over chunks of sequences in LDS) rather
// than reading a plan written by another launch.
//
// A wave walks its share in segments that stay inside one column group.  Per
// segment it loads the page ids with one vector load and the query columns
// into MFMA B operands, then streams the tiles as 64-position halves straight
// into A-operand registers (16 B per lane per load, 64 B contiguous per row
// per instruction) with the next half in flight while the current one is
// multiplied.  S^T = K Q^T puts the columns on the MFMA N side; rows
// (positions) reduce with an in-lane max plus two cross-lane steps.
// ---------------------------------------------------------------------------
constexpr int kIdxWaves = 4;
constexpr int kIdxThreads = 64 * kIdxWaves;
constexpr int kMaxSegment = 64;   // blocks per segment: one page id per lane

// Blocks [lo, hi) that column group cg of a sequence with n new tokens and c
// cached ones must score; empty when none of its rows needs a score.
struct GroupRange {
  int lo, hi;
};

template <int NCT>
__device__ __forceinline__ GroupRange group_range(const IndexerParams& p, int n, int c, int hpi, int cg) {
  const int col0 = cg * 16 * NCT;
  GroupRange r{0, 0};
  if (col0 >= n * hpi) return r;
  const int t_last = min(n, (col0 + 16 * NCT + hpi - 1) / hpi) - 1;
  const int nb_last = (c + t_last) / kBlock + 1;
  if (nb_last <= p.top_k) return r;          // every row selects all its blocks
  r.lo = p.init;
  r.hi = max(r.lo, min(nb_last - p.local, p.nbmax));
  return r;
}

// New tokens (clamped to the host bound, so that every address stays inside
// buffers sized from it) and cached tokens of sequence b.
__device__ __forceinline__ int2 seq_shape(const IndexerParams& p, int b) {
  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  return int2{max(n, 0), p.rg.clen[b]};
}

template <int NCT>
__device__ __forceinline__ int64_t group_units(const IndexerParams& p, int n, int c, int hpi, int ncg) {
  int64_t u = 0;
  for (int cg = 0; cg < ncg; ++cg) {
    const GroupRange r = group_range<NCT>(p, n, c, hpi, cg);
    u += r.hi - r.lo;
  }
  return u;
}

// Sequences whose shape (new and cached tokens, first row) a scorer
// workgroup keeps in LDS from its prefix pass, so that a segment's setup
// needs no second round trip for them; larger batches read them again.
constexpr int kSeqLds = 1024;

template <int NCT, bool FP8>
__global__ __launch_bounds__(kIdxThreads) void indexer_score_kernel(IndexerParams p, int ncg) {
  __shared__ int64_t chunk_pre[kIdxThreads + 1];
  __shared__ int3 seq_lds[kSeqLds];
  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int l16 = lane & 15, g = lane >> 4;
  const int B = p.rg.batch;
  const int hpi = p.H_kv / p.H_ik;           // KV heads per index-K head
  const int cpt = (B + kIdxThreads - 1) / kIdxThreads;   // sequences per chunk

  // units of each chunk of cpt sequences, then an inclusive scan over chunks
  {
    int64_t u = 0;
    const int b_end = min(B, (int)(threadIdx.x + 1) * cpt);
    for (int b = threadIdx.x * cpt; b < b_end; ++b) {
      const int2 nc = seq_shape(p, b);
      if (B <= kSeqLds) seq_lds[b] = int3{nc.x, nc.y, p.rg.offs[b]};
      if (nc.x > 0) u += group_units<NCT>(p, nc.x, nc.y, hpi, ncg) * p.H_ik;
    }
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t v = __shfl_up(u, d);
      if (lane >= d) u += v;
    }
    chunk_pre[threadIdx.x + 1] = u;
    __syncthreads();
    int64_t add = 0;
    for (int w = 0; w < wave; ++w) add += chunk_pre[64 * w + 64];
    __syncthreads();
    chunk_pre[threadIdx.x + 1] = u + add;
    if (threadIdx.x == 0) chunk_pre[0] = 0;
    __syncthreads();
  }
  const int64_t total = chunk_pre[kIdxThreads];
  const int64_t W = (int64_t)gridDim.x * kIdxWaves;
  const int64_t w = (int64_t)blockIdx.x * kIdxWaves + wave;
  const int64_t base = total / W, rem = total % W;
  int64_t s = w * base + min(w, rem);
  const int64_t e = s + base + (w < rem ? 1 : 0);

  constexpr int ESZ = FP8 ? 1 : 2;    // bytes per index-K element
  constexpr int KW = FP8 ? 2 : 4;     // 16-byte loads per lane per position tile
  const char* pool = static_cast<const char*>(p.ik.data);
  const size_t ts = (size_t)p.ik.token_stride * ESZ;
  const size_t ps = (size_t)p.ik.page_stride * ESZ;
  const size_t lane_off = (size_t)l16 * ts + (FP8 ? 32 * g : 16 * g);

  while (s < e) {
    // chunk holding unit s: the last j with chunk_pre[j] <= s
    int lo = 0, hi = kIdxThreads;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (chunk_pre[mid] <= s) lo = mid; else hi = mid;
    }
    // walk the chunk's sequences, then (hk, column group) inside the sequence
    // (new tokens, cached tokens, first row) of sequence bq
    auto shape = [&](int bq) {
      if (B <= kSeqLds) return seq_lds[bq];
      const int2 v = seq_shape(p, bq);
      return int3{v.x, v.y, p.rg.offs[bq]};
    };
    int64_t acc = chunk_pre[lo];
    int b = lo * cpt;
    int3 nc = shape(b);
    int64_t per_hk = nc.x > 0 ? group_units<NCT>(p, nc.x, nc.y, hpi, ncg) : 0;
    while (acc + per_hk * p.H_ik <= s) {
      acc += per_hk * p.H_ik;
      ++b;
      nc = shape(b);
      per_hk = nc.x > 0 ? group_units<NCT>(p, nc.x, nc.y, hpi, ncg) : 0;
    }
    const int n = nc.x, c = nc.y;
    int64_t o = s - acc;
    const int hk = (int)(o / per_hk);
    o -= (int64_t)hk * per_hk;
    int cg = 0;
    GroupRange gr = group_range<NCT>(p, n, c, hpi, 0);
    while (o >= gr.hi - gr.lo) {
      o -= gr.hi - gr.lo;
      ++cg;
      gr = group_range<NCT>(p, n, c, hpi, cg);
    }
    const int blk_lo = gr.lo + (int)o;
    const int nblk = (int)min(min((int64_t)(gr.hi - blk_lo), e - s), (int64_t)kMaxSegment);
    s += nblk;

    const int r0 = nc.z;
    const int col0 = cg * 16 * NCT;
    u32x4 qf[NCT][4];
    int plim[NCT];     // last visible position of the column's token (-1: none)
    int orow[NCT];     // (row, KV head) index of the column
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int cc = col0 + ct * 16 + l16;
      const int t = cc / hpi;
      const int h = hk + p.H_ik * (cc % hpi);
      const bool ok = t < n;
      plim[ct] = ok ? c + t : -1;
      orow[ct] = ok ? (r0 + t) * p.H_kv + h : 0;
      const uint16_t* qp = p.q_idx + (size_t)orow[ct] * kDim;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        // contraction dims of k-step q for lane group g: BF16 32q + 8g + j;
        // FP8 (each lane reads 32 consecutive code bytes) 32g + 8q + j
        const int d0 = FP8 ? 32 * g + 8 * q : 32 * q + 8 * g;
        qf[ct][q] = ok ? ld16(qp + d0) : u32x4{0u, 0u, 0u, 0u};
      }
    }

    // page ids of the segment's blocks, one per lane; out-of-pool ids read
    // page 0 and write no score
    int pg_lane = 0;
    if (lane < nblk) pg_lane = p.rg.table[(size_t)b * p.rg.stride + blk_lo + lane];
    if ((unsigned)pg_lane >= (unsigned)p.ik.num_pages) {
      pg_lane = -1;
      if (lane < nblk) report_error(p.err, kErrPage);
    }
    const char* head_base = pool + (size_t)hk * p.ik.head_stride * ESZ + lane_off;
    const float* scale_head = FP8 ? p.ik.scale + (size_t)hk * p.ik.scale_head_stride : nullptr;

    // One 64-position half tile: BF16 as 4 position tiles x 4 k-steps of
    // MFMA operands; FP8 as 4 position tiles x 32 code bytes (two loads)
    // plus the scales of the 4 C-tile rows this lane holds per position tile.
    struct Half {
      u32x4 k[4][KW];
      f32x4 sc[FP8 ? 4 : 1];
    };
    auto load_half = [&](int u, Half& hf) {
      int pg = __builtin_amdgcn_readlane(pg_lane, u >> 1);
      if (pg < 0) pg = 0;
      const char* src = head_base + (size_t)pg * ps + (size_t)(64 * (u & 1)) * ts;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int q = 0; q < KW; ++q) hf.k[pt][q] = ld16(src + (size_t)(16 * pt) * ts + (FP8 ? 16 : 64) * q);
      if constexpr (FP8) {
        const float* sp = scale_head + (size_t)pg * p.ik.scale_page_stride + 64 * (u & 1) + 4 * g;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) hf.sc[pt] = *reinterpret_cast<const f32x4*>(sp + 16 * pt);
      }
    };

    float mx[NCT];
    auto compute_half = [&](int u, const Half& hf) {
      const int blk = blk_lo + (u >> 1);
      const int pos_base = blk * kBlock + 64 * (u & 1);
      const bool clip = pos_base + 63 > c;   // some position past a token
      if ((u & 1) == 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) mx[ct] = neg_inf();
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        u32x4 kf[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (FP8) {
            const u32x4 w = hf.k[pt][q >> 1];
            kf[q] = fp8x8_to_bf16x8((q & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y});
          } else {
            kf[q] = hf.k[pt][q];
          }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; ++q) acc4 = mfma_bf16(kf[q], qf[ct][q], acc4);
          // FP8: row i of this C tile is position 16 pt + 4 g + i, whose
          // value is code * scale, so its dot product is scaled here
          if constexpr (FP8) acc4 = acc4 * hf.sc[pt];
          if (clip) {
            const int lim = plim[ct] - (pos_base + 16 * pt + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i > lim) acc4[i] = neg_inf();
          }
          mx[ct] = fmaxf(mx[ct], fmaxf(fmaxf(acc4[0], acc4[1]), fmaxf(acc4[2], acc4[3])));
        }
      }
      if (u & 1) {
        const bool page_ok = __builtin_amdgcn_readlane(pg_lane, u >> 1) >= 0;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const float m = colgroup_max(mx[ct]);
          if (page_ok && g == 0 && plim[ct] >= 0) p.scores[(size_t)orow[ct] * p.score_stride + blk] = m;
        }
      }
    };

    // halves 0 .. 2 nblk - 1 with the next one always in flight
    Half kA, kB;
    load_half(0, kA);
    for (int j = 0; j < nblk; ++j) {
      load_half(2 * j + 1, kB);
      compute_half(2 * j, kA);
      if (j + 1 < nblk) load_half(2 * j + 2, kA);
      compute_half(2 * j + 1, kB);
    }
  }
}

// Waves the scorer keeps resident per CU (register-limited occupancy; the
// equal shares assume every wave of the grid is resident at once).
constexpr int score_waves_per_cu(int nct, bool fp8) { return nct >= 4 ? 4 : (fp8 && nct == 1) ? 12 : 8; }

hipError_t launch_indexer_decode(const IndexerParams& p, int num_cus, hipStream_t s) {
  const int hpi = p.H_kv / p.H_ik;
  const int cols = p.rg.max_seq * hpi;
  const int nct = cols <= 16 ? 1 : cols <= 32 ? 2 : 4;
  const int ncg = (cols + 16 * nct - 1) / (16 * nct);
  dim3 grid(num_cus * score_waves_per_cu(nct, p.ik_fp8 != 0) / kIdxWaves);
  if (p.ik_fp8) {
    if (nct == 1) hipLaunchKernelGGL((indexer_score_kernel<1, true>), grid, dim3(kIdxThreads), 0, s, p, ncg);
    else if (nct == 2) hipLaunchKernelGGL((indexer_score_kernel<2, true>), grid, dim3(kIdxThreads), 0, s, p, ncg);
    else hipLaunchKernelGGL((indexer_score_kernel<4, true>), grid, dim3(kIdxThreads), 0, s, p, ncg);
  } else {
    if (nct == 1) hipLaunchKernelGGL((indexer_score_kernel<1, false>), grid, dim3(kIdxThreads), 0, s, p, ncg);
    else if (nct == 2) hipLaunchKernelGGL((indexer_score_kernel<2, false>), grid, dim3(kIdxThreads), 0, s, p, ncg);
    else hipLaunchKernelGGL((indexer_score_kernel<4, false>), grid, dim3(kIdxThreads), 0, s, p, ncg);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k selection, one wave per (row, HPW KV heads): HPW = 1, or several
// on the prefill route, where the many rows make the per-wave setup and the
// score loads' latency worth sharing between heads.
//
// Candidates are the blocks [init, nb - local) (everything not forced).  The
// (top_k - |forced|)-th largest score is found as its order-preserving
// 32-bit key by a radix select, eight bits per round from the highest bit
// where candidate keys differ: a round counts the keys that match the bits
// decided so far into 256 LDS bins by their next eight bits and takes the
// highest bin at which the count from the top reaches what is still needed
// (bins summed in 16 groups of 16, each level a 16-lane suffix scan).
// Blocks strictly above the threshold are taken, then the lowest-id blocks
// equal to it until the count is reached.  Output is emitted in ascending id
// order by ballot prefix counts, so no sort is needed: forced-first, chosen
// candidates, forced-newest are already ascending ranges.
// ---------------------------------------------------------------------------

// Sum of lanes j .. 15 of this lane's 16-lane row (lanes past the row add 0).
__device__ __forceinline__ int row_suffix_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x101, 0xf, 0xf, true);   // row_shl:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x102, 0xf, 0xf, true);   // row_shl:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x104, 0xf, 0xf, true);   // row_shl:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x108, 0xf, 0xf, true);   // row_shl:8
  return x;
}

template <int KPL, int HPW>
__global__ __launch_bounds__(256) void topk_kernel(IndexerParams p) {
  // per wave: 256 radix bins, then one bin per lane that takes the adds of
  // keys outside the round (never read), so the adds need no branch
  __shared__ u32x4 hist_lds[4][80];
  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int b = blockIdx.y;
  const int hgroups = (p.H_kv + HPW - 1) / HPW;
  const int idx = blockIdx.x * 4 + wave;
  const int t = idx / hgroups;
  const int h0 = (idx % hgroups) * HPW;
  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  const int clen = p.rg.clen[b];   // requested with the offsets: one round trip
  if (t >= n) return;
  const int nh = min(HPW, p.H_kv - h0);
  const int pos = clen + t;
  const int nb = min(pos / kBlock + 1, p.nbmax);
  const int r = r0 + t;
  int32_t* out0 = p.d_indices + ((size_t)r * p.H_kv + h0) * p.top_k;
  if (nb <= p.top_k) {
    for (int i = lane; i < nh * p.top_k; i += 64) {
      const int k = i % p.top_k;
      out0[i] = k < nb ? k : -1;
    }
    return;
  }
  const int ncand = nb - p.init - p.local;
  const int kfree = p.top_k - p.init - p.local;
  for (int hh = 0; hh < nh; ++hh) {
    int32_t* out = out0 + (size_t)hh * p.top_k;
    for (int i = lane; i < p.init; i += 64) out[i] = i;
    for (int i = lane; i < p.local; i += 64) out[p.init + kfree + i] = nb - p.local + i;
  }
  if (kfree == 0) return;

  const float* sc0 = p.scores + ((size_t)r * p.H_kv + h0) * p.score_stride + p.init;
  const int nslot = (ncand + 63) / 64;
  // Every head's candidate slots are requested before any is used (slots
  // past the end read the last candidate), so one memory latency covers
  // the wave's heads; keys past the candidates are 0, below every real key.
  float v[HPW][KPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
    for (int s = 0; s < KPL; ++s)
      v[hh][s] = HPW == 1 || hh < nh ? sc0[(size_t)hh * p.score_stride + min(s * 64 + lane, ncand - 1)] : 0.f;
  uint32_t* hist = reinterpret_cast<uint32_t*>(hist_lds[wave]);

#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    if (hh >= nh) break;
    int32_t* out = out0 + (size_t)hh * p.top_k;
    uint32_t key[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      const uint32_t k = score_key(v[hh][s]);
      key[s] = s * 64 + lane < ncand ? k : 0u;
    }
    // The search starts below the leading bits that every candidate key
    // shares (sign and exponent of scores of one magnitude, typically six
    // or more bits): the threshold takes the shared value there (a 1 keeps
    // all ncand > kfree keys, a 0 would keep none).  The highest bit where
    // some candidate differs from the first one is found with six ballots
    // over each lane's OR of differences.
    const uint32_t ref = uniform(key[0]);   // lane 0, slot 0: always a candidate
    uint32_t diff = 0u;
#pragma unroll
    for (int s = 0; s < KPL; ++s) diff |= s * 64 + lane < ncand ? key[s] ^ ref : 0u;
    int top = -1;                           // highest differing bit, -1: all keys equal
#pragma unroll
    for (int step = 32; step >= 1; step >>= 1)
      if (top + step <= 31 && ballot((diff >> (top + step)) != 0u)) top += step;
    uint32_t thr = top < 0 ? ref : top == 31 ? 0u : ref & ~((2u << top) - 1u);
    // Radix rounds over bits hb .. hb - w + 1.  Invariant: `gt_keys` keys
    // exceed thr in the bits decided so far, fewer than kfree, and at least
    // kfree - gt_keys of the keys matching thr there remain, so some bin
    // reaches the need and the round's choice exists.  Once exactly kfree
    // keys are at or above the threshold, no lower bit can change which keys
    // those are (equal keys at the boundary never give an exact count), so
    // the search stops there.
    int gt_keys = 0;
    bool exact = false;
    for (int hb = top; hb >= 0;) {
      const int w = min(8, hb + 1), sh = hb + 1 - w;
      const uint32_t hi = hb == 31 ? 0u : ~((2u << hb) - 1u);   // bits already decided
      const uint32_t pre = thr & hi;
      hist_lds[wave][lane] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < KPL; ++s) {
        const bool in = (s * 64 + lane < ncand) & ((key[s] & hi) == pre);
        const uint32_t bin = in ? (key[s] >> sh) & ((1u << w) - 1u) : 256u + lane;
        __hip_atomic_fetch_add(hist + bin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      }
      const int need = kfree - gt_keys;
      // group j = bins 16 j .. 16 j + 15, suffix counts over groups
      int gs = 0;
      if (lane < 16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 c4 = hist_lds[wave][4 * lane + q];
          gs += (int)(c4[0] + c4[1] + c4[2] + c4[3]);
        }
      }
      gs = row_suffix_sum(gs);
      // (bit 0 only guards the count of leading zeros: the invariant puts
      // group 0 and bin 0 of a group at or above the need)
      const int G = 63 - __builtin_clzll(ballot(lane < 16 && gs >= need) | 1ull);
      const int g_above = G == 15 ? 0 : __builtin_amdgcn_readlane(gs, G + 1);
      int bs = lane < 16 ? (int)hist[16 * G + lane] : 0;
      bs = row_suffix_sum(bs);
      const int j = 63 - __builtin_clzll(ballot(lane < 16 && g_above + bs >= need) | 1ull);
      const int n_ge = g_above + __builtin_amdgcn_readlane(bs, j);              // bins >= 16 G + j
      const int n_gt = g_above + (j == 15 ? 0 : __builtin_amdgcn_readlane(bs, j + 1));
      thr |= (uint32_t)(16 * G + j) << sh;
      if (n_ge == need) {
        exact = true;
        break;
      }
      gt_keys += n_gt;
      hb -= w;
    }
    int run = 0;
    if (exact) {
      // the candidates at or above the threshold are exactly the kfree chosen
#pragma unroll
      for (int s = 0; s < KPL; ++s) {
        if (s < nslot) {
          const bool sel = s * 64 + lane < ncand && key[s] >= thr;
          const uint64_t sm = ballot(sel);
          if (sel) out[p.init + run + mask_rank(sm)] = p.init + s * 64 + lane;
          run += __popcll(sm);
        }
      }
      continue;
    }
    // equal keys straddle the cut: all above it, then the lowest ids equal
    // to it (keys past the candidates rank after every candidate)
    int above = 0;
#pragma unroll
    for (int s = 0; s < KPL; ++s) above += __popcll(ballot(key[s] > thr));
    const int need_eq = kfree - above;
    int run_eq = 0;
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
      if (s < nslot) {
        const bool eq = key[s] == thr;
        const uint64_t em = ballot(eq);
        const bool sel = key[s] > thr || (eq && run_eq + mask_rank(em) < need_eq);
        const uint64_t sm = ballot(sel);
        if (sel) out[p.init + run + mask_rank(sm)] = p.init + s * 64 + lane;
        run += __popcll(sm);
        run_eq += __popcll(em);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection reuse across draft steps: a row gather.  One workgroup per 8
// rows (one wave per two rows' worth of ids at width 8 x 64); the source
// row is read once per row and broadcast.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void reuse_kernel(int32_t* out, const int32_t* prev, const int32_t* src,
                                                    int rows, int prev_rows, int width) {
  const int r = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (r >= rows) return;
  const int sr = src[r];
  const bool ok = sr >= 0 && sr < prev_rows;
  int32_t* o = out + (size_t)r * width;
  const int32_t* in = prev + (size_t)(ok ? sr : 0) * width;
  for (int i = threadIdx.x & 31; i < width; i += 32) o[i] = ok ? in[i] : -1;
}

hipError_t launch_indexer_reuse(int32_t* out, const int32_t* prev, const int32_t* src, int rows,
                                int prev_rows, int width, hipStream_t s) {
  hipLaunchKernelGGL(reuse_kernel, dim3((rows + 7) / 8), dim3(256), 0, s, out, prev, src, rows,
                     prev_rows, width);
  return hipGetLastError();
}

hipError_t launch_topk(const IndexerParams& p, hipStream_t s) {
  const int ncand_max = p.nbmax - p.init - p.local;
  // With many rows (the prefill route) one wave takes several KV heads of a
  // token, paying the per-wave setup and the score loads' latency once.
  const bool many = p.rg.max_seq > 8;
  const dim3 block(256);
  auto grid = [&](int hpw) {
    return dim3((unsigned)((p.rg.max_seq * ((p.H_kv + hpw - 1) / hpw) + 3) / 4), (unsigned)p.rg.batch);
  };
  if (ncand_max <= 256) {
    if (many) hipLaunchKernelGGL((topk_kernel<4, 8>), grid(8), block, 0, s, p);
    else hipLaunchKernelGGL((topk_kernel<4, 1>), grid(1), block, 0, s, p);
  } else if (ncand_max <= 1024) {
    if (many) hipLaunchKernelGGL((topk_kernel<16, 2>), grid(2), block, 0, s, p);
    else hipLaunchKernelGGL((topk_kernel<16, 1>), grid(1), block, 0, s, p);
  } else if (ncand_max <= 4096) {
    hipLaunchKernelGGL((topk_kernel<64, 1>), grid(1), block, 0, s, p);
  } else {
    hipLaunchKernelGGL((topk_kernel<128, 1>), grid(1), block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace msa
