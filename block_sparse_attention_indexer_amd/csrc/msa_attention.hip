// Sparse attention over selected KV blocks (decode / speculative decode
// route) with split-K partitions, and the split-K combine.
//
// Semantics ("ferrox_core::block_sparse" page, positions_of_blocks and the
// masked pass it feeds; "msa" page, speculative-decode route): token t of
// sequence b sits at position p = cache_lengths[b] + t and attends to the
// positions j <= p of the blocks its KV head selected, with an ordinary
// softmax; every query head of the GQA group reads the same blocks.
//
// Work item = (sequence, KV head, group of `tpw` tokens, partition).  One
// wave owns an item.  Its MFMA columns are (token, query head) pairs:
// 16 = tpw * G (decode uses one token, so with G = 8 half the columns idle).
// The wave builds the ascending union of its tokens' block lists in LDS
// (with a per-block membership mask), takes its partition's slice of it,
// and streams each block's K and V tiles straight from HBM into MFMA
// operand registers:
//   S^T = K Q^T        A = K rows (positions), B = Q^T  -> C[position][column]
//   O^T += V^T P^T     A = V^T built in registers by 16-bit permutes,
//                      B = P^T, which is exactly the C layout of S^T
// so the softmax statistics of a column stay in the lanes that own it and
// no LDS round trip is needed.  Online softmax runs per 64-position half
// block in log2 units.
//
// Workgroups: one wave per (sequence, KV head) on the decode route; the
// token groups of a (sequence, KV head) in one workgroup when speculative
// rows are split into partitions; and one wave per workgroup, the busy
// token groups first, when speculative rows run in one partition (a CU
// streams at most about 43 GB/s however many of its waves are busy, so the
// busy waves are spread over the CUs).
#include <type_traits>

#include "msa_common.h"
#include "msa_kernels.h"
#include "msa_splitk.h"

namespace msa {

// Exclusive prefix over the wave's lanes of a per-lane count 0 <= v < 64,
// and the wave's total: one ballot per bit of the count, so no cross-lane
// shuffle chain.
__device__ __forceinline__ void wave_prefix_small(int v, int* before, int* total) {
  int bsum = 0, tsum = 0;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const uint64_t bk = ballot((v >> k) & 1);
    bsum += mask_rank(bk) << k;
    tsum += __popcll(bk) << k;
  }
  *before = bsum;
  *total = tsum;
}

template <bool FP8>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(AttnParams p) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  const int ntok_groups = (p.rg.max_seq + p.tpw - 1) / p.tpw;
  const int ntgb = (ntok_groups + W - 1) / W;
  // Group = (sequence, KV head, workgroup of token groups); its np
  // partitions are workgroups whose indices are congruent modulo the XCD
  // count, which the hardware dispatches to one XCD (workgroup i runs on XCD
  // i mod 8), so that the split-K exchange stays inside one L2.  One-wave
  // workgroups of speculative rows (p.tgs > 1, one partition) keep the
  // token groups of a (sequence, KV head) on one XCD as well (below).
  int pi, grp, tgb, sh;   // grp: split-K group (flags); sh: (sequence, KV head)
  if (p.tgs > 1) {
    // One-wave workgroups of speculative rows: XCD x takes the (sequence,
    // KV head) pairs sh = 8 q + x, and its workgroup j the j-th token group
    // that has tokens, counting q-major.  So the busy token groups are the
    // XCD's first workgroups, which the dispatcher spreads over its CUs
    // (consecutive workgroups go to different CUs), and the token groups of
    // one pair sit on one XCD, side by side, where the blocks they share
    // meet in its L2.  Workgroups past the busy token groups have nothing
    // to do.
    const int xcd = blockIdx.x % kXcdCount, j = blockIdx.x / kXcdCount;
    const int pairs = p.rg.batch * p.H_kv;
    int seen = 0;
    sh = -1;
    tgb = 0;
    for (int q0 = 0; q0 * kXcdCount < pairs; q0 += 64) {
      const int sq = (q0 + lane) * kXcdCount + xcd;
      int act = 0;
      if (sq < pairs) {
        const int bq = sq / p.H_kv;
        const int nq = min(p.rg.offs[bq + 1] - p.rg.offs[bq], p.rg.max_seq);
        act = min(p.tgs, (max(nq, 0) + p.tpw - 1) / p.tpw);
      }
      int before = 0, total = 0;
      wave_prefix_small(act, &before, &total);
      const uint64_t hit = ballot(act > 0 && seen + before <= j && j < seen + before + act);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        sh = (q0 + l) * kXcdCount + xcd;
        tgb = j - seen - __builtin_amdgcn_readlane(before, l);
        break;
      }
      seen += total;
    }
    if (sh < 0) return;
    pi = 0;
    grp = sh;                                      // (one partition: no flags)
  } else {
    splitk_slot(blockIdx.x, p.np, &pi, &grp);
    if (grp >= p.rg.batch * p.H_kv * ntgb) return;   // padding of the last XCD round
    tgb = grp % ntgb;
    sh = grp / ntgb;
  }
  const int h = sh % p.H_kv;
  const int b = sh / p.H_kv;

  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);   // keeps rows < rcap
  const int c = p.rg.clen[b];
  // more new tokens than the host bound, or blocks past the table (clipped)
  if (threadIdx.x == 0 && pi == 0 && tgb == 0 && h == 0 &&
      (p.rg.offs[b + 1] - r0 > p.rg.max_seq || (n > 0 && (c + n - 1) / kBlock >= p.nbmax)))
    report_error(p.err, kErrLength);
  const int tok0 = (tgb * W + wave) * p.tpw;
  const int ntok = max(0, min(n - tok0, p.tpw));

  // ---- union of the wave's token selections, ascending, in LDS ----------
  // LDS: one bitmap row of nbw words per token of the TG token groups
  // scheduled together (the workgroup's waves, or with one-wave workgroups
  // every token group of the (sequence, KV head)), then each wave's union.
  const int nbw = (p.nbmax + 31) >> 5;
  const int cap = p.tpw * p.top_k;
  const int TG = W > 1 ? W : p.tgs;
  const int own = W > 1 ? wave : tgb;              // this wave's token group among the TG
  const int row_tok0 = W > 1 ? tgb * W * p.tpw : 0;   // token of bitmap row 0
  uint32_t* bm = lds;
  uint32_t* bm_own = bm + own * p.tpw * nbw;
  int32_t* uid = reinterpret_cast<int32_t*>(lds + TG * p.tpw * nbw + wave * 2 * cap);
  uint32_t* umk = reinterpret_cast<uint32_t*>(uid + cap);
  int nU = 0;
  // One token per wave (decode): when the row's valid ids come first and
  // ascend, as the indexer writes them, the row is the union itself.  Each
  // entry's page is then requested as soon as its id arrives and kept in
  // umk (the token mask is 1), so the page lookup needs no round trip of its
  // own after the union is built.  Other rows take the bitmap below.
  bool ids_in_order = false;
  if (p.tpw == 1 && TG == 1 && ntok == 1) {
    const int nbt = min((c + tok0) / kBlock + 1, p.nbmax);
    const int32_t* lst = p.d_indices + ((size_t)(r0 + tok0) * p.H_kv + h) * p.top_k;
    bool ok = true, seen_invalid = false;
    for (int i0 = 0; i0 < p.top_k; i0 += 64) {
      const int i = i0 + lane;
      const int id = i < p.top_k ? lst[i] : -1;
      const bool valid = id >= 0 && id < nbt;
      const uint64_t vm = ballot(valid);
      // valid entries must form a prefix of the row
      ok = ok && (vm & (vm + 1ull)) == 0ull && !(seen_invalid && vm != 0ull);
      seen_invalid = seen_invalid || vm != ~0ull;
      if (i < p.top_k) {
        uid[i] = id;
        umk[i] = valid ? (uint32_t)p.rg.table[(size_t)b * p.rg.stride + id] : 0u;
      }
      nU += __popcll(vm);
    }
    __syncthreads();   // (one wave) the ids of every lane are in LDS
    // strictly ascending: each valid entry above the one before it
    for (int i0 = 0; i0 < nU; i0 += 64) {
      const int i = i0 + lane;
      if (ballot(i > 0 && i < nU && uid[i - 1] >= uid[i]) != 0ull) ok = false;
    }
    ids_in_order = ok;
    if (!ok) nU = 0;
  }
  if (!ids_in_order) {
    // rows this wave fills: its own token group's, or with one-wave
    // workgroups every token group's
    const int rw0 = W > 1 ? own * p.tpw : 0;
    const int rw1 = W > 1 ? rw0 + p.tpw : TG * p.tpw;
    for (int i = rw0 * nbw + lane; i < rw1 * nbw; i += 64) bm[i] = 0u;
    __syncthreads();
    for (int row = rw0; row < rw1; ++row) {
      const int tok = row_tok0 + row;
      if (tok >= n) break;
      const int nbt = min((c + tok) / kBlock + 1, p.nbmax);
      const int32_t* lst = p.d_indices + ((size_t)(r0 + tok) * p.H_kv + h) * p.top_k;
      for (int i = lane; i < p.top_k; i += 64) {
        const int id = lst[i];
        if (id >= 0 && id < nbt) atomicOr(&bm[row * nbw + (id >> 5)], 1u << (id & 31));
      }
    }
    __syncthreads();
    // Each lane takes one 32-block word: its set bits in ascending order go
    // to consecutive union slots after the lanes below it.  The tokens'
    // words are kept in registers (T: a bound on the wave's tokens, at most
    // 16), and the exclusive prefix of the per-lane counts (at most 32) is
    // summed over six ballots, one per bit of the count.
    auto build = [&](auto tmax) {
      constexpr int T = decltype(tmax)::value;
      for (int w0 = 0; w0 < nbw; w0 += 64) {
        const int w = w0 + lane;
        uint32_t wd[T];
        uint32_t u = 0u;
#pragma unroll
        for (int tl = 0; tl < T; ++tl) {
          wd[tl] = tl < ntok && w < nbw ? bm_own[tl * nbw + w] : 0u;
          u |= wd[tl];
        }
        int before = 0, total = 0;
        wave_prefix_small(__popc(u), &before, &total);
        int pos = nU + before;
        while (u) {
          const int bit = __ffs(u) - 1;
          u &= u - 1u;
          uint32_t mk = 0u;
#pragma unroll
          for (int tl = 0; tl < T; ++tl) mk |= ((wd[tl] >> bit) & 1u) << tl;
          uid[pos] = w * 32 + bit;
          umk[pos] = mk;
          ++pos;
        }
        nU += total;
      }
    };
    if (p.tpw <= 2) build(std::integral_constant<int, 2>{});
    else if (p.tpw <= 4) build(std::integral_constant<int, 4>{});
    else if (p.tpw <= 8) build(std::integral_constant<int, 8>{});
    else build(std::integral_constant<int, 16>{});
  }
  __syncthreads();
  // With several tokens per wave (speculative rows), the waves of one
  // (sequence, KV head) need many of the same blocks: every token's first
  // and newest blocks, and the picks their tokens share.  Such a block costs
  // one HBM fetch only if the waves reach it at about the same moment (an
  // L2 line does not outlive much of another wave's streaming), so the
  // waves walk their unions on one common schedule.  The blocks that more
  // than one wave needs form one global order (most waves first, then by
  // id); step g of every wave is global block g if the wave needs it, else
  // the wave's next block that no other wave needs, while those last.  So
  // wave w's k-th shared block, at global index g, sits at k + min(P, g -
  // k) (P: its private blocks), and its private block j at j + #{shared k :
  // g - k <= j}.  Counting waves per block is bit-sliced over the
  // workgroup's block bitmaps, one 32-block word per lane.  Unions of more
  // than 64 blocks, or bitmaps of more than 64 words, are walked block 0
  // first, then newest first, as are workgroups of more than four waves
  // (the bit-sliced count takes four).  The order of blocks changes only
  // the rounding order of the softmax sums.
  if (p.tpw > 1 && nU > 1) {
    if (TG > 1 && TG <= 4 && nU <= 64 && nbw <= 64) {
      // -- blocks needed by exactly 2, 3 and 4 waves, per 32-block word --
      uint32_t E2 = 0u, E3 = 0u, E4 = 0u;
      if (lane < nbw) {
        uint32_t u[4] = {0u, 0u, 0u, 0u};
        for (int w2 = 0; w2 < TG; ++w2) {
          const uint32_t* bm2 = bm + w2 * p.tpw * nbw;
          uint32_t any = 0u;
          for (int tl = 0; tl < p.tpw; ++tl) any |= bm2[tl * nbw + lane];
          u[w2] = any;
        }
        // per-bit count of four words: bits b0 + 2 b1 + 4 b2
        const uint32_t s01 = u[0] ^ u[1], c01 = u[0] & u[1], s23 = u[2] ^ u[3], c23 = u[2] & u[3];
        const uint32_t b0 = s01 ^ s23, k1 = s01 & s23;
        const uint32_t b1 = c01 ^ c23 ^ k1, b2 = (c01 & c23) | ((c01 ^ c23) & k1);
        E2 = ~b0 & b1 & ~b2;
        E3 = b0 & b1;
        E4 = b2;
      }
      // exclusive prefix counts over words and totals, per class, packed
      // as three 21-bit fields (class c at bit 21 (c - 2))
      uint64_t excl = 0ull, tot = 0ull;
      {
        const uint32_t ew[3] = {E2, E3, E4};
#pragma unroll
        for (int f = 0; f < 3; ++f) {
          int bf = 0, tf = 0;
          wave_prefix_small(__popc(ew[f]), &bf, &tf);
          excl |= (uint64_t)bf << (21 * f);
          tot |= (uint64_t)tf << (21 * f);
        }
      }
      auto field = [](uint64_t v, int c) { return (int)((v >> (21 * (c - 2))) & 0x1FFFFFu); };
      // -- this wave's entries, one per lane --------------------------------
      const bool has = lane < nU;
      const int x = has ? uid[lane] : 0;
      const uint32_t mk = has ? umk[lane] : 0u;
      const int wd = x >> 5;
      const uint32_t e2 = __shfl(E2, wd), e3 = __shfl(E3, wd), e4 = __shfl(E4, wd);
      const uint32_t pw_lo = __shfl((uint32_t)excl, wd), pw_hi = __shfl((uint32_t)(excl >> 32), wd);
      const uint64_t pw = ((uint64_t)pw_hi << 32) | pw_lo;
      const uint32_t bit = 1u << (x & 31);
      const int cls = !has ? 0 : (e4 & bit) ? 4 : (e3 & bit) ? 3 : (e2 & bit) ? 2 : 1;
      const uint32_t ec = cls == 4 ? e4 : cls == 3 ? e3 : e2;
      int gidx = 0;   // global index of a shared block
      if (cls >= 2) {
        for (int c2 = cls + 1; c2 <= 4; ++c2) gidx += field(tot, c2);
        gidx += field(pw, cls) + __popc(ec & (bit - 1u));
      }
      // rank among this wave's shared blocks in the global order (classes
      // high to low, ids ascending within a class), and among its private ones
      int rnk = 0, nshared = 0;
      for (int cl = 4; cl >= 2; --cl) {
        const uint64_t m = ballot(cls == cl);
        if (cls == cl) rnk = nshared + mask_rank(m);
        nshared += __popcll(m);
      }
      {
        const uint64_t m = ballot(cls == 1);
        if (cls == 1) rnk = mask_rank(m);
      }
      const int npriv = nU - nshared;
      const int dgap = gidx - rnk;   // shared: global steps before it not taken by its own shared blocks
      // shared blocks placed before private block rnk (the ballot and the
      // walk over shared lanes run with every lane active)
      int before = 0;
      uint64_t sm = ballot(cls >= 2);
      while (sm) {
        const int t = __builtin_ctzll(sm);
        sm &= sm - 1;
        before += __builtin_amdgcn_readlane(dgap, t) <= rnk;
      }
      const int npos = cls >= 2 ? rnk + min(npriv, dgap) : rnk + before;
      if (has) {
        uid[npos] = x;
        umk[npos] = mk;
      }
    } else {
      const int lo = uid[0] == 0 ? 1 : 0;
      const int len = nU - lo;
      for (int i = lane; i < len / 2; i += 64) {
        const int a = lo + i, z = lo + len - 1 - i;
        const int32_t ia = uid[a], iz = uid[z];
        const uint32_t ma = umk[a], mz = umk[z];
        uid[a] = iz;
        uid[z] = ia;
        umk[a] = mz;
        umk[z] = ma;
      }
    }
  }
  __syncthreads();

  // ---- this partition's slice of the union --------------------------------
  const int per = (nU + p.np - 1) / p.np;
  const int e_lo = min(nU, pi * per);
  const int e_hi = min(nU, e_lo + per);

  // ---- columns: (token, query head) pairs ---------------------------------
  const int tl_col = l16 / p.G;
  const int g_col = l16 % p.G;
  const bool col_ok = tl_col < ntok;
  const int p_col = c + tok0 + tl_col;
  const int qrow = r0 + tok0 + tl_col;
  const int hq = h * p.G + g_col;
  const int p_max = c + tok0 + ntok - 1;

  u32x4 qf[4];
  {
    const uint16_t* qp = p.q + ((size_t)qrow * p.H_q + hq) * kDim;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int d0 = FP8 ? 32 * g + 8 * s : 32 * s + 8 * g;
      qf[s] = col_ok ? ld16(qp + d0) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 O[8];
#pragma unroll
  for (int T = 0; T < 8; ++T) O[T] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = neg_inf(), l_run = 0.f;

  const int esz = FP8 ? 1 : 2;
  const char* kpool = static_cast<const char*>(p.k.data);
  const char* vpool = static_cast<const char*>(p.v.data);
  const size_t kts = (size_t)p.k.token_stride * esz, vts = (size_t)p.v.token_stride * esz;
  const size_t khead = (size_t)h * p.k.head_stride * esz, vhead = (size_t)h * p.v.head_stride * esz;
  const size_t kps = (size_t)p.k.page_stride * esz, vps = (size_t)p.v.page_stride * esz;
  // per-lane byte offsets inside a half block; a page's rows span less than
  // 2 GiB (checked on the host), so 32 bits hold them
  const uint32_t koff = (uint32_t)l16 * (uint32_t)kts + (FP8 ? 32u : 16u) * g;
  const uint32_t voff = (uint32_t)(4 * g) * (uint32_t)vts + (FP8 ? 8u : 16u) * l16;

  // Raw tiles of one 64-position half block.  BF16: K as MFMA A operands
  // (4 position tiles x 4 k-steps), V as 2 chunks x 8 rows of 8 dims per
  // lane.  FP8: the same bytes at half width, widened when consumed.
  constexpr int KW = FP8 ? 2 : 4;
  typedef typename std::conditional<FP8, u32x2, u32x4>::type VRaw;
  u32x4 kraw[4][KW];
  VRaw vraw[2][8];

  // The slice is walked in segments of up to 64 union entries; per segment
  // each lane holds one entry's block id, token mask and page id, so that no
  // table lookup sits between consecutive blocks.  Inside a segment the
  // halves form a pipeline: K of the next half is requested as soon as the
  // scores of the current half have consumed K, V of the next half as soon
  // as P V has consumed V, so one half's worth of loads is always in flight.
  const int nE = e_hi - e_lo;
  for (int s0 = 0; s0 < nE; s0 += 64) {
    const int nS = min(64, nE - s0);
    int blk_lane = 0, pg_lane = -1;
    uint32_t mk_lane = 0u;
    if (lane < nS) {
      blk_lane = uid[e_lo + s0 + lane];
      mk_lane = umk[e_lo + s0 + lane];
      int pg;
      if (ids_in_order) {   // umk holds the page; the one token's mask is 1
        pg = (int)mk_lane;
        mk_lane = 1u;
      } else {
        pg = p.rg.table[(size_t)b * p.rg.stride + blk_lane];
      }
      pg_lane = (unsigned)pg < (unsigned)p.k.num_pages ? pg : -1;   // bad ids: block skipped
      if (pg_lane < 0) report_error(p.err, kErrPage);
    }

    // Addresses = wave-uniform base (page, head, half block, row constant)
    // + a 32-bit per-lane offset, so the loads take the scalar-base form.
    auto page_of = [&](int u) { return max(__builtin_amdgcn_readlane(pg_lane, u >> 1), 0); };
    // A load whose rows all lie past the wave's last visible position in
    // the half is pointed at the half's first rows instead, which other
    // loads of the half fetch anyway (an L2 hit): its values are masked (K)
    // or zeroed (V) later, so it need not fetch anything new from HBM.  The
    // choice is wave-uniform and made on the scalar base, so every load stays
    // unconditional and keeps its one per-lane offset.
    auto last_row = [&](int u) {
      return p_max - (__builtin_amdgcn_readlane(blk_lane, u >> 1) * kBlock + 64 * (u & 1));
    };
    auto issue_k = [&](int u) {
      const char* kb = kpool + (size_t)page_of(u) * kps + khead + (size_t)(64 * (u & 1)) * kts;
      const int lr = last_row(u);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const char* rowb = kb + (size_t)(16 * pt > lr ? 0 : 16 * pt) * kts;
#pragma unroll
        for (int s = 0; s < KW; ++s) kraw[pt][s] = ld16(rowb + koff + (FP8 ? 16 * s : 64 * s));
      }
    };
    auto issue_v = [&](int u) {
      const char* vb = vpool + (size_t)page_of(u) * vps + vhead + (size_t)(64 * (u & 1)) * vts;
      const int lr = last_row(u);
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r0 = 32 * ch + 16 * (j >> 2) + (j & 3);   // the load's rows: r0 + 4 g
          const char* rowb = vb + (size_t)(r0 > lr ? (j & 3) : r0) * vts;
          if constexpr (FP8) vraw[ch][j] = ld8(rowb + voff);
          else vraw[ch][j] = ld16(rowb + voff);
        }
    };

    auto half = [&](int u, auto prefetch) {
      constexpr bool kNext = decltype(prefetch)::value;
      const int i = u >> 1;
      const int blk = __builtin_amdgcn_readlane(blk_lane, i);
      const uint32_t msk = __builtin_amdgcn_readlane(mk_lane, i);
      const bool pvalid = __builtin_amdgcn_readlane(pg_lane, i) >= 0;
      const int plim = (pvalid && col_ok && ((msk >> tl_col) & 1u)) ? p_col : -1;
      const int pos0 = blk * kBlock + 64 * (u & 1);

      // -- S^T = K Q^T ------------------------------------------------------
      u32x4 kf[4][4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (FP8) {
            const u32x4 w = kraw[pt][s >> 1];
            kf[pt][s] = fp8x8_to_bf16x8((s & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y});
          } else {
            kf[pt][s] = kraw[pt][s];
          }
        }
      f32x4 sacc[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        sacc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[pt] = mfma_bf16(kf[pt][s], qf[s], sacc[pt]);
      }
      // fences keep the next half's loads from being hoisted above the
      // instructions that still read the buffers they overwrite
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kNext) issue_k(u + 1);
      __builtin_amdgcn_sched_barrier(0);

      // -- scale, causal/selection mask, online softmax ---------------------
      float hmax = neg_inf();
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int pos = pos0 + 16 * pt + 4 * g + ii;
          const float v = pos <= plim ? sacc[pt][ii] * p.scale_log2 : neg_inf();
          sacc[pt][ii] = v;
          hmax = fmaxf(hmax, v);
        }
      hmax = colgroup_max(hmax);
      const float m_new = fmaxf(m_run, hmax);
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float e2 = exp2f(sacc[pt][ii] - m_use);
          sacc[pt][ii] = e2;
          lsum += e2;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int T = 0; T < 8; ++T) O[T] *= alpha;

      // -- V rows past every token of the wave (or of a skipped block) hold
      //    no data: zero them so that 0 * garbage cannot poison O ---------
      if (!pvalid || pos0 + 63 > p_max) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (!pvalid || pos0 + 32 * ch + 16 * (j >> 2) + 4 * g + (j & 3) > p_max) vraw[ch][j] = VRaw{};
      }
      u32x4 vrow[2][8];
#pragma unroll
      for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (FP8) vrow[ch][j] = fp8x8_to_bf16x8(vraw[ch][j]);
          else vrow[ch][j] = vraw[ch][j];
        }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (FP8 && kNext) issue_v(u + 1);

      // -- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        const f32x4 s0v = sacc[2 * ch], s1v = sacc[2 * ch + 1];
        const u32x4 bp = {pack_bf16(s0v[0], s0v[1]), pack_bf16(s0v[2], s0v[3]),
                          pack_bf16(s1v[0], s1v[1]), pack_bf16(s1v[2], s1v[3])};
#pragma unroll
        for (int T = 0; T < 8; ++T) {
          u32x4 a;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            a[q] = pick_halves(vrow[ch][2 * q][T >> 1], vrow[ch][2 * q + 1][T >> 1], T & 1);
          O[T] = mfma_bf16(a, bp, O[T]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!FP8 && kNext) issue_v(u + 1);
      __builtin_amdgcn_sched_barrier(0);
    };

    issue_k(0);
    issue_v(0);
    const int nh = 2 * nS;
    for (int u = 0; u < nh - 1; ++u) half(u, std::true_type{});
    half(nh - 1, std::false_type{});
  }

  // ---- epilogue: normalise and store --------------------------------------
  const float l_tot = colgroup_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (p.np == 1) {
    if (!col_ok) return;
    uint16_t* op = p.out + ((size_t)qrow * p.H_q + hq) * kDim + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = {pack_bf16(O[0][i] * inv, O[1][i] * inv), pack_bf16(O[2][i] * inv, O[3][i] * inv),
                       pack_bf16(O[4][i] * inv, O[5][i] * inv), pack_bf16(O[6][i] * inv, O[7][i] * inv)};
      *reinterpret_cast<u32x4*>(op + 8 * i) = v;
    }
    return;
  }
  // Split-K: store this partition's normalised partial and its log-sum-exp
  // (natural log), keyed on the ragged row; the group's last partition
  // merges (msa_splitk.h: the exchange stays in the group's XCD).
  const size_t col = (size_t)qrow * p.H_q + hq;
  const size_t pstride = (size_t)p.rcap * p.H_q;
  if (col_ok) {
    float* op = p.part_o + ((size_t)pi * pstride + col) * kDim + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4*>(op + 8 * i) = f32x4{O[0][i] * inv, O[1][i] * inv, O[2][i] * inv, O[3][i] * inv};
      *reinterpret_cast<f32x4*>(op + 8 * i + 4) = f32x4{O[4][i] * inv, O[5][i] * inv, O[6][i] * inv, O[7][i] * inv};
    }
    if (g == 0) p.part_lse[(size_t)pi * pstride + col] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : neg_inf();
  }
  __shared__ int merge_sh[3];
  uint64_t* flags = p.ready + (size_t)grp * p.np;
  if (!splitk_arrive(flags, pi, p.np, p.epoch)) return;
  // each wave merges its own columns: l16 < nc (columns are token-major)
  const int nc = min(16, ntok * p.G);
  const int ncp = nc <= 2 ? 2 : nc <= 4 ? 4 : nc <= 8 ? 8 : 16;
  auto row_of = [&](int cc) { return r0 + tok0 + cc / p.G; };
  auto head_of = [&](int cc) { return h * p.G + cc % p.G; };
  switch (ncp) {
    case 2: splitk_merge<1>(flags, p.epoch, merge_sh, p.part_o, p.part_lse, p.out, p.H_q, p.rcap, p.np, nc, row_of, head_of, lane); break;
    case 4: splitk_merge<2>(flags, p.epoch, merge_sh, p.part_o, p.part_lse, p.out, p.H_q, p.rcap, p.np, nc, row_of, head_of, lane); break;
    case 8: splitk_merge<4>(flags, p.epoch, merge_sh, p.part_o, p.part_lse, p.out, p.H_q, p.rcap, p.np, nc, row_of, head_of, lane); break;
    default: splitk_merge<8>(flags, p.epoch, merge_sh, p.part_o, p.part_lse, p.out, p.H_q, p.rcap, p.np, nc, row_of, head_of, lane); break;
  }
}

size_t attention_decode_lds_bytes(const AttnParams& p) {
  const int nbw = (p.nbmax + 31) / 32;
  const int tg = p.ntg > 1 ? p.ntg : p.tgs;
  return ((size_t)tg * p.tpw * nbw + (size_t)p.ntg * 2 * p.tpw * p.top_k) * sizeof(uint32_t);
}

hipError_t launch_attention_decode(const AttnParams& p, bool fp8, hipStream_t s) {
  const int ntok_groups = (p.rg.max_seq + p.tpw - 1) / p.tpw;
  const int ntgb = (ntok_groups + p.ntg - 1) / p.ntg;
  const size_t nwg = p.tgs > 1 ? (size_t)kXcdCount * ((p.rg.batch * p.H_kv + kXcdCount - 1) / kXcdCount) * p.tgs
                               : splitk_workgroups((size_t)p.rg.batch * p.H_kv * ntgb, p.np);
  const size_t lds = attention_decode_lds_bytes(p);
  dim3 grid((unsigned)nwg), block(64 * p.ntg);
  if (fp8) hipLaunchKernelGGL(attn_decode_kernel<true>, grid, block, lds, s, p);
  else hipLaunchKernelGGL(attn_decode_kernel<false>, grid, block, lds, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K combine: out = sum_pi exp(lse_pi - LSE) o_pi / sum_pi exp(lse_pi -
// LSE), partitions with lse = -inf skipped.  One workgroup per (row slot,
// 8 query heads); 32 lanes per head, 4 dims per lane.  Lane i of a head's
// group reads lse of partitions i and i + 32, so the weights come from one
// load and a 32-lane reduction; the partial outputs are then read with all
// loads of a pass in flight.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int hgroups = (p.H_q + 7) >> 3;
  const int rs = blockIdx.x / hgroups;
  const int hq = (blockIdx.x % hgroups) * 8 + (threadIdx.x >> 5);
  const int b = rs / p.max_seq, t = rs % p.max_seq;
  const int r0 = p.offs[b];
  if (t >= min(p.offs[b + 1] - r0, p.max_seq) || hq >= p.H_q) return;
  const int r = r0 + t;
  const int sub = threadIdx.x & 31;
  const size_t stride = (size_t)p.rcap * p.H_q;          // between partitions
  const size_t base = (size_t)r * p.H_q + hq;
  const float* po = p.part_o + base * kDim + 4 * sub;
  // the first eight partitions' outputs are requested together with the
  // lse values (one memory round trip after the offsets, not two); a
  // partition's weight is applied with a select, so a partial of weight 0
  // never enters the sum
  // (unconditional loads: a partition past np re-reads partition 0 and is
  // masked below; under a branch the compiler would wait after each load)
  f32x4 v0[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    v0[k] = *reinterpret_cast<const f32x4*>(po + (k < p.np ? k : 0) * stride * kDim);
  const float l0 = sub < p.np ? p.part_lse[sub * stride + base] : neg_inf();
  const float l1 = sub + 32 < p.np ? p.part_lse[(sub + 32) * stride + base] : neg_inf();
  float M = fmaxf(l0, l1);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 32));
  const float w0 = l0 == neg_inf() ? 0.f : __expf(l0 - M);
  const float w1 = l1 == neg_inf() ? 0.f : __expf(l1 - M);
  float den = w0 + w1;
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) den += __shfl_xor(den, o, 32);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float w = __shfl(w0, k, 32);
    if (k < p.np && w != 0.f) acc += w * v0[k];
  }
  for (int pi0 = 8; pi0 < p.np; pi0 += 8) {
    f32x4 v[8];
    float w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int pi = pi0 + k;
      w[k] = pi < 32 ? __shfl(w0, pi, 32) : __shfl(w1, pi - 32, 32);
      v[k] = pi < p.np ? *reinterpret_cast<const f32x4*>(po + pi * stride * kDim)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (pi0 + k < p.np && w[k] != 0.f) acc += w[k] * v[k];
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const u32x2 o = {pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(p.out + base * kDim + 4 * sub) = o;
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  dim3 grid((unsigned)((size_t)p.batch * p.max_seq * ((p.H_q + 7) / 8)));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace msa
