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
// Block-max scorer, streaming index-K pages from HBM.
//
// Workgroup = 4 waves; each wave scores kBpw consecutive blocks of one
// sequence against up to 16 * NCT columns.  A column is one (token, KV head)
// pair whose KV head reads index-K head hk (one shared head, or one per KV
// head).  Per block the wave loads the 128 x 128 BF16 tile straight into
// MFMA A-operand registers (16 B per lane per load, 64 B contiguous per row
// per instruction), computes S^T = K Q^T with the columns on the MFMA N side,
// then reduces rows (positions) with in-lane max plus two cross-lane steps.
// ---------------------------------------------------------------------------
constexpr int kIdxWaves = 4;
constexpr int kBpw = 2;

template <int NCT>
__global__ __launch_bounds__(256) void indexer_score_kernel(IndexerParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int b = blockIdx.y;
  const int hk = blockIdx.z % p.H_ik;
  const int cg = blockIdx.z / p.H_ik;
  const int r0 = p.rg.offs[b];
  // Rows past the host bound never exist; the clamp keeps every address in
  // the buffers sized from the bounds.
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  const int hpi = p.H_kv / p.H_ik;          // KV heads per index-K head
  const int col0 = cg * 16 * NCT;           // first column of this group
  if (n <= 0 || col0 >= n * hpi) return;
  const int c = p.rg.clen[b];
  // Tokens of this column group and the blocks any of them may need scored.
  const int t_last = min(n, (col0 + 16 * NCT + hpi - 1) / hpi) - 1;
  const int nb_last = (c + t_last) / kBlock + 1;
  if (nb_last <= p.top_k) return;           // every row selects all its blocks
  const int blk_hi = min(nb_last - p.local, p.nbmax);

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
    for (int s = 0; s < 4; ++s) qf[ct][s] = ok ? ld16(qp + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
  }

  const int blk0 = (blockIdx.x * kIdxWaves + wave) * kBpw;
  const uint16_t* pool = static_cast<const uint16_t*>(p.ik.data);
  for (int bi = 0; bi < kBpw; ++bi) {
    const int blk = blk0 + bi;
    if (blk < p.init || blk >= blk_hi) continue;
    const int page = uniform(p.rg.table[(size_t)b * p.rg.stride + blk]);
    if ((unsigned)page >= (unsigned)p.ik.num_pages) continue;
    const uint16_t* base = pool + (size_t)page * p.ik.page_stride + (size_t)hk * p.ik.head_stride;
    u32x4 kf[8][4];
#pragma unroll
    for (int pt = 0; pt < 8; ++pt)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[pt][s] = ld16(base + (size_t)(16 * pt + l16) * p.ik.token_stride + 32 * s + 8 * g);

    const bool clip = blk * kBlock + kBlock - 1 > c;   // some position past a token
    float mx[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) mx[ct] = neg_inf();
#pragma unroll
    for (int pt = 0; pt < 8; ++pt) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_bf16(kf[pt][s], qf[ct][s], acc);
        if (clip) {
          const int pos0 = blk * kBlock + 16 * pt + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (pos0 + i > plim[ct]) acc[i] = neg_inf();
        }
        mx[ct] = fmaxf(mx[ct], fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])));
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float m = colgroup_max(mx[ct]);
      if (g == 0 && plim[ct] >= 0) p.scores[(size_t)orow[ct] * p.score_stride + blk] = m;
    }
  }
}

hipError_t launch_indexer_decode(const IndexerParams& p, hipStream_t s) {
  const int hpi = p.H_kv / p.H_ik;
  const int cols = p.rg.max_seq * hpi;
  const int nct = cols <= 16 ? 1 : cols <= 32 ? 2 : 4;
  const int ncg = (cols + 16 * nct - 1) / (16 * nct);
  dim3 grid((p.nbmax + kIdxWaves * kBpw - 1) / (kIdxWaves * kBpw), p.rg.batch, p.H_ik * ncg);
  if (nct == 1) hipLaunchKernelGGL(indexer_score_kernel<1>, grid, dim3(256), 0, s, p);
  else if (nct == 2) hipLaunchKernelGGL(indexer_score_kernel<2>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(indexer_score_kernel<4>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k selection, one wave per (row, KV head).
//
// Candidates are the blocks [init, nb - local) (everything not forced).  The
// (top_k - |forced|)-th largest score is found by building its
// order-preserving 32-bit key one bit at a time from the top (each step
// counts keys >= the trial value with a wave ballot).  Blocks strictly above
// the threshold are taken, then the lowest-id blocks equal to it until the
// count is reached.  Output is emitted in ascending id order by ballot
// prefix counts, so no sort is needed: forced-first, chosen candidates,
// forced-newest are already ascending ranges.
// ---------------------------------------------------------------------------
template <int KPL>
__global__ __launch_bounds__(256) void topk_kernel(IndexerParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.y;
  const int idx = blockIdx.x * 4 + wave;
  const int t = idx / p.H_kv;
  const int h = idx % p.H_kv;
  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);
  if (t >= n) return;
  const int pos = p.rg.clen[b] + t;
  const int nb = min(pos / kBlock + 1, p.nbmax);
  const int r = r0 + t;
  int32_t* out = p.d_indices + ((size_t)r * p.H_kv + h) * p.top_k;
  if (nb <= p.top_k) {
    for (int i = lane; i < p.top_k; i += 64) out[i] = i < nb ? i : -1;
    return;
  }
  const int ncand = nb - p.init - p.local;
  const int kfree = p.top_k - p.init - p.local;
  for (int i = lane; i < p.init; i += 64) out[i] = i;
  for (int i = lane; i < p.local; i += 64) out[p.init + kfree + i] = nb - p.local + i;
  if (kfree == 0) return;

  const float* sc = p.scores + ((size_t)r * p.H_kv + h) * p.score_stride + p.init;
  const int nslot = (ncand + 63) / 64;
  uint32_t key[KPL];
#pragma unroll
  for (int s = 0; s < KPL; ++s) {
    const int i = s * 64 + lane;
    key[s] = (s < nslot && i < ncand) ? score_key(sc[i]) : 0u;
  }
  uint32_t thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int s = 0; s < KPL; ++s)
      if (s < nslot) cnt += __popcll(ballot(key[s] >= cand));
    if (cnt >= kfree) thr = cand;
  }
  int above = 0;
#pragma unroll
  for (int s = 0; s < KPL; ++s)
    if (s < nslot) above += __popcll(ballot(key[s] > thr));
  const int need_eq = kfree - above;
  int run = 0, run_eq = 0;
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

hipError_t launch_topk(const IndexerParams& p, hipStream_t s) {
  const int ncand_max = p.nbmax - p.init - p.local;
  dim3 grid((p.rg.max_seq * p.H_kv + 3) / 4, p.rg.batch);
  if (ncand_max <= 256) hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, s, p);
  else if (ncand_max <= 1024) hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, s, p);
  else if (ncand_max <= 4096) hipLaunchKernelGGL(topk_kernel<64>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(topk_kernel<128>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace msa
