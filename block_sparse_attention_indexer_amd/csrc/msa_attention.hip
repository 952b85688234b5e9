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
#include <type_traits>

#include "msa_common.h"
#include "msa_kernels.h"

namespace msa {

template <bool FP8>
__global__ __launch_bounds__(256, 2) void attn_decode_kernel(AttnParams p) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;

  const int ntok_groups = (p.rg.max_seq + p.tpw - 1) / p.tpw;
  const int ntgb = (ntok_groups + W - 1) / W;
  int x = blockIdx.x;
  const int pi = x % p.np;
  x /= p.np;
  const int tgb = x % ntgb;
  x /= ntgb;
  const int h = x % p.H_kv;
  const int b = x / p.H_kv;

  const int r0 = p.rg.offs[b];
  const int n = min(p.rg.offs[b + 1] - r0, p.rg.max_seq);   // keeps rows < rcap
  const int c = p.rg.clen[b];
  const int tok0 = (tgb * W + wave) * p.tpw;
  const int ntok = max(0, min(n - tok0, p.tpw));

  // ---- union of the wave's token selections, ascending, in LDS ----------
  const int nbw = (p.nbmax + 31) >> 5;
  const int cap = p.tpw * p.top_k;
  uint32_t* bm = lds + wave * (p.tpw * nbw + 2 * cap);
  int32_t* uid = reinterpret_cast<int32_t*>(bm + p.tpw * nbw);
  uint32_t* umk = reinterpret_cast<uint32_t*>(uid + cap);
  for (int i = lane; i < p.tpw * nbw; i += 64) bm[i] = 0u;
  __syncthreads();
  for (int tl = 0; tl < ntok; ++tl) {
    const int tok = tok0 + tl;
    const int nbt = min((c + tok) / kBlock + 1, p.nbmax);
    const int32_t* lst = p.d_indices + ((size_t)(r0 + tok) * p.H_kv + h) * p.top_k;
    for (int i = lane; i < p.top_k; i += 64) {
      const int id = lst[i];
      if (id >= 0 && id < nbt) atomicOr(&bm[tl * nbw + (id >> 5)], 1u << (id & 31));
    }
  }
  __syncthreads();
  int nU = 0;
  for (int w0 = 0; w0 < nbw; w0 += 64) {
    const int w = w0 + lane;
    uint32_t u = 0u;
    if (w < nbw)
      for (int tl = 0; tl < ntok; ++tl) u |= bm[tl * nbw + w];
    const int cnt = __popc(u);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int pos = nU + incl - cnt;
    while (u) {
      const int bit = __ffs(u) - 1;
      u &= u - 1u;
      uint32_t mk = 0u;
      for (int tl = 0; tl < ntok; ++tl) mk |= ((bm[tl * nbw + w] >> bit) & 1u) << tl;
      uid[pos] = w * 32 + bit;
      umk[pos] = mk;
      ++pos;
    }
    nU += __shfl(incl, 63);
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
      const int pg = p.rg.table[(size_t)b * p.rg.stride + blk_lane];
      pg_lane = (unsigned)pg < (unsigned)p.k.num_pages ? pg : -1;   // bad ids: block skipped
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
  if (!col_ok) return;
  if (p.np == 1) {
    uint16_t* op = p.out + ((size_t)qrow * p.H_q + hq) * kDim + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4 v = {pack_bf16(O[0][i] * inv, O[1][i] * inv), pack_bf16(O[2][i] * inv, O[3][i] * inv),
                       pack_bf16(O[4][i] * inv, O[5][i] * inv), pack_bf16(O[6][i] * inv, O[7][i] * inv)};
      *reinterpret_cast<u32x4*>(op + 8 * i) = v;
    }
  } else {
    const size_t row = ((size_t)pi * p.rcap + qrow) * p.H_q + hq;
    float* op = p.part_o + row * kDim + 32 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4*>(op + 8 * i) = f32x4{O[0][i] * inv, O[1][i] * inv, O[2][i] * inv, O[3][i] * inv};
      *reinterpret_cast<f32x4*>(op + 8 * i + 4) = f32x4{O[4][i] * inv, O[5][i] * inv, O[6][i] * inv, O[7][i] * inv};
    }
    if (g == 0) p.part_lse[row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : neg_inf();
  }
}

size_t attention_decode_lds_bytes(const AttnParams& p) {
  const int nbw = (p.nbmax + 31) / 32;
  return (size_t)p.ntg * (p.tpw * nbw + 2 * p.tpw * p.top_k) * sizeof(uint32_t);
}

hipError_t launch_attention_decode(const AttnParams& p, bool fp8, hipStream_t s) {
  const int ntok_groups = (p.rg.max_seq + p.tpw - 1) / p.tpw;
  const int ntgb = (ntok_groups + p.ntg - 1) / p.ntg;
  const size_t nwg = (size_t)p.rg.batch * p.H_kv * ntgb * p.np;
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
