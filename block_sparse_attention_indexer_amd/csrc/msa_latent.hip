// Latent sparse attention ("Struct_latent_sparse_attention_ragged_paged" page
// of the MAX Mojo docs): every cached entry is one latent vector that is both
// key and value, read from a sliding-window leaf (a range of positions) and a
// compressed leaf (a per-query list of entries), with a per-head sink logit
// in the softmax denominator.
//
// One workgroup of four waves owns (row, latent head, group of up to 64
// query heads, split-K partition).  The row's entries are numbered window
// positions first, then list slots; a partition takes a contiguous run of
// 32-entry tiles of that numbering.  The workgroup first resolves each of
// its entries to the address of its latent vector (in LDS).  The waves then
// take the partition's tiles in turn (wave w: tiles w, w + 4, ...), each
// streaming its own tiles through its own ring of LDS stages with
// global->LDS DMA, a whole ring of tiles in flight (four BF16 tiles, eight
// FP8 ones), so no wave waits for another inside the loop.  A wave holds
// all of the group's query heads as MFMA
// columns (up to four 16-column tiles): S^T = X . Q^T over a tile (X the
// 32 latent rows), an online softmax over the rows, then O^T += X^T . P^T
// with X^T read from the same LDS tile by transposing reads -- keys and
// values are one tile, fetched once, and every operand read feeds one MFMA
// per column tile.  At the end the four waves' softmax states are merged
// through LDS.
//
// The tile is stored row-major, one row per entry: BF16 leaves 256 bytes,
// 16-byte column c of row pos at c ^ f(pos), f(pos) = ((pos & 7) << 1) |
// ((pos >> 3) & 1), which keeps the transposing value reads free of LDS
// bank conflicts (the 16-byte key reads measure 2-way conflicted with it);
// FP8 e4m3 leaves 128 bytes, column c at c ^ fp8_vswz(pos), the codes being
// widened to BF16 (exactly) as the MFMA operands are read.
//
// Entries a partition does not attend (a list value outside [0, leaf
// length), the padding after the row's last entry) are still fetched -- from
// the row's own query vector -- so that every wave issues the same number of
// DMAs per tile and the vmcnt waits stay exact; their scores are masked to
// -inf, so their probability is exactly 0.  For BF16 leaves those stand-in
// bytes are finite; for FP8 leaves they could decode as NaN, so the wave
// zeroes such rows of its tile before reading it.
//
// The sink joins one wave's running softmax in the row's partition 0 as one more
// logit with no value (max = sink, sum = 1 before any entry), so neither the
// merge of the four waves nor the split-K merge needs anything extra.  With
// several partitions, the group's last partition merges their results in
// the same launch (msa_splitk.h).
#include <algorithm>

#include "msa_common.h"
#include "msa_kernels.h"
#include "msa_latent.h"
#include "msa_splitk.h"
#include "msa_lds.h"

namespace msa {

constexpr int kLatWaves = 4;
constexpr int kLatRingBytes = 4 * kLatentTile * 256;           // per wave: 32 KiB
constexpr float kLatLazy = 8.f;   // log2 headroom before the running max moves

struct LatentLds {
  // per-wave tile rings; after the loop, each wave's merged-state area
  char ring[kLatWaves][kLatRingBytes];
  // first byte of each entry's latent vector, or null: not attended; after
  // the loop, the waves' per-column max and sum
  const char* src[kLatentMaxSlots];
  // the group's query vectors, [head][128] BF16 (read into registers once)
  char q[64 * 256];
};

__device__ __forceinline__ int lat_swz(int pos) { return ((pos & 7) << 1) | ((pos >> 3) & 1); }

// entries a lookup-table row of `stride` pages addresses
__device__ __forceinline__ int tab_cap(int stride) {
  return stride > (0x7FFFFFFF >> 7) ? 0x7FFFFFFF : stride << 7;
}

// o *= s in place in the accumulation registers.  The accumulators live in
// AGPRs (they are MFMA results and operands); written as plain C++, the
// multiply makes the compiler copy every accumulator to VGPRs at the top of
// each tile, whether or not the (rare) rescale runs.  The last MFMA that
// wrote o is a whole score phase earlier; the trailing s_nop covers the
// AGPR-write -> MFMA-read wait states of the next accumulation.
__device__ __forceinline__ void scale_acc(f32x4& o, float s) {
  float x0 = o[0], x1 = o[1], x2 = o[2], x3 = o[3];
  float t0, t1, t2, t3;
  __asm__ volatile(
      "v_accvgpr_read_b32 %4, %0\n\t"
      "v_accvgpr_read_b32 %5, %1\n\t"
      "v_accvgpr_read_b32 %6, %2\n\t"
      "v_accvgpr_read_b32 %7, %3\n\t"
      "v_mul_f32 %4, %8, %4\n\t"
      "v_mul_f32 %5, %8, %5\n\t"
      "v_mul_f32 %6, %8, %6\n\t"
      "v_mul_f32 %7, %8, %7\n\t"
      "v_accvgpr_write_b32 %0, %4\n\t"
      "v_accvgpr_write_b32 %1, %5\n\t"
      "v_accvgpr_write_b32 %2, %6\n\t"
      "v_accvgpr_write_b32 %3, %7\n\t"
      "s_nop 4"
      : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "=&v"(t0), "=&v"(t1), "=&v"(t2), "=&v"(t3)
      : "v"(s));
  o = f32x4{x0, x1, x2, x3};
}

// Wait until at most n tiles of kDma DMAs each are still in flight (the
// count must be an immediate, hence the cases).
template <int kDma>
__device__ __forceinline__ void wait_tiles(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDma)); break;
    case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kDma)); break;
    case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kDma)); break;
    case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * kDma)); break;
    case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm(5 * kDma)); break;
    case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm(6 * kDma)); break;
    case 7: __builtin_amdgcn_s_waitcnt(vmcnt_imm(7 * kDma)); break;
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(8 * kDma)); break;
  }
}

template <int NCT, bool FP8>
__global__ __launch_bounds__(64 * kLatWaves, 1) void latent_attn_kernel(LatentParams p) {
  constexpr int RB = FP8 ? 128 : 256;                 // bytes per entry row
  constexpr int ESZ = FP8 ? 1 : 2;                    // bytes per element
  constexpr int kTileBytes = kLatentTile * RB;
  constexpr int kDma = kTileBytes / 1024;             // DMAs per tile: 8 (BF16), 4 (FP8)
  constexpr int kLanesPerRow = RB / 16;
  constexpr int kRowsPerDma = 64 / kLanesPerRow;
  constexpr int kStages = kLatRingBytes / kTileBytes;  // tiles in flight per wave: 4, 8
  static_assert(kStages <= 8 && kStages * kDma <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(16))) LatentLds L;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform((int)(tid >> 6));
  const int l16 = lane & 15, g = lane >> 4;

  // group = (row slot, latent head, column group); its np partitions share
  // an XCD (msa_splitk.h)
  int pi, id;
  splitk_slot(blockIdx.x, p.np, &pi, &id);
  if (id >= p.batch * p.max_seq * p.H_lat * p.ncg) return;   // padding of the last XCD round
  const int grp = id;
  // this partition among all of the row's (with leaves of two storage
  // types, the window leaf's partitions come from one launch, the list's
  // from a second one)
  const int gpi = p.pi_base + pi;
  const int cg = id % p.ncg;
  id /= p.ncg;
  const int hl = id % p.H_lat;
  id /= p.H_lat;
  const int b = id / p.max_seq, t = id % p.max_seq;
  // the sequence's lengths are read together with its row offsets (one
  // memory round trip, not two), and so are the sinks
  bool col_ok[NCT];
  float sink_v[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    col_ok[ct] = cg * 64 + 16 * ct + l16 < p.G;
    sink_v[ct] = p.sink[hl * p.G + (col_ok[ct] ? cg * 64 + 16 * ct + l16 : 0)];
  }
  const int r0 = p.offs[b], r1 = p.offs[b + 1];
  // lengths past what a sequence's lookup table addresses (bad device data)
  // are clipped to it, so no table read leaves the table's row (the host
  // checked that the window leaf's table covers max_seq new positions more)
  const int swa_len = p.window > 0 ? min(p.swa.clen[b], tab_cap(p.swa.stride) - p.max_seq) : 0;
  const int comp_len = p.top_c > 0 ? min(p.comp.clen[b], tab_cap(p.comp.stride)) : 0;
  if (threadIdx.x == 0 && pi == 0 && hl == 0 && cg == 0 && t == 0 &&
      ((p.window > 0 && swa_len < p.swa.clen[b]) || (p.top_c > 0 && comp_len < p.comp.clen[b]) ||
       r1 - r0 > p.max_seq))
    report_error(p.err, kErrLength);
  if (t >= min(r1 - r0, p.max_seq)) return;
  const int r = r0 + t;

  // ---- queries: the group's heads as NCT 16-column MFMA tiles -------------------
  // They reach LDS by DMA right ahead of the first tiles and registers after
  // that; loaded into registers here, they would sit on the path of the list
  // and page-table loads (loads return in order).
  const uint16_t* qrow = p.q + (size_t)r * p.H * kDim;
  u32x4 qf[NCT][4];

  // ---- this partition's entries ---------------------------------------------
  const int pos = swa_len + t;
  const int n_swa = p.window > 0 ? max(0, min(p.window, pos + 1)) : 0;
  const int lo = pos - n_swa + 1;
  const int nent = n_swa + p.top_c;
  const int ntiles_row = (nent + kLatentTile - 1) / kLatentTile;
  const int e0 = (int)((int64_t)ntiles_row * pi / p.np);
  const int e1 = (int)((int64_t)ntiles_row * (pi + 1) / p.np);
  const int ntile = e1 - e0;
  const int s0 = e0 * kLatentTile;
  const int s1 = min(nent, e1 * kLatentTile);
  const int32_t* lst = p.lists + ((size_t)r * p.H_lat + hl) * p.top_c;
  // Resolve every entry of the partition to the address of its latent
  // vector.  Every load is issued unconditionally (slots that need none read
  // a harmless int instead) and the loaded values are merged with masks, not
  // branches, so a thread's loads are all in flight together: the partition
  // pays two memory round trips, not two per entry.
  {
    constexpr int kPer = kLatentMaxSlots / (64 * kLatWaves);
    const int32_t* swa_tab = p.swa.table + (size_t)b * p.swa.stride;
    const int32_t* comp_tab = p.comp.table + (size_t)b * p.comp.stride;
    const char* swa_base = static_cast<const char*>(p.swa.pool.data);
    const char* comp_base = static_cast<const char*>(p.comp.pool.data);
    if (swa_base) swa_base += (size_t)hl * p.swa.pool.head_stride * ESZ;
    if (comp_base) comp_base += (size_t)hl * p.comp.pool.head_stride * ESZ;
    int ent[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = s0 + tid + 64 * kLatWaves * k;
      const bool listed = s < s1 && s >= n_swa;
      const int v = *(listed ? lst + (s - n_swa) : p.offs);
      const int m = -(int)listed;
      ent[k] = (v & m) | ((s < n_swa ? lo + s : -1) & ~m);
    }
    int pg[kPer];
    bool att[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = s0 + tid + 64 * kLatWaves * k;
      const int e = ent[k];
      const bool win = s < s1 && s < n_swa;
      const bool cmp = s < s1 && s >= n_swa && e >= 0 && e < comp_len;
      const int v = *(win ? swa_tab + (e >> 7) : cmp ? comp_tab + (e >> 7) : p.offs);
      const int m = -(int)(win || cmp);
      pg[k] = (v & m) | ~m;
      att[k] = win || cmp;
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = s0 + tid + 64 * kLatWaves * k;
      const int i = tid + 64 * kLatWaves * k;
      if (i < ntile * kLatentTile) {
        const char* a = nullptr;
        // a page id outside the pool (bad table data) is skipped like an
        // invalid entry, so no read leaves the pool
        const int npages = s < n_swa ? p.swa.pool.num_pages : p.comp.pool.num_pages;
        if (att[k] && (unsigned)pg[k] >= (unsigned)npages) report_error(p.err, kErrPage);
        if ((unsigned)pg[k] < (unsigned)npages)
          a = s < n_swa ? swa_base + (size_t)pg[k] * p.swa.pool.page_stride * ESZ +
                              (size_t)(ent[k] & 127) * p.swa.pool.token_stride * ESZ
                        : comp_base + (size_t)pg[k] * p.comp.pool.page_stride * ESZ +
                              (size_t)(ent[k] & 127) * p.comp.pool.token_stride * ESZ;
        L.src[i] = a;
      }
    }
  }

  f32x4 O[8][NCT];
  float m_run[NCT], l_run[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) O[dt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[ct] = neg_inf();
    l_run[ct] = 0.f;
    if (gpi == 0 && wave == 0 && col_ok[ct]) {
      const float sk = sink_v[ct];
      if (sk != neg_inf()) {
        m_run[ct] = sk * kLog2e;
        l_run[ct] = g == 0 ? 1.f : 0.f;   // counted once per column
      }
    }
  }
  const float sc = p.scale_log2;
  // every load so far has landed before the first DMA is issued, so that the
  // compiler's own waits for them never have to drain the tile ring
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // ---- this wave's tiles ----------------------------------------------------------
  // DMA i of a tile fetches rows kRowsPerDma * i onwards; lane L lands in row
  // kRowsPerDma * i + L / kLanesPerRow at physical column L % kLanesPerRow,
  // which holds logical column (L % kLanesPerRow) ^ swizzle(row).  Rows that
  // are not attended fetch 16 bytes of the row's first query vector instead.
  auto swz = [](int pos) { return FP8 ? fp8_vswz(pos) : lat_swz(pos); };
  char* ring = L.ring[wave];
  const int my_n = ntile > wave ? (ntile - wave + kLatWaves - 1) / kLatWaves : 0;
  const char* dummy = reinterpret_cast<const char*>(qrow) + 16 * l16;
  const int drow = lane / kLanesPerRow, dcol = lane % kLanesPerRow;
  uint32_t colb[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) colb[i] = (uint32_t)((dcol ^ swz(kRowsPerDma * i + drow)) << 4);
  auto issue = [&](int j) {
    const int tb = (wave + kLatWaves * j) * kLatentTile;
    char* stage = ring + (j % kStages) * kTileBytes;
    const char* a[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) a[i] = L.src[tb + kRowsPerDma * i + drow];
#pragma unroll
    for (int i = 0; i < kDma; ++i) dma16(a[i] ? a[i] + colb[i] : dummy, stage + kRowsPerDma * i * RB);
  };

  // lane-constant LDS offsets.
  // BF16 K A-operand: row 16pt + l16, logical column 4s + g.
  // FP8 K A-operands: row 16pt + l16, logical column g + 4h holds the 16
  //   bytes of k-steps 2h and 2h + 1.
  // BF16 X^T A-operand (transposing read h, dim tile dt): source lane (l16,
  //   g) reads row 16h + 4g + l16 / 4 at dims 16dt + 4(l16 % 4), so output
  //   lane (m, g) receives dim 16dt + m of rows 16h + 4g + k -- the P^T
  //   B-operand layout.
  // FP8 X^T A-operand (one 8-bit transposing read, dim tile dt): source lane
  //   l16 reads the row of position k = l16 / 2, 16(k / 4) + 4g + k % 4, at
  //   dims 16dt + 8(l16 % 2); within a 16-lane group output lane i, element
  //   k is byte i % 8 of source lane i / 8 + 2k, so lane (m, g) receives dim
  //   16dt + m of the same eight rows as the BF16 reads.
  const int kq = FP8 ? l16 * RB : l16 * RB + ((g ^ lat_swz(l16)) << 4);
  int vq;
  if constexpr (FP8) {
    const int k = l16 >> 1;
    const int vr8 = 16 * (k >> 2) + 4 * g + (k & 3);
    vq = vr8 * RB + (fp8_vswz(vr8) << 4) + 8 * (l16 & 1);
  } else {
    const int vrow = 4 * g + (l16 >> 2);
    vq = vrow * RB + ((((l16 & 3) >> 1) ^ lat_swz(vrow)) << 4) + 8 * (l16 & 1);
  }

  // the queries: wave w < NCT fetches heads 16w .. 16w + 15 of the group
  // (four per DMA; a head past the group fetches head 0's vector instead)
  if (wave < NCT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hq = 16 * wave + 4 * i + (lane >> 4);
      const int head = cg * 64 + hq < p.G ? hl * p.G + cg * 64 + hq : hl * p.G;
      dma16(reinterpret_cast<const char*>(qrow + (size_t)head * kDim) + 16 * l16,
            L.q + (16 * wave + 4 * i) * 256);
    }
  }
#pragma unroll
  for (int j = 0; j < kStages; ++j)
    if (j < my_n) issue(j);
  // the query DMAs are older than the tiles': they have landed once at most
  // the tiles' remain; then every wave's are visible after the barrier
  wait_tiles<kDma>(min(my_n, kStages));
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // contraction dims of k-step s for lane group g: BF16 32s + 8g + j;
      // FP8 (a lane's 16 key bytes cover two k-steps) 16g + 64(s/2) + 8(s%2) + j
      const int d0 = FP8 ? 16 * g + 64 * (s >> 1) + 8 * (s & 1) : 32 * s + 8 * g;
      const u32x4 v = *reinterpret_cast<const u32x4*>(L.q + (16 * ct + l16) * 256 + 2 * d0);
      qf[ct][s] = col_ok[ct] ? v : u32x4{0u, 0u, 0u, 0u};
    }

  for (int j = 0; j < my_n; ++j) {
    // this wave's DMAs of tile j are done once at most those of the younger
    // tiles in flight remain (the wave reads only what it fetched itself)
    wait_tiles<kDma>(min(my_n - 1 - j, kStages - 1));

    char* tile = ring + (j % kStages) * kTileBytes;
    const int tb = (wave + kLatWaves * j) * kLatentTile;
    const uint32_t live = (uint32_t)ballot(lane < kLatentTile && L.src[tb + (lane & 31)] != nullptr);
    if constexpr (FP8) {
      // rows that are not attended hold stand-in bytes: zero them (this
      // wave's own DMAs of the tile have landed; its LDS operations run in
      // order, so the reads below see the zeros)
      if (live != 0xFFFFFFFFu) {
#pragma unroll
        for (int k = 0; k < kTileBytes / 16 / 64; ++k) {
          const int idx = lane + 64 * k;
          if (!((live >> (idx / kLanesPerRow)) & 1u))
            *reinterpret_cast<u32x4*>(tile + idx * 16) = u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
    // The key operands are requested together (one LDS latency per tile);
    // the transposed value reads are issued right behind the score MFMAs, so
    // they land while the scores and the softmax run.  (LDS results return
    // in order and the wait counter saturates at 15, so requesting the
    // values first would make the first MFMA wait for them.)
    u32x4 ka[2][4];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 16 * pt + l16;
          const u32x4 w = *reinterpret_cast<const u32x4*>(tile + kq + 16 * pt * RB +
                                                          (((g + 4 * h) ^ fp8_vswz(row)) << 4));
          ka[pt][2 * h] = fp8x8_to_bf16x8(u32x2{w.x, w.y});
          ka[pt][2 * h + 1] = fp8x8_to_bf16x8(u32x2{w.z, w.w});
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          ka[pt][s] = *reinterpret_cast<const u32x4*>(tile + 16 * pt * RB + (kq ^ (s << 6)));
      }
    }
    // this lane's rows of the tile are 16pt + 4g + i: bit 4pt + i of m8
    const uint32_t lg = live >> (4 * g);
    const uint32_t m8 = (lg & 0xFu) | ((lg >> 12) & 0xF0u);
    const bool full = live == 0xFFFFFFFFu;
    __builtin_amdgcn_sched_barrier(0);
    f32x4 S[2][NCT];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          S[pt][ct] = mfma_bf16(ka[pt][s], qf[ct][s], s == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : S[pt][ct]);
    __builtin_amdgcn_sched_barrier(0);
    u32x2 va[8][2];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if constexpr (FP8) {
        va[dt][0] = lds_tr_b8(tile + (vq ^ (dt << 4)));
      } else {
        const char* base = tile + (vq ^ (dt << 5));
        va[dt][0] = lds_tr_b16(base);
        va[dt][1] = lds_tr_b16(base + 16 * RB);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    if (!full) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((m8 >> (4 * pt + i)) & 1u))
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) S[pt][ct][i] = neg_inf();
    }
    bool any_move = false;
    float alpha[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float hmax = fmaxf(fmaxf(fmaxf(S[0][ct][0], S[0][ct][1]), fmaxf(S[0][ct][2], S[0][ct][3])),
                         fmaxf(fmaxf(S[1][ct][0], S[1][ct][1]), fmaxf(S[1][ct][2], S[1][ct][3])));
      hmax = colgroup_max(hmax) * sc;
      // lazy rescaling: the reference max only moves when a score would
      // exceed it by more than 2^kLatLazy
      const bool move = col_ok[ct] && hmax > m_run[ct] + kLatLazy;
      const float m_new = move ? hmax : m_run[ct];
      const float m_use = m_new == neg_inf() ? 0.f : m_new;
      const float off = col_ok[ct] ? m_use : __builtin_inff();
      alpha[ct] = move ? fast_exp2(m_run[ct] - m_use) : 1.f;
      any_move |= move;
      float lsum = 0.f;
#pragma unroll
      for (int pt = 0; pt < 2; ++pt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e2 = fast_exp2(__builtin_fmaf(S[pt][ct][i], sc, -off));
          S[pt][ct][i] = e2;
          lsum += e2;
        }
      l_run[ct] = l_run[ct] * alpha[ct] + lsum;
      m_run[ct] = m_new;
    }
    // O is still zero on the wave's first tile; later moves are rare (the
    // lazy threshold)
    if (j > 0 && __builtin_amdgcn_ballot_w64(any_move)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) scale_acc(O[dt][ct], alpha[ct]);
    }
    u32x4 bp[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      bp[ct] = u32x4{pack_bf16(S[0][ct][0], S[0][ct][1]), pack_bf16(S[0][ct][2], S[0][ct][3]),
                     pack_bf16(S[1][ct][0], S[1][ct][1]), pack_bf16(S[1][ct][2], S[1][ct][3])};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x4 a = FP8 ? fp8x8_to_bf16x8(va[dt][0]) : u32x4{va[dt][0].x, va[dt][0].y, va[dt][1].x, va[dt][1].y};
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) O[dt][ct] = mfma_bf16(a, bp[ct], O[dt][ct]);
    }
    // the stage of tile j is free once this wave's reads of it have
    // returned (the MFMAs above consumed them)
    if (j + kStages < my_n) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      issue(j + kStages);
    }
  }

  // ---- merge the four waves' states ------------------------------------------
  // Wave w stores its column max and sum (src area) and its unnormalised O
  // (its ring, [ct][dt][lane] f32x4); wave ct then merges column tile ct:
  // M = max_w m_w, O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.
  float l_tot[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) l_tot[ct] = colgroup_sum(l_run[ct]);
  __syncthreads();   // every wave is done with its ring and the entry list
  float* stat = reinterpret_cast<float*>(L.src);                  // [w][ct][2][16]
  f32x4* ow = reinterpret_cast<f32x4*>(L.ring[wave]);
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) ow[(ct * 8 + dt) * 64 + lane] = O[dt][ct];
    if (g == 0) {
      stat[((wave * NCT + ct) * 2 + 0) * 16 + l16] = m_run[ct];
      stat[((wave * NCT + ct) * 2 + 1) * 16 + l16] = l_tot[ct];
    }
  }
  __syncthreads();
  // waves 0 .. NCT - 1 each merge the four waves' states of one column tile
  const int ct = min(wave, NCT - 1);
  if (wave < NCT && col_ok[ct]) {
    float mw[kLatWaves], M = neg_inf();
#pragma unroll
    for (int w = 0; w < kLatWaves; ++w) {
      mw[w] = stat[((w * NCT + ct) * 2 + 0) * 16 + l16];
      M = fmaxf(M, mw[w]);
    }
    float lsum = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kLatWaves; ++w) {
      const float sw = (mw[w] == neg_inf()) ? 0.f : fast_exp2(mw[w] - M);
      lsum += sw * stat[((w * NCT + ct) * 2 + 1) * 16 + l16];
      const f32x4* src = reinterpret_cast<const f32x4*>(L.ring[w]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] += sw * src[(ct * 8 + dt) * 64 + lane];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;

    // ---- store: O^T tile dt, C row 4g + i is dim 16dt + 4g + i --------------------
    const size_t hrow = (size_t)r * p.H + hl * p.G + cg * 64 + 16 * ct + l16;
    if (p.np_total == 1) {
      uint16_t* op = p.out + hrow * kDim + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<u32x2*>(op + 16 * dt) =
            u32x2{pack_bf16(o[dt][0] * inv, o[dt][1] * inv), pack_bf16(o[dt][2] * inv, o[dt][3] * inv)};
    } else {
      const size_t prow = (size_t)gpi * p.rcap * p.H + hrow;
      float* op = p.part_o + prow * kDim + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(op + 16 * dt) = o[dt] * inv;
      if (g == 0) p.part_lse[prow] = lsum > 0.f ? (M + __log2f(lsum)) * kLn2 : neg_inf();
    }
  }
  if (p.np_total == 1) return;
  // split-K: the group's last partition merges the partials of its (up to)
  // 64 query heads, 4 threads per head
  uint64_t* flags = p.ready + (size_t)grp * p.np_total;
  if (!splitk_arrive(flags, gpi, p.np_total, p.epoch)) return;
  const int nc = min(64, p.G - cg * 64);
  // (the wave-merge statistics are dead past the arrival's barrier)
  splitk_merge<8>(flags, p.epoch, reinterpret_cast<int*>(stat), p.part_o, p.part_lse, p.out, p.H,
                  p.rcap, p.np_total, nc, [&](int) { return r; },
                  [&](int c) { return hl * p.G + cg * 64 + c; }, tid);
}

template <bool FP8>
static void launch_latent_t(const LatentParams& p, dim3 grid, dim3 block, hipStream_t s) {
  const int cols = std::min(64, p.G);   // heads of the widest column group
  if (cols <= 16) hipLaunchKernelGGL((latent_attn_kernel<1, FP8>), grid, block, 0, s, p);
  else if (cols <= 32) hipLaunchKernelGGL((latent_attn_kernel<2, FP8>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((latent_attn_kernel<4, FP8>), grid, block, 0, s, p);
}

hipError_t launch_latent(const LatentParams& p, hipStream_t s) {
  const size_t nwg = splitk_workgroups((size_t)p.batch * p.max_seq * p.H_lat * p.ncg, p.np);
  const dim3 grid((unsigned)nwg), block(64 * kLatWaves);
  if (p.fp8) launch_latent_t<true>(p, grid, block, s);
  else launch_latent_t<false>(p, grid, block, s);
  return hipGetLastError();
}

}  // namespace msa
