"""CPU oracle for block-sparse paged attention: the indexer's block selection
and the sparse attention pass over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The product path (the HIP library and
its Python binding) never does, and this module imports nothing from it.

It is written from the method's statement on these pages:

* "ferrox_core::block_sparse" (docs.rs), section "Four rules", and its
  function summaries ``block_sparse_select`` / ``positions_of_blocks``: the
  selection semantics (block score is the max over a block's positions, the
  raw dot product with no softmax scale, one selection per KV head read by
  the whole GQA group, forced first/newest blocks) and the attention as an
  ordinary masked pass over the selected positions.
* "ferrox_core::block_sparse", section "The block size is an ABI, not a
  tuning knob": blocks are 128 tokens and coincide with KV pages.
* "DeepSeekSparseAttentionConfig" (TensorRT-LLM API reference), field
  ``indexer_k_dtype``: an FP8 index-K cache holds one e4m3 code per element
  and one float32 scale per 128 elements (per token at head dim 128).
* "msa" (MAX Mojo module docs, graph-op bindings for the MiniMax-M3 MSA
  kernels), intro and routes paragraphs: BF16 index-K, BF16 or scale-free FP8
  e4m3 main KV, FP32 accumulation, a token's position is its sequence's cache
  length plus its index among the new tokens, block id ``blk`` starts at
  logical position ``128 * blk``, causality is per token.

Readings where the pages are silent (each is listed with its reason in the
design notes): top_k counts the forced blocks; "newest" is relative to the
token's own position; a block's score only ranges over positions the token
may see (j <= p); equal scores go to the lower block id; padding is -1.

Precision: dot products of BF16 / e4m3 values are formed from the exact
decoded values and accumulated in float32, as the pages state for the
kernels; both selection and attention use float32 accumulation.

Every function follows one definition step by step, with no blocking or
fusion beyond what that step states.  Inputs are numpy arrays of the raw
storage bits (uint16 for BF16, uint8 for e4m3) so that decoding is also the
oracle's own.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

BLOCK = 128


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float32 values.  A BF16 number is the upper half
    of an IEEE binary32 word, so widening is exact: shift left by 16."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _e4m3fn_table() -> np.ndarray:
    """Value of each of the 256 OCP FP8 E4M3 ('fn' variant) codes.

    Format: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 encodes subnormals m/8 * 2^-6.  There is no infinity; the codes
    S.1111.111 are NaN, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    tab = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            tab[code] = np.nan
        elif e == 0:
            tab[code] = s * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            tab[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


E4M3FN_TABLE = _e4m3fn_table()


def decode_e4m3fn(bits: np.ndarray) -> np.ndarray:
    """e4m3fn bit patterns -> float32 values (exact: every e4m3 value is a
    float32 value)."""
    return E4M3FN_TABLE[np.asarray(bits).astype(np.intp)].astype(np.float32)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "fp8_e4m3":
        return decode_e4m3fn(bits)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Selection ("ferrox_core::block_sparse", section "Four rules")
# ---------------------------------------------------------------------------

def visible_blocks(p: int) -> int:
    """Blocks a token at position p may see: 0 .. p // 128."""
    return p // BLOCK + 1


def forced_blocks(nb: int, init_blocks: int, local_blocks: int) -> list:
    """Fourth rule: the first `init_blocks` and the newest `local_blocks` of
    the token's nb visible blocks are always selected, before any scoring."""
    first = set(range(0, min(init_blocks, nb)))
    newest = set(range(max(0, nb - local_blocks), nb))
    return sorted(first | newest)


def index_k_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """FP8 index-K ("DeepSeekSparseAttentionConfig" page, indexer_k_dtype):
    one e4m3 code per element and one float32 scale per token; the value is
    code * scale.  codes [n, D] raw e4m3 bits, scales [n] float32; the
    products are exact in float64."""
    return decode_e4m3fn(codes).astype(np.float64) * scales.astype(np.float64)[:, None]


def position_scores(q_idx: np.ndarray, ik_rows: np.ndarray) -> np.ndarray:
    """Second rule: the raw dot product q_idx . k_idx of every position, with
    no softmax scale.  q_idx [D] and ik_rows [n, D] are float32 values of
    BF16 numbers; products are exact in float32, sums accumulate in float32."""
    return ik_rows.astype(np.float32) @ q_idx.astype(np.float32)


def block_scores(pos_scores: np.ndarray, p: int, blocks) -> dict:
    """First rule: a block's score is the MAX of its positions' scores (not
    the mean or the sum), over the positions j <= p the token may see."""
    out = {}
    for blk in blocks:
        lo = blk * BLOCK
        hi = min(lo + BLOCK, p + 1)
        out[blk] = float(np.max(pos_scores[lo:hi]))
    return out


@dataclass
class Selection:
    blocks: list          # ascending selected block ids
    decisive: bool        # k-th and (k+1)-th candidate scores clearly apart
    kth_score: float      # score of the last freely chosen block (nan if none)
    scores: dict          # candidate block -> score


def block_sparse_select(nb: int, scores: dict, top_k: int, init_blocks: int,
                        local_blocks: int, rel_gap: float = 1e-3) -> Selection:
    """The blocks one KV head may read for one query position, ascending.

    F = forced blocks.  If nb <= top_k every visible block is read.  Otherwise
    the top_k - |F| highest-scoring blocks outside F join F; equal scores go
    to the lower block id.  `decisive` is False when the last chosen score
    and the first rejected one differ by at most `rel_gap` relative, the only
    case in which a different but equally valid selection exists under
    rounding.
    """
    F = forced_blocks(nb, init_blocks, local_blocks)
    if nb <= top_k:
        return Selection(list(range(nb)), True, float("nan"), {})
    free = top_k - len(F)
    cands = [blk for blk in range(nb) if blk not in set(F)]
    ranked = sorted(cands, key=lambda blk: (-scores[blk], blk))
    chosen = ranked[:free]
    decisive = True
    kth = float("nan")
    if free > 0:
        kth = scores[ranked[free - 1]]
        if free < len(ranked):
            nxt = scores[ranked[free]]
            decisive = (kth - nxt) > rel_gap * max(abs(kth), abs(nxt))
    return Selection(sorted(set(F) | set(chosen)), decisive, kth,
                     {blk: scores[blk] for blk in cands})


def positions_of_blocks(blocks, p: int) -> np.ndarray:
    """The positions a block selection covers, ascending and causally
    clipped to j <= p."""
    pos = []
    for blk in sorted(blocks):
        for j in range(blk * BLOCK, blk * BLOCK + BLOCK):
            if j <= p:
                pos.append(j)
    return np.asarray(pos, dtype=np.int64)


# ---------------------------------------------------------------------------
# Attention: an ordinary masked softmax pass over the selected positions
# ---------------------------------------------------------------------------

def masked_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """softmax(scale * q K^T) V for query rows q [G, D] over key/value rows
    K, V [n, D], float32 accumulation.  Returns (out [G, D], lse [G]) where
    lse is the natural log of the softmax denominator including the max
    shift, i.e. log sum_j exp(scale * q.k_j).  With no positions the output
    is 0 and lse is -inf (an empty selection has no softmax)."""
    G, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((G, D), np.float32), np.full(G, -np.inf, np.float32)
    z = (q.astype(np.float32) @ K.astype(np.float32).T) * np.float32(scale)
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    l = w.sum(axis=1, keepdims=True)
    out = (w @ V.astype(np.float32)) / l
    lse = (m + np.log(l))[:, 0]
    return out.astype(np.float32), lse.astype(np.float32)


def splitk_combine(part_o: np.ndarray, part_lse: np.ndarray) -> np.ndarray:
    """Merge per-partition results of one softmax: each partition pi holds its
    own normalised output o_pi and log-denominator lse_pi.  The merged output
    is sum_pi exp(lse_pi - LSE) o_pi with LSE = log sum_pi exp(lse_pi);
    partitions with lse = -inf (no positions) carry no weight.  Shapes:
    part_o [np, ..., D], part_lse [np, ...]."""
    lse = part_lse.astype(np.float64)
    M = np.max(lse, axis=0)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(lse), np.exp(lse - safe), 0.0)
    den = w.sum(axis=0)
    num = (w[..., None] * part_o.astype(np.float64)).sum(axis=0)
    out = np.where(den[..., None] > 0, num / np.where(den > 0, den, 1.0)[..., None], 0.0)
    return out.astype(np.float32)


# ---------------------------------------------------------------------------
# Paged cache access and the full ragged problem
# ---------------------------------------------------------------------------

@dataclass
class Problem:
    """Host numpy copies of a problem's inputs (raw storage bits)."""

    q: np.ndarray                 # uint16 [R, H_q, D]
    q_idx: np.ndarray             # uint16 [R, H_kv, D]
    index_k: np.ndarray           # uint16 [P, H_ik, 128, D]
    k_cache: np.ndarray           # uint16 or uint8 [P, H_kv, 128, D]
    v_cache: np.ndarray
    kv_dtype: str                 # "bf16" or "fp8_e4m3"
    input_row_offsets: np.ndarray  # int [B+1]
    cache_lengths: np.ndarray     # int [B]
    kv_lookup_table: np.ndarray   # int [B, stride]
    top_k: int
    init_blocks: int
    local_blocks: int
    scale: float
    ik_dtype: str = "bf16"        # index-K: "bf16", or "fp8_e4m3" codes + scales
    index_k_scale: np.ndarray = None   # float32 [P, H_ik, 128] for FP8 index-K

    @property
    def num_kv_heads(self):
        return self.k_cache.shape[1]

    @property
    def group(self):
        return self.q.shape[1] // self.num_kv_heads


def row_position(pb: Problem, r: int):
    """Sequence b, position p and visible block count nb of ragged row r: the
    token's position is its sequence's cache length plus its index among the
    sequence's new tokens."""
    offs = pb.input_row_offsets
    b = int(np.searchsorted(offs, r, side="right") - 1)
    t = r - int(offs[b])
    p = int(pb.cache_lengths[b]) + t
    return b, p, visible_blocks(p)


def gather_rows(pool: np.ndarray, lookup_row: np.ndarray, head: int, n: int) -> np.ndarray:
    """Logical positions 0..n-1 of one head of one sequence: position j sits
    in page lookup_row[j // 128] at slot j % 128."""
    nblk = (n + BLOCK - 1) // BLOCK
    pages = np.asarray(lookup_row[:nblk], dtype=np.intp)
    tiles = pool[pages, head]                     # [nblk, 128, D]
    return tiles.reshape(nblk * BLOCK, -1)[:n]


def select_row(pb: Problem, r: int) -> list:
    """Selections of ragged row r for every KV head.  Third rule: each KV
    head h has its own index query q_idx[r, h] and its own selection, with
    no reduction across heads; it scores against index-K head h mod H_ik
    (one index-K head shared by all, or one per KV head)."""
    b, p, nb = row_position(pb, r)
    H_kv = pb.q_idx.shape[1]
    H_ik = pb.index_k.shape[1]
    if nb <= pb.top_k:
        return [block_sparse_select(nb, {}, pb.top_k, pb.init_blocks, pb.local_blocks)
                for _ in range(H_kv)]
    F = set(forced_blocks(nb, pb.init_blocks, pb.local_blocks))
    cands = [blk for blk in range(nb) if blk not in F]
    sels = [None] * H_kv
    for hk in range(H_ik):
        codes = gather_rows(pb.index_k, pb.kv_lookup_table[b], hk, p + 1)
        if pb.ik_dtype == "fp8_e4m3":
            sc = gather_rows(pb.index_k_scale[..., None], pb.kv_lookup_table[b], hk, p + 1)[:, 0]
            rows = index_k_values(codes, sc)
        else:
            rows = decode_bf16(codes)
        for h in range(hk, H_kv, H_ik):
            if pb.ik_dtype == "fp8_e4m3":
                # values are no longer BF16-exact: score in float64
                s = rows @ decode_bf16(pb.q_idx[r, h]).astype(np.float64)
            else:
                s = position_scores(decode_bf16(pb.q_idx[r, h]), rows)
            sels[h] = block_sparse_select(nb, block_scores(s, p, cands), pb.top_k,
                                          pb.init_blocks, pb.local_blocks)
    return sels


def indexer(pb: Problem, rows=None):
    """Top-k block ids per (row, KV head), ascending, padded with -1.
    Returns (d_indices [len(rows), H_kv, top_k] int32, selections)."""
    R = pb.q_idx.shape[0]
    rows = list(range(R) if rows is None else rows)
    H_kv = pb.q_idx.shape[1]
    out = np.full((len(rows), H_kv, pb.top_k), -1, dtype=np.int32)
    sels = []
    for i, r in enumerate(rows):
        per_head = select_row(pb, r)
        for h, sel in enumerate(per_head):
            out[i, h, :len(sel.blocks)] = sel.blocks
        sels.append(per_head)
    return out, sels


def attention_row(pb: Problem, r: int, h: int, blocks) -> tuple:
    """Attention of the GQA group of KV head h (query heads h*G .. h*G+G-1)
    for row r over the positions covered by `blocks` (ids < 0 ignored),
    causally clipped at the row's position."""
    b, p, nb = row_position(pb, r)
    blocks = [int(x) for x in blocks if x >= 0]
    pos = positions_of_blocks(blocks, p)
    G = pb.group
    qv = decode_bf16(pb.q[r, h * G:(h + 1) * G])
    if pos.size == 0:
        return masked_attention(qv, np.zeros((0, qv.shape[1])), np.zeros((0, qv.shape[1])), pb.scale)
    pages = np.asarray(pb.kv_lookup_table[b], dtype=np.intp)[pos // BLOCK]
    K = decode(pb.k_cache[pages, h, pos % BLOCK], pb.kv_dtype)
    V = decode(pb.v_cache[pages, h, pos % BLOCK], pb.kv_dtype)
    return masked_attention(qv, K, V, pb.scale)


def attention(pb: Problem, d_indices: np.ndarray, rows=None) -> np.ndarray:
    """Output [len(rows), H_q, D] (float32) for the given block ids.
    d_indices is indexed like the rows argument: d_indices[i] belongs to
    rows[i]."""
    R = pb.q.shape[0]
    rows = list(range(R) if rows is None else rows)
    H_kv = pb.num_kv_heads
    G = pb.group
    D = pb.q.shape[2]
    out = np.zeros((len(rows), H_kv * G, D), dtype=np.float32)
    for i, r in enumerate(rows):
        for h in range(H_kv):
            o, _ = attention_row(pb, r, h, d_indices[i, h])
            out[i, h * G:(h + 1) * G] = o
    return out


def problem_from_inputs(inp, rows_needed=None) -> Problem:
    """Host copies of an `Inputs` object's tensors as raw storage bits."""
    import torch

    def bits(t):
        if t.dtype == torch.bfloat16:
            return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.detach().contiguous().view(torch.uint8).cpu().numpy()

    wl = inp.wl
    return Problem(
        q=bits(inp.q), q_idx=bits(inp.q_idx), index_k=bits(inp.index_k),
        k_cache=bits(inp.k_cache), v_cache=bits(inp.v_cache), kv_dtype=wl.kv_dtype,
        ik_dtype=wl.ik_dtype,
        index_k_scale=(None if inp.index_k_scale is None
                       else inp.index_k_scale.detach().contiguous().cpu().numpy()),
        input_row_offsets=inp.input_row_offsets.cpu().numpy().astype(np.int64),
        cache_lengths=inp.cache_lengths.cpu().numpy().astype(np.int64),
        kv_lookup_table=inp.kv_lookup_table.cpu().numpy().astype(np.int64),
        top_k=wl.top_k, init_blocks=wl.init_blocks, local_blocks=wl.local_blocks,
        scale=wl.softmax_scale)


def problem_for_sequences(inp, seqs) -> tuple:
    """Host copy of only the sequences `seqs` of an `Inputs` object: their
    pages are copied and renumbered, rows are renumbered in order.  Returns
    (problem, original_rows) where original_rows[i] is the ragged row of the
    full problem that row i of the sub-problem stands for.  This only moves
    data; values and positions are unchanged."""
    import torch

    def bits(t):
        if t.dtype == torch.bfloat16:
            return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return t.detach().contiguous().view(torch.uint8).cpu().numpy()

    wl = inp.wl
    offs = inp.input_row_offsets.cpu().numpy().astype(np.int64)
    table = inp.kv_lookup_table.cpu().numpy().astype(np.int64)
    clen = inp.cache_lengths.cpu().numpy().astype(np.int64)
    seqs = [int(b) for b in seqs]
    pages = np.unique(np.concatenate([table[b] for b in seqs]))
    remap = {int(pg): i for i, pg in enumerate(pages)}
    sub_table = np.vectorize(lambda x: remap[int(x)])(table[seqs]).astype(np.int64)
    idx = torch.from_numpy(pages).to(inp.index_k.device)
    rows = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in seqs])
    ridx = torch.from_numpy(rows).to(inp.q.device)
    sub_offs = np.zeros(len(seqs) + 1, dtype=np.int64)
    sub_offs[1:] = np.cumsum([offs[b + 1] - offs[b] for b in seqs])
    pb = Problem(
        q=bits(inp.q[ridx]), q_idx=bits(inp.q_idx[ridx]), index_k=bits(inp.index_k[idx]),
        k_cache=bits(inp.k_cache[idx]), v_cache=bits(inp.v_cache[idx]), kv_dtype=wl.kv_dtype,
        ik_dtype=wl.ik_dtype,
        index_k_scale=(None if inp.index_k_scale is None
                       else inp.index_k_scale[idx].detach().contiguous().cpu().numpy()),
        input_row_offsets=sub_offs, cache_lengths=clen[seqs], kv_lookup_table=sub_table,
        top_k=wl.top_k, init_blocks=wl.init_blocks, local_blocks=wl.local_blocks,
        scale=wl.softmax_scale)
    return pb, rows
