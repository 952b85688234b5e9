"""Seeded synthetic inputs for block-sparse paged attention.

This module draws random numbers and lays them out in the paged-cache format.
It holds none of the method's arithmetic: no scoring, no selection, no
softmax.  Both the HIP path and the CPU oracle consume the tensors it builds,
which is the only thing the two sides share.

Layout (all tensors are torch tensors on the requested device):

* ``q``        bf16 ``[R, H_q, 128]``   attention queries, ragged rows
* ``q_idx``    bf16 ``[R, H_kv, 128]``  indexer queries, one per KV head
* ``index_k``  bf16 ``[P, H_ik, 128, 128]`` index-K page pool, or (FP8
  index-K) float8_e4m3fn codes of that shape with ``index_k_scale`` float32
  ``[P, H_ik, 128]``, both views of one buffer of 132 bytes per token
* ``k_cache`` / ``v_cache`` bf16 or float8_e4m3fn ``[P, H_kv, 128, 128]``
* ``input_row_offsets`` int32 ``[B+1]``, ``cache_lengths`` int32 ``[B]``,
  ``kv_lookup_table`` int32 ``[B, lookup_stride]``

Row ``r = input_row_offsets[b] + t`` is new token ``t`` of sequence ``b``.  Its
key/value (and index key) are already stored at logical position
``cache_lengths[b] + t``.  Logical position ``j`` of sequence ``b`` lives in
page ``kv_lookup_table[b, j // 128]`` at slot ``j % 128``.

Poisoning: slots at or past a sequence's length in its last page, pool pages
no sequence uses, and one extra "trap" page that every unused lookup entry
points at are filled with NaN.  An out-of-range read therefore shows up as NaN
in a result rather than as a silently plausible number.

Value recipe: every tensor is drawn from its own ``torch.Generator`` seeded
from the workload seed, as float32 N(0, sigma), then rounded to its storage
type by torch's round-to-nearest-even cast (FP8 values are clamped to the
e4m3 finite range first).  Integer choices (lengths, page permutation, boosted
rows) come from ``numpy.random.Generator(PCG64(seed))``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

BLOCK = 128       # tokens per KV block == tokens per page
HEAD_DIM = 128    # head dim of q, k, v, q_idx, k_idx
FP8_MAX = 448.0   # largest finite e4m3fn magnitude


@dataclass(frozen=True)
class Workload:
    """A named problem: per-sequence lengths, head counts, selection knobs."""

    name: str
    new_lens: tuple          # n_b: new query tokens per sequence
    cache_lens: tuple        # c_b: tokens cached before this step's tokens
    num_kv_heads: int
    group: int               # GQA group size G (H_q = G * H_kv)
    top_k: int
    init_blocks: int
    local_blocks: int
    kv_dtype: str = "bf16"   # "bf16" or "fp8_e4m3"
    ik_dtype: str = "bf16"   # index-K: "bf16" or "fp8_e4m3" (codes + per-token scale)
    kv_sigma: float = 1.0
    num_ik_heads: int = 1    # index-K heads stored in the cache: 1 or H_kv
    boost_frac: float = 0.0  # fraction of index-K rows multiplied by `boost`
    boost: float = 4.0
    pool_pages: Optional[int] = None  # None: exactly the pages in use
    seed: int = 0
    scale: Optional[float] = None     # None: 1/sqrt(128)

    @property
    def batch(self) -> int:
        return len(self.new_lens)

    @property
    def num_q_heads(self) -> int:
        return self.group * self.num_kv_heads

    @property
    def total_rows(self) -> int:
        return int(sum(self.new_lens))

    @property
    def max_seq_length(self) -> int:
        return int(max(self.new_lens))

    @property
    def max_cache_length(self) -> int:
        return int(max(self.cache_lens))

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(HEAD_DIM)

    def seq_lens(self):
        return [int(c) + int(n) for c, n in zip(self.cache_lens, self.new_lens)]

    def pages_per_seq(self):
        return [(L + BLOCK - 1) // BLOCK for L in self.seq_lens()]

    @property
    def lookup_stride(self) -> int:
        return max(self.pages_per_seq())


# ---------------------------------------------------------------------------
# The five benchmark workloads and small variants of the same shapes.
# ---------------------------------------------------------------------------

def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def decode_small(seed: int = 0) -> Workload:
    """Decode, batch 1, 1 KV head x GQA 4, context 2048 (16 blocks) in a
    randomly permuted pool of 32 pages, top-k 4 (init 1, local 1)."""
    return Workload("decode_b1_ctx2048_gqa4_topk4", new_lens=(1,), cache_lens=(2047,),
                    num_kv_heads=1, group=4, top_k=4, init_blocks=1, local_blocks=1,
                    pool_pages=32, seed=seed)


def decode_batch64(seed: int = 0, batch: int = 64, lo: int = 4096, hi: int = 32768) -> Workload:
    """Decode, batch 64, 8 KV heads x GQA 8, context lengths uniform in
    [4096, 32768] (including the new token), top-k 16 (init 1, local 2),
    5% of index-K rows multiplied by 4."""
    L = _rng(seed).integers(lo, hi, size=batch, endpoint=True)
    return Workload(f"decode_b{batch}_ctx{lo // 1024}k-{hi // 1024}k_topk16",
                    new_lens=tuple([1] * batch), cache_lens=tuple(int(x) - 1 for x in L),
                    num_kv_heads=8, group=8, top_k=16, init_blocks=1, local_blocks=2,
                    boost_frac=0.05, seed=seed)


def spec_decode(seed: int = 0, batch: int = 32, lo: int = 8192, hi: int = 65536) -> Workload:
    """Speculative decode: batch 32, 2-8 draft tokens per sequence appended at
    cache lengths uniform in [8192, 65536], 8 KV heads x GQA 8, top-k 32
    (init 1, local 4)."""
    g = _rng(seed)
    n = g.integers(2, 8, size=batch, endpoint=True)
    c = g.integers(lo, hi, size=batch, endpoint=True)
    return Workload(f"specdecode_b{batch}_draft2-8_ctx{lo // 1024}k-{hi // 1024}k_topk32",
                    new_lens=tuple(int(x) for x in n), cache_lens=tuple(int(x) for x in c),
                    num_kv_heads=8, group=8, top_k=32, init_blocks=1, local_blocks=4,
                    seed=seed)


def prefill_ragged(seed: int = 0, new=(1024, 4096, 8192, 16384),
                   cached=(0, 2048, 0, 16384)) -> Workload:
    """Ragged prefill: 4 sequences of {1024, 4096, 8192, 16384} new tokens
    after {0, 2048, 0, 16384} cached ones, 8 KV heads x GQA 8, top-k 64
    (init 1, local 4)."""
    return Workload(f"prefill_{len(new)}seq_{sum(new)}tok_topk64", new_lens=tuple(new),
                    cache_lens=tuple(cached), num_kv_heads=8, group=8, top_k=64,
                    init_blocks=1, local_blocks=4, seed=seed)


def prefill_ragged_dense(seed: int = 0) -> Workload:
    """The ragged prefill's first three sequences alone ({1024, 4096, 8192} new
    tokens after {0, 2048, 0}): every token sees at most 64 blocks, so its
    selection is every visible block -- dense causal attention."""
    return replace(prefill_ragged(seed, new=(1024, 4096, 8192), cached=(0, 2048, 0)),
                   name="prefill_3seq_13312tok_dense_causal")


def prefill_ragged_sparse(seed: int = 0) -> Workload:
    """The ragged prefill's last sequence alone (16384 new tokens after 16384
    cached): 129..256 visible blocks per token, 64 selected."""
    return replace(prefill_ragged(seed, new=(16384,), cached=(16384,)),
                   name="prefill_1seq_16384tok_after_16384_topk64")


def decode_fp8_long(seed: int = 0, batch: int = 16, ctx: int = 131072) -> Workload:
    """Long-context decode with scale-free FP8 e4m3 K/V (N(0, 0.5) clamped to
    the e4m3 range) and BF16 index-K: batch 16, context 131072 (1024 blocks),
    8 KV heads x GQA 8, top-k 64 (init 1, local 4)."""
    return Workload(f"decode_fp8_b{batch}_ctx{ctx // 1024}k_topk64",
                    new_lens=tuple([1] * batch), cache_lens=tuple([ctx - 1] * batch),
                    num_kv_heads=8, group=8, top_k=64, init_blocks=1, local_blocks=4,
                    kv_dtype="fp8_e4m3", kv_sigma=0.5, seed=seed)


def decode_fp8_long_fp8ik(seed: int = 0) -> Workload:
    """The long-context FP8 decode with an FP8 index-K cache as well (e4m3
    codes + one float32 scale per token, 132 bytes per token instead of 256):
    batch 16, context 131072, 8 KV heads x GQA 8, top-k 64 (init 1, local 4)."""
    wl = decode_fp8_long(seed)
    return replace(wl, name="decode_fp8kv_fp8ik_b16_ctx128k_topk64", ik_dtype="fp8_e4m3")


WORKLOADS = {
    "decode_small": decode_small,
    "decode_batch64": decode_batch64,
    "spec_decode": spec_decode,
    "prefill_ragged": prefill_ragged,
    "prefill_ragged_dense": prefill_ragged_dense,
    "prefill_ragged_sparse": prefill_ragged_sparse,
    "decode_fp8_long": decode_fp8_long,
    "decode_fp8_long_fp8ik": decode_fp8_long_fp8ik,
}


# ---------------------------------------------------------------------------
# Tensor construction
# ---------------------------------------------------------------------------

@dataclass
class Inputs:
    """Device tensors of one problem plus the host-side scalars that size it."""

    wl: Workload
    q: torch.Tensor
    q_idx: torch.Tensor
    index_k: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    input_row_offsets: torch.Tensor
    cache_lengths: torch.Tensor
    kv_lookup_table: torch.Tensor
    page_of: list = field(default_factory=list)   # host copy: page ids per sequence
    index_k_scale: Optional[torch.Tensor] = None  # float32 [P, H_ik, 128] for FP8 index-K

    @property
    def device(self):
        return self.q.device


def _gen(device, seed: int, tag: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 7919) & 0x7FFF_FFFF_FFFF)
    return g


def _fill_normal(t: torch.Tensor, gen: torch.Generator, sigma: float, fp8: bool,
                 chunk_elems: int = 1 << 26) -> None:
    """Fill `t` (any shape, contiguous) with N(0, sigma) rounded to its dtype."""
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        x = torch.randn(e - s, generator=gen, device=t.device, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        if fp8:
            x.clamp_(-FP8_MAX, FP8_MAX)
        flat[s:e] = x.to(t.dtype)


def make_inputs(wl: Workload, device="cpu") -> Inputs:
    """Build the tensors of workload `wl` on `device`, deterministically."""
    device = torch.device(device)
    B = wl.batch
    H_kv, H_q, H_ik = wl.num_kv_heads, wl.num_q_heads, wl.num_ik_heads
    if H_ik not in (1, H_kv):
        raise ValueError("index-K heads must be 1 or the KV head count")
    pages = wl.pages_per_seq()
    used = sum(pages)
    pool = wl.pool_pages if wl.pool_pages is not None else used
    if pool < used:
        raise ValueError("pool smaller than the pages in use")
    P = pool + 1          # + one NaN trap page at the end
    trap = pool

    g = _rng(wl.seed + 1)
    perm = g.permutation(pool)
    page_of = []
    table = np.full((B, wl.lookup_stride), trap, dtype=np.int32)
    pos = 0
    for b in range(B):
        ids = perm[pos:pos + pages[b]].astype(np.int32)
        pos += pages[b]
        page_of.append(ids)
        table[b, :pages[b]] = ids

    kv_torch = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float8_e4m3fn
    fp8 = wl.kv_dtype != "bf16"

    R = wl.total_rows
    q = torch.empty((R, H_q, HEAD_DIM), dtype=torch.bfloat16, device=device)
    q_idx = torch.empty((R, H_kv, HEAD_DIM), dtype=torch.bfloat16, device=device)
    index_k = torch.empty((P, H_ik, BLOCK, HEAD_DIM), dtype=torch.bfloat16, device=device)
    k_cache = torch.empty((P, H_kv, BLOCK, HEAD_DIM), dtype=kv_torch, device=device)
    v_cache = torch.empty((P, H_kv, BLOCK, HEAD_DIM), dtype=kv_torch, device=device)

    _fill_normal(q, _gen(device, wl.seed, 1), 1.0, False)
    _fill_normal(q_idx, _gen(device, wl.seed, 2), 1.0, False)
    _fill_normal(index_k, _gen(device, wl.seed, 3), 1.0, False)
    _fill_normal(k_cache, _gen(device, wl.seed, 4), wl.kv_sigma, fp8)
    _fill_normal(v_cache, _gen(device, wl.seed, 5), wl.kv_sigma, fp8)

    # Boost a random fraction of index-K rows (one row = one logical position
    # of one sequence, all index heads) by an exact power-of-two factor.
    if wl.boost_frac > 0.0:
        hits_page, hits_slot = [], []
        for b in range(B):
            L = wl.seq_lens()[b]
            m = np.nonzero(g.random(L) < wl.boost_frac)[0]
            hits_page.append(page_of[b][m // BLOCK])
            hits_slot.append(m % BLOCK)
        hp = torch.from_numpy(np.concatenate(hits_page).astype(np.int64)).to(device)
        hs = torch.from_numpy(np.concatenate(hits_slot).astype(np.int64)).to(device)
        if hp.numel():
            rows = index_k[hp, :, hs, :].float() * wl.boost
            index_k[hp, :, hs, :] = rows.to(torch.bfloat16)

    # FP8 index-K: the same values stored as e4m3 codes with one float32 scale
    # per (page, head, slot), scale = max |value| / 448 over the slot's 128
    # dims (1 for an all-zero slot), code = value / scale rounded to nearest
    # even by torch's cast.  Page layout: each head's 128 x 128 code bytes
    # followed by its 128 scales, i.e. 132 bytes per token.
    index_k_scale = None
    if wl.ik_dtype == "fp8_e4m3":
        head_bytes = BLOCK * HEAD_DIM + BLOCK * 4
        store = torch.empty((P, H_ik, head_bytes), dtype=torch.uint8, device=device)
        codes = store[:, :, :BLOCK * HEAD_DIM].view(torch.float8_e4m3fn).unflatten(2, (BLOCK, HEAD_DIM))
        index_k_scale = store[:, :, BLOCK * HEAD_DIM:].view(torch.float32)
        for p0 in range(0, P, 1024):
            vals = index_k[p0:p0 + 1024].float()
            amax = vals.abs().amax(dim=-1)
            sc = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
            codes[p0:p0 + 1024] = (vals / sc.unsqueeze(-1)).to(torch.float8_e4m3fn)
            index_k_scale[p0:p0 + 1024] = sc
        index_k = codes
    elif wl.ik_dtype != "bf16":
        raise ValueError(f"unsupported index-K dtype {wl.ik_dtype}")

    # Poison every slot that no sequence may read.
    nan = float("nan")
    unused = np.setdiff1d(np.arange(pool), np.concatenate(page_of) if page_of else [])
    poison_pages = torch.from_numpy(np.append(unused, trap).astype(np.int64)).to(device)
    for t in (index_k, k_cache, v_cache):
        t[poison_pages] = nan
    if index_k_scale is not None:
        index_k_scale[poison_pages] = nan
    for b in range(B):
        L = wl.seq_lens()[b]
        if L % BLOCK:
            last = int(page_of[b][-1])
            for t in (index_k, k_cache, v_cache):
                t[last, :, L % BLOCK:, :] = nan
            if index_k_scale is not None:
                index_k_scale[last, :, L % BLOCK:] = nan

    offs = np.zeros(B + 1, dtype=np.int32)
    offs[1:] = np.cumsum(wl.new_lens)
    return Inputs(
        wl=wl, q=q, q_idx=q_idx, index_k=index_k, k_cache=k_cache, v_cache=v_cache,
        input_row_offsets=torch.from_numpy(offs).to(device),
        cache_lengths=torch.tensor(wl.cache_lens, dtype=torch.int32, device=device),
        kv_lookup_table=torch.from_numpy(table).to(device),
        page_of=page_of, index_k_scale=index_k_scale,
    )


def shrink(wl: Workload, **kw) -> Workload:
    """A copy of `wl` with some fields replaced (for small test variants)."""
    return replace(wl, **kw)
