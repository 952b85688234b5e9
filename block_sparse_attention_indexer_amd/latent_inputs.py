"""Seeded synthetic inputs for latent sparse attention over two paged leaves.

Like ``inputs``, this module only draws random numbers and lays them out; it
holds none of the method's arithmetic.  Both the HIP path and the CPU oracle
consume the tensors it builds.

Layout (torch tensors on the requested device):

* ``q``           bf16 ``[R, H, 128]``           queries, ragged rows
* ``swa_pool``    bf16 / float8_e4m3fn ``[P_s, H_lat, 128, 128]``  window leaf
* ``comp_pool``   bf16 / float8_e4m3fn ``[P_c, H_lat, 128, 128]``  compressed leaf
* ``swa_lookup_table`` / ``comp_lookup_table`` int32 ``[B, stride]``
* ``swa_cache_lengths`` / ``comp_cache_lengths`` int32 ``[B]``
* ``comp_indices`` int32 ``[R, H_lat, top_c]``   per-row entry lists
* ``attn_sink``   float32 ``[H]``
* ``input_row_offsets`` int32 ``[B + 1]``

Row r = offsets[b] + t is new token t of sequence b at window-leaf position
swa_cache_lengths[b] + t.  Window-leaf position j of sequence b is slot
j % 128 of page swa_lookup_table[b, j // 128]; compressed entry e is slot
e % 128 of page comp_lookup_table[b, e // 128].

Only the window leaf's pages that some new token's window reaches are
allocated; every other lookup entry points at a trap page of NaN, and window
positions no token of the step may see (before the earliest window start,
after the last new token) are NaN too.  Compressed entries at or past
comp_cache_lengths[b] and unused pool pages are NaN.  A read of anything the
operation must not read therefore shows up as NaN in a result.

Entry lists: for each (row, latent head) min(top_c, comp_len) distinct
entries drawn uniformly from [0, comp_len) and sorted, padded with -1; a
workload may then overwrite a fraction of the slots with out-of-range values
(comp_len + k, or a negative number other than -1) or with a copy of another
slot's entry.

Value recipe: latent vectors N(0, sigma) (FP8: clamped to the e4m3 range),
queries N(0, 1), sinks N(sink_mean, 1) in float32; every tensor from its own
``torch.Generator``; integer choices from ``numpy.random.Generator(PCG64)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch

from .inputs import _fill_normal, _gen, _rng

PAGE = 128
HEAD_DIM = 128


@dataclass(frozen=True)
class LatentWorkload:
    name: str
    new_lens: tuple            # new query tokens per sequence
    swa_cache_lens: tuple      # window-leaf positions cached before the new tokens
    comp_lens: tuple           # entries in the compressed leaf per sequence
    num_heads: int             # query heads H
    num_latent_heads: int = 1  # H_lat (query head g reads latent head g // (H / H_lat))
    window: int = 128
    top_c: int = 512           # list slots per (row, latent head)
    swa_dtype: str = "bf16"
    comp_dtype: str = "bf16"
    sigma: float = 1.0
    sink_mean: float = 0.0
    sink_neg_inf_frac: float = 0.0   # fraction of heads whose sink is -inf (no sink)
    bad_frac: float = 0.0      # fraction of list slots overwritten with out-of-range values
    dup_frac: float = 0.0      # fraction of list slots overwritten with another slot's entry
    seed: int = 0
    scale: Optional[float] = None    # None: 1/sqrt(128)

    @property
    def batch(self) -> int:
        return len(self.new_lens)

    @property
    def total_rows(self) -> int:
        return int(sum(self.new_lens))

    @property
    def max_seq_length(self) -> int:
        return int(max(self.new_lens))

    @property
    def group(self) -> int:
        return self.num_heads // self.num_latent_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(HEAD_DIM)

    @property
    def max_swa_cache_length(self) -> int:
        return int(max(self.swa_cache_lens))

    @property
    def max_comp_length(self) -> int:
        return int(max(self.comp_lens))

    def window_span(self, b: int):
        """[lo, hi] window-leaf positions sequence b's new tokens may see."""
        c, n = int(self.swa_cache_lens[b]), int(self.new_lens[b])
        lo = max(0, c - self.window + 1) if self.window > 0 else c + n
        return lo, c + n - 1


def latent_decode(seed: int = 0, batch: int = 64, heads: int = 64, window: int = 128,
                  top_c: int = 2048, lo: int = 32768, hi: int = 131072) -> LatentWorkload:
    """Decode over a shared latent: batch 64, 64 query heads on one latent
    head of dim 128, window 128, 2048 listed compressed entries per token,
    contexts uniform in [32k, 128k] with a compressed leaf of context / 4
    entries."""
    g = _rng(seed)
    ctx = g.integers(lo, hi, size=batch, endpoint=True)
    return LatentWorkload(
        f"latent_decode_b{batch}_h{heads}_win{window}_topc{top_c}_ctx{lo // 1024}k-{hi // 1024}k",
        new_lens=tuple([1] * batch), swa_cache_lens=tuple(int(x) - 1 for x in ctx),
        comp_lens=tuple(int(x) // 4 for x in ctx), num_heads=heads, window=window,
        top_c=top_c, sink_mean=2.0, seed=seed)


def latent_decode_fp8(seed: int = 0, **kw) -> LatentWorkload:
    """latent_decode with both leaves stored as FP8 e4m3 (half the bytes per
    latent vector)."""
    w = latent_decode(seed, **kw)
    return replace(w, name=w.name.replace("latent_decode", "latent_decode_fp8"),
                   swa_dtype="fp8_e4m3", comp_dtype="fp8_e4m3")


LATENT_WORKLOADS = {"latent_decode": latent_decode, "latent_decode_fp8": latent_decode_fp8}


@dataclass
class LatentInputs:
    wl: LatentWorkload
    q: torch.Tensor
    input_row_offsets: torch.Tensor
    comp_indices: torch.Tensor
    attn_sink: torch.Tensor
    swa_pool: torch.Tensor
    swa_lookup_table: torch.Tensor
    swa_cache_lengths: torch.Tensor
    comp_pool: torch.Tensor
    comp_lookup_table: torch.Tensor
    comp_cache_lengths: torch.Tensor


def _torch_dtype(name: str):
    if name == "bf16":
        return torch.bfloat16
    if name == "fp8_e4m3":
        return torch.float8_e4m3fn
    raise ValueError(f"unsupported leaf dtype {name}")


def make_latent_inputs(wl: LatentWorkload, device="cpu") -> LatentInputs:
    device = torch.device(device)
    B, H, H_lat = wl.batch, wl.num_heads, wl.num_latent_heads
    if H % H_lat:
        raise ValueError("query heads must be a multiple of latent heads")
    g = _rng(wl.seed + 11)
    nan = float("nan")

    # window leaf: the logical pages some new token's window reaches
    # the table covers the host bounds: max cached positions + max new tokens
    swa_stride = max(1, (wl.max_swa_cache_length + wl.max_seq_length + PAGE - 1) // PAGE)
    spans = [wl.window_span(b) for b in range(B)]
    swa_need = [list(range(lo // PAGE, hi // PAGE + 1)) if hi >= lo else [] for lo, hi in spans]
    n_swa = sum(len(x) for x in swa_need)
    perm = g.permutation(n_swa + 1)            # + one unused page
    swa_trap = n_swa + 1
    swa_table = np.full((B, swa_stride), swa_trap, np.int32)
    k = 0
    for b in range(B):
        for lp in swa_need[b]:
            swa_table[b, lp] = perm[k]
            k += 1

    # compressed leaf: every page of each sequence's entries
    comp_pages = [(n + PAGE - 1) // PAGE for n in wl.comp_lens]
    comp_stride = max(1, max(comp_pages))
    n_comp = sum(comp_pages)
    perm_c = g.permutation(n_comp + 1)
    comp_trap = n_comp + 1
    comp_table = np.full((B, comp_stride), comp_trap, np.int32)
    k = 0
    for b in range(B):
        comp_table[b, :comp_pages[b]] = perm_c[k:k + comp_pages[b]]
        k += comp_pages[b]

    sd, cd = _torch_dtype(wl.swa_dtype), _torch_dtype(wl.comp_dtype)
    R = wl.total_rows
    q = torch.empty((R, H, HEAD_DIM), dtype=torch.bfloat16, device=device)
    swa_pool = torch.empty((swa_trap + 1, H_lat, PAGE, HEAD_DIM), dtype=sd, device=device)
    comp_pool = torch.empty((comp_trap + 1, H_lat, PAGE, HEAD_DIM), dtype=cd, device=device)
    _fill_normal(q, _gen(device, wl.seed, 21), 1.0, False)
    _fill_normal(swa_pool, _gen(device, wl.seed, 22), wl.sigma, sd != torch.bfloat16)
    _fill_normal(comp_pool, _gen(device, wl.seed, 23), wl.sigma, cd != torch.bfloat16)
    sink = torch.empty((H,), dtype=torch.float32, device=device)
    sink.normal_(generator=_gen(device, wl.seed, 24)).add_(wl.sink_mean)
    if wl.sink_neg_inf_frac > 0:
        m = torch.from_numpy(g.random(H) < wl.sink_neg_inf_frac).to(device)
        sink[m] = -float("inf")

    # poison: trap and unused pages, window positions outside every window,
    # compressed entries past the leaf's length
    swa_used = swa_table[swa_table != swa_trap]
    swa_unused = np.setdiff1d(np.arange(swa_trap + 1), swa_used)
    swa_pool[torch.from_numpy(swa_unused.astype(np.int64)).to(device)] = nan
    for b in range(B):
        lo, hi = spans[b]
        if hi < lo:
            continue
        first, last = int(swa_table[b, lo // PAGE]), int(swa_table[b, hi // PAGE])
        if lo % PAGE:
            swa_pool[first, :, :lo % PAGE] = nan
        if (hi + 1) % PAGE:
            swa_pool[last, :, (hi + 1) % PAGE:] = nan
    comp_unused = np.setdiff1d(np.arange(comp_trap + 1), comp_table[comp_table != comp_trap])
    comp_pool[torch.from_numpy(comp_unused.astype(np.int64)).to(device)] = nan
    for b in range(B):
        n = wl.comp_lens[b]
        if n % PAGE:
            comp_pool[int(comp_table[b, comp_pages[b] - 1]), :, n % PAGE:] = nan

    # entry lists
    offs = np.zeros(B + 1, np.int32)
    offs[1:] = np.cumsum(wl.new_lens)
    lists = np.full((R, H_lat, wl.top_c), -1, np.int32)
    for b in range(B):
        n = wl.comp_lens[b]
        k = min(wl.top_c, n)
        for r in range(offs[b], offs[b + 1]):
            for hl in range(H_lat):
                if k:
                    lists[r, hl, :k] = np.sort(g.choice(n, size=k, replace=False))
                if wl.bad_frac > 0:
                    m = g.random(wl.top_c) < wl.bad_frac
                    bad = np.where(g.random(wl.top_c) < 0.5, n + g.integers(0, 1 << 20, wl.top_c),
                                   -g.integers(2, 1 << 20, wl.top_c))
                    lists[r, hl, m] = bad[m]
                if wl.dup_frac > 0 and k > 1:
                    m = g.random(wl.top_c) < wl.dup_frac
                    lists[r, hl, m] = lists[r, hl, g.integers(0, k, wl.top_c)][m]
    return LatentInputs(
        wl=wl, q=q, input_row_offsets=torch.from_numpy(offs).to(device),
        comp_indices=torch.from_numpy(lists).to(device), attn_sink=sink,
        swa_pool=swa_pool, swa_lookup_table=torch.from_numpy(swa_table).to(device),
        swa_cache_lengths=torch.tensor(wl.swa_cache_lens, dtype=torch.int32, device=device),
        comp_pool=comp_pool, comp_lookup_table=torch.from_numpy(comp_table).to(device),
        comp_cache_lengths=torch.tensor(wl.comp_lens, dtype=torch.int32, device=device))


def shrink(wl: LatentWorkload, **kw) -> LatentWorkload:
    return replace(wl, **kw)
