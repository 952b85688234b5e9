"""CPU oracle for latent sparse attention over two paged leaves.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module.  The product path (the HIP library and
its Python binding) never does, and this module imports nothing from it.

Written from the "Struct_latent_sparse_attention_ragged_paged" page of the
MAX Mojo docs (the struct summary and the argument list of ``execute``):
attention in which one latent vector per cached entry serves as both key and
value, read from two paged leaves -- a sliding-window leaf addressed by a
range of positions and a compressed leaf addressed by an explicit list of
entries per query -- with a per-head attention sink that enters the softmax
denominator.  The ragged rows (``input_row_offsets``), the per-leaf cache
lengths and page lookup tables and the softmax ``scale`` are that page's
arguments; ``window`` is its window parameter.

Readings where the page is silent (each is listed with its reason in the
design notes):

* head dim 128 and 128 entries per page, as on the MSA pages; the latent
  cache has one head per latent head (usually one, shared by every query
  head); query head g reads latent head g // (H / H_lat);
* token t of sequence b sits at position p = swa_cache_lengths[b] + t, and
  the window leaf supplies positions max(0, p - window + 1) .. p (window 0:
  none);
* the compressed leaf supplies, for row r and latent head hl, every listed
  entry e = comp_indices[r][hl][k] with 0 <= e < comp_cache_lengths[b], once
  per occurrence in the list; other values (-1 padding, out of range) are
  skipped; there is no causal clip on compressed entries;
* the sink is a logit in the units of the scaled scores with no value:
  out = sum_j exp(z_j) v_j / (sum_j exp(z_j) + exp(sink)), z_j = scale q.k_j;
  a sink of -inf removes it;
* both leaves are BF16 or scale-free FP8 e4m3, decoded exactly.

Precision: the page fixes none, so everything is float64 from the exactly
decoded storage values.  Each function follows one step of the definition
with no blocking or fusion.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle.msa_oracle import decode

PAGE = 128
HEAD_DIM = 128


@dataclass
class LatentProblem:
    """Host copies of one latent problem (raw storage bits for the data)."""

    q: np.ndarray                 # uint16 bf16 bits [R, H, D]
    offsets: np.ndarray           # int [B + 1]
    swa_cache_lengths: np.ndarray  # int [B]
    comp_cache_lengths: np.ndarray  # int [B]
    swa_pool: np.ndarray          # bits [P_s, H_lat, 128, D]
    swa_table: np.ndarray         # int [B, S_s]
    comp_pool: np.ndarray         # bits [P_c, H_lat, 128, D]
    comp_table: np.ndarray        # int [B, S_c]
    comp_indices: np.ndarray      # int [R, H_lat, top_c]
    attn_sink: np.ndarray         # float32 [H]
    window: int
    scale: float
    swa_dtype: str = "bf16"
    comp_dtype: str = "bf16"

    @property
    def num_heads(self) -> int:
        return self.q.shape[1]

    @property
    def num_latent_heads(self) -> int:
        return self.swa_pool.shape[1]


def row_position(pb: LatentProblem, r: int):
    """(sequence b, new-token index t, position p) of ragged row r."""
    b = int(np.searchsorted(pb.offsets, r, side="right") - 1)
    t = r - int(pb.offsets[b])
    return b, t, int(pb.swa_cache_lengths[b]) + t


def window_positions(p: int, window: int) -> np.ndarray:
    """Positions the sliding-window leaf supplies to a token at p: the last
    `window` positions up to and including p."""
    return np.arange(max(0, p - window + 1), p + 1) if window > 0 else np.arange(0)


def listed_entries(pb: LatentProblem, r: int, hl: int, b: int) -> np.ndarray:
    """Compressed-leaf entries of row r, latent head hl: every listed value in
    [0, comp_cache_lengths[b]), in list order, each occurrence kept."""
    lst = pb.comp_indices[r, hl].astype(np.int64)
    return lst[(lst >= 0) & (lst < int(pb.comp_cache_lengths[b]))]


def leaf_rows(pool: np.ndarray, table_row: np.ndarray, head: int, idx: np.ndarray,
              dtype: str) -> np.ndarray:
    """Latent vectors of logical entries idx of one sequence in a paged leaf:
    entry i is slot i % 128 of page table_row[i // 128].  float64 [n, D]."""
    if idx.size == 0:
        return np.zeros((0, pool.shape[-1]), np.float64)
    pages = table_row[idx // PAGE]
    return decode(pool[pages, head, idx % PAGE, :], dtype).astype(np.float64)


def sink_softmax_attention(q: np.ndarray, kv: np.ndarray, sink: np.ndarray, scale: float):
    """Attention of queries q [G, D] over entries kv [n, D] that are both key
    and value, with one sink logit per query in the denominator:
    out[g] = sum_j exp(z_gj) kv_j / (sum_j exp(z_gj) + exp(sink_g)),
    z = scale * q kv^T.  Computed with the common max subtracted."""
    G, D = q.shape
    z = scale * (q @ kv.T)                                   # [G, n]
    zmax = z.max(axis=1) if kv.shape[0] else np.full(G, -np.inf)
    m = np.maximum(zmax, sink)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(z - m[:, None])
    den = w.sum(axis=1) + np.exp(sink - m)
    num = w @ kv
    return np.where(den[:, None] > 0, num / np.where(den > 0, den, 1.0)[:, None], 0.0)


def row_entries(pb: LatentProblem, r: int, hl: int) -> np.ndarray:
    """Every latent vector row r's latent head hl attends: the window leaf's
    positions, then the compressed leaf's listed entries.  float64 [n, D]."""
    b, _, p = row_position(pb, r)
    swa = leaf_rows(pb.swa_pool, pb.swa_table[b], hl, window_positions(p, pb.window), pb.swa_dtype)
    comp = leaf_rows(pb.comp_pool, pb.comp_table[b], hl, listed_entries(pb, r, hl, b), pb.comp_dtype)
    return np.concatenate([swa, comp], axis=0)


def latent_attention(pb: LatentProblem, rows=None) -> np.ndarray:
    """Output [len(rows), H, D] (float64): for each row and latent head, the
    sink softmax attention of that head's query heads over row_entries."""
    rows = range(pb.q.shape[0]) if rows is None else rows
    rows = list(rows)
    H, H_lat = pb.num_heads, pb.num_latent_heads
    G = H // H_lat
    out = np.zeros((len(rows), H, pb.q.shape[2]), np.float64)
    for i, r in enumerate(rows):
        for hl in range(H_lat):
            kv = row_entries(pb, r, hl)
            q = decode(pb.q[r, hl * G:(hl + 1) * G], "bf16").astype(np.float64)
            sink = pb.attn_sink[hl * G:(hl + 1) * G].astype(np.float64)
            out[i, hl * G:(hl + 1) * G] = sink_softmax_attention(q, kv, sink, float(pb.scale))
    return out


# ---------------------------------------------------------------------------
# Host copies of device inputs
# ---------------------------------------------------------------------------

def _bits(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(f"unexpected storage type {t.dtype}")


def problem_for_sequences(inp, seqs, rows=None) -> tuple:
    """A LatentProblem holding every row of the given sequences but only the
    pages that `rows` (original ragged row numbers; None: all rows of those
    sequences) read -- their window pages and listed compressed pages,
    renumbered densely, every other lookup entry pointing at a page of NaN --
    and `orig`, the original row number of each of its rows.  Only the rows
    named in `rows` may be evaluated on it.  Page renumbering leaves results
    unchanged (they do not depend on which physical page holds a logical
    page)."""
    import torch
    seqs = sorted(int(b) for b in seqs)
    offs = inp.input_row_offsets.cpu().numpy().astype(np.int64)
    swa_cl = inp.swa_cache_lengths.cpu().numpy().astype(np.int64)
    comp_cl = inp.comp_cache_lengths.cpu().numpy().astype(np.int64)
    swa_tab = inp.swa_lookup_table.cpu().numpy()
    comp_tab = inp.comp_lookup_table.cpu().numpy()
    lists = inp.comp_indices.cpu().numpy()
    wl = inp.wl
    orig = np.concatenate([np.arange(offs[b], offs[b + 1]) for b in seqs]).astype(np.int64)
    new_offs = np.concatenate([[0], np.cumsum([offs[b + 1] - offs[b] for b in seqs])])
    wanted = set(orig.tolist()) if rows is None else {int(r) for r in rows}

    def need_of(b, which):
        ps = set()
        for r in range(offs[b], offs[b + 1]):
            if r not in wanted:
                continue
            if which == "swa":
                p = swa_cl[b] + (r - offs[b])
                ps.update(int(j) // PAGE for j in window_positions(p, wl.window))
            else:
                lst = lists[r].reshape(-1).astype(np.int64)
                lst = lst[(lst >= 0) & (lst < comp_cl[b])]
                ps.update(int(e) // PAGE for e in lst)
        return ps

    def build(table, which):
        phys, maps = [], []
        for b in seqs:
            need = need_of(b, which)
            m = {}
            for lp in sorted(need):
                m[lp] = len(phys)
                phys.append(int(table[b, lp]))
            maps.append(m)
        trap = len(phys)
        new_tab = np.full((len(seqs), table.shape[1]), trap, np.int64)
        for i, m in enumerate(maps):
            for lp, k in m.items():
                new_tab[i, lp] = k
        return phys, new_tab

    def gather(pool, phys):
        idx = torch.tensor(phys, dtype=torch.long, device=pool.device)
        got = _bits(pool.index_select(0, idx))
        trap = np.full((1,) + got.shape[1:], 0xFFFF if got.dtype == np.uint16 else 0x7F, got.dtype)
        return np.concatenate([got, trap], axis=0)

    s_phys, s_tab = build(swa_tab, "swa")
    c_phys, c_tab = build(comp_tab, "comp")
    pb = LatentProblem(
        q=_bits(inp.q[torch.from_numpy(orig).to(inp.q.device)]),
        offsets=new_offs.astype(np.int64),
        swa_cache_lengths=swa_cl[seqs], comp_cache_lengths=comp_cl[seqs],
        swa_pool=gather(inp.swa_pool, s_phys), swa_table=s_tab,
        comp_pool=gather(inp.comp_pool, c_phys), comp_table=c_tab,
        comp_indices=lists[orig].astype(np.int64),
        attn_sink=inp.attn_sink.cpu().numpy().astype(np.float32),
        window=wl.window, scale=wl.softmax_scale,
        swa_dtype=wl.swa_dtype, comp_dtype=wl.comp_dtype)
    return pb, orig


def problem_from_inputs(inp) -> LatentProblem:
    """The whole problem (every row) as host copies; for small inputs."""
    import torch
    return LatentProblem(
        q=_bits(inp.q), offsets=inp.input_row_offsets.cpu().numpy().astype(np.int64),
        swa_cache_lengths=inp.swa_cache_lengths.cpu().numpy().astype(np.int64),
        comp_cache_lengths=inp.comp_cache_lengths.cpu().numpy().astype(np.int64),
        swa_pool=_bits(inp.swa_pool), swa_table=inp.swa_lookup_table.cpu().numpy().astype(np.int64),
        comp_pool=_bits(inp.comp_pool), comp_table=inp.comp_lookup_table.cpu().numpy().astype(np.int64),
        comp_indices=inp.comp_indices.cpu().numpy().astype(np.int64),
        attn_sink=inp.attn_sink.cpu().numpy().astype(np.float32),
        window=inp.wl.window, scale=inp.wl.softmax_scale,
        swa_dtype=inp.wl.swa_dtype, comp_dtype=inp.wl.comp_dtype)
