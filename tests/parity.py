"""Comparison helpers shared by the GPU parity tests and the smoke check.

Selection parity: a (row, KV head) is *decisive* when the oracle's last
chosen and first rejected candidate scores differ by more than 1e-3
relative; there the GPU's block ids must be bit-identical.  Elsewhere the
GPU selection must still be a valid selection (forced blocks, ascending,
the right size) that differs from the oracle's only inside the near-tie
band: every free block it picks scores at least the oracle's cut less 1e-3
relative, and every block scoring more than the cut plus 1e-3 relative is
picked.

Attention parity: BF16 outputs within atol + rtol * |ref| of the oracle
(1e-2 / 1e-2 for BF16 KV, 3e-2 / 3e-2 for FP8 KV), run on the oracle's own
block ids so that selection and attention are checked separately.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import msa_oracle as O

TOL = {"bf16": (1e-2, 1e-2), "fp8_e4m3": (3e-2, 3e-2)}


def check_selection(pb, rows, d_gpu_rows, sels, rel_gap=1e-3):
    """Returns (n_decisive, n_relaxed); raises AssertionError on a mismatch."""
    nd = nr = 0
    top_k = pb.top_k
    for i, r in enumerate(rows):
        _, p, nb = O.row_position(pb, r)
        F = set(O.forced_blocks(nb, pb.init_blocks, pb.local_blocks))
        for h, sel in enumerate(sels[i]):
            got = [int(x) for x in d_gpu_rows[i, h]]
            if sel.decisive:
                nd += 1
                want = sel.blocks + [-1] * (top_k - len(sel.blocks))
                assert got == want, f"row {r} head {h}: gpu {got} != oracle {want}"
                continue
            nr += 1
            valid = [x for x in got if x >= 0]
            assert got[len(valid):] == [-1] * (top_k - len(valid)), (r, h, got)
            assert valid == sorted(set(valid)), (r, h, got)
            assert len(valid) == min(top_k, nb), (r, h, got)
            assert F <= set(valid), (r, h, got)
            # every free block the GPU picked scores at least the cut (less
            # the band), and every block scoring clearly above the cut was
            # picked: only blocks inside the near-tie band may be exchanged
            band = rel_gap * abs(sel.kth_score) + 1e-6
            lo, hi = sel.kth_score - band, sel.kth_score + band
            picked = set(valid) - F
            for x in picked:
                assert sel.scores[x] >= lo, (r, h, x, sel.scores[x], sel.kth_score)
            for x, s in sel.scores.items():
                if s > hi:
                    assert x in picked, (f"row {r} head {h}: block {x} scores {s} above the "
                                         f"cut {sel.kth_score} but the gpu dropped it", got)
    return nd, nr


def check_attention(gpu, ref, kv_dtype, what=""):
    atol, rtol = TOL[kv_dtype]
    gpu = gpu.float().cpu().numpy() if isinstance(gpu, torch.Tensor) else gpu
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"first {idx.tolist()}: gpu {gpu[tuple(idx[0])]} ref {ref[tuple(idx[0])]}")
    return float(err.max()) if err.size else 0.0


def sample_rows(pb, per_seq=None, seed=0):
    """Row indices of a sub-problem: all rows, or per_seq rows of every
    sequence including its first and last."""
    offs = pb.input_row_offsets
    rows = []
    rng = np.random.default_rng(seed)
    for b in range(len(offs) - 1):
        lo, hi = int(offs[b]), int(offs[b + 1])
        if hi <= lo:
            continue
        if per_seq is None or hi - lo <= per_seq:
            rows.extend(range(lo, hi))
        else:
            pick = set([lo, hi - 1]) | set(rng.choice(np.arange(lo, hi), per_seq - 2, replace=False).tolist())
            rows.extend(sorted(pick))
    return rows
