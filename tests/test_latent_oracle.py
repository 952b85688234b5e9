"""Pins of the latent sparse attention oracle against facts that do not come
from the oracle's own formula: library attention and softmax routines,
closed forms for one or two entries, invariances the definition implies
(leaf interchange, list order, invalid entries, page placement), and
sensitivity exactly at the window and leaf-length boundaries.

The definition pinned is the one of the "Struct_latent_sparse_attention_
ragged_paged" page of the MAX Mojo docs (shared K=V latent, window leaf by
position range, compressed leaf by per-query entry list, per-head sink in
the denominator) with the readings stated in the oracle's header.
"""
import numpy as np
import pytest
import scipy.special
import torch

from block_sparse_attention_indexer_amd import latent_inputs as LI
from oracle import latent_oracle as L
from oracle.msa_oracle import decode_bf16

D = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bits (round to nearest even, via torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def values(bits):
    return decode_bf16(bits).astype(np.float64)


def make(rng, *, new_lens=(1,), swa_cache=(300,), comp_lens=(200,), H=4, H_lat=1, window=16,
         top_c=8, sink=None, lists=None):
    """A small LatentProblem with identity-free page tables (pages permuted)."""
    B = len(new_lens)
    R = sum(new_lens)
    sp = max((c + n + 127) // 128 for c, n in zip(swa_cache, new_lens))
    cp = max(1, max((n + 127) // 128 for n in comp_lens))
    P_s, P_c = B * sp, B * cp
    swa_pool = bf16_bits(rng.standard_normal((P_s, H_lat, 128, D)))
    comp_pool = bf16_bits(rng.standard_normal((P_c, H_lat, 128, D)))
    swa_table = rng.permutation(P_s).reshape(B, sp)
    comp_table = rng.permutation(P_c).reshape(B, cp)
    offs = np.concatenate([[0], np.cumsum(new_lens)])
    if lists is None:
        lists = np.full((R, H_lat, top_c), -1, np.int64)
        for b in range(B):
            for r in range(offs[b], offs[b + 1]):
                for hl in range(H_lat):
                    k = min(top_c, comp_lens[b])
                    lists[r, hl, :k] = rng.choice(comp_lens[b], size=k, replace=False)
    if sink is None:
        sink = rng.standard_normal(H).astype(np.float32)
    return L.LatentProblem(
        q=bf16_bits(rng.standard_normal((R, H, D))), offsets=offs,
        swa_cache_lengths=np.array(swa_cache), comp_cache_lengths=np.array(comp_lens),
        swa_pool=swa_pool, swa_table=swa_table, comp_pool=comp_pool, comp_table=comp_table,
        comp_indices=np.asarray(lists, np.int64), attn_sink=np.asarray(sink, np.float32),
        window=window, scale=1 / np.sqrt(D))


def latent_vec(pb, leaf, b, idx, hl=0):
    pool, table = (pb.swa_pool, pb.swa_table) if leaf == "swa" else (pb.comp_pool, pb.comp_table)
    return values(pool[table[b, idx // 128], hl, idx % 128])


def test_reduces_to_dense_causal_attention():
    """No sink (-inf), no listed entries and a window covering the whole
    prefix: ordinary causal attention with K = V = the latent sequence,
    which torch's scaled_dot_product_attention computes (float64, CPU)."""
    rng = np.random.default_rng(1)
    c, n = 250, 7
    pb = make(rng, new_lens=(n,), swa_cache=(c,), comp_lens=(0,), window=10_000,
              sink=np.full(4, -np.inf, np.float32))
    out = L.latent_attention(pb)
    seq = np.stack([latent_vec(pb, "swa", 0, j) for j in range(c + n)])   # [c+n, D]
    q = values(pb.q)                                                       # [n, H, D]
    mask = np.arange(c + n)[None, :] <= (c + np.arange(n))[:, None]        # [n, c+n]
    kv = torch.from_numpy(seq)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2)[None], kv, kv, attn_mask=torch.from_numpy(mask),
        scale=pb.scale)[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_sink_is_an_extra_logit_without_value():
    """softmax over [z_1 .. z_n, sink] (scipy) with the sink's weight dropped."""
    rng = np.random.default_rng(2)
    pb = make(rng, swa_cache=(40,), comp_lens=(300,), window=9, top_c=20)
    out = L.latent_attention(pb)
    kv = np.concatenate([np.stack([latent_vec(pb, "swa", 0, j) for j in range(32, 41)]),
                         np.stack([latent_vec(pb, "comp", 0, e) for e in pb.comp_indices[0, 0]])])
    for h in range(4):
        z = pb.scale * (kv @ values(pb.q[0, h]))
        w = scipy.special.softmax(np.append(z, float(pb.attn_sink[h])))[:-1]
        np.testing.assert_allclose(out[0, h], w @ kv, rtol=1e-12, atol=1e-13)


def test_single_entry_closed_form():
    """One window entry, nothing listed: out = v * sigmoid(z - sink)."""
    rng = np.random.default_rng(3)
    pb = make(rng, swa_cache=(77,), comp_lens=(0,), window=1)
    out = L.latent_attention(pb)
    v = latent_vec(pb, "swa", 0, 77)
    for h in range(4):
        z = pb.scale * float(v @ values(pb.q[0, h]))
        lam = scipy.special.expit(z - float(pb.attn_sink[h]))
        np.testing.assert_allclose(out[0, h], lam * v, rtol=1e-12, atol=1e-14)


def test_duplicate_entry_counts_per_occurrence():
    """Window 0 and the list [e, e]: out = v_e * sigmoid(z + ln 2 - sink)."""
    rng = np.random.default_rng(4)
    lists = np.array([[[17, 17, -1, -1]]])
    pb = make(rng, swa_cache=(5,), comp_lens=(40,), window=0, lists=lists)
    out = L.latent_attention(pb)
    v = latent_vec(pb, "comp", 0, 17)
    for h in range(4):
        z = pb.scale * float(v @ values(pb.q[0, h]))
        lam = scipy.special.expit(z + np.log(2.0) - float(pb.attn_sink[h]))
        np.testing.assert_allclose(out[0, h], lam * v, rtol=1e-12, atol=1e-14)


def test_leaves_are_interchangeable():
    """The same vectors reached through the window leaf or through the
    compressed leaf's list give the same output: both leaves feed one
    softmax."""
    rng = np.random.default_rng(5)
    W, c = 24, 200
    a = make(rng, swa_cache=(c,), comp_lens=(0,), window=W, top_c=W)
    b = L.LatentProblem(**{**a.__dict__})
    b.window = 0
    b.comp_pool, b.comp_table = a.swa_pool, a.swa_table
    b.comp_cache_lengths = np.array([c + 1])
    b.comp_indices = np.arange(c - W + 1, c + 1)[None, None, :]
    np.testing.assert_allclose(L.latent_attention(a), L.latent_attention(b), rtol=1e-13, atol=1e-14)


def test_list_order_and_invalid_values_do_not_matter():
    rng = np.random.default_rng(6)
    a = make(rng, swa_cache=(90,), comp_lens=(150,), window=5, top_c=12)
    b = L.LatentProblem(**{**a.__dict__})
    lst = a.comp_indices[0, 0]
    junk = np.array([-1, -7, 150, 151, 1 << 30])
    b.comp_indices = np.concatenate([rng.permutation(lst), junk])[None, None, :]
    np.testing.assert_allclose(L.latent_attention(a), L.latent_attention(b), rtol=1e-13, atol=1e-14)


def test_page_placement_does_not_matter():
    rng = np.random.default_rng(7)
    a = make(rng, new_lens=(3, 2), swa_cache=(130, 260), comp_lens=(200, 300), window=40, top_c=30)
    b = L.LatentProblem(**{**a.__dict__})
    for pool_name, tab_name in (("swa_pool", "swa_table"), ("comp_pool", "comp_table")):
        pool, tab = getattr(a, pool_name), getattr(a, tab_name)
        perm = rng.permutation(pool.shape[0])          # new page k holds old page perm[k]
        inv = np.argsort(perm)
        setattr(b, pool_name, pool[perm])
        setattr(b, tab_name, inv[tab])
    np.testing.assert_allclose(L.latent_attention(a), L.latent_attention(b), rtol=0, atol=0)


def test_window_boundary_is_exact():
    """Changing the vector just outside the window leaves the output alone;
    changing the first one inside moves it."""
    rng = np.random.default_rng(8)
    W, c = 10, 100
    a = make(rng, swa_cache=(c,), comp_lens=(0,), window=W)
    base = L.latent_attention(a)
    for j, moves in ((c - W, False), (c - W + 1, True), (c, True)):
        b = L.LatentProblem(**{**a.__dict__})
        b.swa_pool = a.swa_pool.copy()
        b.swa_pool[a.swa_table[0, j // 128], 0, j % 128] = bf16_bits(rng.standard_normal(D) * 3)
        assert (np.abs(L.latent_attention(b) - base).max() > 1e-6) == moves, j


def test_comp_length_boundary_is_exact():
    """Entry comp_len - 1 is attended, entry comp_len is not (and NaN there
    stays out of the result)."""
    rng = np.random.default_rng(9)
    n = 64
    lists = np.array([[[n - 1, n, -1]]])
    a = make(rng, swa_cache=(30,), comp_lens=(n,), window=3, lists=lists)
    a.comp_pool = a.comp_pool.copy()
    a.comp_pool[a.comp_table[0, n // 128], 0, n % 128] = 0xFFFF          # NaN at entry n
    out = L.latent_attention(a)
    assert np.isfinite(out).all()
    b = L.LatentProblem(**{**a.__dict__})
    b.comp_indices = np.array([[[-1, n, -1]]])
    assert np.abs(L.latent_attention(b) - out).max() > 1e-6


def test_sink_limits():
    """A sink far above every score drives the output to 0; a sink far below
    equals no sink (-inf); with no sink the output is a convex combination."""
    rng = np.random.default_rng(10)
    a = make(rng, swa_cache=(60,), comp_lens=(100,), window=8, top_c=10,
             sink=np.full(4, -np.inf, np.float32))
    none = L.latent_attention(a)
    b = L.LatentProblem(**{**a.__dict__})
    b.attn_sink = np.full(4, -1e4, np.float32)
    np.testing.assert_allclose(L.latent_attention(b), none, rtol=1e-14, atol=0)
    b.attn_sink = np.full(4, 1e3, np.float32)
    assert np.abs(L.latent_attention(b)).max() < 1e-300
    kv = L.row_entries(a, 0, 0)
    assert (none >= kv.min(axis=0) - 1e-12).all() and (none <= kv.max(axis=0) + 1e-12).all()


def test_query_heads_read_their_latent_head():
    """With two latent heads, query heads 0..G-1 read latent head 0 and
    G..2G-1 latent head 1: each half equals a one-latent-head problem."""
    rng = np.random.default_rng(11)
    a = make(rng, new_lens=(2,), swa_cache=(140,), comp_lens=(260,), H=6, H_lat=2, window=20,
             top_c=16)
    out = L.latent_attention(a)
    for hl in range(2):
        b = L.LatentProblem(**{**a.__dict__})
        b.q = a.q[:, 3 * hl:3 * hl + 3]
        b.swa_pool = a.swa_pool[:, hl:hl + 1]
        b.comp_pool = a.comp_pool[:, hl:hl + 1]
        b.comp_indices = a.comp_indices[:, hl:hl + 1]
        b.attn_sink = a.attn_sink[3 * hl:3 * hl + 3]
        np.testing.assert_allclose(out[:, 3 * hl:3 * hl + 3], L.latent_attention(b), rtol=0, atol=0)


def test_empty_row_gives_zero():
    rng = np.random.default_rng(12)
    a = make(rng, swa_cache=(10,), comp_lens=(5,), window=0, lists=np.full((1, 1, 4), -1))
    assert (L.latent_attention(a) == 0).all()
    a.attn_sink = np.full(4, -np.inf, np.float32)
    assert (L.latent_attention(a) == 0).all()


def test_host_copy_of_generated_inputs_is_consistent():
    """The page-subset host copy of generated inputs gives the same result as
    the full copy, and no NaN-poisoned slot is ever read."""
    wl = LI.LatentWorkload("t", new_lens=(3, 1, 2), swa_cache_lens=(300, 5, 129),
                           comp_lens=(700, 0, 130), num_heads=4, window=40, top_c=24,
                           sink_mean=1.0, bad_frac=0.1, dup_frac=0.1, seed=3)
    inp = LI.make_latent_inputs(wl, "cpu")
    full = L.latent_attention(L.problem_from_inputs(inp))
    assert np.isfinite(full).all()
    rows = [0, 2, 4, 5]
    pb, orig = L.problem_for_sequences(inp, [0, 2], rows)
    sub = L.latent_attention(pb, [int(np.nonzero(orig == r)[0][0]) for r in rows])
    np.testing.assert_allclose(sub, full[rows], rtol=0, atol=0)


def test_fp8_leaves_equal_their_bf16_encoding():
    """Every e4m3 value is exactly a BF16 value, so a problem whose leaves are
    stored as FP8 codes (generated inputs, NaN-poisoned slots included) must
    give bit for bit the output of the same problem with the leaves re-encoded
    as BF16 -- pinning the FP8 leaf path (codes, dtype plumbing, page-subset
    copies) to the BF16 one.  The codes are decoded here by torch's own cast,
    not by the oracle's table."""
    wl = LI.LatentWorkload("t8", new_lens=(2, 1, 3), swa_cache_lens=(260, 40, 1000),
                           comp_lens=(500, 90, 0), num_heads=8, num_latent_heads=2, window=48,
                           top_c=40, sink_mean=1.0, bad_frac=0.1, dup_frac=0.1, seed=8,
                           swa_dtype="fp8_e4m3", comp_dtype="fp8_e4m3", sigma=2.0)
    inp = LI.make_latent_inputs(wl, "cpu")
    pb8 = L.problem_from_inputs(inp)
    pb16 = L.LatentProblem(**{**pb8.__dict__})
    for leaf in ("swa_pool", "comp_pool"):
        codes = torch.from_numpy(getattr(pb8, leaf).copy()).view(torch.float8_e4m3fn)
        setattr(pb16, leaf, codes.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    pb16.swa_dtype = pb16.comp_dtype = "bf16"
    out8 = L.latent_attention(pb8)
    assert np.isfinite(out8).all()
    np.testing.assert_array_equal(out8, L.latent_attention(pb16))
    # the page-subset copy agrees too
    rows = [0, 3, 5]
    pb, orig = L.problem_for_sequences(inp, [0, 2], rows)
    sub = L.latent_attention(pb, [int(np.nonzero(orig == r)[0][0]) for r in rows])
    np.testing.assert_array_equal(sub, out8[rows])
