"""Pins for the CPU oracle: each test checks it against something other than
itself -- hand-worked fixtures, a library routine, brute force, closed forms
or an invariant the selection rules imply.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLK = O.BLOCK


# ---------------------------------------------------------------------------
# helpers: small problems built directly as storage bits
# ---------------------------------------------------------------------------

def to_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def fp8_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def make_problem(rng, new_lens, cache_lens, H_kv=2, G=2, H_ik=1, D=16, top_k=3,
                 init=1, local=1, kv_dtype="bf16", extra_pages=3, scale=None, poison=True,
                 ik_dtype="bf16"):
    B = len(new_lens)
    L = [c + n for c, n in zip(cache_lens, new_lens)]
    pages = [(x + BLK - 1) // BLK for x in L]
    P = sum(pages) + extra_pages
    perm = rng.permutation(P)
    stride = max(pages)
    table = np.full((B, stride), perm[-1], dtype=np.int64)
    pos = 0
    for b in range(B):
        table[b, :pages[b]] = perm[pos:pos + pages[b]]
        pos += pages[b]
    R = sum(new_lens)

    def bf(*shape):
        return to_bf16_bits(rng.standard_normal(shape))

    if kv_dtype == "bf16":
        k = bf(P, H_kv, BLK, D)
        v = bf(P, H_kv, BLK, D)
    else:
        def f8(*shape):
            x = np.clip(rng.standard_normal(shape) * 0.5, -448, 448).astype(np.float32)
            return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        k = f8(P, H_kv, BLK, D)
        v = f8(P, H_kv, BLK, D)
    ik = bf(P, H_ik, BLK, D)
    ik_scale = None
    if ik_dtype == "fp8_e4m3":
        # codes of N(0,1) values with one scale per token, max |value| -> 448
        vals = rng.standard_normal((P, H_ik, BLK, D)).astype(np.float32)
        ik_scale = (np.abs(vals).max(axis=-1) / 448.0).astype(np.float32)
        ik = fp8_bits(vals / ik_scale[..., None])
    if poison:
        nan16 = np.uint16(0x7FC0)
        nan8 = np.uint8(0x7F)
        used = set(table[b, i] for b in range(B) for i in range(pages[b]))
        nan_ik = nan8 if ik_dtype == "fp8_e4m3" else nan16
        for pg in range(P):
            if pg not in used:
                ik[pg] = nan_ik
                if ik_scale is not None:
                    ik_scale[pg] = np.nan
                k[pg] = nan16 if kv_dtype == "bf16" else nan8
                v[pg] = nan16 if kv_dtype == "bf16" else nan8
        for b in range(B):
            if L[b] % BLK:
                pg = table[b, pages[b] - 1]
                ik[pg, :, L[b] % BLK:] = nan_ik
                if ik_scale is not None:
                    ik_scale[pg, :, L[b] % BLK:] = np.nan
                k[pg, :, L[b] % BLK:] = nan16 if kv_dtype == "bf16" else nan8
                v[pg, :, L[b] % BLK:] = nan16 if kv_dtype == "bf16" else nan8
    offs = np.zeros(B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(new_lens)
    return O.Problem(q=bf(R, H_kv * G, D), q_idx=bf(R, H_kv, D), index_k=ik, k_cache=k,
                     v_cache=v, kv_dtype=kv_dtype, input_row_offsets=offs,
                     cache_lengths=np.asarray(cache_lens, dtype=np.int64),
                     kv_lookup_table=table, top_k=top_k, init_blocks=init,
                     local_blocks=local, scale=(1 / math.sqrt(D)) if scale is None else scale,
                     ik_dtype=ik_dtype, index_k_scale=ik_scale)


def logical(pb, pool, b, h, n):
    """Positions 0..n-1 of head h of sequence b, looked up one by one in the
    page table (independently of the oracle's own gather)."""
    rows = [pool[int(pb.kv_lookup_table[b][j // BLK]), h, j % BLK] for j in range(n)]
    return np.stack(rows) if rows else np.zeros((0, pool.shape[-1]), pool.dtype)


# ---------------------------------------------------------------------------
# storage formats vs torch's conversions (library routines)
# ---------------------------------------------------------------------------

def test_bf16_decode_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.decode_bf16(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.nanmax(np.abs(ours)) == 448.0
    assert int(np.isnan(ours).sum()) == 2        # S.1111.111 only


# ---------------------------------------------------------------------------
# hand-worked fixtures
# ---------------------------------------------------------------------------

def test_golden_selection_cases():
    fx = json.load(open(os.path.join(GOLDEN, "selection_hand_worked.json")))
    for case in fx["cases"]:
        nb = case["nb"]
        p = nb * BLK - 1
        pos = np.full(nb * BLK, -1e30, dtype=np.float32)
        for blk, vals in case["block_position_scores"].items():
            b0 = int(blk) * BLK
            pos[b0:b0 + len(vals)] = vals
        F = set(O.forced_blocks(nb, case["init"], case["local"]))
        cands = [b for b in range(nb) if b not in F]
        sel = O.block_sparse_select(nb, O.block_scores(pos, p, cands), case["top_k"],
                                    case["init"], case["local"])
        assert sel.blocks == case["expected"], case["comment"]
    for fs in fx["forced_sets"]:
        assert O.forced_blocks(fs["nb"], fs["init"], fs["local"]) == fs["expected"]


def test_golden_attention_closed_form():
    fx = json.load(open(os.path.join(GOLDEN, "attention_closed_form.json")))
    for case in fx["cases"]:
        out, lse = O.masked_attention(np.array(case["q"]), np.array(case["K"]),
                                      np.array(case["V"]), case["scale"])
        np.testing.assert_allclose(out, case["expected_out"], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(lse, case["expected_lse"], rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# brute force on tiny inputs
# ---------------------------------------------------------------------------

def brute_force(pb):
    """Pure-Python loops: per-position dot products, block maxima, a
    selection characterised by the exchange condition, and an explicit
    [rows x positions] mask for the attention."""
    B = len(pb.cache_lengths)
    H_kv, G = pb.num_kv_heads, pb.group
    H_ik = pb.index_k.shape[1]
    D = pb.q.shape[2]
    outs, sels = {}, {}
    for b in range(B):
        c = int(pb.cache_lengths[b])
        n = int(pb.input_row_offsets[b + 1] - pb.input_row_offsets[b])
        L = c + n
        for t in range(n):
            r = int(pb.input_row_offsets[b]) + t
            p = c + t
            nb = p // BLK + 1
            for h in range(H_kv):
                if pb.ik_dtype == "fp8_e4m3":
                    codes = O.decode_e4m3fn(logical(pb, pb.index_k, b, h % H_ik, L)).astype(np.float64)
                    scl = logical(pb, pb.index_k_scale[..., None], b, h % H_ik, L)[:, 0]
                    ik = np.array([[codes[j, d] * float(scl[j]) for d in range(D)] for j in range(L)])
                else:
                    ik = O.decode_bf16(logical(pb, pb.index_k, b, h % H_ik, L)).astype(np.float64)
                qi = O.decode_bf16(pb.q_idx[r, h]).astype(np.float64)
                score = {}
                for blk in range(nb):
                    best = -math.inf
                    for j in range(blk * BLK, min(blk * BLK + BLK, p + 1)):
                        s = sum(qi[d] * ik[j, d] for d in range(D))
                        best = max(best, s)
                    score[blk] = best
                forced = set(range(min(pb.init_blocks, nb))) | set(range(max(0, nb - pb.local_blocks), nb))
                if nb <= pb.top_k:
                    S = set(range(nb))
                else:
                    free = [x for x in range(nb) if x not in forced]
                    k_free = pb.top_k - len(forced)
                    S = None
                    for T in itertools.combinations(free, k_free):
                        rest = [y for y in free if y not in T]
                        if all(score[x] > score[y] or (score[x] == score[y] and x < y)
                               for x in T for y in rest):
                            S = forced | set(T)
                            break
                    assert S is not None
                sels[(r, h)] = sorted(S)
                K = O.decode(logical(pb, pb.k_cache, b, h, L), pb.kv_dtype).astype(np.float64)
                V = O.decode(logical(pb, pb.v_cache, b, h, L), pb.kv_dtype).astype(np.float64)
                mask = [((j // BLK) in S) and j <= p for j in range(L)]
                for g in range(G):
                    qv = O.decode_bf16(pb.q[r, h * G + g]).astype(np.float64)
                    z = [pb.scale * sum(qv[d] * K[j, d] for d in range(D)) if mask[j] else None
                         for j in range(L)]
                    m = max(x for x in z if x is not None)
                    w = [math.exp(x - m) if x is not None else 0.0 for x in z]
                    tot = sum(w)
                    outs[(r, h * G + g)] = [sum(w[j] * V[j, d] for j in range(L) if mask[j]) / tot
                                            for d in range(D)]
    return sels, outs


@pytest.mark.parametrize("seed,kv", [(1, "bf16"), (2, "bf16"), (3, "fp8_e4m3")])
def test_brute_force_tiny(seed, kv):
    rng = np.random.default_rng(seed)
    pb = make_problem(rng, new_lens=[1, 3, 2], cache_lens=[520, 300, 0], H_kv=2, G=3,
                      D=8, top_k=3, init=1, local=1, kv_dtype=kv)
    sels, outs = brute_force(pb)
    d, _ = O.indexer(pb)
    out = O.attention(pb, d)
    for (r, h), S in sels.items():
        got = [x for x in d[r, h] if x >= 0]
        assert got == S, (r, h)
    for (r, g), ref in outs.items():
        np.testing.assert_allclose(out[r, g], ref, rtol=2e-5, atol=2e-5)


def test_brute_force_tiny_separate_index_heads():
    rng = np.random.default_rng(11)
    pb = make_problem(rng, new_lens=[2], cache_lens=[600], H_kv=2, G=2, H_ik=2, D=8,
                      top_k=4, init=1, local=2)
    sels, _ = brute_force(pb)
    d, _ = O.indexer(pb)
    for (r, h), S in sels.items():
        assert [x for x in d[r, h] if x >= 0] == S


@pytest.mark.parametrize("seed,H_ik", [(21, 1), (22, 2)])
def test_brute_force_tiny_fp8_index_k(seed, H_ik):
    rng = np.random.default_rng(seed)
    pb = make_problem(rng, new_lens=[1, 3], cache_lens=[700, 260], H_kv=2, G=2, H_ik=H_ik,
                      D=8, top_k=3, init=1, local=1, ik_dtype="fp8_e4m3")
    sels, _ = brute_force(pb)
    d, _ = O.indexer(pb)
    for (r, h), S in sels.items():
        assert [x for x in d[r, h] if x >= 0] == S, (r, h)


# ---------------------------------------------------------------------------
# FP8 index-K: codes times a per-token scale
# ---------------------------------------------------------------------------

def test_fp8_index_k_with_power_of_two_scales_equals_bf16_values():
    # e4m3 values times 2^e are BF16-exact: the FP8 path must then select
    # exactly what the BF16 path selects on those values
    rng = np.random.default_rng(31)
    pb8 = make_problem(rng, new_lens=[1, 2], cache_lens=[2500, 1800], H_kv=2, G=2, D=16,
                       top_k=5, init=1, local=1, ik_dtype="fp8_e4m3", poison=False)
    P, H_ik = pb8.index_k.shape[:2]
    pb8.index_k = fp8_bits(rng.standard_normal(pb8.index_k.shape) * 8)
    pb8.index_k_scale = (2.0 ** rng.integers(-6, 4, size=(P, H_ik, BLK))).astype(np.float32)
    vals = O.decode_e4m3fn(pb8.index_k).astype(np.float64) * pb8.index_k_scale[..., None]
    bits = to_bf16_bits(vals)
    assert (O.decode_bf16(bits).astype(np.float64) == vals).all()      # exact
    pb16 = O.Problem(**{**pb8.__dict__, "index_k": bits, "ik_dtype": "bf16", "index_k_scale": None})
    d8, s8 = O.indexer(pb8)
    d16, s16 = O.indexer(pb16)
    n = 0
    for i in range(d8.shape[0]):
        for h in range(d8.shape[1]):
            if s8[i][h].decisive and s16[i][h].decisive:
                assert (d8[i, h] == d16[i, h]).all()
                n += 1
    assert n >= d8.shape[0] * d8.shape[1] - 1


def test_fp8_index_k_needle_through_the_scale_alone():
    # one position's codes are ordinary; only its scale is raised -- the
    # score must follow code . q times the scale
    rng = np.random.default_rng(32)
    pb = make_problem(rng, new_lens=[1], cache_lens=[24 * BLK - 1], H_kv=2, G=2, D=16,
                      top_k=4, init=1, local=1, ik_dtype="fp8_e4m3")
    b, h, target = 0, 0, 13
    qv = O.decode_bf16(pb.q_idx[0, h])
    j = target * BLK + 40
    page = pb.kv_lookup_table[b, j // BLK]
    pb.index_k[page, 0, j % BLK] = fp8_bits(np.sign(qv) * 64.0)     # aligned with q, |code| 64
    pb.index_k_scale[page, 0, j % BLK] = 1e3
    d, _ = O.indexer(pb)
    assert target in d[0, h]


def test_fp8_index_k_common_scale_factor_invariance():
    rng = np.random.default_rng(33)
    pb = make_problem(rng, new_lens=[2, 1], cache_lens=[1500, 2600], D=16, top_k=4,
                      init=1, local=1, ik_dtype="fp8_e4m3")
    d0, _ = O.indexer(pb)
    base = pb.index_k_scale.copy()
    for f in (2.0 ** -5, 2.0 ** 7):
        pb.index_k_scale = (base * f).astype(np.float32)
        d1, _ = O.indexer(pb)
        assert (d0 == d1).all()


# ---------------------------------------------------------------------------
# invariants of the selection rules
# ---------------------------------------------------------------------------

def test_selection_invariants_random():
    rng = np.random.default_rng(5)
    for trial in range(6):
        init = int(rng.integers(0, 3))
        local = int(rng.integers(0, 3))
        top_k = init + local + int(rng.integers(1, 4))
        pb = make_problem(rng, new_lens=[1, 4], cache_lens=[int(rng.integers(0, 2000)),
                                                            int(rng.integers(0, 2000))],
                          D=16, top_k=top_k, init=init, local=local)
        d, sels = O.indexer(pb)
        for r in range(d.shape[0]):
            _, p, nb = O.row_position(pb, r)
            F = O.forced_blocks(nb, init, local)
            for h in range(d.shape[1]):
                row = list(d[r, h])
                valid = [x for x in row if x >= 0]
                assert row[len(valid):] == [-1] * (top_k - len(valid))
                assert valid == sorted(set(valid))           # ascending, unique
                assert len(valid) == min(top_k, nb)          # size
                assert len(valid) > 0                        # never empty
                assert set(F) <= set(valid)                  # forced present
                assert all(0 <= x < nb for x in valid)       # causal


def test_needle_forces_its_block():
    rng = np.random.default_rng(7)
    pb = make_problem(rng, new_lens=[1], cache_lens=[20 * BLK - 1], H_kv=2, G=2, D=16,
                      top_k=4, init=1, local=1)
    b, h, target = 0, 1, 9
    qv = O.decode_bf16(pb.q_idx[0, h])
    j = target * BLK + 77
    page = pb.kv_lookup_table[b, j // BLK]
    pb.index_k[page, 0, j % BLK] = to_bf16_bits(qv * 8.0)     # exact power-of-two multiple
    d, _ = O.indexer(pb)
    assert target in d[0, h]


def test_scale_invariance_power_of_two():
    rng = np.random.default_rng(8)
    pb = make_problem(rng, new_lens=[2, 1], cache_lens=[1500, 900], D=16, top_k=4,
                      init=1, local=1)
    d0, _ = O.indexer(pb)
    for f in (0.25, 4.0):
        pb.q_idx = to_bf16_bits(O.decode_bf16(pb.q_idx) * f)
        d1, _ = O.indexer(pb)
        pb.q_idx = to_bf16_bits(O.decode_bf16(pb.q_idx) / f)
        assert (d0 == d1).all()


def test_all_equal_scores_pick_lowest_free_ids():
    rng = np.random.default_rng(9)
    pb = make_problem(rng, new_lens=[1], cache_lens=[12 * BLK + 5], D=16, top_k=5,
                      init=1, local=2, poison=False)
    pb.index_k[:] = to_bf16_bits(np.ones(16))
    d, sels = O.indexer(pb)
    # nb = 13: forced {0, 11, 12}; two free slots go to the lowest ids 1, 2
    expect = [0, 1, 2, 11, 12]
    for h in range(d.shape[1]):
        assert list(d[0, h]) == expect
        assert not sels[0][h].decisive


def test_per_head_independence_under_head_permutation():
    rng = np.random.default_rng(10)
    H_kv, G = 3, 2
    pb = make_problem(rng, new_lens=[2], cache_lens=[1000], H_kv=H_kv, G=G, H_ik=H_kv,
                      D=16, top_k=3)
    d0, _ = O.indexer(pb)
    o0 = O.attention(pb, d0)
    perm = np.array([2, 0, 1])
    qperm = np.concatenate([np.arange(h * G, h * G + G) for h in perm])
    pb.q_idx = pb.q_idx[:, perm].copy()
    pb.index_k = pb.index_k[:, perm].copy()
    pb.k_cache = pb.k_cache[:, perm].copy()
    pb.v_cache = pb.v_cache[:, perm].copy()
    pb.q = pb.q[:, qperm].copy()
    d1, _ = O.indexer(pb)
    o1 = O.attention(pb, d1)
    assert (d1 == d0[:, perm]).all()
    assert np.array_equal(o1, o0[:, qperm])


def test_page_permutation_invariance_bitwise():
    rng = np.random.default_rng(12)
    pb = make_problem(rng, new_lens=[1, 3], cache_lens=[1100, 700], D=16, top_k=4, kv_dtype="fp8_e4m3")
    d0, _ = O.indexer(pb)
    o0 = O.attention(pb, d0)
    P = pb.k_cache.shape[0]
    perm = rng.permutation(P)            # new page i holds old page perm[i]
    inv = np.argsort(perm)
    for name in ("index_k", "k_cache", "v_cache"):
        setattr(pb, name, getattr(pb, name)[perm].copy())
    pb.kv_lookup_table = inv[pb.kv_lookup_table]
    d1, _ = O.indexer(pb)
    o1 = O.attention(pb, d1)
    assert (d0 == d1).all()
    assert np.array_equal(o0, o1)


def test_score_ignores_positions_after_the_token():
    # local = 0 makes the token's own block a scored candidate; a huge value
    # planted past the token's position must not count.
    rng = np.random.default_rng(13)
    c = 6 * BLK + 10
    pb = make_problem(rng, new_lens=[1], cache_lens=[c], H_kv=1, G=1, D=16, top_k=2,
                      init=1, local=0, poison=False)
    qv = O.decode_bf16(pb.q_idx[0, 0])
    page = pb.kv_lookup_table[0, 6]
    pb.index_k[page, 0, 100] = to_bf16_bits(qv * 64.0)    # position 6*128+100 > p
    _, sels = O.indexer(pb)
    sel = sels[0][0]
    rows = O.decode_bf16(O.gather_rows(pb.index_k, pb.kv_lookup_table[0], 0, c + 1))
    visible_max = float(np.max(rows[6 * BLK:c + 1] @ qv))
    assert sel.scores[6] == pytest.approx(visible_max, rel=1e-6)


# ---------------------------------------------------------------------------
# attention special cases
# ---------------------------------------------------------------------------

def test_dense_when_topk_covers_all_blocks_matches_sdpa():
    rng = np.random.default_rng(14)
    new, cached = [3, 5, 1], [300, 0, 700]
    pb = make_problem(rng, new_lens=new, cache_lens=cached, H_kv=2, G=2, D=32, top_k=8,
                      init=1, local=1, scale=0.3)
    d, _ = O.indexer(pb)
    out = O.attention(pb, d)
    for b in range(3):
        L = new[b] + cached[b]
        rows = np.arange(pb.input_row_offsets[b], pb.input_row_offsets[b + 1])
        for h in range(2):
            K = torch.from_numpy(O.decode_bf16(logical(pb, pb.k_cache, b, h, L)).astype(np.float64))
            V = torch.from_numpy(O.decode_bf16(logical(pb, pb.v_cache, b, h, L)).astype(np.float64))
            qh = torch.from_numpy(O.decode_bf16(pb.q[rows, h * 2:h * 2 + 2]).astype(np.float64))
            qh = qh.permute(1, 0, 2)                               # [G, n, D]
            pos_q = torch.arange(new[b]) + cached[b]
            mask = torch.arange(L)[None, :] <= pos_q[:, None]      # causal with cache offset
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh, K[None].expand(2, L, -1), V[None].expand(2, L, -1), attn_mask=mask, scale=0.3)
            np.testing.assert_allclose(out[rows, h * 2:h * 2 + 2], ref.permute(1, 0, 2).numpy(),
                                       rtol=1e-5, atol=1e-5)


def test_constant_values_and_gqa_mapping():
    rng = np.random.default_rng(15)
    H_kv, G = 3, 4
    pb = make_problem(rng, new_lens=[2], cache_lens=[400], H_kv=H_kv, G=G, D=16, top_k=2,
                      poison=False)
    consts = [1.5, -2.0, 0.375]
    for h in range(H_kv):
        pb.v_cache[:, h] = to_bf16_bits(np.full(16, consts[h]))
    d, _ = O.indexer(pb)
    out = O.attention(pb, d)
    for g in range(H_kv * G):
        np.testing.assert_allclose(out[:, g], consts[g // G], rtol=1e-6)


def test_zero_query_gives_mean_over_positions_per_token():
    # q = 0 makes every weight equal, so out = mean of V over the positions
    # the token may see; pins position = cache_length + token index.
    rng = np.random.default_rng(16)
    c, n = 250, 6
    pb = make_problem(rng, new_lens=[n], cache_lens=[c], H_kv=1, G=2, D=16, top_k=8)
    pb.q[:] = to_bf16_bits(np.zeros(16))
    d, _ = O.indexer(pb)
    out = O.attention(pb, d)
    V = O.decode_bf16(logical(pb, pb.v_cache, 0, 0, c + n)).astype(np.float64)
    for t in range(n):
        np.testing.assert_allclose(out[t, 0], V[:c + t + 1].mean(axis=0), rtol=1e-5, atol=1e-6)


def test_first_token_of_fresh_sequence_reads_only_position_zero():
    rng = np.random.default_rng(17)
    pb = make_problem(rng, new_lens=[1, 2], cache_lens=[0, 129], H_kv=2, G=2, D=16, top_k=1,
                      init=1, local=0)
    d, _ = O.indexer(pb)
    out = O.attention(pb, d)
    V0 = O.decode_bf16(logical(pb, pb.v_cache, 0, 1, 1))[0]
    np.testing.assert_allclose(out[0, 2], V0, rtol=1e-6)
    np.testing.assert_allclose(out[0, 3], V0, rtol=1e-6)


def test_splitk_combine_equals_unsplit():
    rng = np.random.default_rng(18)
    G, D, n = 4, 16, 300
    q = rng.standard_normal((G, D)).astype(np.float32)
    K = rng.standard_normal((n, D)).astype(np.float32)
    V = rng.standard_normal((n, D)).astype(np.float32)
    full, full_lse = O.masked_attention(q, K, V, 0.25)
    cuts = [0, 0, 37, 128, 128, 300, 300]         # includes empty partitions
    parts = [O.masked_attention(q, K[a:b], V[a:b], 0.25) for a, b in zip(cuts[:-1], cuts[1:])]
    po = np.stack([p[0] for p in parts])
    pl = np.stack([p[1] for p in parts])
    assert np.isneginf(pl[0]).all()
    np.testing.assert_allclose(O.splitk_combine(po, pl), full, rtol=1e-5, atol=1e-6)
    # lse merges the same way: log sum exp of the parts
    merged = np.log(np.sum(np.exp(pl.astype(np.float64)), axis=0))
    np.testing.assert_allclose(merged, full_lse, rtol=1e-5)


def test_poisoned_slots_never_reach_results():
    rng = np.random.default_rng(19)
    pb = make_problem(rng, new_lens=[3, 1], cache_lens=[261, 1000], D=16, top_k=3,
                      kv_dtype="fp8_e4m3")
    d, _ = O.indexer(pb)
    out = O.attention(pb, d)
    assert np.isfinite(out).all()


def test_own_block_at_block_boundaries():
    # init 0, local 1, top_k 1: the selection is exactly the block holding
    # the token.  Positions straddle block edges; expected ids by hand.
    cases = [(0, 0), (126, 0), (127, 0), (128, 1), (255, 1), (256, 2), (383, 2)]
    rng = np.random.default_rng(20)
    for c, own in cases:
        pb = make_problem(rng, new_lens=[1], cache_lens=[c], H_kv=1, G=1, D=8, top_k=1,
                          init=0, local=1)
        d, _ = O.indexer(pb)
        assert list(d[0, 0]) == [own], c
    # two new tokens on either side of an edge (positions 127 and 128)
    pb = make_problem(rng, new_lens=[2], cache_lens=[127], H_kv=1, G=1, D=8, top_k=1,
                      init=0, local=1)
    d, _ = O.indexer(pb)
    assert [list(x[0]) for x in d] == [[0], [1]]
