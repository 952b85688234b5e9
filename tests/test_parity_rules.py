"""CPU checks of the parity machinery itself: the selection comparison rule,
and the host copies (`problem_from_inputs`, `problem_for_sequences`) that
every GPU parity test builds its oracle problem from."""
import types

import numpy as np
import pytest
import torch

import parity
from block_sparse_attention_indexer_amd import inputs as I
from oracle import msa_oracle as O


# --- the selection rule ------------------------------------------------------

def _one_row(scores, nb, top_k=4, init=1, local=1):
    """A one-row problem whose token sees nb blocks, and the oracle's
    selection for the given candidate scores."""
    pb = types.SimpleNamespace(input_row_offsets=np.array([0, 1]),
                               cache_lengths=np.array([(nb - 1) * 128 + 10]),
                               top_k=top_k, init_blocks=init, local_blocks=local)
    sel = O.block_sparse_select(nb, scores, top_k, init, local)
    return pb, sel


def _check(pb, sel, ids):
    row = np.asarray([ids + [-1] * (pb.top_k - len(ids))], dtype=np.int32)[:, None, :]
    return parity.check_selection(pb, [0], row, [[sel]])


def test_non_decisive_row_rejects_a_dropped_clear_winner():
    # forced {0, 5}; candidates 1..4; block 1 is far above the cut, blocks
    # 2 and 3 are a near-tie at the cut
    pb, sel = _one_row({1: 10.0, 2: 5.0, 3: 4.9999, 4: 1.0}, nb=6)
    assert sel.blocks == [0, 1, 2, 5] and not sel.decisive
    assert _check(pb, sel, [0, 1, 2, 5]) == (0, 1)
    assert _check(pb, sel, [0, 1, 3, 5]) == (0, 1)      # the tie exchanged: valid
    with pytest.raises(AssertionError):
        _check(pb, sel, [0, 2, 3, 5])                   # block 1 dropped
    with pytest.raises(AssertionError):
        _check(pb, sel, [0, 1, 4, 5])                   # a block below the band
    with pytest.raises(AssertionError):
        _check(pb, sel, [0, 1, 2])                      # forced block 5 missing
    with pytest.raises(AssertionError):
        _check(pb, sel, [1, 0, 2, 5])                   # not ascending


def test_decisive_row_must_be_bit_identical():
    pb, sel = _one_row({1: 10.0, 2: 5.0, 3: 3.0, 4: 1.0}, nb=6)
    assert sel.decisive
    assert _check(pb, sel, [0, 1, 2, 5]) == (1, 0)
    with pytest.raises(AssertionError):
        _check(pb, sel, [0, 1, 3, 5])


def test_row_with_every_block_visible_takes_all():
    pb, sel = _one_row({}, nb=3)
    assert sel.decisive and sel.blocks == [0, 1, 2]
    assert _check(pb, sel, [0, 1, 2]) == (1, 0)
    with pytest.raises(AssertionError):
        _check(pb, sel, [0, 2])


# --- the host copies of generated inputs -------------------------------------

def _torch_logical(t, page_of, b, h, n):
    """Logical positions 0..n-1 of sequence b, head h, read from the
    generator's own host page list with torch indexing (float32 values)."""
    pages = torch.as_tensor(np.asarray(page_of[b][:(n + 127) // 128], dtype=np.int64))
    return t[pages, h].float().reshape(-1, t.shape[-1])[:n].numpy()


def _small(kv="bf16", ik="bf16", H_ik=1):
    return I.Workload("hostcopy", new_lens=(3, 0, 1, 5), cache_lens=(300, 20, 900, 129),
                      num_kv_heads=2, group=2, top_k=3, init_blocks=1, local_blocks=1,
                      kv_dtype=kv, ik_dtype=ik, kv_sigma=0.5 if kv != "bf16" else 1.0,
                      num_ik_heads=H_ik, pool_pages=20, seed=4)


@pytest.mark.parametrize("kv,ik,H_ik", [("bf16", "bf16", 1), ("fp8_e4m3", "fp8_e4m3", 2)])
def test_problem_from_inputs_holds_the_tensors_values(kv, ik, H_ik):
    """Every value the oracle reads through the full copy (queries by row,
    caches by logical position through the lookup table) equals what torch
    reads from the generated tensors through the generator's page list."""
    wl = _small(kv, ik, H_ik)
    inp = I.make_inputs(wl, "cpu")
    pb = O.problem_from_inputs(inp)
    np.testing.assert_array_equal(O.decode_bf16(pb.q), inp.q.float().numpy())
    np.testing.assert_array_equal(O.decode_bf16(pb.q_idx), inp.q_idx.float().numpy())
    assert pb.input_row_offsets.tolist() == [0, 3, 3, 4, 9]
    assert pb.cache_lengths.tolist() == list(wl.cache_lens)
    assert (pb.top_k, pb.init_blocks, pb.local_blocks, pb.scale) == (3, 1, 1, wl.softmax_scale)
    for b, L in enumerate(wl.seq_lens()):
        for h in range(2):
            for pool, t in ((pb.k_cache, inp.k_cache), (pb.v_cache, inp.v_cache)):
                got = O.decode(O.gather_rows(pool, pb.kv_lookup_table[b], h, L), kv)
                np.testing.assert_array_equal(got, _torch_logical(t, inp.page_of, b, h, L))
        for h in range(H_ik):
            codes = O.gather_rows(pb.index_k, pb.kv_lookup_table[b], h, L)
            want = _torch_logical(inp.index_k, inp.page_of, b, h, L)
            np.testing.assert_array_equal(O.decode(codes, ik), want)
            if ik != "bf16":
                sc = O.gather_rows(pb.index_k_scale[..., None], pb.kv_lookup_table[b], h, L)[:, 0]
                np.testing.assert_array_equal(
                    sc, _torch_logical(inp.index_k_scale[..., None], inp.page_of, b, h, L)[:, 0])
                assert np.isfinite(sc).all()


@pytest.mark.parametrize("kv,ik,H_ik", [("bf16", "bf16", 1), ("fp8_e4m3", "fp8_e4m3", 2)])
def test_subset_copy_equals_full_copy_restricted(kv, ik, H_ik):
    """The page-subset copy of some sequences reads, position by position and
    row by row, what the full copy reads for those sequences; its rows map
    back to the full rows; and the oracle's selections and outputs on it are
    bit-identical to the full problem's on the same rows."""
    wl = _small(kv, ik, H_ik)
    inp = I.make_inputs(wl, "cpu")
    full = O.problem_from_inputs(inp)
    seqs = [3, 1, 0]                        # out of order, with an empty sequence
    pb, orig = O.problem_for_sequences(inp, seqs)
    assert orig.tolist() == [4, 5, 6, 7, 8, 0, 1, 2]
    assert pb.input_row_offsets.tolist() == [0, 5, 5, 8]
    assert pb.cache_lengths.tolist() == [129, 20, 300]
    # fewer pages than the full pool: only the listed sequences' own
    used = set(np.concatenate([np.asarray(inp.page_of[b]) for b in seqs]).tolist())
    assert pb.k_cache.shape[0] <= len(used) + 1
    for i, r in enumerate(orig):
        np.testing.assert_array_equal(pb.q[i], full.q[r])
        np.testing.assert_array_equal(pb.q_idx[i], full.q_idx[r])
        assert O.row_position(pb, i)[1:] == O.row_position(full, int(r))[1:]
    for i, b in enumerate(seqs):
        L = wl.seq_lens()[b]
        for name, H in (("k_cache", 2), ("v_cache", 2), ("index_k", H_ik)):
            for h in range(H):
                np.testing.assert_array_equal(
                    O.gather_rows(getattr(pb, name), pb.kv_lookup_table[i], h, L),
                    O.gather_rows(getattr(full, name), full.kv_lookup_table[b], h, L))
        if ik != "bf16":
            for h in range(H_ik):
                np.testing.assert_array_equal(
                    O.gather_rows(pb.index_k_scale[..., None], pb.kv_lookup_table[i], h, L),
                    O.gather_rows(full.index_k_scale[..., None], full.kv_lookup_table[b], h, L))
    d_sub, _ = O.indexer(pb)
    d_full, _ = O.indexer(full, orig.tolist())
    np.testing.assert_array_equal(d_sub, d_full)
    np.testing.assert_array_equal(O.attention(pb, d_sub),
                                  O.attention(full, d_full, orig.tolist()))
