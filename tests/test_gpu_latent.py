"""GPU parity of latent sparse attention: msa_latent_attention_paged through
the C ABI against the float64 oracle, element by element, within the BF16
bar (1e-2 absolute + 1e-2 relative), on seeded inputs whose non-attended
slots hold NaN (so a read of anything outside the window, past a leaf's
length or through an invalid list value shows up)."""
import numpy as np
import pytest
import torch

import parity
from block_sparse_attention_indexer_amd import binding as B
from block_sparse_attention_indexer_amd import latent_inputs as LI
from oracle import latent_oracle as L

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def check(wl, num_partitions=0, seqs=None, rows_per_seq=None):
    say(f"[case] {wl.name} B={wl.batch} H={wl.num_heads} H_lat={wl.num_latent_heads} "
        f"win={wl.window} top_c={wl.top_c} np={num_partitions}")
    inp = LI.make_latent_inputs(wl, DEV)
    out = B.run_latent(inp, num_partitions=num_partitions)
    torch.cuda.synchronize()
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    offs = inp.input_row_offsets.cpu().numpy()
    rows = []
    rng = np.random.default_rng(0)
    for b in seqs:
        rs = np.arange(offs[b], offs[b + 1])
        if rows_per_seq is not None and len(rs) > rows_per_seq:
            rs = np.sort(rng.choice(rs, rows_per_seq, replace=False))
        rows.extend(int(r) for r in rs)
    pb, orig = L.problem_for_sequences(inp, seqs, rows)
    local = [int(np.nonzero(orig == r)[0][0]) for r in rows]
    ref = L.latent_attention(pb, local)
    got = out[torch.tensor(rows, device=DEV, dtype=torch.long)]
    assert torch.isfinite(got.float()).all(), "non-finite output"
    # the FP8 bar when a leaf the call reads is FP8
    read = ([wl.swa_dtype] if wl.window else []) + ([wl.comp_dtype] if wl.top_c else [])
    err = parity.check_attention(got, ref, "fp8_e4m3" if "fp8_e4m3" in read else "bf16", wl.name)
    say(f"  rows={len(rows)} max|err|={err:.3e}")
    return inp, out


def wl(name, new, swa, comp, H=16, H_lat=1, window=32, top_c=100, **kw):
    return LI.LatentWorkload(name, new_lens=tuple(new), swa_cache_lens=tuple(swa),
                             comp_lens=tuple(comp), num_heads=H, num_latent_heads=H_lat,
                             window=window, top_c=top_c, **kw)


def test_decode_small():
    check(wl("lat_small", [1] * 4, [300, 40, 5000, 127], [900, 10, 1300, 0], sink_mean=1.0,
             bad_frac=0.05, dup_frac=0.05, seed=1))


@pytest.mark.parametrize("np_", [1, 2, 3, 7])
def test_explicit_partitions(np_):
    check(wl("lat_np", [1] * 3, [700, 2000, 64], [3000, 500, 260], H=64, window=128, top_c=700,
             sink_mean=2.0, seed=2), num_partitions=np_)


def test_sixty_four_heads_per_latent_head():
    check(wl("lat_g64", [1] * 6, [4000, 10, 129, 9000, 300, 70000], [1000, 3, 40, 2000, 75, 17000],
             H=64, window=128, top_c=512, sink_mean=3.0, seed=3))


def test_two_column_groups_and_partial_waves():
    # 160 heads: one full group of 64, one of 64, one of 32 (two idle waves)
    check(wl("lat_g160", [1] * 3, [500, 6000, 33], [2000, 800, 9], H=160, window=100, top_c=300,
             sink_mean=1.5, seed=4))


def test_several_latent_heads():
    check(wl("lat_hlat", [1, 2, 1], [1000, 200, 50], [400, 700, 31], H=48, H_lat=3, window=48,
             top_c=96, bad_frac=0.1, seed=5))


def test_multi_token_rows_share_windows():
    check(wl("lat_multi", [5, 1, 8, 3], [400, 127, 0, 1000], [600, 50, 0, 900], H=32, window=64,
             top_c=80, sink_mean=0.5, seed=6))


def test_prefill_rows():
    check(wl("lat_prefill", [300, 45], [0, 512], [300, 128], H=16, window=128, top_c=64,
             seed=7), rows_per_seq=40)


def test_window_only_and_list_only():
    check(wl("lat_win_only", [1, 2], [900, 30], [0, 0], H=16, window=200, top_c=0, seed=8))
    check(wl("lat_list_only", [1, 3], [900, 30], [500, 700], H=16, window=0, top_c=150, seed=9))


def test_sinks_absent_large_and_empty_rows():
    # some heads without a sink, large sinks elsewhere, a sequence whose list
    # is all invalid and whose window is empty (window 0): output from the sink alone = 0
    check(wl("lat_sinks", [1, 1, 2], [100, 4000, 7], [0, 2000, 64], H=32, window=16, top_c=40,
             sink_mean=6.0, sink_neg_inf_frac=0.3, bad_frac=0.2, seed=10))
    w0 = wl("lat_empty", [1, 1], [10, 20], [0, 0], H=16, window=0, top_c=8, sink_mean=1.0,
            sink_neg_inf_frac=0.5, seed=11)
    inp, out = check(w0)
    assert (out.float() == 0).all()


def test_latent_decode_workload_full():
    check(LI.latent_decode())


def test_rows_past_the_batch_are_untouched():
    w = wl("lat_untouched", [2, 1], [300, 50], [200, 100], H=16, window=32, top_c=40, seed=12)
    inp = LI.make_latent_inputs(w, DEV)
    out = torch.full((w.total_rows + 3, w.num_heads, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    B.run_latent(inp, output=out, num_partitions=2)
    torch.cuda.synchronize()
    assert (out[w.total_rows:].float() == 7.0).all()
    assert torch.isfinite(out[:w.total_rows].float()).all()


def test_page_placement_gives_identical_results():
    w = wl("lat_perm", [1, 3], [1500, 260], [800, 300], H=32, window=64, top_c=120, seed=13)
    inp = LI.make_latent_inputs(w, DEV)
    a = B.run_latent(inp, num_partitions=2).clone()
    for pool, tab in (("swa_pool", "swa_lookup_table"), ("comp_pool", "comp_lookup_table")):
        P = getattr(inp, pool).shape[0]
        perm = torch.randperm(P, generator=torch.Generator().manual_seed(5)).to(DEV)
        inv = torch.argsort(perm)
        setattr(inp, pool, getattr(inp, pool)[perm].contiguous())
        setattr(inp, tab, inv[getattr(inp, tab).long()].to(torch.int32).contiguous())
    b = B.run_latent(inp, num_partitions=2)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


FP8 = dict(swa_dtype="fp8_e4m3", comp_dtype="fp8_e4m3")


@pytest.mark.parametrize("np_", [0, 3])
def test_fp8_leaves_decode(np_):
    # invalid and repeated list values leave rows of a tile unattended (their
    # stand-in bytes must not reach the result); 64 heads on one latent head
    check(wl("lat_fp8", [1] * 5, [300, 40, 5000, 127, 20000], [900, 10, 1300, 0, 6000], H=64,
             window=128, top_c=600, sink_mean=1.5, bad_frac=0.1, dup_frac=0.05, seed=21, **FP8),
          num_partitions=np_)


def test_fp8_leaves_heads_and_rows():
    # 3 latent heads of 16 query heads, multi-token rows; 40 query heads
    # (a partial column tile) on a second case
    check(wl("lat_fp8_hlat", [1, 4, 2], [1000, 200, 50], [400, 700, 31], H=48, H_lat=3, window=48,
             top_c=96, sink_neg_inf_frac=0.3, bad_frac=0.1, seed=22, **FP8))
    check(wl("lat_fp8_g40", [1, 1], [3000, 77], [800, 90], H=40, window=100, top_c=200, seed=23,
             **FP8))


def test_fp8_window_only_and_list_only():
    check(wl("lat_fp8_win", [1, 2], [900, 30], [0, 0], H=16, window=200, top_c=0, seed=24, **FP8))
    check(wl("lat_fp8_list", [1, 3], [900, 30], [500, 700], H=16, window=0, top_c=150, seed=25,
             **FP8))


def test_fp8_prefill_rows():
    check(wl("lat_fp8_prefill", [300, 45], [0, 512], [300, 128], H=16, window=128, top_c=64,
             seed=26, **FP8), rows_per_seq=40)


def test_fp8_latent_decode_workload_full():
    check(LI.latent_decode_fp8())


MIXED = (dict(swa_dtype="bf16", comp_dtype="fp8_e4m3"), dict(swa_dtype="fp8_e4m3", comp_dtype="bf16"))


@pytest.mark.parametrize("types", [0, 1])
@pytest.mark.parametrize("np_", [0, 1, 2, 5])
def test_leaves_of_two_storage_types(types, np_):
    # the window leaf in one type and the compressed leaf in the other: one
    # launch per leaf, the second merging both launches' partials; a row in
    # its first window positions, invalid and repeated list values, a sink
    check(wl(f"lat_mixed{types}_np{np_}", [1, 3, 2, 1], [700, 90, 1500, 0], [900, 150, 2000, 40],
             H=64, window=96, top_c=300, sink_mean=1.0, sink_neg_inf_frac=0.25, bad_frac=0.05,
             dup_frac=0.05, seed=40 + types, **MIXED[types]), num_partitions=np_)


def test_leaves_of_two_storage_types_at_the_decode_workload_shape():
    from dataclasses import replace
    check(replace(LI.latent_decode(), name="latent_decode_mixed", swa_dtype="fp8_e4m3"),
          seqs=[0, 17, 63])


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_running_max_moves_between_tiles(dtype):
    # a softmax scale of 6/sqrt(128) spreads the scores by tens of units (the
    # values stay of unit size, so the usual bar holds), so a wave's running
    # maximum moves by more than its lazy threshold after its first tile and
    # the accumulators are rescaled inside the loop (about a hundred times in
    # this case)
    check(wl(f"lat_moves_{dtype}", [1] * 4, [3000, 700, 9000, 100], [4000, 1500, 2500, 600], H=64,
             window=128, top_c=1024, scale=6.0 / 128 ** 0.5, seed=27, swa_dtype=dtype,
             comp_dtype=dtype),
          num_partitions=1)


def test_page_ids_outside_the_pool_are_skipped():
    # table entries pointing past the pool (or negative) make the entries on
    # those pages count as not attended: the same output as listing none of
    # them, and no read outside the pool
    w = wl("lat_badpage", [1, 2], [700, 300], [900, 500], H=32, window=64, top_c=150, seed=31)
    inp = LI.make_latent_inputs(w, DEV)
    P = inp.comp_pool.shape[0]
    tab = inp.comp_lookup_table.clone()
    lists = inp.comp_indices.clone()
    bad = {0: 2, 1: 1}                      # sequence -> logical page made bad
    inp.comp_lookup_table[0, bad[0]] = P + 1000
    inp.comp_lookup_table[1, bad[1]] = -7
    B.msa_device_errors(clear=True)
    got = B.run_latent(inp, num_partitions=2).clone()
    assert B.msa_device_errors() == B.MSA_DEVERR_PAGE
    offs = inp.input_row_offsets.cpu().tolist()
    for b, lp in bad.items():
        rows = lists[offs[b]:offs[b + 1]]
        rows[(rows >= 128 * lp) & (rows < 128 * (lp + 1))] = -1
    inp.comp_lookup_table.copy_(tab)
    inp.comp_indices.copy_(lists)
    ref = B.run_latent(inp, num_partitions=2)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    assert torch.equal(got, ref)


def test_lengths_past_the_lookup_table_stay_inside_it():
    # a sequence whose device lengths exceed what its lookup tables address
    # (bad data: its own result is undefined) must not disturb any other
    # sequence's rows, which stay bit-identical to a clean call
    w = wl("lat_badlen", [1, 2, 1], [700, 300, 1200], [900, 500, 300], H=16, window=64, top_c=120,
           seed=32)
    inp = LI.make_latent_inputs(w, DEV)
    B.msa_device_errors(clear=True)
    clean = B.run_latent(inp, num_partitions=2).clone()
    assert B.msa_device_errors() == 0
    inp.swa_cache_lengths[0] = 10 ** 9
    inp.comp_cache_lengths[0] = 10 ** 9
    got = B.run_latent(inp, num_partitions=2)
    torch.cuda.synchronize()
    assert B.msa_device_errors() == B.MSA_DEVERR_LENGTH
    assert torch.equal(got[1:], clean[1:])
