"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case generates seeded inputs on the GPU, runs msa_indexer_paged and
msa_attention_paged, and compares rows with the oracle element by element
(every row of the decode and speculative workloads; sampled rows of a
sequence only on the prefill route): block ids bit-exact on decisive rows
(valid, and different only inside the near-tie band at the score cut,
elsewhere), attention within the BF16 / FP8 tolerances on the oracle's
own ids, and end to end on rows whose every head is decisive.
"""
import numpy as np
import pytest
import torch

import parity
from block_sparse_attention_indexer_amd import binding as B
from block_sparse_attention_indexer_amd import inputs as I
from oracle import msa_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run_and_check(wl, seqs=None, per_seq=None, num_partitions=0, shared=False, chunk=None):
    """Run the indexer and attention on the GPU, then compare sequences
    `seqs` (default: every sequence) with the oracle, `chunk` sequences at a
    time (each chunk's pages copied to the host on their own, so full-size
    workloads are compared whole without holding their caches twice)."""
    say(f"[case] {wl.name} B={wl.batch} seqs={'all' if seqs is None else seqs} "
        f"per_seq={per_seq} np={num_partitions} shared={shared}")
    inp = I.make_inputs(wl, DEV)
    d_gpu = B.run_indexer(inp)
    out_gpu = B.run_attention(inp, d_gpu, num_partitions=num_partitions, shared=shared)
    torch.cuda.synchronize()
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    chunk = chunk or len(seqs) or 1
    parts = []
    nd = nr = 0
    for c0 in range(0, len(seqs), chunk):
        pb, orig_rows = O.problem_for_sequences(inp, seqs[c0:c0 + chunk])
        sub = parity.sample_rows(pb, per_seq)
        d_ref, sels = O.indexer(pb, sub)
        grows = torch.as_tensor(orig_rows[sub], device=DEV, dtype=torch.long)
        a, b = parity.check_selection(pb, sub, d_gpu[grows].cpu().numpy(), sels)
        nd, nr = nd + a, nr + b
        ref = O.attention(pb, d_ref, sub)
        dec = [i for i, s in enumerate(sels) if all(x.decisive for x in s)]
        parts.append((grows, d_ref, ref, dec))
        del pb
        if len(seqs) > chunk:
            say(f"  sequences {c0}..{min(len(seqs), c0 + chunk) - 1}: selections checked")
    d_mix = d_gpu.clone()
    for grows, d_ref, _, _ in parts:
        d_mix[grows] = torch.from_numpy(d_ref).to(DEV)
    out_mix = B.run_attention(inp, d_mix, num_partitions=num_partitions, shared=shared)
    torch.cuda.synchronize()
    err = 0.0
    nrows = 0
    for grows, _, ref, dec in parts:
        err = max(err, parity.check_attention(out_mix[grows], ref, wl.kv_dtype, wl.name))
        if dec:
            parity.check_attention(out_gpu[grows[dec]], ref[dec], wl.kv_dtype,
                                   wl.name + " end-to-end")
        nrows += len(grows)
    say(f"  rows={nrows} decisive heads={nd} relaxed={nr} max|err|={err:.3e}")
    return inp, d_gpu, out_gpu


def wl_custom(name, new, cached, H_kv=2, G=8, top_k=6, init=1, local=2, kv="bf16", H_ik=1,
              boost=0.0, seed=3, ik="bf16"):
    return I.Workload(name, new_lens=tuple(new), cache_lens=tuple(cached), num_kv_heads=H_kv,
                      group=G, top_k=top_k, init_blocks=init, local_blocks=local, kv_dtype=kv,
                      kv_sigma=0.5 if kv != "bf16" else 1.0, num_ik_heads=H_ik, boost_frac=boost,
                      seed=seed, ik_dtype=ik)


# --- the five workloads ------------------------------------------------------

def test_decode_small_full():
    run_and_check(I.decode_small())


def test_decode_batch64_full():
    run_and_check(I.decode_batch64(), chunk=16)


def test_spec_decode_full():
    run_and_check(I.spec_decode(), chunk=4)


def test_prefill_ragged_small():
    wl = I.prefill_ragged(new=(300, 1100, 40, 2100), cached=(0, 2048, 5000, 16384))
    run_and_check(wl, per_seq=40)


def test_prefill_ragged_full_sampled():
    run_and_check(I.prefill_ragged(), per_seq=24)


def test_decode_fp8_long_full():
    run_and_check(I.decode_fp8_long(), chunk=2)


# --- shape variants and edge cases -----------------------------------------

@pytest.mark.parametrize("G", [2, 4, 8])
def test_spec_one_partition_one_wave_workgroups(G):
    # one partition: with 2 to 4 token groups per (sequence, KV head) each
    # token group runs as its own one-wave workgroup, placed on its
    # sequence's XCD, computing the common block schedule itself
    run_and_check(wl_custom(f"g{G}_spec_np1", [3, 8, 1, 5, 2], [3000, 127, 5000, 2500, 90000], G=G,
                            top_k=7), num_partitions=1)


def test_spec_one_wave_workgroups_many_pairs():
    # 72 sequences x 8 KV heads = 576 (sequence, KV head) pairs, 72 per XCD:
    # a workgroup's search for its token group crosses a 64-pair chunk
    g = np.random.default_rng(11)
    new = [int(x) for x in g.integers(1, 9, size=72)]
    cached = [int(x) for x in g.integers(200, 4000, size=72)]
    run_and_check(wl_custom("spec_np1_many", new, cached, H_kv=8, G=8, top_k=6, seed=12),
                  num_partitions=1, chunk=24)


@pytest.mark.parametrize("G", [1, 2, 4, 16])
def test_group_sizes_decode_and_spec(G):
    run_and_check(wl_custom(f"g{G}_decode", [1, 1, 1], [3000, 129, 5000], G=G))
    run_and_check(wl_custom(f"g{G}_spec", [3, 8, 1, 5], [3000, 127, 5000, 2500], G=G, top_k=5))


def test_separate_index_heads_and_no_forced_blocks():
    run_and_check(wl_custom("ik_per_head", [1, 4], [4000, 2600], H_kv=4, H_ik=4, init=0, local=0,
                            top_k=3))
    run_and_check(wl_custom("local_only", [2, 1], [1300, 2000], init=0, local=1, top_k=2))


def test_fp8_spec_and_boosted_rows():
    run_and_check(wl_custom("fp8_spec", [2, 7], [6000, 700], kv="fp8_e4m3", top_k=8, local=4))
    run_and_check(wl_custom("boost", [1, 1, 1, 1], [4095, 4096, 9000, 300], boost=0.05))


def test_empty_and_zero_length_sequences():
    wl = wl_custom("zero_len", [1, 0, 3, 0], [900, 700, 2000, 10], top_k=4)
    run_and_check(wl)
    run_and_check(wl, shared=True)
    # prefill route: empty sequences between long and one-token ones (empty
    # plan slots and index tiles, a sequence with no cache)
    run_and_check(wl_custom("zero_len_prefill", [0, 40, 0, 1, 17], [500, 3000, 0, 128, 0], top_k=4))
    inp = I.make_inputs(wl, DEV)
    rg = B.ragged(inp.input_row_offsets[:1], inp.cache_lengths[:0], inp.kv_lookup_table[:0], 0, 0)
    d = torch.empty((0, 2, 4), dtype=torch.int32, device=DEV)
    B.msa_indexer_paged(d, inp.q_idx, inp.index_k, rg, 2, 4, 1, 2)


@pytest.mark.parametrize("np_", [1, 2, 3, 7])
def test_explicit_partitions(np_):
    run_and_check(wl_custom(f"np{np_}", [1, 2, 5], [8000, 3000, 255], top_k=9), num_partitions=np_)


def test_split_k_at_full_size():
    # the automatic plan keeps these batches in one partition; force a split
    run_and_check(I.decode_batch64(), seqs=[2, 33, 63], num_partitions=4)
    run_and_check(I.spec_decode(), seqs=[1, 30], num_partitions=3)


def test_many_sequences_per_scorer_chunk():
    # more sequences than scorer threads: each prefix chunk spans several
    rng = np.random.default_rng(11)
    n = 300
    cached = rng.integers(300, 3000, size=n)
    new = rng.integers(0, 3, size=n)
    wl = wl_custom("b300", new.tolist(), cached.tolist(), top_k=4, seed=11)
    run_and_check(wl, seqs=[0, 1, 2, 255, 256, 257, 298, 299])


def test_maximum_context_and_top_k():
    # MSA_MAX_BLOCKS blocks (1 Mi positions) and MSA_MAX_TOPK blocks per row:
    # the widest top-k (8188 candidates) and the largest attention unions
    full = B.MSA_MAX_BLOCKS * 128
    run_and_check(wl_custom("max_decode", [1, 1], [full - 1, 3000 * 128 + 5], H_kv=2, G=2,
                            top_k=B.MSA_MAX_TOPK, init=1, local=4))
    run_and_check(wl_custom("max_prefill", [16], [full - 16], H_kv=1, G=4,
                            top_k=B.MSA_MAX_TOPK, init=1, local=4), per_seq=6)
    # speculative rows through msa_attention_paged_shared: 8 tokens' fresh
    # top-512 selections give a union of thousands of blocks per tile, so the
    # 4-wave kernel's LDS ring of plan entries refills many times
    run_and_check(wl_custom("max_spec_shared", [8, 5], [full - 8, 3000 * 128 + 5], H_kv=1, G=4,
                            top_k=B.MSA_MAX_TOPK, init=1, local=4), per_seq=4, shared=True)


def test_top_k_over_a_few_thousand_candidates():
    # 1025..4096 candidates: the 64-keys-per-lane top-k
    run_and_check(wl_custom("kpl64", [1, 3, 1], [3500 * 128, 2100 * 128 + 77, 1400 * 128], H_kv=2,
                            top_k=100, init=2, local=3))


@pytest.mark.parametrize("np_", [0, 1])
@pytest.mark.parametrize("case", ["union64", "bitmap65", "mixed_paths"])
def test_speculative_block_schedule_edges(case, np_):
    # The waves of a speculative (sequence, KV head) walk their unions on one
    # common schedule when a wave's union has at most 64 blocks and the block
    # bitmaps at most 64 words, else block 0 first and then newest first.
    # union64: no forced blocks and 32 picks from ~1500 candidates, so two
    #   tokens' unions are mostly exactly 64 blocks; 3 to 4 waves per
    #   workgroup (5 to 8 draft tokens, two per wave).
    # bitmap65: one context of 2049 blocks makes the bitmaps 65 words: every
    #   wave takes the fallback order.
    # mixed_paths: 40 picks per token, so some waves of a workgroup hold
    #   more than 64 blocks and take the fallback while the others follow
    #   the schedule.
    # np_ = 0 lets the planner split these small batches (workgroups of the
    # token groups of one (sequence, KV head)); np_ = 1 gives one-wave
    # workgroups that each compute the schedule from every token group.
    if case == "union64":
        wl = wl_custom("sched_union64", [5, 6, 8, 3], [190000, 150000, 120000, 170000], H_kv=1,
                       top_k=32, init=0, local=0, seed=21)
    elif case == "bitmap65":
        wl = wl_custom("sched_bitmap65", [4, 2], [2049 * 128 + 5, 3000], H_kv=1, top_k=32,
                       init=1, local=2, seed=22)
    else:
        wl = wl_custom("sched_mixed", [7, 4, 2], [100000, 50000, 9000], H_kv=2, top_k=40,
                       init=1, local=1, seed=23)
    run_and_check(wl, chunk=1, num_partitions=np_)


def test_two_column_groups_per_sequence():
    # 16 KV heads sharing one index head x 8 draft tokens = 128 columns
    run_and_check(wl_custom("cg2", [8, 3, 6], [3000, 5000, 700], H_kv=16, G=1, top_k=5))


def test_tie_break_lower_id_on_all_equal_scores():
    wl = wl_custom("ties", [1, 2], [20 * 128 + 3, 9 * 128], top_k=6, init=1, local=2)
    inp = I.make_inputs(wl, DEV)
    inp.index_k.copy_(torch.ones_like(inp.index_k))
    d = B.run_indexer(inp).cpu().numpy()
    # row 0: nb 21 -> forced {0, 19, 20}, free {1, 2, 3}; rows 1, 2: nb 10, 10
    assert list(d[0, 0]) == [0, 1, 2, 3, 19, 20]
    assert list(d[1, 1]) == [0, 1, 2, 3, 8, 9]
    assert list(d[2, 0]) == [0, 1, 2, 3, 8, 9]


@pytest.mark.parametrize("name,new,cached,top_k", [
    ("decode_kpl4", [1, 1], [3000, 200 * 128 + 5], 40),
    ("decode_kpl16", [1], [900 * 128], 40),
    ("decode_kpl64", [1], [3000 * 128 + 17], 64),
    ("decode_kpl128", [1], [5000 * 128], 100),
    ("spec", [3, 5], [900 * 128, 150 * 128 + 9], 40),
    ("prefill", [40, 12], [2000, 250 * 128], 30),
])
def test_tied_block_scores_select_lowest_ids(name, new, cached, top_k):
    # Index keys constant over a block, c_b times a unit vector with c_b a
    # small integer of either sign, so every block score is exactly c_b q[0]
    # in any precision: large groups of equal scores, the cut falling inside
    # one, and scores of both signs.  The selection is then unique (equal
    # scores go to the lower block id) and must match the oracle exactly.
    wl = wl_custom(f"tiedscores_{name}", new, cached, top_k=top_k, init=1, local=2, seed=31)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    P = inp.index_k.shape[0]
    c = torch.from_numpy(np.random.default_rng(5).integers(-20, 21, size=P)).to(DEV, torch.float32)
    inp.index_k.zero_()
    inp.index_k[:, :, :, 0] = c.view(P, 1, 1).to(torch.bfloat16)
    d_gpu = B.run_indexer(inp).cpu().numpy()
    pb, orig_rows = O.problem_for_sequences(inp, range(wl.batch))
    d_ref, _ = O.indexer(pb)
    assert np.array_equal(d_gpu[orig_rows], d_ref)


@pytest.mark.parametrize("name,new,cached,top_k,np_", [
    ("decode", [1, 1, 1, 1], [3000, 200 * 128 + 5, 900 * 128, 40], 40, 0),
    ("decode_split", [1, 1], [900 * 128, 3000 * 128 + 17], 64, 4),
    ("spec", [3, 8, 1], [900 * 128, 150 * 128 + 9, 5000], 24, 0),
])
def test_selection_row_order_gives_bitwise_identical_results(name, new, cached, top_k, np_):
    # The same selection written in another order (ids shuffled, the -1
    # padding spread among them) is the same set of blocks: the decode rows
    # then leave the in-order fast path for the bitmap, and every output must
    # stay bit-identical to the indexer's ascending rows.
    wl = wl_custom(f"roworder_{name}", new, cached, top_k=top_k, init=1, local=2, seed=41)
    say(f"[case] {wl.name} np={np_}")
    inp = I.make_inputs(wl, DEV)
    d = B.run_indexer(inp)
    o0 = B.run_attention(inp, d, num_partitions=np_).clone()
    g = torch.Generator().manual_seed(7)
    dp = d.cpu()
    perm = torch.stack([torch.randperm(top_k, generator=g) for _ in range(dp.shape[0] * dp.shape[1])])
    dp = torch.gather(dp.reshape(-1, top_k), 1, perm).reshape(dp.shape).contiguous()
    assert not torch.equal(dp, d.cpu())
    o1 = B.run_attention(inp, dp.to(DEV), num_partitions=np_)
    torch.cuda.synchronize()
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


def test_page_permutation_gives_bitwise_identical_results():
    wl = wl_custom("perm", [1, 3], [7000, 2000], top_k=8)
    inp = I.make_inputs(wl, DEV)
    d0 = B.run_indexer(inp)
    o0 = B.run_attention(inp, d0)
    P = inp.k_cache.shape[0]
    perm = torch.randperm(P, generator=torch.Generator().manual_seed(1)).to(DEV)
    inv = torch.argsort(perm)
    for name in ("index_k", "k_cache", "v_cache"):
        setattr(inp, name, getattr(inp, name)[perm].contiguous())
    inp.kv_lookup_table = inv[inp.kv_lookup_table.long()].to(torch.int32).contiguous()
    d1 = B.run_indexer(inp)
    o1 = B.run_attention(inp, d1)
    torch.cuda.synchronize()
    assert torch.equal(d0, d1)
    assert torch.equal(o0.view(torch.int16), o1.view(torch.int16))


@pytest.mark.parametrize("route", ["decode", "prefill", "spec_shared"])
def test_bad_page_ids_stay_inside_their_sequence(route):
    # page ids outside the pool in one sequence's lookup table (bad data: that
    # sequence's result is undefined) must leave every other sequence's
    # selection and output bit-identical to a clean call; every kernel reads
    # page 0 or skips the block instead, so no read leaves the pools
    new = {"decode": [1, 1, 1], "prefill": [40, 100, 9], "spec_shared": [3, 8, 2]}[route]
    shared = route == "spec_shared"
    wl = wl_custom(f"badpage_{route}", new, [3000, 5000, 700], top_k=6)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    B.msa_device_errors(clear=True)
    d0 = B.run_indexer(inp).clone()
    o0 = B.run_attention(inp, d0, shared=shared).clone()
    assert B.msa_device_errors() == 0             # clean data reports nothing
    P = inp.k_cache.shape[0]
    inp.kv_lookup_table[0, 3] = P + 50
    inp.kv_lookup_table[0, 10] = -3
    d1 = B.run_indexer(inp)
    o1 = B.run_attention(inp, d1, shared=shared)
    torch.cuda.synchronize()
    assert B.msa_device_errors() == B.MSA_DEVERR_PAGE   # ... and the bad ids are reported
    r1 = int(inp.input_row_offsets[1])
    assert torch.equal(d0[r1:], d1[r1:])
    assert torch.equal(o0[r1:].view(torch.int16), o1[r1:].view(torch.int16))
    assert torch.isfinite(o1.float()).all()


@pytest.mark.parametrize("route", ["decode", "spec_shared", "prefill"])
def test_lengths_past_the_lookup_table_stay_inside_it(route):
    # the last sequence's device length (10^6) runs far past its lookup-table
    # row, under a host bound on cache lengths four times the real one (so
    # the host bound alone would allow blocks past the table): every kernel
    # clips block counts to the table's width, so no read leaves the table,
    # and the other sequences' ids and outputs stay bit-identical
    new = {"decode": [1, 1, 1], "spec_shared": [3, 8, 2], "prefill": [40, 100, 9]}[route]
    wl = wl_custom(f"longlen_{route}", new, [3000, 5000, 700], top_k=6)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    rg = B.ragged(inp.input_row_offsets, inp.cache_lengths, inp.kv_lookup_table,
                  wl.max_seq_length, 4 * wl.max_cache_length)
    attention = B.msa_attention_paged_shared if route == "spec_shared" else B.msa_attention_paged

    def step():
        d = torch.empty((wl.total_rows, wl.num_kv_heads, wl.top_k), dtype=torch.int32, device=DEV)
        B.msa_indexer_paged(d, inp.q_idx, inp.index_k, rg, wl.num_kv_heads, wl.top_k,
                            wl.init_blocks, wl.local_blocks, index_k_scale=inp.index_k_scale)
        out = torch.empty((wl.total_rows, wl.num_q_heads, 128), dtype=torch.bfloat16, device=DEV)
        attention(out, inp.q, d, inp.k_cache, inp.v_cache, rg, wl.num_q_heads, wl.num_kv_heads,
                  wl.top_k, wl.softmax_scale)
        return d, out

    B.msa_device_errors(clear=True)
    d_tight = B.run_indexer(inp).clone()
    d0, o0 = step()
    assert B.msa_device_errors() == 0             # the loose host bound is not an error
    inp.cache_lengths[-1] = 10 ** 6
    d1, o1 = step()
    torch.cuda.synchronize()
    assert B.msa_device_errors() & B.MSA_DEVERR_LENGTH
    assert torch.equal(d0, d_tight)              # the loose host bound changes nothing
    rl = int(inp.input_row_offsets[-2])
    assert torch.equal(d0[:rl], d1[:rl])
    assert torch.equal(o0[:rl].view(torch.int16), o1[:rl].view(torch.int16))
    assert torch.isfinite(o0.float()).all()


@pytest.mark.parametrize("mode", ["paged", "shared", "prefill"])
def test_rows_fully_written_and_no_ids_gives_zero(mode):
    # decode + speculative rows through either entry point, or a prefill batch
    # (whose tiles with no visible block are not in the work list)
    shared = mode == "shared"
    new = [1, 40] if mode == "prefill" else [1, 4]
    wl = wl_custom("poison", new, [3000, 500], top_k=5)
    say(f"[case] {wl.name} {mode}")
    inp = I.make_inputs(wl, DEV)
    d = B.run_indexer(inp)
    out = torch.full((wl.total_rows + 3, wl.num_q_heads, 128), float("nan"), dtype=torch.bfloat16,
                     device=DEV)
    B.run_attention(inp, d, output=out, shared=shared)
    torch.cuda.synchronize()
    assert torch.isfinite(out[:wl.total_rows].float()).all()
    assert torch.isnan(out[wl.total_rows:].float()).all()
    none = torch.full_like(d, -1)
    B.run_attention(inp, none, output=out, shared=shared)
    torch.cuda.synchronize()
    assert (out[:wl.total_rows].float() == 0).all()
    # only blocks past every row's position: no visible position either
    future = torch.full_like(d, -1)
    future[:, :, 0] = 1000
    out.fill_(float("nan"))
    B.run_attention(inp, future, output=out, shared=shared)
    torch.cuda.synchronize()
    assert (out[:wl.total_rows].float() == 0).all()
    assert torch.isnan(out[wl.total_rows:].float()).all()


def test_splitk_combine_standalone():
    rng = np.random.default_rng(4)
    np_, Bt, S, H = 5, 3, 4, 6
    offs = np.array([0, 2, 2, 6], dtype=np.int32)
    rcap = Bt * S
    po = rng.standard_normal((np_, rcap, H, 128)).astype(np.float32)
    pl = (rng.standard_normal((np_, rcap, H)) * 3).astype(np.float32)
    pl[1] = -np.inf
    pl[:, 0, 0] = -np.inf                     # a row/head with no positions at all
    out = torch.full((6, H, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    B.msa_splitk_combine(out, torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV),
                         torch.from_numpy(offs).to(DEV), Bt, S, np_, H)
    torch.cuda.synchronize()
    # global rows are keyed on the ragged row: rows 0..5 live at 0..5
    ref = O.splitk_combine(po[:, :6], pl[:, :6])
    parity.check_attention(out, ref, "bf16", "combine")
    assert (out[0, 0].float() == 0).all()


# --- prefill route variants --------------------------------------------------

@pytest.mark.parametrize("G", [1, 2, 4, 16])
def test_prefill_group_sizes(G):
    # tiles of 32 tokens up to G = 8, of 16 at G = 16 (one 16-column MFMA
    # tile per wave)
    run_and_check(wl_custom(f"prefill_g{G}", [40, 100, 9], [0, 3000, 700], G=G, top_k=6),
                  per_seq=30)


@pytest.mark.parametrize("G,kv", [(8, "bf16"), (16, "bf16"), (8, "fp8_e4m3")])
def test_prefill_dense_and_sparse_tiles(G, kv):
    # sequences 0 and 1 see at most top-k blocks (dense-causal tiles, which
    # run on their own kernel at G = 8 and 16), sequence 2 sees 32-34 (sparse
    # tiles); the tiles of the call are split between the two kernels
    run_and_check(wl_custom(f"prefill_dense_mix_g{G}_{kv}", [200, 64, 300], [0, 900, 4000], G=G,
                            top_k=8, kv=kv), per_seq=None)


@pytest.mark.parametrize("G", [8, 16])
def test_prefill_dense_causal_long_unions(G):
    # every token sees 501..504 blocks and chooses them all (top-k 512):
    # dense-causal tiles whose unions refill the kernel's LDS ring of plan
    # entries, on the 8-wave kernel
    run_and_check(wl_custom(f"prefill_dense_long_g{G}", [300], [64000], H_kv=1, G=G,
                            top_k=B.MSA_MAX_TOPK, init=1, local=4), per_seq=4)


def test_prefill_short_context_selection_with_holes():
    # A caller's selection may leave out visible blocks even where top-k
    # covers them all: such tiles are not dense-causal.  Ids in another
    # order and -1 slots; the output must follow the ids given.
    wl = wl_custom("prefill_holes", [150, 90], [100, 600], top_k=8)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    d = B.run_indexer(inp)
    torch.cuda.synchronize()
    d_cpu = d.cpu().numpy().copy()
    rng = np.random.default_rng(5)
    for r in range(d_cpu.shape[0]):
        for h in range(d_cpu.shape[1]):
            row = d_cpu[r, h]
            valid = row[row >= 0]
            if r % 3 == 0 and len(valid) > 1:      # drop one chosen block
                valid = np.delete(valid, rng.integers(len(valid)))
            row[:] = -1
            row[:len(valid)] = rng.permutation(valid)
    d_mod = torch.from_numpy(d_cpu).to(DEV)
    out = B.run_attention(inp, d_mod)
    torch.cuda.synchronize()
    pb, orig_rows = O.problem_for_sequences(inp, list(range(wl.batch)))
    rows = np.arange(len(orig_rows))
    ref = O.attention(pb, d_cpu[orig_rows], rows)
    err = parity.check_attention(out[torch.as_tensor(orig_rows, device=DEV)], ref, wl.kv_dtype,
                                 wl.name)
    say(f"  max|err|={err:.3e}")


def test_prefill_fp8_kv():
    run_and_check(wl_custom("prefill_fp8", [70, 33], [2500, 0], kv="fp8_e4m3", top_k=7, local=3),
                  per_seq=30)


def test_prefill_index_head_per_kv_head_and_no_forced_blocks():
    run_and_check(wl_custom("prefill_ik_per_head", [300, 20], [1000, 5000], H_kv=2, H_ik=2,
                            top_k=5, init=0, local=0), per_seq=40)
    run_and_check(wl_custom("prefill_local_only", [150], [3000], top_k=4, init=0, local=1),
                  per_seq=40)


def test_prefill_tile_edges():
    # lengths around the 32-token tile and the 128-token block
    run_and_check(wl_custom("prefill_edges", [9, 31, 32, 33, 129], [127, 128, 0, 4000, 255],
                            top_k=4), per_seq=None)


# --- FP8 index-K (e4m3 codes + one float32 scale per token) ---------------

def test_fp8_index_k_decode_and_spec():
    run_and_check(wl_custom("ik8_decode", [1, 1, 1], [5000, 300, 9000], ik="fp8_e4m3", boost=0.05))
    run_and_check(wl_custom("ik8_spec", [3, 8, 1, 5], [3000, 2500, 700, 4000], top_k=8,
                            ik="fp8_e4m3"))
    run_and_check(wl_custom("ik8_heads", [1, 4], [4000, 2600], H_kv=4, H_ik=4, init=0, local=0,
                            top_k=3, ik="fp8_e4m3"))


def test_fp8_index_k_prefill():
    run_and_check(wl_custom("ik8_prefill", [200, 45, 300], [1000, 5000, 0], top_k=5,
                            ik="fp8_e4m3"), per_seq=30)
    run_and_check(wl_custom("ik8_prefill_heads", [130, 40], [3000, 9000], H_kv=2, H_ik=2, G=4,
                            top_k=6, ik="fp8_e4m3"), per_seq=30)


def test_fp8_index_k_long_context_full():
    run_and_check(I.decode_fp8_long_fp8ik(), chunk=2)


# --- selection reuse across draft steps ---------------------------------------

def first_row_sources(inp):
    """Each row's source for a reuse step: its sequence's first row."""
    offs = inp.input_row_offsets.cpu().numpy()
    return np.concatenate([np.full(offs[b + 1] - offs[b], offs[b])
                           for b in range(len(offs) - 1)]).astype(np.int32)


def oracle_reused_ids(inp, wl):
    """The oracle's selection of every row, then each row given its
    sequence's first row's ids; with the problem and its global rows."""
    pb, orig = O.problem_for_sequences(inp, list(range(wl.batch)))
    rows = list(range(len(orig)))
    d_ref, _ = O.indexer(pb, rows)
    full = np.full((wl.total_rows, wl.num_kv_heads, wl.top_k), -1, dtype=np.int32)
    full[orig] = d_ref
    return pb, orig, rows, full, full[first_row_sources(inp)]


def test_reuse_gathers_rows_and_feeds_attention():
    # every draft token reuses its sequence's first token's selection; two
    # extra rows name out-of-range sources and must come back empty
    wl = wl_custom("reuse", [3, 8, 1, 5], [6000, 2500, 700, 4000], top_k=8)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    pb, orig, rows, prev, reused = oracle_reused_ids(inp, wl)
    d_prev = torch.from_numpy(prev).to(DEV)
    src_t = torch.from_numpy(first_row_sources(inp)).to(DEV)
    d = torch.empty_like(d_prev)
    B.msa_indexer_reuse(d, d_prev, src_t)
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), reused)
    bad = torch.tensor([-1, d_prev.shape[0]], dtype=torch.int32, device=DEV)
    d_bad = torch.empty((2,) + tuple(d_prev.shape[1:]), dtype=torch.int32, device=DEV)
    B.msa_indexer_reuse(d_bad, d_prev, bad)
    torch.cuda.synchronize()
    assert (d_bad == -1).all()
    # attention on the reused selections, each row with its own causal clip
    out = B.run_attention(inp, d)
    torch.cuda.synchronize()
    ref = O.attention(pb, reused[orig], rows)
    parity.check_attention(out[torch.as_tensor(orig, device=DEV)], ref, wl.kv_dtype, "reuse")


# --- msa_attention_paged_shared: speculative rows sharing one selection -------

@pytest.mark.parametrize("G,kv", [(8, "bf16"), (8, "fp8_e4m3"), (16, "bf16"), (16, "fp8_e4m3"),
                                  (1, "bf16"), (4, "bf16")])
def test_shared_entry_on_reused_selections(G, kv):
    # draft tokens reuse their sequence's first token's blocks; at group size
    # 16 a tile holds 4 tokens, so 5-8 token sequences span a full tile and a
    # ragged one; a 1-token sequence and one inside its first block ride along
    wl = wl_custom(f"shared_G{G}_{kv}", [3, 8, 1, 5, 2, 7], [6000, 2500, 700, 4000, 20, 12000],
                   G=G, top_k=8, kv=kv)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    pb, orig, rows, _, reused = oracle_reused_ids(inp, wl)
    d = torch.from_numpy(reused).to(DEV)
    out = B.run_attention(inp, d, shared=True)
    out_p = B.run_attention(inp, d)
    torch.cuda.synchronize()
    ref = O.attention(pb, reused[orig], rows)
    g = torch.as_tensor(orig, device=DEV)
    err = parity.check_attention(out[g], ref, kv, wl.name)
    err_p = parity.check_attention(out_p[g], ref, kv, wl.name + " msa_attention_paged")
    say(f"  rows={len(rows)} max|err| shared={err:.3e} paged={err_p:.3e}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_e4m3"])
def test_shared_entry_on_fresh_selections(kv):
    # rows of a sequence select different blocks: the union grows, the result
    # is the same operation's
    wl = wl_custom(f"shared_fresh_{kv}", [3, 8, 1, 5], [6000, 2500, 700, 4000], top_k=8, kv=kv,
                   seed=11)
    say(f"[case] {wl.name}")
    inp = I.make_inputs(wl, DEV)
    pb, orig, rows, fresh, _ = oracle_reused_ids(inp, wl)
    out = B.run_attention(inp, torch.from_numpy(fresh).to(DEV), shared=True)
    torch.cuda.synchronize()
    ref = O.attention(pb, fresh[orig], rows)
    err = parity.check_attention(out[torch.as_tensor(orig, device=DEV)], ref, kv, wl.name)
    say(f"  rows={len(rows)} max|err|={err:.3e}")


def test_shared_entry_at_full_spec_size():
    # the speculative workload's shape (batch 32, 2-8 drafts, contexts 8k-64k,
    # top-k 32) as the reuse bench step runs it, every sequence: the first
    # row of each sequence feeds every row of that sequence
    wl = I.spec_decode()
    say(f"[case] {wl.name} shared, reused")
    inp = I.make_inputs(wl, DEV)
    d = torch.full((wl.total_rows, wl.num_kv_heads, wl.top_k), -1, dtype=torch.int32, device=DEV)
    parts = []
    for c0 in range(0, wl.batch, 4):
        seqs = list(range(c0, min(wl.batch, c0 + 4)))
        pb, orig = O.problem_for_sequences(inp, seqs)
        rows = list(range(len(orig)))
        d_ref, _ = O.indexer(pb, rows)
        offs = pb.input_row_offsets
        src = np.concatenate([np.full(offs[b + 1] - offs[b], offs[b]) for b in range(len(seqs))])
        reused = d_ref[src]
        g = torch.as_tensor(orig, device=DEV)
        d[g] = torch.from_numpy(reused).to(DEV)
        parts.append((g, O.attention(pb, reused, rows)))
    out = B.run_attention(inp, d, shared=True)
    torch.cuda.synchronize()
    err = max(parity.check_attention(out[g], ref, wl.kv_dtype, wl.name) for g, ref in parts)
    say(f"  rows={wl.total_rows} max|err|={err:.3e}")
