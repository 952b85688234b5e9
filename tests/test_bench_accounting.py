"""bench.py's accounting, on the CPU.

Every roofline `achieved` figure bench.py prints is the algorithmic work of a
call (bytes or flops, counted from the selections the step made) divided by
the call's duration.  These tests check that count against one taken position
by position from the oracle's definitions (visible blocks, forced blocks, the
positions a block covers, the latent leaves' entries), on reduced copies of
the benchmark workloads with random valid selections; and that bench.py
refuses more than one GPU before it touches any.
"""
import os
import subprocess
import sys
from dataclasses import replace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from block_sparse_attention_indexer_amd import inputs as I  # noqa: E402
from block_sparse_attention_indexer_amd import latent_inputs as LI  # noqa: E402
from oracle import latent_oracle as LO  # noqa: E402
from oracle import msa_oracle as O  # noqa: E402

D = 128


def random_selections(wl, rng, shuffle):
    """[R, H_kv, top_k] ids: for each row and KV head, the forced blocks plus
    a random choice of the others (every visible block when there are no more
    than top_k), padded with -1; in ascending order, or shuffled with the
    padding mixed in (the accounting must not depend on the order)."""
    d = np.full((wl.total_rows, wl.num_kv_heads, wl.top_k), -1, dtype=np.int32)
    r = 0
    for b in range(wl.batch):
        for t in range(wl.new_lens[b]):
            nb = O.visible_blocks(wl.cache_lens[b] + t)
            F = O.forced_blocks(nb, wl.init_blocks, wl.local_blocks)
            for h in range(wl.num_kv_heads):
                if nb <= wl.top_k:
                    ids = list(range(nb))
                else:
                    rest = [x for x in range(nb) if x not in set(F)]
                    ids = sorted(F + rng.choice(rest, wl.top_k - len(F), replace=False).tolist())
                row = np.array(ids + [-1] * (wl.top_k - len(ids)), dtype=np.int32)
                if shuffle:
                    row = rng.permutation(row)
                d[r, h] = row
            r += 1
    return d


def counted_work(wl, d):
    """The same four quantities counted position by position:
    - gathered-KV bytes: per sequence and KV head, every distinct position
      some new token of the sequence attends, K and V, 128 elements each;
    - attention flops: 4 * 128 per (query head, attended position);
    - index-K bytes: per sequence and index-K head, the 128-position tiles of
      the newest token's candidate blocks (visible and not forced), 256 bytes
      per position for BF16 index-K, 128 codes + a float32 scale for FP8;
    - indexer flops: 2 * 128 per (KV head, candidate position) of every
      token that scores (more visible blocks than top_k)."""
    esz = 2 if wl.kv_dtype == "bf16" else 1
    ik_pos = 2 * D if wl.ik_dtype == "bf16" else D + 4
    kv = attn = ik = idx = 0
    r = 0
    for b in range(wl.batch):
        seen = [set() for _ in range(wl.num_kv_heads)]
        nb_last = 0
        for t in range(wl.new_lens[b]):
            p = wl.cache_lens[b] + t
            nb = O.visible_blocks(p)
            nb_last = max(nb_last, nb)
            for h in range(wl.num_kv_heads):
                blocks = [int(x) for x in d[r, h] if x >= 0]
                pos = O.positions_of_blocks(blocks, p)
                seen[h].update(pos.tolist())
                attn += 4 * D * wl.group * len(pos)
            if nb > wl.top_k:
                cand = nb - len(O.forced_blocks(nb, wl.init_blocks, wl.local_blocks))
                idx += 2 * D * wl.num_kv_heads * cand * O.BLOCK
            r += 1
        kv += sum(len(s) for s in seen) * 2 * D * esz
        if nb_last > wl.top_k:
            cand = nb_last - len(O.forced_blocks(nb_last, wl.init_blocks, wl.local_blocks))
            ik += cand * O.BLOCK * ik_pos * wl.num_ik_heads
    return dict(kv_bytes=kv, ik_bytes=ik, attn_flops=attn, idx_flops=idx)


# reduced copies of the benchmark workloads: same head counts, group sizes,
# top-k, forced blocks and storage types, fewer and shorter sequences
SMALL = {
    "decode_small": I.decode_small(),
    "decode_batch64": I.decode_batch64(batch=5, lo=600, hi=5000),
    "spec_decode": I.spec_decode(batch=4, lo=3000, hi=12000),
    "prefill_ragged": I.prefill_ragged(new=(37, 300, 5), cached=(0, 2100, 9000)),
    "decode_fp8_long": I.decode_fp8_long(batch=2, ctx=9000),
    "decode_fp8_long_fp8ik": replace(I.decode_fp8_long(batch=2, ctx=9000), ik_dtype="fp8_e4m3"),
    "spec_index_head_per_kv_head": replace(I.spec_decode(batch=3, lo=3000, hi=12000), num_ik_heads=8),
}


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("shuffle", [False, True])
def test_algorithmic_work_matches_a_position_count(name, shuffle):
    wl = SMALL[name]
    d = random_selections(wl, np.random.default_rng(7), shuffle)
    got = bench.algorithmic_work(wl, d)
    want = counted_work(wl, d)
    assert got == want
    # the workloads exercise what they should: scoring happened, and (in
    # the prefill) tokens of one sequence share blocks
    assert want["ik_bytes"] > 0 and want["kv_bytes"] > 0
    if name == "prefill_ragged":
        assert want["kv_bytes"] < want["attn_flops"] // (4 * D * wl.group) * 2 * D * 2


def test_algorithmic_work_of_a_row_subset():
    # rows= restricts the count to the rows whose ids are given
    wl = SMALL["spec_decode"]
    d = random_selections(wl, np.random.default_rng(3), False)
    offs = np.concatenate([[0], np.cumsum(wl.new_lens)])
    b = 2
    rows = np.arange(offs[b], offs[b + 1])
    one = replace(wl, new_lens=(wl.new_lens[b],), cache_lens=(wl.cache_lens[b],))
    assert bench.algorithmic_work(wl, d[rows], rows=rows) == counted_work(one, d[rows])


@pytest.mark.parametrize("dtypes", [("bf16", "bf16"), ("fp8_e4m3", "fp8_e4m3"), ("bf16", "fp8_e4m3")])
def test_latent_work_matches_the_oracle_entries(dtypes):
    wl = replace(LI.latent_decode(batch=3, heads=16, window=8, top_c=40, lo=300, hi=1200),
                 new_lens=(1, 3, 2), num_latent_heads=2, bad_frac=0.2, dup_frac=0.2,
                 swa_dtype=dtypes[0], comp_dtype=dtypes[1])
    inp = LI.make_latent_inputs(wl, "cpu")
    pb = LO.problem_from_inputs(inp)
    esz = {"bf16": 2, "fp8_e4m3": 1}
    ent = nbytes = 0
    for r in range(wl.total_rows):
        b, _, p = LO.row_position(pb, r)
        for hl in range(wl.num_latent_heads):
            n_swa = len(LO.window_positions(p, wl.window))
            n_comp = len(LO.listed_entries(pb, r, hl, b))
            ent += n_swa + n_comp
            nbytes += D * (n_swa * esz[wl.swa_dtype] + n_comp * esz[wl.comp_dtype])
    got = bench.latent_work(inp)
    assert got["entries"] == ent
    assert got["latent_bytes"] == nbytes
    assert got["flops"] == ent * 4 * D * (wl.num_heads // wl.num_latent_heads)


def test_more_than_one_gpu_is_refused_before_any_device_call():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_counter_rows_are_summed_per_dispatch(tmp_path):
    # rocprofv3 reports a counter once per instance (e.g. per XCD) of a
    # dispatch; the record takes the sum per dispatch, per kernel
    rows = [("copyBuffer", 1, "FETCH_SIZE", 100.0), ("copyBuffer", 1, "FETCH_SIZE", 28.0),
            ("msa::attn_decode_kernel<false>", 2, "FETCH_SIZE", 5.0),
            ("msa::attn_decode_kernel<false>", 2, "FETCH_SIZE", 7.0),
            ("msa::attn_decode_kernel<false>", 3, "FETCH_SIZE", 11.0),
            ("msa::attn_decode_kernel<false>", 3, "WRITE_SIZE", 99.0)]
    path = tmp_path / "run_counter_collection.csv"
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for k, d, c, v in rows:
            f.write(f'{d},"{k}",{c},{v}\n')
    per = bench._counter_per_dispatch(str(path), "FETCH_SIZE")
    assert per == {"copyBuffer": [128.0], "msa::attn_decode_kernel<false>": [12.0, 11.0]}
    assert bench._counter_per_dispatch(str(path), "WRITE_SIZE") == {"msa::attn_decode_kernel<false>": [99.0]}


def test_call_counter_sums_every_instance_of_the_call_kernel():
    # the prefill route launches two instances of the union-tile kernel per
    # call (dense-causal tiles, then the rest) besides its plan and schedule
    per = {"copyBuffer": [1000.0],
           "msa::attn_prefill3_kernel<false, 2, 8, false>": [10.0, 12.0],
           "msa::attn_prefill3_kernel<false, 1, 16, false>": [100.0, 102.0],
           "msa::prefill_plan_kernel": [1.0, 3.0], "msa::attn_schedule_kernel": [2.0, 2.0]}
    assert bench.call_counter_kib(per, "prefill_ragged") == (11.0 + 101.0 + 2.0 + 2.0, 4, 4.0)
    per = {"msa::attn_decode_kernel<true>": [5.0, 7.0], "copyBuffer": [1.0]}
    assert bench.call_counter_kib(per, "decode_fp8_long") == (6.0, 2, 0.0)


def traffic_records():
    out = []
    for f in sorted(os.listdir(bench.PROFILES)):
        if f.endswith("_traffic.json"):
            out.append(f)
    return out


@pytest.mark.parametrize("fname", traffic_records())
def test_traffic_records_are_consistent(fname, monkeypatch):
    """A committed record's HBM bytes are its two counters (KiB per launch)
    scaled by the calibration copy's readings, and bench.py uses the record
    only while the kernel sources hash to the value stored in it."""
    import json
    rec = json.load(open(os.path.join(bench.PROFILES, fname)))
    cal = rec["calibration"]
    hbm = (rec["fetch_size_kib_per_launch"] * 1024 * cal["fetch_scale"] +
           rec["write_size_kib_per_launch"] * 1024 * cal["write_scale"])
    assert abs(rec["hbm_bytes_per_launch"] - hbm) <= 1
    assert rec["hbm_over_algorithmic"] == pytest.approx(
        rec["hbm_bytes_per_launch"] / rec["algorithmic_gathered_kv_bytes_per_launch"], rel=1e-6)
    # the calibration: a 1 GiB copy reads FETCH_SIZE KiB and writes WRITE_SIZE KiB
    assert 0.5 <= cal["fetch_scale"] <= 4 and 0.5 <= cal["write_scale"] <= 4
    kernel = fname.split("_traffic.json")[0]
    workload = next(w for w in list(I.WORKLOADS) + ["spec_decode_reuse", "latent_decode", "latent_decode_fp8"]
                    if kernel.endswith("_" + w) and kernel[:-len(w) - 1] == bench.kernel_of(w))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w=workload: rec["kernel_source_sha256_16"])
    assert bench.traffic_record(workload) == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w=workload: "0" * 16)
    assert bench.traffic_record(workload) is None
