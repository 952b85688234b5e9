#!/usr/bin/env python3
"""Benchmark of the block-sparse paged attention hot path on one MI355X.

One step = the whole path over one batch of synthetic inputs already resident
in HBM: msa_indexer_paged (block-max scoring + top-k) then
msa_attention_paged (sparse attention, plus the split-K combine when the row
is split).  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Default: the top-level fields are decode, batch 64, 8 KV heads x GQA 8,
context lengths uniform in [4096, 32768], top-k 16 (init 1, local 2), BF16
KV.  Its metric is the gathered-KV bytes the step must move divided by the
step time (GB/s), with query tokens per second beside it.  The same line's
"workloads" object holds every other workload measured in the same process
with the same step count (the small decode, speculative decode, the ragged
prefill -- which reports attention TFLOP/s -- and its dense-causal and
sparse sequences on their own, the FP8 128k decode, and the FP8 index-K,
selection-reuse and latent variants), each with its own
roofline objects and a shorter oracle baseline.

Timing: W untimed warmup steps, then exactly K steps bracketed by a device
synchronize and two HIP events on the launch stream, with nothing else
enqueued between them; value and ms_per_step come from the host wall clock
over those K steps.

Roofline: the dominant kernel is the sparse-attention kernel.  Its duration
is one attention call as the library enqueues it (the kernel, plus the
split-K combine when the row is split), measured live with HIP events on the
launch stream around each call of K more steps run after the timed region
(so each call sees the caches as a step leaves them); achieved = algorithmic
bytes (or flops) of one call / that duration.  The same steps time the
indexer call against its own roof (indexer_roofline).  cold_cache_ms adds
the median of single calls after a 512 MiB read sweep of L2 and the
last-level cache.

Latent workloads (--workload latent_decode, latent_decode_fp8): one step is
one msa_latent_attention_paged call; the metric is the latent bytes it must
gather (window positions and valid listed entries, 256 bytes each in BF16,
128 in FP8) per second.  The steps rotate over input sets of the same shape with different
data, so that the data of consecutive steps does not stay in the GPU's
last-level cache.

CPU baseline: the oracle (plain NumPy, as written -- not tuned) timed on the
host cores on a bounded sample of the same workload's rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="decode_small | decode_batch64 | spec_decode | prefill_ragged | "
                         "decode_fp8_long | decode_fp8_long_fp8ik | spec_decode_reuse | "
                         "latent_decode | latent_decode_fp8 | all (one line each).  Default: "
                         "one line for decode_batch64 whose 'workloads' object holds every "
                         "other workload, measured in the same process")
    ap.add_argument("--other-cpu-seconds", type=float, default=2.0,
                    help="oracle budget of each workload inside the default line's 'workloads'")
    ap.add_argument("--other-cold-runs", type=int, default=5,
                    help="cold-cache runs of each workload inside the default line's 'workloads'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle work to sample for the CPU baseline")
    ap.add_argument("--partitions", type=int, default=0, help="split-K partitions (0 = auto)")
    ap.add_argument("--cold-runs", type=int, default=30,
                    help="runs of the cold-cache per-call timing (median reported)")
    ap.add_argument("--entry", choices=("auto", "paged"), default="auto",
                    help="attention entry point of a reuse step: auto = msa_attention_paged_shared, "
                         "paged = msa_attention_paged (for comparison)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (a kernel of known "
                         "traffic, to scale FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="instead of timing: turn the rocprofv3 counter_collection.csv files of a "
                         "FETCH_SIZE run and a WRITE_SIZE run (both with --copy-calibration) into "
                         "the attention kernel's HBM traffic record for --workload")
    ap.add_argument("--traffic-out", default=None,
                    help="where --traffic-record writes its JSON (default: stdout)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work, counted from the selections the step actually made
# ---------------------------------------------------------------------------

def algorithmic_work(wl, d_idx, rows=None):
    """Gathered-KV bytes (union over a sequence's new tokens per KV head),
    index-K bytes (non-forced candidate positions, once per sequence and
    index-K head), attention flops (4 * D per (query head, position)) and
    indexer flops (2 * D per (index head, candidate position)).  d_idx[i]
    belongs to rows[i] (all rows in order when rows is None)."""
    esz = 1 if wl.kv_dtype != "bf16" else 2
    offs = np.concatenate([[0], np.cumsum(wl.new_lens)])
    rows = np.arange(wl.total_rows) if rows is None else np.asarray(rows)
    kv_bytes = ik_bytes = attn_flops = idx_flops = 0
    for b in range(wl.batch):
        sel = np.nonzero((rows >= offs[b]) & (rows < offs[b + 1]))[0]
        if sel.size == 0:
            continue
        p = wl.cache_lens[b] + (rows[sel] - offs[b])
        nb = p // 128 + 1
        ids = d_idx[sel]                                  # [n, H_kv, top_k]
        vis = np.where(ids >= 0, np.clip(p[:, None, None] - 128 * ids + 1, 0, 128), 0)
        attn_flops += 4 * 128 * wl.group * int(vis.sum())
        nbl = int(nb.max())
        for h in range(wl.num_kv_heads):
            cov = np.zeros(nbl + 1, dtype=np.int64)
            m = ids[:, h] >= 0
            np.maximum.at(cov, np.clip(ids[:, h][m], 0, nbl), vis[:, h][m])
            kv_bytes += int(cov.sum()) * 128 * 2 * esz
        if nbl > wl.top_k:
            # bytes per index-K position: 128 BF16 values, or 128 e4m3 codes
            # plus a float32 scale
            ik_pos = 132 if wl.ik_dtype == "fp8_e4m3" else 256
            ik_bytes += max(0, nbl - wl.local_blocks - wl.init_blocks) * 128 * ik_pos * wl.num_ik_heads
            k = np.where(nb > wl.top_k, nb - wl.local_blocks - wl.init_blocks, 0)
            idx_flops += 2 * 128 * wl.num_kv_heads * 128 * int(k.sum())
    return dict(kv_bytes=kv_bytes, ik_bytes=ik_bytes, attn_flops=attn_flops, idx_flops=idx_flops)


def latent_work(inp):
    """Latent bytes one call must gather: for every row and latent head, its
    window positions plus its listed entries inside the compressed leaf (each
    occurrence), 256 bytes each for a BF16 leaf and 128 for an FP8 e4m3 leaf
    (one vector of 128); and flops, 4 * 128 per (query head, entry)."""
    wl = inp.wl
    offs = inp.input_row_offsets.cpu().numpy()
    swa_c = inp.swa_cache_lengths.cpu().numpy()
    comp_c = inp.comp_cache_lengths.cpu().numpy()
    lists = inp.comp_indices.cpu().numpy()
    ent = nbytes = 0
    esz = {"bf16": 2, "fp8_e4m3": 1}
    for b in range(wl.batch):
        for r in range(offs[b], offs[b + 1]):
            p = int(swa_c[b]) + (r - offs[b])
            n_swa = min(wl.window, p + 1) if wl.window > 0 else 0
            lst = lists[r]
            n_comp = int(((lst >= 0) & (lst < comp_c[b])).sum())
            ent += wl.num_latent_heads * n_swa + n_comp
            nbytes += 128 * (wl.num_latent_heads * n_swa * esz[wl.swa_dtype] +
                             n_comp * esz[wl.comp_dtype])
    return {"entries": ent, "latent_bytes": nbytes,
            "flops": ent * 4 * 128 * (wl.num_heads // wl.num_latent_heads)}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of rows
# ---------------------------------------------------------------------------

def cpu_baseline(inp, wl, prefill, seconds):
    """The oracle, as written, on the host cores: a first pass over every
    sequence (all of its rows for decode, 16 sampled rows per sequence for
    prefill), then, while the time budget lasts, more of the same work:
    further passes over the same rows for decode, further distinct sampled
    rows for prefill.  Only the oracle's selection + attention is timed."""
    from oracle import msa_oracle as O
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:  # pragma: no cover - reporting only
        threads = 1
    order = [int(b) for b in np.random.default_rng(0).permutation(wl.batch)]
    offs = inp.input_row_offsets.cpu().numpy()
    perms = {b: np.random.default_rng(b).permutation(int(offs[b + 1] - offs[b])) for b in order}
    state = {"spent": 0.0, "rows": 0, "kv": 0, "flops": 0}

    def timed(pb, orig, rows):
        t0 = time.perf_counter()
        d, _ = O.indexer(pb, rows)
        O.attention(pb, d, rows)
        dt = time.perf_counter() - t0
        w = algorithmic_work(wl, d, rows=[int(orig[r]) for r in rows])
        state["spent"] += dt
        state["kv"] += w["kv_bytes"]
        state["flops"] += w["attn_flops"]
        state["rows"] += len(rows)
        return dt

    # pass 1: every sequence once
    for b in order:
        rows = sorted(perms[b][:16].tolist()) if prefill else list(range(len(perms[b])))
        pb, orig = O.problem_for_sequences(inp, [b])
        timed(pb, orig, rows)
    t1 = state["spent"]
    passes = 1
    if t1 < seconds:
        # the rest of the budget, in equal shares per sequence: decode repeats
        # the sequence's rows, prefill takes further distinct sampled rows
        share = (seconds - t1) / len(order)
        for b in order:
            pb, orig = O.problem_for_sequences(inp, [b])
            used, nxt, k = 0.0, 16, 0
            while used < share:
                if prefill:
                    rows = sorted(perms[b][nxt:nxt + 16].tolist())
                    if not rows:
                        break
                    nxt += 16
                else:
                    rows = list(range(len(perms[b])))
                used += timed(pb, orig, rows)
                k += 1
            passes = max(passes, 1 + k)
    extra = (f"up to {16 * passes} sampled rows per sequence, " if prefill
             else f"up to {passes} passes per sequence, ")
    spent = state["spent"]
    if prefill:
        value, unit = state["flops"] / spent / 1e12, "TFLOP/s"
    else:
        value, unit = state["kv"] / spent / 1e9, "GB/s"
    return {"value": value, "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{state['rows']} row evaluations over all {wl.batch} sequences ({extra}"
                      f"{spent:.1f} s of oracle time), selection + attention",
            "query_tok_s": state["rows"] / spent,
            "affinity_cpus": len(os.sched_getaffinity(0)), "os_cpus": os.cpu_count()}


# ---------------------------------------------------------------------------
# the measured step
# ---------------------------------------------------------------------------

def is_latent(workload):
    return workload.startswith("latent")


def is_reuse(workload):
    return workload.endswith("_reuse")


def is_prefill(workload):
    return workload.startswith("prefill")


def kernel_of(workload):
    """The dominant kernel of one attention call: the union-tile kernel on
    the prefill route and for a reuse step (whose msa_attention_paged_shared
    runs its speculative rows through it), else the decode kernel."""
    if is_latent(workload):
        return "latent_attn_kernel"
    return "attn_prefill3_kernel" if is_reuse(workload) or is_prefill(workload) else "attn_decode_kernel"


def call_extra_kernels(workload):
    """The other kernels one attention call launches: the plan and schedule
    kernels of the union-tile route (split-K partials are merged inside the
    attention kernels, so no combine launch)."""
    if is_reuse(workload) or is_prefill(workload):
        return ("prefill_plan_kernel", "attn_schedule_kernel")
    return ()


def reuse_sources(inp):
    """Source row of every row of a reuse step: its sequence's first row."""
    import torch
    offs = inp.input_row_offsets.cpu().numpy()
    src = np.concatenate([np.full(offs[b + 1] - offs[b], offs[b]) for b in range(len(offs) - 1)])
    return torch.from_numpy(src.astype(np.int32)).to(inp.input_row_offsets.device)


def kernel_source_hash(workload="decode_batch64"):
    h = hashlib.sha256()
    if is_latent(workload):
        files = ("msa_latent.hip", "msa_latent.h", "msa_lds.h", "msa_splitk.h", "msa_common.h",
                 "msa_kernels.h")
    elif is_reuse(workload) or is_prefill(workload):
        files = ("msa_prefill.hip", "msa_lds.h", "msa_common.h", "msa_kernels.h")
    else:
        files = ("msa_attention.hip", "msa_splitk.h", "msa_common.h", "msa_kernels.h")
    for f in files:
        h.update(open(os.path.join(ROOT, "block_sparse_attention_indexer_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


FLUSH_BYTES = 512 * 2**20   # more than L2 (8 x 4 MB) plus the 256 MB last-level cache


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence.
    A default event (torch.cuda.Event) releases to system scope when it is
    recorded, which writes back and invalidates the GPU caches between the
    calls it brackets: time that the calls never spend inside a step, and a
    cache state they never meet there.  The functions come from the HIP
    runtime the process has already loaded (torch's, which libmsa shares)."""
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        import ctypes
        rc = self._lib().hipEventRecord(self._ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self._ev:
            self._hip.hipEventDestroy(self._ev)


def cold_call_ms(fn, stream, runs):
    """Median time of one call of `fn` on `stream` (HIP events around it),
    each run preceded, outside the events, by a read of a 512 MiB scratch
    buffer that evicts L2 and the last-level cache.  The sweep reads rather
    than writes: a written sweep leaves up to 256 MB of dirty lines whose
    write-back then lands inside the timed call.  None when runs is 0
    (profiled runs pass --cold-runs 0 so that the trace holds only calls made
    within steps)."""
    import torch
    if runs <= 0:
        return None
    scratch = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    scratch.sum()                 # write-back of the zeroing happens here
    torch.cuda.synchronize()
    times = []
    for i in range(runs):
        scratch.sum()
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del scratch
    return float(np.median(times))


def traffic_record(workload):
    """HBM traffic per launch of the attention kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{kernel_of(workload)}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


COPY_BYTES = 1 << 30     # the --copy-calibration copy reads and writes 1 GiB


def _counter_per_dispatch(path, counter):
    """{kernel name: [counter value per dispatch]} from a counter_collection.csv
    (rows of one dispatch are summed over the instances they are reported for)."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def call_counter_kib(per, workload):
    """One attention call's counter value from {kernel name: [value per
    dispatch]}: the mean per dispatch of every instance of the call's kernel
    (the prefill route runs its dense-causal tiles on a second instance),
    summed, plus the mean of each of the call's other kernels.  Returns
    (per call, dispatches of the kernel, the other kernels' part)."""
    inst = {name: vals for name, vals in per.items() if kernel_of(workload) in name}
    extra = 0.0
    for k in call_extra_kernels(workload):
        vals = [v for name, vs in per.items() if k in name for v in vs]
        extra += float(np.mean(vals)) if vals else 0.0
    total = float(sum(np.mean(vals) for vals in inst.values())) + extra
    return total, sum(len(v) for v in inst.values()), extra


def write_traffic_record(args):
    """HBM bytes per launch of the attention kernel: FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch) scaled by what the same counters read for the 1 GiB
    calibration copy, next to the algorithmic gathered-KV bytes of the launch."""
    import torch

    from block_sparse_attention_indexer_amd import binding as B
    from block_sparse_attention_indexer_amd import inputs as I

    fetch_csv, write_csv = args.traffic_record
    scaled = {}
    raw = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        per = _counter_per_dispatch(path, counter)
        copy = max(v for name, vals in per.items() if "copy" in name.lower() for v in vals)
        per_call, ndisp, extra = call_counter_kib(per, args.workload)
        if not ndisp:
            raise SystemExit(f"no {kernel_of(args.workload)} dispatch in {path}")
        scale = COPY_BYTES / (copy * 1024.0)
        raw[counter] = (per_call, copy, scale, ndisp, extra)
        scaled[counter] = per_call * 1024.0 * scale

    if is_latent(args.workload):
        from block_sparse_attention_indexer_amd import latent_inputs as LI
        lw = LI.LATENT_WORKLOADS[args.workload]()
        algo = latent_work(LI.make_latent_inputs(lw, "cpu"))["latent_bytes"]
        wl_name = lw.name
    else:
        wl = I.WORKLOADS[args.workload[:-len("_reuse")] if is_reuse(args.workload) else args.workload]()
        inp = I.make_inputs(wl, "cuda")
        d = B.run_indexer(inp)
        if is_reuse(args.workload):
            d = d[reuse_sources(inp).long()]
        torch.cuda.synchronize()
        algo = algorithmic_work(wl, d.cpu().numpy())["kv_bytes"]
        wl_name = wl.name
    hbm = scaled["FETCH_SIZE"] + scaled["WRITE_SIZE"]
    cmd = ("rocprofv3 --pmc {c} --kernel-include-regex "
           f"'{'|'.join((kernel_of(args.workload),) + call_extra_kernels(args.workload))}|copy|elementwise' "
           "--output-format csv -d $OUT/pmc_{w}_{l} -o run -- python3 $R/bench.py "
           "--workload {w} --steps 2 --warmup 1 --no-cpu-baseline --cold-runs 0 --copy-calibration")
    rec = {
        "kernel": (f"msa::{kernel_of(args.workload)}" if not raw["FETCH_SIZE"][4] else
                   "one attention call: " + " + ".join(
                       f"msa::{k}" for k in (kernel_of(args.workload),) + call_extra_kernels(args.workload))),
        "workload": f"{args.workload} ({wl_name})",
        "fetch_size_kib_per_launch": raw["FETCH_SIZE"][0],
        "write_size_kib_per_launch": raw["WRITE_SIZE"][0],
        "other_kernels_fetch_write_kib_per_launch": [raw["FETCH_SIZE"][4], raw["WRITE_SIZE"][4]],
        "dispatches_averaged": raw["FETCH_SIZE"][3],
        "calibration": {
            "fetch_scale": raw["FETCH_SIZE"][2], "write_scale": raw["WRITE_SIZE"][2],
            "how": (f"the same runs include one plain 1 GiB device-to-device copy (bench.py "
                    f"--copy-calibration): FETCH_SIZE reads {raw['FETCH_SIZE'][1]:.0f} KiB and "
                    f"WRITE_SIZE {raw['WRITE_SIZE'][1]:.0f} KiB for 1048576 KiB moved each way"),
        },
        "hbm_bytes_per_launch": int(round(hbm)),
        "algorithmic_gathered_kv_bytes_per_launch": int(algo),
        "hbm_over_algorithmic": hbm / algo if algo else None,
        "kernel_source_sha256_16": kernel_source_hash(args.workload),
        "commands": [cmd.format(c="FETCH_SIZE", w=args.workload, l="fetch"),
                     cmd.format(c="WRITE_SIZE", w=args.workload, l="write"),
                     f"python3 $R/bench.py --workload {args.workload} --traffic-record "
                     f"$OUT/pmc_{args.workload}_fetch/run_counter_collection.csv "
                     f"$OUT/pmc_{args.workload}_write/run_counter_collection.csv"],
        "note": ("counter runs on an MI355X from /tmp with TMPDIR=/tmp; $R is the repository "
                 "root and $OUT the directory the counter files go to. HBM bytes beyond the algorithmic gathered-KV bytes are q, the block ids, "
                 "page-table entries, the output (and split-K partials when the row is split), "
                 "the unused rows of partly filled blocks and blocks that several token groups "
                 "of one sequence load separately."),
    }
    if is_prefill(args.workload):
        # q in and the output out: rows x query heads x 128 dims of BF16 each
        qo = 2 * wl.total_rows * wl.num_q_heads * 128 * 2
        rec["algorithmic_q_and_output_bytes_per_launch"] = int(qo)
        rec["hbm_over_algorithmic_with_q_and_output"] = hbm / (algo + qo)
        rec["note"] += (" On the prefill route q and the output (rows x query heads x 256 B "
                        "each) dominate the call's own HBM bytes; the union blocks every tile "
                        "stages into LDS come from L2 and the last-level cache, not HBM.")
    text = json.dumps(rec, indent=2) + "\n"
    if args.traffic_out:
        open(args.traffic_out, "w").write(text)
    else:
        sys.stdout.write(text)


def run(workload, args):
    import torch

    from block_sparse_attention_indexer_amd import binding as B
    from block_sparse_attention_indexer_amd import inputs as I

    # "<workload>_reuse": a draft step that reuses an earlier step's block
    # selection (each row takes its sequence's first row's ids) instead of
    # running the indexer
    reuse = is_reuse(workload)
    wl = I.WORKLOADS[workload[:-len("_reuse")] if reuse else workload]()
    # the reuse step's rows of a sequence share one selection: the shared entry
    # point reads each sequence's blocks once for all of its tokens
    shared = reuse and args.entry != "paged"
    prefill = wl.max_seq_length > 8
    inp = I.make_inputs(wl, "cuda")
    rg = B.ragged_of_inputs(inp)
    stream = torch.cuda.current_stream()
    d = torch.empty((wl.total_rows, wl.num_kv_heads, wl.top_k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.total_rows, wl.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    np_ = B.msa_attention_partitions(rg, wl.num_q_heads, wl.num_kv_heads, wl.top_k, args.partitions)
    ws_i = torch.empty(max(1, B.msa_indexer_workspace_bytes(rg, wl.num_kv_heads, wl.top_k)),
                       dtype=torch.uint8, device="cuda")
    ws_a = torch.empty(max(1, B.msa_attention_workspace_bytes(rg, wl.num_q_heads, wl.num_kv_heads,
                                                              wl.top_k, np_)),
                       dtype=torch.uint8, device="cuda")

    def indexer():
        B.msa_indexer_paged(d, inp.q_idx, inp.index_k, rg, wl.num_kv_heads, wl.top_k,
                            wl.init_blocks, wl.local_blocks, ws_i, stream,
                            index_k_scale=inp.index_k_scale)

    if reuse:
        indexer()
        d_prev = d.clone()
        src = reuse_sources(inp)

        def indexer():      # noqa: F811 - the draft step's selection
            B.msa_indexer_reuse(d, d_prev, src, stream)

    attention_entry = B.msa_attention_paged_shared if shared else B.msa_attention_paged

    def attention():
        attention_entry(out, inp.q, d, inp.k_cache, inp.v_cache, rg, wl.num_q_heads,
                        wl.num_kv_heads, wl.top_k, wl.softmax_scale, np_, ws_a, stream)

    for _ in range(args.warmup):
        indexer()
        attention()
    torch.cuda.synchronize()
    K = args.steps

    # The timed region: K whole steps, nothing else on the stream.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(K):
        indexer()
        attention()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_step_ms = t_start.elapsed_time(t_end) / K

    # Per-call averages in the step's own context: K more steps after the
    # timed region, with timing-only HIP events (no cache write-back at
    # record) around each call on the launch stream (kept out of the timed
    # region, where they would add gaps).  Repeating one call alone would let
    # its data stay in the 256 MB last-level cache (the FP8 128k attention
    # reads 268 MB), which never happens within a step, where the other
    # call's reads evict it.
    ev = [[TimingEvent() for _ in range(3)] for _ in range(K)]
    for e in ev:
        e[0].record(stream)
        indexer()
        e[1].record(stream)
        attention()
        e[2].record(stream)
    torch.cuda.synchronize()
    idx_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    att_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K

    cold = {"indexer_call": cold_call_ms(indexer, stream, args.cold_runs),
            "attention_call": cold_call_ms(attention, stream, args.cold_runs),
            "runs": args.cold_runs, "flush": f"{FLUSH_BYTES >> 20} MiB read", "statistic": "median"}

    # Split-K partials are merged inside the attention kernel (no combine
    # launch), so the attention call is the attention kernel.
    work = algorithmic_work(wl, d.cpu().numpy())
    if reuse:
        # the reused selection reads no index-K and scores nothing
        work["ik_bytes"] = work["idx_flops"] = 0
    ms = wall / K * 1e3
    tok_s = wl.total_rows / (wall / K)
    # The roofline's duration is one attention call: the attention kernel
    # alone on the decode routes (split-K partials are merged inside it); on
    # the prefill route it also holds the plan and schedule launches.
    if prefill:
        metric_value = work["attn_flops"] / (wall / K) / 1e12
        unit = "TFLOP/s"
        achieved = work["attn_flops"] / (att_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                "traffic": traffic_record(workload),
                "kernel": "prefill attention call: prefill_plan_kernel + attn_schedule_kernel + "
                          "attn_prefill3_kernel"}
    else:
        metric_value = work["kv_bytes"] / (wall / K) / 1e9
        unit = "GB/s"
        achieved = work["kv_bytes"] / (att_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS,
                "traffic": traffic_record(workload) if shared == reuse else None,
                "kernel": ("attention call (msa_attention_paged_shared): prefill_plan_kernel + "
                           "attn_schedule_kernel + attn_prefill3_kernel (4 waves)") if shared else
                          "attn_decode_kernel" if np_ == 1 else
                          "attn_decode_kernel (split-K, partials merged in-kernel)"}
    # The indexer call (scorer + top-k) against its own roof: index-K bytes
    # over HBM peak on the decode routes, scoring flops over BF16 MFMA peak
    # on the prefill route.  A reuse step runs no indexer, and rows that see
    # no more than top_k blocks score nothing.
    if reuse or idx_ms <= 0 or (work["ik_bytes"] == 0 and work["idx_flops"] == 0):
        idx_roof = None
    elif prefill:
        a_idx = work["idx_flops"] / (idx_ms * 1e-3) / 1e12
        idx_roof = {"bound": "mfma", "achieved": a_idx, "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": a_idx / BF16_MFMA_PEAK_TFLOPS,
                    "call": "indexer_schedule_kernel + indexer_score_prefill_kernel + topk_kernel"}
    else:
        a_idx = work["ik_bytes"] / (idx_ms * 1e-3) / 1e9
        idx_roof = {"bound": "hbm", "achieved": a_idx, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": a_idx / HBM_PEAK_GBPS, "call": "indexer_score_kernel + topk_kernel"}
    res = {
        "metric": "decode gathered-KV GB/s (% HBM peak) + query tok/s; prefill TFLOP/s (% MFMA)",
        "value": metric_value, "unit": unit, "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if wl.kv_dtype == "bf16" else "fp8_e4m3 kv / bf16",
        "data": "synthetic",
        "config": {"workload": wl.name + (" draft step, top-k reused from each sequence's first "
                                          "draft token" if reuse else ""),
                   "batch": wl.batch, "new_tokens": wl.total_rows,
                   "max_context": max(wl.seq_lens()), "kv_heads": wl.num_kv_heads,
                   "gqa": wl.group, "top_k": wl.top_k, "init_blocks": wl.init_blocks,
                   "local_blocks": wl.local_blocks, "kv_dtype": wl.kv_dtype,
                   "index_k_heads": wl.num_ik_heads, "index_k_dtype": wl.ik_dtype,
                   "split_k_partitions": 1 if shared else np_,
                   "attention_entry": attention_entry.__name__},
        "query_tok_s": tok_s,
        "hbm_frac_of_step": (work["kv_bytes"] + work["ik_bytes"]) / (wall / K) / 1e9 / HBM_PEAK_GBPS,
        "gpu_ms_per_step": gpu_step_ms,
        "kernels_ms": {"indexer_call": idx_ms, "attention_call": att_ms},
        "algorithmic": work,
        "roofline": roof,
        "indexer_roofline": idx_roof,
        "cold_cache_ms": cold,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, wl, prefill, args.cpu_seconds)
    return res


def run_latent(workload, args):
    import torch
    from dataclasses import replace

    from block_sparse_attention_indexer_amd import binding as B
    from block_sparse_attention_indexer_amd import latent_inputs as LI

    wl = LI.LATENT_WORKLOADS[workload]()
    first = LI.make_latent_inputs(wl, "cuda")
    work = latent_work(first)
    # enough input sets of the same shape (different data and lists) that the
    # data the rotating steps read spans more than twice the 256 MB last-level
    # cache
    nsets = max(1, -(-2 * 256 * 2**20 // work["latent_bytes"]))
    sets = [first] + [LI.make_latent_inputs(replace(wl, seed=wl.seed + 1000 + k), "cuda")
                      for k in range(1, nsets)]
    stream = torch.cuda.current_stream()
    np_ = B.msa_latent_partitions(wl.batch, wl.max_seq_length, wl.num_heads, wl.num_latent_heads,
                                  wl.window, wl.top_c, args.partitions)
    ws = torch.empty(max(1, B.msa_latent_workspace_bytes(wl.batch, wl.max_seq_length, wl.num_heads,
                                                         wl.num_latent_heads, wl.window, wl.top_c,
                                                         np_)), dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.total_rows, wl.num_heads, 128), dtype=torch.bfloat16, device="cuda")
    leaves = [B.latent_leaves_of_inputs(inp) for inp in sets]

    def step(k):
        inp = sets[k % nsets]
        swa, comp = leaves[k % nsets]
        B.msa_latent_attention_paged(out, inp.q, inp.input_row_offsets, wl.batch,
                                     wl.max_seq_length, inp.comp_indices, inp.attn_sink, swa, comp,
                                     wl.num_heads, wl.num_latent_heads, wl.window, wl.softmax_scale,
                                     np_, ws, stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for k in range(K):
        step(k)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = t_start.elapsed_time(t_end) / K
    ms = wall / K * 1e3
    value = work["latent_bytes"] / (wall / K) / 1e9
    # the roofline's duration: one call as the library enqueues it (kernel +
    # split-K combine), from the events around the timed steps
    achieved = work["latent_bytes"] / (gpu_ms * 1e-3) / 1e9
    cold = {"latent_call": cold_call_ms(lambda: step(0), stream, args.cold_runs),
            "runs": args.cold_runs, "flush": f"{FLUSH_BYTES >> 20} MiB read", "statistic": "median"}
    res = {
        "metric": "decode gathered-KV GB/s (% HBM peak) + query tok/s; prefill TFLOP/s (% MFMA)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + " (latent sparse attention: shared K=V latent, window "
                                         "leaf + compressed leaf by per-token entry list, "
                                         "per-head sink)",
                   "batch": wl.batch, "new_tokens": wl.total_rows, "query_heads": wl.num_heads,
                   "latent_heads": wl.num_latent_heads, "head_dim": 128, "window": wl.window,
                   "top_c": wl.top_c, "context": [min(wl.swa_cache_lens) + 1, max(wl.swa_cache_lens) + 1],
                   "compressed_leaf_entries": [min(wl.comp_lens), max(wl.comp_lens)],
                   "leaf_dtype": wl.swa_dtype, "split_k_partitions": np_,
                   "input_sets_rotated": nsets},
        "query_tok_s": wl.total_rows / (wall / K),
        "gpu_ms_per_step": gpu_ms,
        "algorithmic": work,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_record(workload),
                     "kernel": "latent call: latent_attn_kernel" +
                               (" (split-K, partials merged in-kernel)" if np_ > 1 else "")},
        "cold_cache_ms": cold,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = latent_cpu_baseline(first, args.cpu_seconds)
    return res


def latent_cpu_baseline(inp, seconds):
    """The latent oracle, as written, on the host cores: every sequence's rows
    once, then further passes over them while the time budget lasts (only the
    oracle's attention is timed, not the host copies of its inputs)."""
    from oracle import latent_oracle as LO
    try:
        import threadpoolctl
        threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                      if i.get("user_api") == "blas")
    except Exception:  # pragma: no cover - reporting only
        threads = 1
    wl = inp.wl
    esz = {"bf16": 2, "fp8_e4m3": 1}
    offs = inp.input_row_offsets.cpu().numpy()
    probs = []
    for b in range(wl.batch):
        pb, orig = LO.problem_for_sequences(inp, [b], list(range(offs[b], offs[b + 1])))
        nb = 0
        for r in range(len(orig)):
            bb, _, p = LO.row_position(pb, r)
            nb += 128 * sum(esz[wl.swa_dtype] * len(LO.window_positions(p, pb.window)) +
                            esz[wl.comp_dtype] * len(LO.listed_entries(pb, r, hl, bb))
                            for hl in range(pb.num_latent_heads))
        probs.append((pb, len(orig), nb))
    spent, nbytes, rows, passes = 0.0, 0, 0, 0
    while spent < seconds:
        for pb, n, nb in probs:
            t0 = time.perf_counter()
            LO.latent_attention(pb, range(n))
            spent += time.perf_counter() - t0
            nbytes += nb
            rows += n
        passes += 1
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} passes over all {wl.batch} sequences' rows ({rows} row evaluations, "
                      f"{spent:.1f} s of oracle time)",
            "query_tok_s": rows / spent,
            "affinity_cpus": len(os.sched_getaffinity(0)), "os_cpus": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        sys.stderr.write("bench.py measures one GPU only: there is no multi-GPU path; "
                         "run with --gpus 1\n")
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.traffic_record:
        args.workload = args.workload or "decode_batch64"
        write_traffic_record(args)
        return
    everything = ["decode_small", "decode_batch64", "spec_decode", "prefill_ragged",
                  "prefill_ragged_dense", "prefill_ragged_sparse", "decode_fp8_long", "decode_fp8_long_fp8ik", "spec_decode_reuse", "latent_decode",
                  "latent_decode_fp8"]

    def one(name, a):
        res = run_latent(name, a) if is_latent(name) else run(name, a)
        torch.cuda.empty_cache()
        return res

    if args.workload is None:
        # the headline workload, then every other one in the same process
        # (shorter oracle and cold-cache budgets), folded into one line
        head = one("decode_batch64", args)
        sub = argparse.Namespace(**{**vars(args), "cpu_seconds": args.other_cpu_seconds,
                                    "cold_runs": args.other_cold_runs})
        others = {}
        for name in everything:
            if name == "decode_batch64":
                continue
            r = one(name, sub)
            others[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "query_tok_s",
                                              "gpu_ms_per_step", "dtype", "config", "kernels_ms",
                                              "roofline", "indexer_roofline", "algorithmic",
                                              "cold_cache_ms", "cpu_baseline") if k in r}
            sys.stderr.write(f"{name}: {r['value']:.1f} {r['unit']}, {r['ms_per_step']:.4f} ms/step, "
                             f"roofline frac {r['roofline']['frac']:.3f}\n")
        head["workloads"] = others
        print(json.dumps(head), flush=True)
    else:
        names = everything if args.workload == "all" else [args.workload]
        for name in names:
            print(json.dumps(one(name, args)), flush=True)
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")    # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        sys.stderr.write(f"copy calibration: {src.numel() * 4} bytes read and written\n")


if __name__ == "__main__":
    main()
