"""msa_attention_paged_noalloc (the entry point for callers that cannot
allocate device memory) against msa_attention_paged: the same kernels on the
same inputs, so the outputs must be bit-identical.  Two calls in a row on
each route, the second with a smaller input, so the second call runs on the
scratch contents the first one left."""
import pytest
import torch

from block_sparse_attention_indexer_amd import binding as B
from block_sparse_attention_indexer_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda"


def wl(name, new, cached, top_k=6, kv="bf16", seed=3):
    return I.Workload(name, new_lens=tuple(new), cache_lens=tuple(cached), num_kv_heads=2, group=8,
                      top_k=top_k, init_blocks=1, local_blocks=2, kv_dtype=kv,
                      kv_sigma=0.5 if kv != "bf16" else 1.0, seed=seed)


def compare(w, num_partitions):
    print(f"[case] {w.name} B={w.batch} np={num_partitions}", flush=True)
    inp = I.make_inputs(w, DEV)
    rg = B.ragged_of_inputs(inp)
    d = B.run_indexer(inp)
    shape = (w.total_rows + 2, w.num_q_heads, 128)
    ref = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    got = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
    args = (inp.q, d, inp.k_cache, inp.v_cache, rg, w.num_q_heads, w.num_kv_heads, w.top_k,
            w.softmax_scale, num_partitions)
    B.msa_attention_paged(ref, *args)
    B.msa_attention_paged_noalloc(got, *args)
    torch.cuda.synchronize()
    n = w.total_rows
    assert torch.isfinite(got[:n].float()).all()
    assert torch.equal(got[:n].view(torch.int16), ref[:n].view(torch.int16))
    assert torch.isnan(got[n:].float()).all()
    need = B.msa_attention_workspace_bytes(rg, w.num_q_heads, w.num_kv_heads, w.top_k,
                                           num_partitions)
    return need


@pytest.mark.parametrize("route", ["decode_split_k", "spec_auto", "prefill", "prefill_fp8"])
def test_noalloc_matches_paged_on_two_calls(route):
    if route == "decode_split_k":
        big = wl("na_decode_big", [1] * 12, [3000 + 700 * i for i in range(12)], top_k=9)
        small = wl("na_decode_small", [1] * 5, [900, 4000, 130, 2500, 6000], top_k=9, seed=4)
        np_ = 4
    elif route == "spec_auto":
        big = wl("na_spec_big", [3, 8, 1, 5, 2], [6000, 2500, 700, 4000, 9000])
        small = wl("na_spec_small", [2, 4], [3000, 1200], seed=5)
        np_ = 0
    elif route == "prefill":
        big = wl("na_prefill_big", [300, 1100, 40], [0, 2048, 5000])
        small = wl("na_prefill_small", [50, 20], [700, 0], seed=6)
        np_ = 0
    else:
        big = wl("na_prefill8_big", [200, 70], [2500, 0], kv="fp8_e4m3")
        small = wl("na_prefill8_small", [33], [900], kv="fp8_e4m3", seed=7)
        np_ = 0
    need_big = compare(big, np_)
    need_small = compare(small, np_)
    assert 0 < need_small <= need_big <= B.MSA_NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_shapes_beyond_its_scratch():
    w = wl("na_too_big", [1] * 4, [3000] * 4)
    inp = I.make_inputs(w, DEV)
    rg = B.ragged_of_inputs(inp)
    rg.batch = 2048                # host bound only: nothing is launched
    out = torch.empty((4, w.num_q_heads, 128), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((4, w.num_kv_heads, w.top_k), dtype=torch.int32, device=DEV)
    with pytest.raises(B.MsaError) as e:
        B.msa_attention_paged_noalloc(out, inp.q, d, inp.k_cache, inp.v_cache, rg, w.num_q_heads,
                                      w.num_kv_heads, w.top_k, w.softmax_scale, 64)
    assert e.value.status == -8
