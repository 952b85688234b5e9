"""HIP graph capture of a whole step (indexer + attention) through the C ABI.

Launch shapes depend only on host-side bounds and the library records no
memset or allocation, so a captured step must replay with the inputs current
at replay time.  Each case captures once, then replays several times with new
queries written eagerly between replays, and requires every replay to match
an eager step on the same inputs bit for bit (the kernels are deterministic:
every output element is produced by one fixed sequence of operations).
"""
import pytest
import torch

from block_sparse_attention_indexer_amd import binding as B
from block_sparse_attention_indexer_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _wl(name, new, cached, H_kv=2, G=8, top_k=6, kv="bf16"):
    return I.Workload(name, new_lens=tuple(new), cache_lens=tuple(cached), num_kv_heads=H_kv,
                      group=G, top_k=top_k, init_blocks=1, local_blocks=2, kv_dtype=kv,
                      kv_sigma=0.5 if kv != "bf16" else 1.0, seed=21)


# (problem, requested partitions, attention entry point)
CASES = {
    "decode_split": (_wl("g_decode", [1, 1, 1, 1], [9000, 3000, 130, 20000]), 3, False),
    "spec": (_wl("g_spec", [3, 8, 1, 5], [6000, 2500, 700, 4000], top_k=8), 0, False),
    "spec_shared": (_wl("g_spec_shared", [3, 8, 1, 5], [6000, 2500, 700, 4000], top_k=8), 0, True),
    "prefill": (_wl("g_prefill", [200, 45, 300], [1000, 5000, 0], top_k=5), 0, False),
    "prefill_fp8": (_wl("g_prefill8", [100, 70], [3000, 600], top_k=5, kv="fp8_e4m3"), 0, False),
}


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_matches_eager(case):
    wl, np_req, shared = CASES[case]
    attention = B.msa_attention_paged_shared if shared else B.msa_attention_paged
    print(f"[case] graph {case}", flush=True)
    inp = I.make_inputs(wl, DEV)
    rg = B.ragged_of_inputs(inp)
    np_ = B.msa_attention_partitions(rg, wl.num_q_heads, wl.num_kv_heads, wl.top_k, np_req)
    ws_i = torch.empty(max(1, B.msa_indexer_workspace_bytes(rg, wl.num_kv_heads, wl.top_k)),
                       dtype=torch.uint8, device=DEV)
    ws_a = torch.empty(max(1, B.msa_attention_workspace_bytes(rg, wl.num_q_heads, wl.num_kv_heads,
                                                              wl.top_k, np_)),
                       dtype=torch.uint8, device=DEV)
    d = torch.empty((wl.total_rows, wl.num_kv_heads, wl.top_k), dtype=torch.int32, device=DEV)
    out = torch.empty((wl.total_rows, wl.num_q_heads, 128), dtype=torch.bfloat16, device=DEV)

    def step(d_buf, out_buf):
        B.msa_indexer_paged(d_buf, inp.q_idx, inp.index_k, rg, wl.num_kv_heads, wl.top_k,
                            wl.init_blocks, wl.local_blocks, ws_i)
        attention(out_buf, inp.q, d_buf, inp.k_cache, inp.v_cache, rg, wl.num_q_heads,
                  wl.num_kv_heads, wl.top_k, wl.softmax_scale, np_, ws_a)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(d, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(d, out)
    torch.cuda.synchronize()

    gen = torch.Generator(device=DEV)
    gen.manual_seed(99)
    d_e = torch.empty_like(d)
    out_e = torch.empty_like(out)
    for rep in range(3):
        inp.q.copy_(torch.randn(inp.q.shape, generator=gen, device=DEV).to(inp.q.dtype))
        inp.q_idx.copy_(torch.randn(inp.q_idx.shape, generator=gen, device=DEV).to(inp.q_idx.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        d_g, out_g = d.clone(), out.clone()
        step(d_e, out_e)
        torch.cuda.synchronize()
        assert torch.equal(d_g, d_e), f"{case} replay {rep}: block ids differ from eager"
        assert torch.equal(out_g.view(torch.int16), out_e.view(torch.int16)), \
            f"{case} replay {rep}: output differs from eager"
        assert torch.isfinite(out_g.float()).all()
    print(f"  {case}: 3 replays identical to eager (np={np_})", flush=True)


@pytest.mark.parametrize("np_req", [1, 3])
def test_latent_graph_replay_matches_eager(np_req):
    """The latent call (and, when split, its combine) captured once and
    replayed with new queries and new entry lists written between replays."""
    from block_sparse_attention_indexer_amd import latent_inputs as LI
    print(f"[case] latent graph np={np_req}", flush=True)
    wl = LI.LatentWorkload("g_latent", new_lens=(1, 3, 2), swa_cache_lens=(900, 4000, 130),
                           comp_lens=(600, 1500, 40), num_heads=64, window=96, top_c=200,
                           sink_mean=1.0, bad_frac=0.05, seed=23)
    inp = LI.make_latent_inputs(wl, DEV)
    swa, comp = B.latent_leaves_of_inputs(inp)
    np_ = B.msa_latent_partitions(wl.batch, wl.max_seq_length, wl.num_heads, 1, wl.window,
                                  wl.top_c, np_req)
    ws = torch.empty(max(1, B.msa_latent_workspace_bytes(wl.batch, wl.max_seq_length, wl.num_heads,
                                                         1, wl.window, wl.top_c, np_)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty((wl.total_rows, wl.num_heads, 128), dtype=torch.bfloat16, device=DEV)

    def step(out_buf):
        B.msa_latent_attention_paged(out_buf, inp.q, inp.input_row_offsets, wl.batch,
                                     wl.max_seq_length, inp.comp_indices, inp.attn_sink, swa, comp,
                                     wl.num_heads, 1, wl.window, wl.softmax_scale, np_, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(out)
    torch.cuda.synchronize()

    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    out_e = torch.empty_like(out)
    offs = inp.input_row_offsets.cpu().tolist()
    for rep in range(3):
        inp.q.copy_(torch.randn(inp.q.shape, generator=gen, device=DEV).to(inp.q.dtype))
        # new lists: valid entries of each sequence's compressed leaf, some -1
        for b in range(wl.batch):
            n = wl.comp_lens[b]
            rows = offs[b + 1] - offs[b]
            lst = torch.randint(-1, max(n, 1), (rows, 1, wl.top_c), generator=gen, device=DEV)
            inp.comp_indices[offs[b]:offs[b + 1]] = lst.to(torch.int32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out_g = out.clone()
        step(out_e)
        torch.cuda.synchronize()
        assert torch.isfinite(out_g.float()).all(), f"replay {rep}"
        assert torch.equal(out_g, out_e), f"replay {rep}: graph output differs from eager"


def test_calls_on_concurrent_streams_match_sequential():
    """Calls keep no state between them: a split-K decode step, a prefill step
    (persistent work list) and a split latent call enqueued on three streams
    at once give, bit for bit, what they give one after another."""
    from block_sparse_attention_indexer_amd import latent_inputs as LI
    print("[case] concurrent streams", flush=True)
    w_dec = _wl("cs_decode", [1, 1, 1, 1], [9000, 3000, 130, 20000])
    w_pre = _wl("cs_prefill", [200, 45, 300], [1000, 5000, 0], top_k=5)
    w_lat = LI.LatentWorkload("cs_latent", new_lens=(1, 3, 2), swa_cache_lens=(900, 4000, 130),
                              comp_lens=(600, 1500, 40), num_heads=64, window=96, top_c=200,
                              sink_mean=1.0, bad_frac=0.05, seed=29)

    def msa_buffers(wl, np_req):
        inp = I.make_inputs(wl, DEV)
        rg = B.ragged_of_inputs(inp)
        np_ = B.msa_attention_partitions(rg, wl.num_q_heads, wl.num_kv_heads, wl.top_k, np_req)
        wsi = torch.empty(max(1, B.msa_indexer_workspace_bytes(rg, wl.num_kv_heads, wl.top_k)),
                          dtype=torch.uint8, device=DEV)
        wsa = torch.empty(max(1, B.msa_attention_workspace_bytes(rg, wl.num_q_heads,
                                                                 wl.num_kv_heads, wl.top_k, np_)),
                          dtype=torch.uint8, device=DEV)
        d = torch.empty((wl.total_rows, wl.num_kv_heads, wl.top_k), dtype=torch.int32, device=DEV)
        out = torch.empty((wl.total_rows, wl.num_q_heads, 128), dtype=torch.bfloat16, device=DEV)

        def step(stream=None):
            B.run_indexer(inp, d_indices=d, workspace=wsi, stream=stream)
            B.run_attention(inp, d, output=out, num_partitions=np_, workspace=wsa, stream=stream)
        return step, (d, out)

    step_dec, res_dec = msa_buffers(w_dec, 3)
    step_pre, res_pre = msa_buffers(w_pre, 0)
    lat = LI.make_latent_inputs(w_lat, DEV)
    np_l = B.msa_latent_partitions(w_lat.batch, w_lat.max_seq_length, w_lat.num_heads, 1,
                                   w_lat.window, w_lat.top_c, 3)
    ws_l = torch.empty(max(1, B.msa_latent_workspace_bytes(w_lat.batch, w_lat.max_seq_length,
                                                           w_lat.num_heads, 1, w_lat.window,
                                                           w_lat.top_c, np_l)),
                       dtype=torch.uint8, device=DEV)
    out_l = torch.empty((w_lat.total_rows, w_lat.num_heads, 128), dtype=torch.bfloat16, device=DEV)

    def step_lat(stream=None):
        B.run_latent(lat, output=out_l, num_partitions=np_l, workspace=ws_l, stream=stream)

    steps = (step_dec, step_pre, step_lat)
    results = (res_dec, res_pre, (out_l,))
    for f in steps:
        f()
    torch.cuda.synchronize()
    ref = [[t.clone() for t in r] for r in results]
    streams = [torch.cuda.Stream() for _ in steps]
    for rep in range(3):
        for r in results:
            for t in r:
                t.fill_(-1 if t.dtype == torch.int32 else float("nan"))
        torch.cuda.synchronize()
        for f, s in zip(steps, streams):
            f(s)
        torch.cuda.synchronize()
        for r, rr in zip(results, ref):
            for t, tt in zip(r, rr):
                a = t.view(torch.int16) if t.dtype == torch.bfloat16 else t
                b = tt.view(torch.int16) if tt.dtype == torch.bfloat16 else tt
                assert torch.equal(a, b), f"rep {rep}: a concurrent call differs from its sequential run"
    print("  3 rounds of concurrent calls identical to sequential ones", flush=True)
