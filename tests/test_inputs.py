"""The seeded input generator: determinism, shapes, page table, poisoning."""
import numpy as np
import torch

from block_sparse_attention_indexer_amd import inputs as I


def test_workload_shapes():
    wl = I.decode_small()
    assert (wl.batch, wl.num_kv_heads, wl.group, wl.top_k) == (1, 1, 4, 4)
    assert wl.seq_lens() == [2048] and wl.pages_per_seq() == [16]
    wl = I.decode_batch64()
    assert wl.batch == 64 and all(4096 <= L <= 32768 for L in wl.seq_lens())
    wl = I.spec_decode()
    assert all(2 <= n <= 8 for n in wl.new_lens) and all(8192 <= c <= 65536 for c in wl.cache_lens)
    wl = I.prefill_ragged()
    assert wl.total_rows == 29696 and wl.max_seq_length == 16384
    wl = I.decode_fp8_long()
    assert wl.pages_per_seq() == [1024] * 16 and wl.kv_dtype == "fp8_e4m3"


def test_small_inputs_deterministic_and_poisoned():
    wl = I.decode_small()
    a = I.make_inputs(wl, "cpu")
    b = I.make_inputs(wl, "cpu")
    for name in ("q", "q_idx", "index_k", "k_cache", "v_cache", "kv_lookup_table"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.int32 else x,
                           y.view(torch.uint8) if y.dtype != torch.int32 else y)
    table = a.kv_lookup_table[0].numpy()
    assert len(set(table.tolist())) == 16 and table.max() < 32
    assert a.index_k.shape == (33, 1, 128, 128)
    used = set(table.tolist())
    for pg in range(33):
        page = a.k_cache[pg].float()
        assert torch.isnan(page).all().item() == (pg not in used)


def test_partial_last_page_poisoned_and_fp8():
    wl = I.shrink(I.decode_fp8_long(), new_lens=(1, 3), cache_lens=(300, 129),
                  name="fp8_tiny")
    inp = I.make_inputs(wl, "cpu")
    assert inp.k_cache.dtype == torch.float8_e4m3fn
    L = wl.seq_lens()
    for b in range(2):
        last = inp.page_of[b][-1]
        k = inp.k_cache[last].float()
        assert torch.isnan(k[:, L[b] % 128:]).all()
        assert torch.isfinite(k[:, :L[b] % 128]).all()
        assert k[:, :L[b] % 128].abs().max() <= 448


def test_boost_rows_are_exact_multiples():
    wl = I.shrink(I.decode_batch64(batch=2, lo=600, hi=700), boost_frac=0.5, name="boost")
    plain = I.make_inputs(I.shrink(wl, boost_frac=0.0), "cpu").index_k.float()
    boosted = I.make_inputs(wl, "cpu").index_k.float()
    ok = torch.isnan(plain) | (boosted == plain) | (boosted == 4 * plain)
    assert ok.all()
    assert (boosted == 4 * plain).logical_and(plain != 0).any()
