"""The C ABI library: it loads, exports every declared entry point, and its
host-side validation rejects bad arguments before touching any device.
CPU only: none of these calls reaches a kernel launch or a device query."""
import ctypes
import functools
import re

import pytest
import torch

from block_sparse_attention_indexer_amd import binding as B

OK, NULL, SHAPE, PARAM, DTYPE, WORKSPACE = 0, -1, -2, -3, -4, -5
FAKE = 1 << 20        # a 16-byte aligned non-null address that is never dereferenced


def test_library_exports_every_declared_function():
    lib = B.library()
    names = B.header_functions()
    assert {"msa_indexer_paged", "msa_attention_paged", "msa_splitk_combine"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_binding_constants_match_header():
    text = open(B.HEADER).read()
    for name in ("MSA_MAX_SPEC_DRAFT", "MSA_MAX_BLOCKS", "MSA_MAX_TOPK", "MSA_MAX_KV_HEADS",
                 "MSA_DEVERR_PAGE", "MSA_DEVERR_LENGTH", "MSA_DTYPE_BF16",
                 "MSA_DTYPE_FP8_E4M3", "MSA_LATENT_MAX_TOPC"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m, name
        assert int(m.group(1)) == getattr(B, name), name
    m = re.search(r"\bMSA_LATENT_MAX_WINDOW\s*=\s*1\s*<<\s*(\d+)", text)
    assert m and 1 << int(m.group(1)) == B.MSA_LATENT_MAX_WINDOW
    m = re.search(r"\bMSA_NOALLOC_SCRATCH_BYTES\s*=\s*(\d+)\s*\*\s*1024\s*\*\s*1024", text)
    assert m and int(m.group(1)) << 20 == B.MSA_NOALLOC_SCRATCH_BYTES


def rg(batch=2, max_seq=1, max_cache=4000, stride=40, null=False):
    p = None if null else FAKE
    return B.Ragged(p, p, p, stride, batch, max_seq, max_cache)


def cache(dtype=B.MSA_DTYPE_BF16, heads=1, page=128, dim=128, tok=128, data=FAKE):
    return B.PagedCache(data, dtype, 100, heads, page, dim, 0, heads * 128 * tok, 128 * tok, tok)


def indexer(r, c, heads=8, top_k=16, init=1, local=2, ws=0, d=FAKE, q=FAKE):
    return B.library().msa_indexer_paged(d, q, ctypes.byref(c), ctypes.byref(r), heads, top_k, init,
                                         local, FAKE if ws else None, ws, None)


ATTENTION_ENTRIES = ("msa_attention_paged", "msa_attention_paged_shared")


def attention(r, k, v, hq=64, hkv=8, top_k=16, np_=0, ws=0, out=FAKE, scale=0.1,
              entry="msa_attention_paged"):
    return getattr(B.library(), entry)(out, FAKE, FAKE, ctypes.byref(k), ctypes.byref(v),
                                       ctypes.byref(r), hq, hkv, top_k, scale, np_,
                                       FAKE if ws else None, ws, None)


def test_indexer_validation():
    assert indexer(rg(), cache(), d=None) == NULL
    assert indexer(rg(null=True), cache()) == NULL
    assert indexer(rg(), cache(data=None)) == NULL
    assert indexer(rg(), cache(page=64)) == SHAPE
    assert indexer(rg(), cache(dim=64)) == SHAPE
    assert indexer(rg(), cache(heads=3)) == SHAPE
    assert indexer(rg(), cache(tok=100)) == SHAPE            # unaligned stride
    assert indexer(rg(), cache(data=FAKE + 2)) == SHAPE      # unaligned base
    assert indexer(rg(), cache(tok=1 << 23)) == SHAPE        # a page's rows span >= 2 GiB
    assert indexer(rg(), cache(dtype=B.MSA_DTYPE_FP8_E4M3)) == NULL   # FP8 without its scales
    assert indexer(rg(), cache(dtype=7)) == DTYPE
    assert indexer(rg(), cache(), top_k=0) == PARAM
    assert indexer(rg(), cache(), top_k=2, init=2, local=1) == PARAM
    assert indexer(rg(), cache(), init=-1) == PARAM
    assert indexer(rg(max_cache=8192 * 128), cache()) == SHAPE
    assert indexer(rg(), cache()) == NULL                    # scores buffer missing
    assert indexer(rg(batch=0), cache()) == OK               # empty batch: no-op
    need = B.msa_indexer_workspace_bytes(rg(), 8, 16)
    assert need >= 2 * 8 * 32 * 4
    assert indexer(rg(), cache(), ws=need - 1) == WORKSPACE
    assert B.msa_indexer_workspace_bytes(rg(max_cache=1000), 8, 16) == 0   # nb <= top_k


def test_kv_head_count_is_bounded_on_every_route():
    # more than 256 KV heads per index-K head do not fit the prefill scorer's
    # tile: rejected by the size query and the entry points on every route,
    # before any arithmetic on the count
    for max_seq in (1, 4, 64):
        r = rg(max_seq=max_seq)
        assert B.msa_indexer_workspace_bytes(r, 256, 16) > 0
        for heads in (257, 300, 1 << 20):
            assert B.msa_indexer_workspace_bytes(r, heads, 16) == 0
            assert indexer(r, cache(), heads=heads) == SHAPE
            assert indexer(r, cache(heads=heads), heads=heads) == SHAPE
            k, v = cache(heads=heads), cache(heads=heads)
            for entry in ATTENTION_ENTRIES:
                assert attention(r, k, v, hq=heads, hkv=heads, entry=entry) == SHAPE
            assert B.msa_attention_workspace_bytes(r, heads, heads, 16, 0) == 0


def test_index_k_scale_rules():
    # FP8 index-K needs its per-token scales; BF16 index-K and K/V take none
    c8 = cache(dtype=B.MSA_DTYPE_FP8_E4M3)
    assert indexer(rg(), c8) == NULL                                  # scales missing
    c8.scale, c8.scale_page_stride, c8.scale_head_stride = FAKE, 4224, 4224
    assert indexer(rg(), c8) == NULL                                  # passes to the workspace check
    c8.scale = FAKE + 4
    assert indexer(rg(), c8) == SHAPE                                 # unaligned scales
    c8.scale, c8.scale_head_stride = FAKE, 4222
    assert indexer(rg(), c8) == SHAPE                                 # stride not a multiple of 4
    c16 = cache()
    c16.scale = FAKE
    assert indexer(rg(), c16) == DTYPE                                # BF16 index-K with scales
    k, v = cache(heads=8), cache(heads=8)
    k.scale = FAKE
    assert attention(rg(), k, v) == DTYPE                             # K/V are scale-free


def test_binding_describes_the_fp8_index_k_page_layout():
    # 128 x 128 codes then 128 float32 scales per (page, head): 132 B per token
    P, H = 3, 2
    store = torch.zeros((P, H, 128 * 128 + 128 * 4), dtype=torch.uint8)
    codes = store[:, :, :128 * 128].view(torch.float8_e4m3fn).unflatten(2, (128, 128))
    scales = store[:, :, 128 * 128:].view(torch.float32)
    c = B.paged_cache(codes, scales)
    assert c.dtype == B.MSA_DTYPE_FP8_E4M3
    assert (c.page_stride, c.head_stride, c.token_stride) == (H * 16896, 16896, 128)
    assert (c.scale_page_stride, c.scale_head_stride) == (H * 4224, 4224)
    assert c.scale - c.data == 128 * 128


def test_reuse_validation():
    lib = B.library()
    assert lib.msa_indexer_reuse(FAKE, FAKE, FAKE, 0, 0, 8, 16, None) == OK       # no rows
    assert lib.msa_indexer_reuse(None, FAKE, FAKE, 4, 2, 8, 16, None) == NULL
    assert lib.msa_indexer_reuse(FAKE, FAKE, None, 4, 2, 8, 16, None) == NULL
    assert lib.msa_indexer_reuse(FAKE, FAKE, FAKE, -1, 2, 8, 16, None) == PARAM
    assert lib.msa_indexer_reuse(FAKE, FAKE, FAKE, 4, 2, 0, 16, None) == PARAM
    assert lib.msa_indexer_reuse(FAKE, FAKE, FAKE, 4, 2, 8, 0, None) == PARAM
    assert lib.msa_indexer_reuse(FAKE, FAKE, FAKE, 4, 2, 8, 513, None) == PARAM
    assert lib.msa_indexer_reuse(FAKE, FAKE, FAKE, 1 << 20, 2, 64, 512, None) == SHAPE


@pytest.mark.parametrize("entry", ATTENTION_ENTRIES)
def test_attention_validation(entry):
    k = cache(heads=8)
    v = cache(heads=8)
    attention = functools.partial(globals()["attention"], entry=entry)
    assert attention(rg(), k, v, out=None) == NULL
    assert attention(rg(), k, v, hq=60) == SHAPE
    assert attention(rg(), k, v, hq=8 * 32) == SHAPE              # group 32 unsupported
    assert attention(rg(), cache(heads=4), v) == SHAPE
    assert attention(rg(), cache(heads=8, dtype=B.MSA_DTYPE_FP8_E4M3), v) == DTYPE
    assert attention(rg(), k, v, top_k=0) == PARAM
    assert attention(rg(), k, v, np_=65) == PARAM
    assert attention(rg(), k, v, scale=float("nan")) == PARAM
    assert attention(rg(), cache(heads=8, tok=1 << 23), v) == SHAPE   # page span >= 2 GiB
    assert attention(rg(), k, v, scale=0.0) == PARAM
    assert attention(rg(), k, v, scale=-0.1) == PARAM
    assert attention(rg(), k, v, scale=float("inf")) == PARAM
    assert attention(rg(), k, v, np_=4) == NULL                 # partials missing
    need = B.msa_attention_workspace_bytes(rg(), 64, 8, 16, 4)
    assert attention(rg(), k, v, np_=4, ws=need - 1) == WORKSPACE
    assert attention(rg(batch=0), k, v) == OK


def test_device_errors_validation():
    assert B.library().msa_device_errors(None, 1, None) == NULL


def noalloc(r, k, v, hq=64, hkv=8, top_k=16, np_=0, scale=0.1):
    return B.library().msa_attention_paged_noalloc(FAKE, FAKE, FAKE, ctypes.byref(k), ctypes.byref(v),
                                                   ctypes.byref(r), hq, hkv, top_k, scale, np_, None)


def test_noalloc_entry_validation_and_scratch_limit():
    SCRATCH = -8
    k, v = cache(heads=8), cache(heads=8)
    # argument errors are reported as by msa_attention_paged
    assert noalloc(rg(), k, v, top_k=0) == PARAM
    assert noalloc(rg(), k, v, hq=60) == SHAPE
    assert noalloc(rg(), k, v, scale=0.0) == PARAM
    assert noalloc(rg(batch=0), k, v) == OK
    # a shape whose workspace exceeds the fixed array is rejected before any
    # launch or device query (explicit partition count: host-only sizing)
    big = rg(batch=2048, max_seq=1)
    need = B.msa_attention_workspace_bytes(big, 64, 8, 16, 8)
    assert need > B.MSA_NOALLOC_SCRATCH_BYTES
    assert noalloc(big, k, v, np_=8) == SCRATCH
    assert B.status_string(SCRATCH) != "unknown status"
    # the ragged prefill (29,696 tokens, 8 KV heads, top-k 64) fits
    pre = B.Ragged(FAKE, FAKE, FAKE, 256, 4, 16384, 16384)
    assert 0 < B.msa_attention_workspace_bytes(pre, 64, 8, 64, 1) <= B.MSA_NOALLOC_SCRATCH_BYTES


def test_shared_speculative_steps_need_the_union_plan():
    # One partition needs no partials, but the shared entry point's union-tile
    # plan for 2-8 token rows still needs workspace; the query covers both.
    k, v = cache(heads=8), cache(heads=8)
    spec = rg(max_seq=4)
    need = B.msa_attention_workspace_bytes(spec, 64, 8, 16, 1)
    assert need > 0
    assert attention(spec, k, v, np_=1, entry="msa_attention_paged_shared") == NULL
    assert attention(spec, k, v, np_=1, ws=need - 1, entry="msa_attention_paged_shared") == WORKSPACE
    assert attention(spec, k, v, np_=64, ws=need - 1, entry="msa_attention_paged_shared") == WORKSPACE
    # decode rows (one token) take the split-K route under either entry point
    dec = rg(max_seq=1)
    assert B.msa_attention_workspace_bytes(dec, 64, 8, 16, 1) == 0
    # the union plan grows with the sequences' tokens per tile at group size 16
    assert (B.msa_attention_workspace_bytes(rg(max_seq=8), 256, 16, 16, 1)
            > B.msa_attention_workspace_bytes(rg(max_seq=4), 256, 16, 16, 1))


def test_partition_planning_is_host_only():
    r = rg(batch=64, max_seq=1, max_cache=32767)
    assert B.msa_attention_partitions(r, 64, 8, 16, 3) == 3
    assert B.msa_attention_partitions(r, 64, 8, 16, 1) == 1
    pre = rg(batch=4, max_seq=16384, max_cache=16384)
    assert B.msa_attention_partitions(pre, 64, 8, 64, 0) == 1     # prefill never splits
    assert B.msa_attention_workspace_bytes(pre, 64, 8, 64, 0) >= 0
    ws = B.msa_attention_workspace_bytes(r, 64, 8, 16, 4)
    assert ws >= 4 * 64 * 64 * 129 * 4
    with pytest.raises(B.MsaError):
        B.msa_attention_partitions(r, 64, 8, 16, 99)


def test_combine_validation():
    lib = B.library()
    assert lib.msa_splitk_combine(FAKE, FAKE, FAKE, FAKE, 2, 1, 0, 8, None) == PARAM
    assert lib.msa_splitk_combine(None, FAKE, FAKE, FAKE, 2, 1, 2, 8, None) == NULL
    assert lib.msa_splitk_combine(FAKE, FAKE, FAKE, FAKE, 0, 1, 2, 8, None) == OK


def leaf(heads=1, stride=40, max_cache=4000, dtype=B.MSA_DTYPE_BF16, null_table=False, pages=100):
    c = cache(dtype=dtype, heads=heads)
    c.num_pages = pages
    return B.LatentLeaf(c, FAKE, None if null_table else FAKE, stride, max_cache)


def latent(swa, comp, batch=2, max_seq=1, top_c=512, heads=64, lat=1, window=128, np_=2, ws=1 << 30,
           scale=0.1, out=FAKE, lists=FAKE, sink=FAKE):
    return B.library().msa_latent_attention_paged(
        out, FAKE, FAKE, batch, max_seq, lists, top_c, sink,
        None if swa is None else ctypes.byref(swa), None if comp is None else ctypes.byref(comp),
        heads, lat, window, scale, np_, FAKE if ws else None, ws, None)


def test_latent_validation():
    """Every check runs before a device query, so a valid call here would only
    fail at the device lookup (-7) -- each case below fails earlier."""
    s, c = leaf(), leaf(stride=40)
    assert latent(s, c, out=None) == NULL
    assert latent(s, c, sink=None) == NULL
    assert latent(None, c) == NULL                             # window > 0 needs the window leaf
    assert latent(s, None) == NULL                             # a list needs the compressed leaf
    assert latent(s, c, lists=None) == NULL
    assert latent(s, leaf(null_table=True)) == NULL
    assert latent(s, c, heads=60, lat=8) == SHAPE              # not a multiple
    assert latent(s, c, lat=2) == SHAPE                        # leaves hold one latent head
    assert latent(leaf(stride=31), c) == SHAPE                 # table too short for the window leaf
    assert latent(s, leaf(stride=31, max_cache=4000)) == SHAPE
    assert latent(leaf(pages=(1 << 24) + 1), c) == SHAPE
    assert latent(s, c, window=-1) == PARAM
    assert latent(s, c, window=(1 << 20) + 1) == PARAM
    assert latent(s, c, top_c=16385) == PARAM
    assert latent(s, c, np_=65) == PARAM
    assert latent(s, c, scale=0.0) == PARAM
    assert latent(s, c, scale=float("nan")) == PARAM
    assert latent(leaf(dtype=7), c) == DTYPE
    f8 = leaf(dtype=B.MSA_DTYPE_FP8_E4M3)
    # leaves of two types: accepted, and they need the split-K workspace even
    # when one partition is asked for
    assert latent(s, f8, ws=0) == NULL
    assert latent(f8, c, ws=0, np_=1) == NULL
    assert B.msa_latent_workspace_bytes(2, 1, 64, 1, 128, 512, 1) > 0
    # both FP8, or one FP8 leaf with the other not read: passes the type check
    assert latent(f8, leaf(dtype=B.MSA_DTYPE_FP8_E4M3), ws=0) == NULL
    assert latent(f8, None, top_c=0, lists=None, np_=1, ws=0) not in (NULL, SHAPE, PARAM, DTYPE)
    assert latent(None, f8, window=0, ws=0) == NULL
    need = B.msa_latent_workspace_bytes(2, 1, 64, 1, 128, 512, 2)
    assert need >= 2 * 2 * 64 * 129 * 4
    assert latent(s, c, ws=need - 1) == WORKSPACE
    assert latent(s, c, ws=0) == NULL
    assert latent(s, c, batch=0) == OK
    # window 0 and no list: neither leaf is needed
    assert latent(None, None, window=0, top_c=0, lists=None, np_=1, ws=0) not in (NULL, SHAPE, PARAM)


def test_latent_partition_planning():
    # one partition's entries must fit 2048 list slots: 10 000 entries need >= 5
    assert B.library().msa_latent_partitions(4, 1, 64, 1, 128, 9872, 4) == PARAM
    assert B.msa_latent_partitions(4, 1, 64, 1, 128, 9872, 5) == 5
    assert B.msa_latent_partitions(4, 1, 64, 1, 128, 9872, 0) >= 5
    assert B.msa_latent_partitions(64, 1, 64, 1, 128, 1920, 1) == 1    # 32 tiles fit one
    # one partition and one leaf: no workspace; both leaves: the query
    # reserves the two partitions that leaves of two types would take
    assert B.msa_latent_workspace_bytes(64, 1, 64, 1, 0, 1920, 1) == 0
    assert B.msa_latent_workspace_bytes(64, 1, 64, 1, 128, 1920, 1) > 0
    assert B.library().msa_latent_partitions(64, 1, 64, 1, 128, 1921, 1) == PARAM
    with pytest.raises(B.MsaError):
        B.msa_latent_partitions(4, 1, 64, 3, 128, 16, 0)


def test_host_calls_from_many_threads_agree():
    # ctypes drops the GIL for the call, so these run concurrently in the
    # library: sizing queries and argument checks keep no shared state
    from concurrent.futures import ThreadPoolExecutor
    shapes = [rg(batch=b, max_seq=s, max_cache=c, stride=(c + s + 127) // 128 + 1)
              for b, s, c in ((2, 1, 4000), (64, 1, 32767), (4, 8, 9000), (3, 300, 5000))]
    k, v = cache(heads=8), cache(heads=8)

    def one(i):
        r = shapes[i % len(shapes)]
        return (B.msa_attention_workspace_bytes(r, 64, 8, 16, 3),
                B.msa_indexer_workspace_bytes(r, 8, 16),
                B.msa_attention_partitions(r, 64, 8, 16, 5),
                attention(r, k, v, np_=4, ws=0),
                attention(r, k, v, hq=60))

    expect = [one(i) for i in range(len(shapes))]
    with ThreadPoolExecutor(max_workers=8) as ex:
        got = list(ex.map(one, range(4000)))
    assert all(g == expect[i % len(shapes)] for i, g in enumerate(got))
