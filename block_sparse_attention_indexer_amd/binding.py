"""ctypes binding of libmsa (include/msa.h): argument marshalling only.

Every function here forwards torch tensors' device addresses, strides and
the current HIP stream to the C entry point of the same name and raises
``MsaError`` on a non-zero status.  No step of the computation happens in
Python; there is no fallback when the library is missing -- importing the
library fails loudly instead.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libmsa.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "msa.h")

MSA_DTYPE_BF16 = 0
MSA_DTYPE_FP8_E4M3 = 1
BLOCK = 128
HEAD_DIM = 128
MSA_MAX_SPEC_DRAFT = 8    # largest new-token count routed as speculative decode
MSA_MAX_BLOCKS = 8192     # most blocks one sequence may hold
MSA_MAX_TOPK = 512        # largest top_k
MSA_MAX_KV_HEADS = 256    # most KV heads of one call
MSA_NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # msa_attention_paged_noalloc's fixed workspace
MSA_DEVERR_PAGE = 1       # device error word: a page id outside the pool
MSA_DEVERR_LENGTH = 2     # device error word: a length beyond the bounds or the table


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({status_string(status)})")
        self.status = status


class PagedCache(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("page_stride", ctypes.c_int64),
        ("head_stride", ctypes.c_int64),
        ("token_stride", ctypes.c_int64),
        ("scale", ctypes.c_void_p),
        ("scale_page_stride", ctypes.c_int64),
        ("scale_head_stride", ctypes.c_int64),
    ]


class Ragged(ctypes.Structure):
    _fields_ = [
        ("input_row_offsets", ctypes.c_void_p),
        ("cache_lengths", ctypes.c_void_p),
        ("kv_lookup_table", ctypes.c_void_p),
        ("lookup_stride", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("max_seq_length", ctypes.c_int32),
        ("max_cache_length", ctypes.c_int32),
    ]


class LatentLeaf(ctypes.Structure):
    _fields_ = [
        ("cache", PagedCache),
        ("cache_lengths", ctypes.c_void_p),
        ("lookup_table", ctypes.c_void_p),
        ("lookup_stride", ctypes.c_int32),
        ("max_cache_length", ctypes.c_int32),
    ]


MSA_LATENT_MAX_TOPC = 16384
MSA_LATENT_MAX_WINDOW = 1 << 20

_lib = None

_SIGNATURES = {
    "msa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "msa_indexer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Ragged), ctypes.c_int32, ctypes.c_int32]),
    "msa_indexer_paged": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(PagedCache), ctypes.POINTER(Ragged),
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "msa_indexer_reuse": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
    "msa_attention_partitions": (ctypes.c_int, [
        ctypes.POINTER(Ragged), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "msa_attention_workspace_bytes": (ctypes.c_size_t, [
        ctypes.POINTER(Ragged), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    "msa_attention_paged": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(PagedCache),
        ctypes.POINTER(PagedCache), ctypes.POINTER(Ragged), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p]),
    "msa_attention_paged_shared": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(PagedCache),
        ctypes.POINTER(PagedCache), ctypes.POINTER(Ragged), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
        ctypes.c_void_p]),
    "msa_attention_paged_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(PagedCache),
        ctypes.POINTER(PagedCache), ctypes.POINTER(Ragged), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]),
    "msa_device_errors": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int, ctypes.c_void_p]),
    "msa_latent_partitions": (ctypes.c_int, [ctypes.c_int32] * 7),
    "msa_latent_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32] * 7),
    "msa_latent_attention_paged": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(LatentLeaf),
        ctypes.POINTER(LatentLeaf), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "msa_splitk_combine": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]),
}


def library(path: str = LIB_PATH):
    """Load libmsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"libmsa.so not built at {path}; run "
                               "`python -m block_sparse_attention_indexer_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def header_functions(path: str = HEADER):
    """Names of the functions include/msa.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(msa_[a-z_0-9]+)\s*\(",
                                 text, flags=re.M)))


def status_string(status: int) -> str:
    return library().msa_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MsaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def paged_cache(pool: torch.Tensor, scale: torch.Tensor = None) -> PagedCache:
    """Describe a page pool tensor [pages, heads, 128, 128] (any strides, last
    dim contiguous) of dtype bfloat16 or float8_e4m3fn, and for an FP8
    index-K cache its per-token scales, float32 [pages, heads, 128] with a
    contiguous last dim."""
    if pool.dim() != 4 or pool.stride(3) != 1:
        raise ValueError("page pool must be [pages, heads, 128, 128] with a contiguous last dim")
    if pool.dtype == torch.bfloat16:
        dt = MSA_DTYPE_BF16
    elif pool.dtype == torch.float8_e4m3fn:
        dt = MSA_DTYPE_FP8_E4M3
    else:
        raise ValueError(f"unsupported cache dtype {pool.dtype}")
    P, H, S, Dm = pool.shape
    sp, ss0, ss1 = None, 0, 0
    if scale is not None:
        if scale.dtype != torch.float32 or scale.dim() != 3 or scale.stride(2) != 1:
            raise ValueError("scales must be float32 [pages, heads, 128] with a contiguous last dim")
        sp, ss0, ss1 = scale.data_ptr(), scale.stride(0), scale.stride(1)
    return PagedCache(pool.data_ptr(), dt, P, H, S, Dm, 0, pool.stride(0), pool.stride(1),
                      pool.stride(2), sp, ss0, ss1)


def ragged(input_row_offsets, cache_lengths, kv_lookup_table, max_seq_length: int,
           max_cache_length: int) -> Ragged:
    """Describe a ragged batch from int32 device tensors and host bounds."""
    for t in (input_row_offsets, cache_lengths, kv_lookup_table):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("row offsets, cache lengths and lookup table must be contiguous int32")
    return Ragged(input_row_offsets.data_ptr(), cache_lengths.data_ptr(), kv_lookup_table.data_ptr(),
                  kv_lookup_table.shape[1], cache_lengths.shape[0], int(max_seq_length),
                  int(max_cache_length))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def msa_indexer_workspace_bytes(rg: Ragged, num_kv_heads: int, top_k: int) -> int:
    return library().msa_indexer_workspace_bytes(ctypes.byref(rg), num_kv_heads, top_k)


def msa_attention_partitions(rg: Ragged, num_q_heads: int, num_kv_heads: int, top_k: int,
                             num_partitions: int = 0) -> int:
    n = library().msa_attention_partitions(ctypes.byref(rg), num_q_heads, num_kv_heads, top_k,
                                           num_partitions)
    if n < 0:
        raise MsaError(n, "msa_attention_partitions")
    return n


def msa_attention_workspace_bytes(rg: Ragged, num_q_heads: int, num_kv_heads: int, top_k: int,
                                  num_partitions: int = 0) -> int:
    return library().msa_attention_workspace_bytes(ctypes.byref(rg), num_q_heads, num_kv_heads,
                                                   top_k, num_partitions)


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def msa_indexer_paged(d_indices, q_idx, index_k, rg: Ragged, num_kv_heads: int, top_k: int,
                      init_blocks: int, local_blocks: int, workspace=None, stream=None,
                      index_k_scale=None):
    """Fill d_indices [rows, H_kv, top_k] (int32) with ascending block ids.
    index_k_scale: the per-token scales of an FP8 index-K cache."""
    cache = paged_cache(index_k, index_k_scale)
    need = msa_indexer_workspace_bytes(rg, num_kv_heads, top_k)
    ws = _workspace(need, q_idx.device, workspace)
    st = library().msa_indexer_paged(_ptr(d_indices), _ptr(q_idx), ctypes.byref(cache),
                                     ctypes.byref(rg), num_kv_heads, top_k, init_blocks,
                                     local_blocks, _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream))
    _check(st, "msa_indexer_paged")
    return d_indices


def msa_indexer_reuse(d_indices, prev_indices, src_row, stream=None):
    """d_indices[r] = prev_indices[src_row[r]] (all KV heads); rows whose source
    is out of range get -1.  int32 tensors [rows, H_kv, top_k],
    [prev_rows, H_kv, top_k] and [rows]."""
    rows, H_kv, top_k = d_indices.shape
    if prev_indices.shape[1:] != (H_kv, top_k) or src_row.shape != (rows,):
        raise ValueError("shapes of d_indices, prev_indices and src_row do not match")
    for t in (d_indices, prev_indices, src_row):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("block ids and source rows must be contiguous int32")
    st = library().msa_indexer_reuse(_ptr(d_indices), _ptr(prev_indices), _ptr(src_row), rows,
                                     prev_indices.shape[0], H_kv, top_k, _stream(stream))
    _check(st, "msa_indexer_reuse")
    return d_indices


def _attention(name, output, q, d_indices, k_cache, v_cache, rg, num_q_heads, num_kv_heads,
               top_k, scale, num_partitions, workspace, stream):
    kc, vc = paged_cache(k_cache), paged_cache(v_cache)
    need = msa_attention_workspace_bytes(rg, num_q_heads, num_kv_heads, top_k, num_partitions)
    ws = _workspace(need, q.device, workspace)
    st = getattr(library(), name)(_ptr(output), _ptr(q), _ptr(d_indices), ctypes.byref(kc),
                                  ctypes.byref(vc), ctypes.byref(rg), num_q_heads, num_kv_heads,
                                  top_k, float(scale), num_partitions, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check(st, name)
    return output


def msa_attention_paged(output, q, d_indices, k_cache, v_cache, rg: Ragged, num_q_heads: int,
                        num_kv_heads: int, top_k: int, scale: float, num_partitions: int = 0,
                        workspace=None, stream=None):
    """Fill output [rows, H_q, 128] (bf16) with attention over the selected blocks."""
    return _attention("msa_attention_paged", output, q, d_indices, k_cache, v_cache, rg,
                      num_q_heads, num_kv_heads, top_k, scale, num_partitions, workspace, stream)


def msa_attention_paged_shared(output, q, d_indices, k_cache, v_cache, rg: Ragged,
                               num_q_heads: int, num_kv_heads: int, top_k: int, scale: float,
                               num_partitions: int = 0, workspace=None, stream=None):
    """msa_attention_paged for speculative steps whose rows of a sequence share
    one selection (e.g. from msa_indexer_reuse): same result, each sequence's
    block union is read once for all its tokens."""
    return _attention("msa_attention_paged_shared", output, q, d_indices, k_cache, v_cache, rg,
                      num_q_heads, num_kv_heads, top_k, scale, num_partitions, workspace, stream)


def msa_attention_paged_noalloc(output, q, d_indices, k_cache, v_cache, rg: Ragged,
                                num_q_heads: int, num_kv_heads: int, top_k: int, scale: float,
                                num_partitions: int = 0, stream=None):
    """msa_attention_paged with no workspace argument: the library's fixed
    per-GPU scratch array serves as the workspace (nothing is allocated)."""
    kc, vc = paged_cache(k_cache), paged_cache(v_cache)
    st = library().msa_attention_paged_noalloc(_ptr(output), _ptr(q), _ptr(d_indices),
                                               ctypes.byref(kc), ctypes.byref(vc),
                                               ctypes.byref(rg), num_q_heads, num_kv_heads, top_k,
                                               float(scale), num_partitions, _stream(stream))
    _check(st, "msa_attention_paged_noalloc")
    return output


def msa_device_errors(clear: bool = True, stream=None) -> int:
    """The device error word (MSA_DEVERR_* bits of bad table data met since
    the last clear), read after the stream's work so far; clears it."""
    bits = ctypes.c_uint32(0)
    st = library().msa_device_errors(ctypes.byref(bits), 1 if clear else 0, _stream(stream))
    _check(st, "msa_device_errors")
    return int(bits.value)


def msa_splitk_combine(output, partial_o, partial_lse, input_row_offsets, batch: int,
                       max_seq_length: int, num_partitions: int, num_q_heads: int, stream=None):
    """Merge split-K partials [np, batch*max_seq, H_q, 128] / [np, batch*max_seq, H_q]."""
    st = library().msa_splitk_combine(_ptr(output), _ptr(partial_o), _ptr(partial_lse),
                                      _ptr(input_row_offsets), batch, max_seq_length,
                                      num_partitions, num_q_heads, _stream(stream))
    _check(st, "msa_splitk_combine")
    return output


def latent_leaf(pool: torch.Tensor, cache_lengths, lookup_table, max_cache_length: int) -> LatentLeaf:
    """Describe one leaf of the latent cache: pool [pages, latent heads, 128,
    128], cache lengths [batch] and page lookup table [batch, stride] (int32)."""
    for t in (cache_lengths, lookup_table):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("cache lengths and lookup table must be contiguous int32")
    return LatentLeaf(paged_cache(pool), _ptr(cache_lengths), _ptr(lookup_table),
                      lookup_table.shape[1], int(max_cache_length))


def msa_latent_partitions(batch: int, max_seq_length: int, num_heads: int, num_latent_heads: int,
                          window: int, top_c: int, num_partitions: int = 0) -> int:
    n = library().msa_latent_partitions(batch, max_seq_length, num_heads, num_latent_heads, window,
                                        top_c, num_partitions)
    if n < 1:
        raise MsaError(n, "msa_latent_partitions")
    return n


def msa_latent_workspace_bytes(batch: int, max_seq_length: int, num_heads: int,
                               num_latent_heads: int, window: int, top_c: int,
                               num_partitions: int = 0) -> int:
    return library().msa_latent_workspace_bytes(batch, max_seq_length, num_heads, num_latent_heads,
                                                window, top_c, num_partitions)


def msa_latent_attention_paged(output, q, input_row_offsets, batch: int, max_seq_length: int,
                               comp_indices, attn_sink, swa: LatentLeaf, comp: LatentLeaf,
                               num_heads: int, num_latent_heads: int, window: int, scale: float,
                               num_partitions: int = 0, workspace=None, stream=None):
    """Fill output [rows, H, 128] (bf16) with latent sparse attention over the
    window leaf `swa` and the compressed leaf `comp` (either may be None when
    window, resp. the list length, is 0).  comp_indices int32 [rows, H_lat,
    top_c] or None; attn_sink float32 [H]."""
    top_c = 0 if comp_indices is None else comp_indices.shape[-1]
    if comp_indices is not None and (comp_indices.dtype != torch.int32 or not comp_indices.is_contiguous()):
        raise ValueError("comp_indices must be contiguous int32")
    if attn_sink.dtype != torch.float32 or not attn_sink.is_contiguous():
        raise ValueError("attn_sink must be contiguous float32")
    need = msa_latent_workspace_bytes(batch, max_seq_length, num_heads, num_latent_heads, window,
                                      top_c, num_partitions)
    ws = _workspace(need, q.device, workspace)
    st = library().msa_latent_attention_paged(
        _ptr(output), _ptr(q), _ptr(input_row_offsets), batch, max_seq_length, _ptr(comp_indices),
        top_c, _ptr(attn_sink), None if swa is None else ctypes.byref(swa),
        None if comp is None else ctypes.byref(comp), num_heads, num_latent_heads, window,
        float(scale), num_partitions, _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "msa_latent_attention_paged")
    return output


# ---------------------------------------------------------------------------
# convenience: run the whole path on an inputs.Inputs problem
# ---------------------------------------------------------------------------

def ragged_of_inputs(inp) -> Ragged:
    wl = inp.wl
    return ragged(inp.input_row_offsets, inp.cache_lengths, inp.kv_lookup_table,
                  wl.max_seq_length, wl.max_cache_length)


def run_indexer(inp, d_indices=None, workspace=None, stream=None):
    wl = inp.wl
    rg = ragged_of_inputs(inp)
    if d_indices is None:
        d_indices = torch.empty((wl.total_rows, wl.num_kv_heads, wl.top_k), dtype=torch.int32,
                                device=inp.device)
    return msa_indexer_paged(d_indices, inp.q_idx, inp.index_k, rg, wl.num_kv_heads, wl.top_k,
                             wl.init_blocks, wl.local_blocks, workspace, stream,
                             index_k_scale=inp.index_k_scale)


def run_attention(inp, d_indices, output=None, num_partitions: int = 0, workspace=None,
                  stream=None, shared: bool = False):
    """Attention of a problem; shared=True calls msa_attention_paged_shared."""
    wl = inp.wl
    rg = ragged_of_inputs(inp)
    if output is None:
        output = torch.empty((wl.total_rows, wl.num_q_heads, HEAD_DIM), dtype=torch.bfloat16,
                             device=inp.device)
    fn = msa_attention_paged_shared if shared else msa_attention_paged
    return fn(output, inp.q, d_indices, inp.k_cache, inp.v_cache, rg, wl.num_q_heads,
              wl.num_kv_heads, wl.top_k, wl.softmax_scale, num_partitions, workspace, stream)


def latent_leaves_of_inputs(inp):
    """(window leaf, compressed leaf) descriptors of a latent_inputs problem."""
    wl = inp.wl
    swa = latent_leaf(inp.swa_pool, inp.swa_cache_lengths, inp.swa_lookup_table,
                      wl.max_swa_cache_length)
    comp = latent_leaf(inp.comp_pool, inp.comp_cache_lengths, inp.comp_lookup_table,
                       wl.max_comp_length)
    return swa, comp


def run_latent(inp, output=None, num_partitions: int = 0, workspace=None, stream=None):
    wl = inp.wl
    swa, comp = latent_leaves_of_inputs(inp)
    if output is None:
        output = torch.empty((wl.total_rows, wl.num_heads, HEAD_DIM), dtype=torch.bfloat16,
                             device=inp.q.device)
    return msa_latent_attention_paged(
        output, inp.q, inp.input_row_offsets, wl.batch, wl.max_seq_length,
        inp.comp_indices if wl.top_c > 0 else None, inp.attn_sink,
        swa if wl.window > 0 else None, comp if wl.top_c > 0 else None, wl.num_heads,
        wl.num_latent_heads, wl.window, wl.softmax_scale, num_partitions, workspace, stream)
