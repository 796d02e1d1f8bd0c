"""DeepSeek Sparse Attention hot path for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI in include/dsa.h (libdsa.so, built in-tree by
`deepseek_sparse_attention_amd.build`).  Every step runs in the library's HIP kernels;
this module only passes device pointers, sizes and torch's current stream, and turns a
non-OK status into DSAError.  There is no CPU fallback: without the built library (or on
a machine without a gfx950 GPU) the calls raise.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "DSAError", "lib", "abi_version", "index_scores", "topk", "index_topk", "sparse_attn", "sparse_attn_noalloc",
    "noalloc_scratch_bytes", "layer_stack",
    "index_scores_paged", "sparse_attn_paged", "indexer_kl", "indexer_kl_workspace_size", "PagedKV", "paged_kv", "OP_ATTN_PAGED", "OP_STACK_PAGED", "OP_INDEXER_KL", "OP_INDEXER_KL_DENSE",
    "workspace_size", "stack_chunk_rows", "check_pattern", "pattern_from_freq", "Shape",
    "KV_BF16", "KV_FP8_E4M3", "KV_MXFP4", "mxfp4_row_bytes", "CACHE_PREFILLED", "STACK_UNFUSED", "CACHE_TOPK_ROWS", "OP_SCORES", "OP_TOPK", "OP_ATTN",
    "OP_STACK", "OP_INDEX_TOPK",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

KV_BF16, KV_FP8_E4M3, KV_MXFP4 = 0, 1, 2
OP_SCORES, OP_TOPK, OP_ATTN, OP_STACK, OP_INDEX_TOPK, OP_ATTN_PAGED, OP_STACK_PAGED = 0, 1, 2, 3, 4, 5, 6
OP_INDEXER_KL, OP_INDEXER_KL_DENSE = 7, 8
CACHE_PREFILLED, STACK_UNFUSED, CACHE_TOPK_ROWS = 1, 2, 4
_STATUS = ["DSA_OK", "DSA_ERR_NULL", "DSA_ERR_SHAPE", "DSA_ERR_UNSUPPORTED", "DSA_ERR_PATTERN",
           "DSA_ERR_WORKSPACE", "DSA_ERR_LAUNCH", "DSA_ERR_DEVICE"]


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = _STATUS[status] if 0 <= status < len(_STATUS) else str(status)
        super().__init__(f"{name}: {message}")


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("Tq", ctypes.c_int), ("Tk", ctypes.c_int),
                ("H_I", ctypes.c_int), ("d_I", ctypes.c_int),
                ("H", ctypes.c_int), ("Hkv", ctypes.c_int), ("Dqk", ctypes.c_int), ("Dv", ctypes.c_int),
                ("k", ctypes.c_int), ("sm_scale", ctypes.c_float), ("kv_dtype", ctypes.c_int),
                ("kv_len", ctypes.c_void_p)]


class LayerIO(ctypes.Structure):
    _fields_ = [("q_idx", ctypes.c_void_p), ("k_idx", ctypes.c_void_p), ("w_idx", ctypes.c_void_p),
                ("q", ctypes.c_void_p), ("kv", ctypes.c_void_p), ("kv_scale", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class PagedKV(ctypes.Structure):
    """dsa_paged_kv: token s of sequence b is pool row block_table[b][s // page_size] * page_size
    + s % page_size."""
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int), ("page_size", ctypes.c_int),
                ("num_pages", ctypes.c_int)]


def paged_kv(block_table, page_size, num_pages):
    """A PagedKV over a device int32 [B, max_blocks] block table.  The descriptor holds a
    reference to the table tensor, so its memory stays allocated while the descriptor lives
    (a raw pointer alone would let torch's allocator hand the memory to the next tensor)."""
    pg = PagedKV(_ptr(block_table), block_table.shape[1], page_size, num_pages)
    pg._table = block_table
    return pg


_lib = None


def lib():
    """The loaded libdsa.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m deepseek_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, U, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_float,
                               ctypes.c_size_t)
        L.dsa_abi_version.restype = I
        L.dsa_last_error.restype = ctypes.c_char_p
        L.dsa_status_string.argtypes = [I]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_index_scores.argtypes = [P, P, P, P, I, I, I, I, I, P, I64, P]
        L.dsa_topk.argtypes = [P, I64, P, I, I, I, I, P, P, SZ, P]
        L.dsa_index_topk.argtypes = [P, P, P, P, I, I, I, I, I, I, F, P, P, SZ, P]
        L.dsa_index_scores_paged.argtypes = [P, P, P, ctypes.POINTER(PagedKV), P, I, I, I, I, I, P, I64, P]
        L.dsa_sparse_attn_paged.argtypes = [P, P, P, I, ctypes.POINTER(PagedKV), P, P, I, I, I, I, I, I, I, F, P, P,
                                            P, SZ, P]
        L.dsa_layer_stack_paged.argtypes = [ctypes.c_char_p, I, P, ctypes.POINTER(Shape), ctypes.POINTER(PagedKV), P,
                                            U, P, SZ, P]
        L.dsa_sparse_attn.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I, I, F, P, P, P, SZ, P]
        L.dsa_sparse_attn_noalloc.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I, I, F, P, P, P]
        L.dsa_noalloc_scratch_bytes.restype = SZ
        L.dsa_layer_stack.argtypes = [ctypes.c_char_p, I, P, ctypes.POINTER(Shape), P, U, P, SZ, P]
        L.dsa_workspace_size.argtypes = [ctypes.POINTER(Shape), I]
        L.dsa_workspace_size.restype = SZ
        L.dsa_stack_chunk_rows.argtypes = [ctypes.POINTER(Shape)]
        L.dsa_stack_chunk_rows.restype = I
        L.dsa_check_pattern.argtypes = [ctypes.c_char_p, I, U]
        L.dsa_pattern_from_freq.argtypes = [I, I, ctypes.c_char_p]
        L.dsa_indexer_kl.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P, P, P, P, P, SZ, P]
        for f in ("dsa_index_scores", "dsa_topk", "dsa_index_topk", "dsa_sparse_attn", "dsa_sparse_attn_noalloc",
                  "dsa_layer_stack",
                  "dsa_check_pattern", "dsa_pattern_from_freq", "dsa_index_scores_paged", "dsa_sparse_attn_paged",
                  "dsa_layer_stack_paged", "dsa_indexer_kl"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise DSAError(status, lib().dsa_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None


def abi_version() -> int:
    return lib().dsa_abi_version()


def index_scores(q_idx, k_idx, w_idx, kv_len=None, scores=None, ld=None, stream=None):
    """dsa_index_scores: returns the fp32 score tensor [B, Tq, ld] (the library writes -inf
    into entries s > p)."""
    B, Tq, H_I, d_I = q_idx.shape
    Tk = k_idx.shape[1]
    ld = Tk if ld is None else ld
    if scores is None:
        scores = torch.empty((B, Tq, ld), dtype=torch.float32, device=q_idx.device)
    _check(lib().dsa_index_scores(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(kv_len), B, Tq, Tk, H_I, d_I,
                                  _ptr(scores), ld, _stream(stream)))
    return scores


def topk(scores, k, Tk=None, kv_len=None, idx=None, ws=None, split=True, stream=None):
    """dsa_topk: int32 [B, Tq, k] ascending, -1 padded.  split=False passes no workspace
    (one workgroup per row); the indices are the same either way."""
    B, Tq, ld = scores.shape
    Tk = ld if Tk is None else Tk
    if idx is None:
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=scores.device)
    nbytes = workspace_size(_shape(B, Tq, Tk, 1, 1, 1, 1, k, 1.0, KV_BF16), OP_TOPK) if split else 0
    ws = _workspace(nbytes, scores.device, ws) if nbytes else None
    _check(lib().dsa_topk(_ptr(scores), ld, _ptr(kv_len), B, Tq, Tk, k, _ptr(idx), _ptr(ws), nbytes,
                          _stream(stream)))
    return idx


def index_topk(q_idx, k_idx, w_idx, k, kv_len=None, oversample=0.0, idx=None, ws=None, stream=None):
    """dsa_index_topk: int32 [B, Tq, k], the indices index_scores + topk would give."""
    B, Tq, H_I, d_I = q_idx.shape
    Tk = k_idx.shape[1]
    if idx is None:
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=q_idx.device)
    shp = _shape(B, Tq, Tk, 1, 1, 1, 1, k, 1.0, KV_BF16, H_I, d_I, kv_len)
    nbytes = workspace_size(shp, OP_INDEX_TOPK)
    ws = _workspace(nbytes, q_idx.device, ws)
    _check(lib().dsa_index_topk(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(kv_len), B, Tq, Tk, H_I, d_I, k,
                                float(oversample), _ptr(idx), _ptr(ws), nbytes, _stream(stream)))
    return idx


def index_scores_paged(q_idx, k_pool, w_idx, pages, Tk, kv_len=None, scores=None, ld=None, stream=None):
    """dsa_index_scores_paged: k_pool bf16 [num_pages * page_size, d_I]; pages a PagedKV."""
    B, Tq, H_I, d_I = q_idx.shape
    ld = Tk if ld is None else ld
    if scores is None:
        scores = torch.empty((B, Tq, ld), dtype=torch.float32, device=q_idx.device)
    _check(lib().dsa_index_scores_paged(_ptr(q_idx), _ptr(k_pool), _ptr(w_idx), ctypes.byref(pages), _ptr(kv_len),
                                        B, Tq, Tk, H_I, d_I, _ptr(scores), ld, _stream(stream)))
    return scores


def sparse_attn_paged(q, kv_pool, idx, sm_scale, pages, Tk, kv_len=None, kv_scale_pool=None, Dv=512, out=None,
                      lse=None, want_lse=True, ws=None, stream=None):
    """dsa_sparse_attn_paged (MLA form): kv_pool [num_pages * page_size, row]: bf16, e4m3 bytes
    (with kv_scale_pool) or MXFP4 bytes (320 per row)."""
    B, Tq, H, Dqk = q.shape
    kvd = _kv_dtype(kv_pool, Dqk, kv_scale_pool)
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, Tq, H, Dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device)
    shp = _shape(B, Tq, Tk, H, 1, Dqk, Dv, k, sm_scale, kvd)
    nbytes = workspace_size(shp, OP_ATTN_PAGED)
    ws = _workspace(nbytes, q.device, ws)
    _check(lib().dsa_sparse_attn_paged(_ptr(q), _ptr(kv_pool), _ptr(kv_scale_pool), kvd, ctypes.byref(pages), _ptr(idx),
                                       _ptr(kv_len), B, Tq, Tk, H, Dqk, Dv, k, sm_scale, _ptr(out), _ptr(lse),
                                       _ptr(ws), nbytes, _stream(stream)))
    return out, lse


def mxfp4_row_bytes(Dqk: int) -> int:
    """Bytes of one MXFP4 latent row of Dqk values (dsa_kv_dtype in include/dsa.h)."""
    return Dqk // 2 + 32


def _kv_dtype(kv, Dqk, kv_scale):
    """Row format of a latent cache tensor: bf16; uint8 rows of Dqk bytes with kv_scale (e4m3);
    uint8 rows of Dqk/2 + 32 bytes without (MXFP4)."""
    if kv.dtype == torch.bfloat16:
        return KV_BF16
    if kv.dtype != torch.uint8:
        raise ValueError(f"latent rows must be bfloat16 or uint8, got {kv.dtype}")
    if kv_scale is not None:
        if kv.shape[-1] != Dqk:
            raise ValueError("fp8 rows (given with kv_scale) must be Dqk bytes wide")
        return KV_FP8_E4M3
    if kv.shape[-1] != mxfp4_row_bytes(Dqk):
        raise ValueError("uint8 rows without kv_scale are MXFP4 and must be Dqk/2 + 32 bytes wide")
    return KV_MXFP4


def indexer_kl(q_idx, k_idx, w_idx, q, k, sm_scale, idx=None, kv_len=None, grads=True, out=None, ws=None,
               stream=None):
    """dsa_indexer_kl: per-row KL(main attention || indexer) and, with grads, the gradients of
    its sum for q_idx, w_idx and k_idx.  idx None: every causal key (dense warm-up).
    Returns (loss fp32 [B,Tq], dq_idx, dw_idx, dk_idx) (gradients None without grads);
    `out` may hold those four tensors, preallocated, and `ws` a uint8 workspace (the key
    gradient's; allocated here when absent or too small)."""
    B, Tq, H_I, d_I = q_idx.shape
    Tk = k_idx.shape[1]
    H, Dqk = q.shape[2], q.shape[3]
    kk = 0 if idx is None else idx.shape[2]
    dev = q_idx.device
    if out is not None:
        loss, dq, dw, dk = out
    else:
        loss = torch.empty((B, Tq), dtype=torch.float32, device=dev)
        dq = dw = dk = None
        if grads:
            dq = torch.empty((B, Tq, H_I, d_I), dtype=torch.float32, device=dev)
            dw = torch.empty((B, Tq, H_I), dtype=torch.float32, device=dev)
            dk = torch.empty((B, Tk, d_I), dtype=torch.float32, device=dev)
    nbytes = 0
    if dk is not None:
        shp = _shape(B, Tq, Tk, H, H, Dqk, Dqk, max(kk, 1), sm_scale, KV_BF16, H_I, d_I)
        nbytes = workspace_size(shp, OP_INDEXER_KL_DENSE if idx is None else OP_INDEXER_KL)
    ws = _workspace(nbytes, dev, ws)
    _check(lib().dsa_indexer_kl(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(k), _ptr(idx), _ptr(kv_len),
                                B, Tq, Tk, H_I, d_I, H, Dqk, kk, ctypes.c_float(sm_scale), _ptr(loss), _ptr(dq),
                                _ptr(dw), _ptr(dk), _ptr(ws), nbytes, _stream(stream)))
    return loss, dq, dw, dk


def indexer_kl_workspace_size(B, Tq, Tk, H_I, d_I, kk=0):
    """Bytes of workspace dsa_indexer_kl needs for key gradients (kk 0: dense warm-up)."""
    shp = _shape(B, Tq, Tk, 1, 1, 32, 32, max(kk, 1), 1.0, KV_BF16, H_I, d_I)
    return workspace_size(shp, OP_INDEXER_KL if kk else OP_INDEXER_KL_DENSE)


def _shape(B, Tq, Tk, H, Hkv, Dqk, Dv, k, sm_scale, kv_dtype, H_I=16, d_I=64, kv_len=None):
    return Shape(B, Tq, Tk, H_I, d_I, H, Hkv, Dqk, Dv, k, sm_scale, kv_dtype, _ptr(kv_len))


def workspace_size(shape: Shape, op: int) -> int:
    return lib().dsa_workspace_size(ctypes.byref(shape), op)


def stack_chunk_rows(shape: Shape) -> int:
    return lib().dsa_stack_chunk_rows(ctypes.byref(shape))


def _workspace(nbytes, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def sparse_attn(q, kv, idx, sm_scale, v=None, kv_scale=None, Dv=None, out=None, lse=None, want_lse=True,
                ws=None, stream=None):
    """dsa_sparse_attn: returns (out bf16 [B,Tq,H,Dv], lse fp32 [B,Tq,H] or None)."""
    B, Tq, H, Dqk = q.shape
    Tk, Hkv = kv.shape[1], kv.shape[2]
    kvd = _kv_dtype(kv, Dqk, kv_scale)
    if v is not None:
        Dv = v.shape[3]
    elif Dv is None:
        raise ValueError("Dv is required when V is taken from the kv rows")
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, Tq, H, Dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device)
    shp = _shape(B, Tq, Tk, H, Hkv, Dqk, Dv, k, sm_scale, kvd)
    nbytes = workspace_size(shp, OP_ATTN)
    ws = _workspace(nbytes, q.device, ws)
    _check(lib().dsa_sparse_attn(_ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(v), kvd, _ptr(idx), B, Tq, Tk, H, Hkv,
                                 Dqk, Dv, k, sm_scale, _ptr(out), _ptr(lse), _ptr(ws), nbytes, _stream(stream)))
    return out, lse


def sparse_attn_noalloc(q, kv, idx, sm_scale, v=None, kv_scale=None, Dv=None, out=None, lse=None, want_lse=True,
                        stream=None):
    """dsa_sparse_attn_noalloc: dsa_sparse_attn with the library's built-in scratch instead of
    a workspace (outputs are allocated here unless given)."""
    B, Tq, H, Dqk = q.shape
    Tk, Hkv = kv.shape[1], kv.shape[2]
    kvd = _kv_dtype(kv, Dqk, kv_scale)
    if v is not None:
        Dv = v.shape[3]
    elif Dv is None:
        raise ValueError("Dv is required when V is taken from the kv rows")
    k = idx.shape[2]
    if out is None:
        out = torch.empty((B, Tq, H, Dv), dtype=torch.bfloat16, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Tq, H), dtype=torch.float32, device=q.device)
    _check(lib().dsa_sparse_attn_noalloc(_ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(v), kvd, _ptr(idx), B, Tq, Tk, H,
                                         Hkv, Dqk, Dv, k, sm_scale, _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def noalloc_scratch_bytes() -> int:
    return lib().dsa_noalloc_scratch_bytes()


def layer_stack(pattern, layers, k, sm_scale, Dv=None, kv_len=None, index_cache=None, prefilled=False,
                H_I=None, d_I=None, ws=None, want_lse=True, unfused=False, pages=None, Tk=None, topk_rows=False,
                stream=None):
    """dsa_layer_stack over `layers` (dicts with q/kv[/v/kv_scale] and, on F layers, q_idx/k_idx/w_idx).

    Returns (outs, lses, index_cache).  Output tensors are allocated unless a layer dict
    carries "out"/"lse".  unfused: 'F' layers take the score-chunk route (STACK_UNFUSED).
    topk_rows (with prefilled): the prefilled cache holds dsa_topk rows (CACHE_TOPK_ROWS).
    pages (a PagedKV) with Tk: k_idx, kv and kv_scale are pools (dsa_layer_stack_paged).
    """
    n = len(layers)
    L0 = layers[0]
    B, Tq, H, Dqk = L0["q"].shape
    if pages is None:
        Tk, Hkv = L0["kv"].shape[1], L0["kv"].shape[2]
    else:
        Hkv = 1
    kvd = _kv_dtype(L0["kv"], Dqk, L0.get("kv_scale"))
    if L0.get("v") is not None:
        Dv = L0["v"].shape[3]
    elif Dv is None:
        raise ValueError("Dv is required when V is taken from the kv rows")
    f0 = next((L for c, L in zip(pattern, layers) if c == "F"), None)
    if f0 is not None:
        H_I, d_I = f0["q_idx"].shape[2], f0["q_idx"].shape[3]
    H_I, d_I = H_I or 16, d_I or 64
    dev = L0["q"].device
    shp = _shape(B, Tq, Tk, H, Hkv, Dqk, Dv, k, sm_scale, kvd, H_I, d_I, kv_len)
    if index_cache is None:
        index_cache = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)
    ios = (LayerIO * n)()
    outs, lses = [], []
    for i, L in enumerate(layers):
        o = L.get("out")
        if o is None:
            o = torch.empty((B, Tq, H, Dv), dtype=torch.bfloat16, device=dev)
        ls = L.get("lse")
        if ls is None and want_lse:
            ls = torch.empty((B, Tq, H), dtype=torch.float32, device=dev)
        outs.append(o)
        lses.append(ls)
        ios[i] = LayerIO(_ptr(L.get("q_idx")), _ptr(L.get("k_idx")), _ptr(L.get("w_idx")), _ptr(L["q"]),
                         _ptr(L["kv"]), _ptr(L.get("kv_scale")), _ptr(L.get("v")), _ptr(o), _ptr(ls))
    nbytes = workspace_size(shp, OP_STACK if pages is None else OP_STACK_PAGED)
    ws = _workspace(nbytes, dev, ws)
    flags = (CACHE_PREFILLED if prefilled else 0) | (STACK_UNFUSED if unfused else 0) | \
        (CACHE_TOPK_ROWS if topk_rows else 0)
    if pages is None:
        _check(lib().dsa_layer_stack(pattern.encode(), n, ios, ctypes.byref(shp), _ptr(index_cache), flags,
                                     _ptr(ws), nbytes, _stream(stream)))
    else:
        _check(lib().dsa_layer_stack_paged(pattern.encode(), n, ios, ctypes.byref(shp), ctypes.byref(pages),
                                           _ptr(index_cache), flags, _ptr(ws), nbytes, _stream(stream)))
    return outs, lses, index_cache


def check_pattern(pattern: str, n_layers: int = None, prefilled: bool = False) -> None:
    n = len(pattern) if n_layers is None else n_layers
    _check(lib().dsa_check_pattern(pattern.encode(), n, CACHE_PREFILLED if prefilled else 0))


def pattern_from_freq(freq: int, n_layers: int) -> str:
    buf = ctypes.create_string_buffer(max(0, n_layers) + 1)
    _check(lib().dsa_pattern_from_freq(freq, n_layers, buf))
    return buf.value.decode()
