"""CPU oracle of the DSA hot path: TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import this
package.  It shares no code with the GPU library and never imports it.

`liboracle.so` (plain C, fp64, see dsa_oracle.c) is built from source by `build()`;
this module marshals torch/numpy arrays into it and adds the layer-stack driver
(IndexCache F/S reuse) and the freq -> pattern rule, written here independently of the
library's own implementation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (always rebuilds)."""
    src = os.path.join(_HERE, "dsa_oracle.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", src, "-o", tmp, "-lm", "-lpthread"])
    os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = D
        L.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_double.restype = D
        L.oracle_e2m1_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_to_double.restype = D
        L.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_to_double.restype = D
        L.oracle_mxfp4_row_bytes.argtypes = [I]
        L.oracle_mxfp4_row_bytes.restype = I64
        L.oracle_mxfp4_value.argtypes = [P, I, I]
        L.oracle_mxfp4_value.restype = D
        L.oracle_index_scores.argtypes = [P, P, P, P, I, I, I, I, I, P, I64, I]
        L.oracle_topk.argtypes = [P, I64, P, I, I, I, I, P, I]
        L.oracle_sparse_attn.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I, I, D, P, P, I]
        L.oracle_dsa_rows.argtypes = [P, P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, D, P, P, I]
        L.oracle_indexer_kl.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, D, P, P, P, P, I]
        L.oracle_indexer_kl_f64.argtypes = L.oracle_indexer_kl.argtypes
        for f in ("oracle_index_scores", "oracle_topk", "oracle_sparse_attn", "oracle_dsa_rows",
                  "oracle_indexer_kl", "oracle_indexer_kl_f64"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(os.cpu_count() or 1, 16))


def _np(x, dtype):
    """Contiguous host numpy array of the raw bits (bf16 -> uint16, fp8 -> uint8)."""
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu").contiguous()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16).numpy().view(np.uint16)
        else:
            x = x.numpy()
    x = np.ascontiguousarray(x)
    assert x.dtype == dtype, (x.dtype, dtype)
    return x


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _kvlen(kv_len, B):
    if kv_len is None:
        return None
    return _np(torch.as_tensor(kv_len, dtype=torch.int32).reshape(B) if not isinstance(kv_len, np.ndarray)
               else kv_len.astype(np.int32), np.int32)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


def e4m3_to_double(code: int) -> float:
    return lib().oracle_e4m3_to_double(code)


def e2m1_to_double(code: int) -> float:
    return lib().oracle_e2m1_to_double(code)


def e8m0_to_double(code: int) -> float:
    return lib().oracle_e8m0_to_double(code)


def mxfp4_row_bytes(D: int) -> int:
    return lib().oracle_mxfp4_row_bytes(D)


def mxfp4_decode_row(row, D: int) -> np.ndarray:
    """The D values of one MXFP4 row (uint8 [D/2 + 32]) as float64."""
    r = np.ascontiguousarray(np.asarray(row, dtype=np.uint8))
    assert r.shape == (mxfp4_row_bytes(D),)
    return np.array([lib().oracle_mxfp4_value(_ptr(r), D, d) for d in range(D)])


def _kv_format(kvn, Dqk, kv_scale):
    """0 bf16, 1 fp8 e4m3 (+ per-token scale), 2 MXFP4 rows (no scale)."""
    if kvn.dtype != np.uint8:
        return 0
    if kv_scale is not None:
        if kvn.shape[-1] != Dqk:
            raise ValueError("fp8 rows must be Dqk bytes wide")
        return 1
    if kvn.shape[-1] != Dqk // 2 + 32 or Dqk % 32:
        raise ValueError("MXFP4 rows must be Dqk/2 + 32 bytes wide (fp8 rows need kv_scale)")
    return 2


def index_scores(q_idx, k_idx, w_idx, kv_len=None, nthreads=None, ld=None) -> np.ndarray:
    """Indexer scores float32 [B, Tq, ld]; entries after the causal bound are -inf."""
    q, k, w = _np(q_idx, np.uint16), _np(k_idx, np.uint16), _np(w_idx, np.uint16)
    B, Tq, H, D = q.shape
    Tk = k.shape[1]
    ld = Tk if ld is None else ld
    out = np.empty((B, Tq, ld), np.float32)
    kl = _kvlen(kv_len, B)
    rc = lib().oracle_index_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(kl), B, Tq, Tk, H, D, _ptr(out), ld,
                                   nthreads or default_threads())
    assert rc == 0, rc
    return out


def topk(scores, k: int, kv_len=None, Tk=None, nthreads=None) -> np.ndarray:
    """Causal top-k of score rows: int32 [B, Tq, k], ascending, -1 padded."""
    s = _np(scores, np.float32)
    B, Tq, ld = s.shape
    Tk = ld if Tk is None else Tk
    out = np.empty((B, Tq, k), np.int32)
    kl = _kvlen(kv_len, B)
    rc = lib().oracle_topk(_ptr(s), ld, _ptr(kl), B, Tq, Tk, k, _ptr(out), nthreads or default_threads())
    assert rc == 0, rc
    return out


def sparse_attn(q, kv, idx, sm_scale, v=None, kv_scale=None, Dv=None, nthreads=None):
    """Attention over selected keys: (out float64 [B,Tq,H,Dv], lse float64 [B,Tq,H]).

    With v None, V is kv[..., :Dv] (Dv must then be given)."""
    qn = _np(q, np.uint16)
    u8 = isinstance(kv, torch.Tensor) and kv.dtype == torch.uint8 or (isinstance(kv, np.ndarray) and kv.dtype == np.uint8)
    kvn = _np(kv, np.uint8 if u8 else np.uint16)
    vn = None if v is None else _np(v, np.uint16)
    sc = None if kv_scale is None else _np(kv_scale, np.float32)
    ix = _np(idx, np.int32)
    B, Tq, H, Dqk = qn.shape
    Tk, Hkv = kvn.shape[1], kvn.shape[2]
    fmt = _kv_format(kvn, Dqk, kv_scale)
    if vn is not None:
        Dv = vn.shape[3]
    elif Dv is None:
        raise ValueError("Dv is required when V is taken from the kv rows")
    k = ix.shape[2]
    out = np.zeros((B, Tq, H, Dv), np.float64)
    lse = np.zeros((B, Tq, H), np.float64)
    rc = lib().oracle_sparse_attn(_ptr(qn), _ptr(kvn), _ptr(sc), _ptr(vn), fmt, _ptr(ix), B, Tq, Tk, H,
                                  Hkv, Dqk, Dv, k, float(sm_scale), _ptr(out), _ptr(lse),
                                  nthreads or default_threads())
    assert rc == 0, rc
    return out, lse


def dsa_rows(q_idx, k_idx, w_idx, q, kv, rows, k, sm_scale, Dv=512, kv_scale=None, nthreads=None):
    """Streamed scores -> top-k -> MLA attention for chosen rows of one prefill sequence."""
    qi, ki, wi, qn = (_np(x, np.uint16) for x in (q_idx, k_idx, w_idx, q))
    u8 = isinstance(kv, torch.Tensor) and kv.dtype == torch.uint8 or (isinstance(kv, np.ndarray) and kv.dtype == np.uint8)
    kvn = _np(kv, np.uint8 if u8 else np.uint16)
    sc = None if kv_scale is None else _np(kv_scale, np.float32)
    rows = np.ascontiguousarray(np.asarray(rows, np.int32))
    H_I, d_I = qi.shape[-2], qi.shape[-1]
    Tk = ki.shape[-2]
    H, Dqk = qn.shape[-2], qn.shape[-1]
    fmt = _kv_format(kvn, Dqk, kv_scale)
    idx = np.empty((len(rows), k), np.int32)
    out = np.empty((len(rows), H, Dv), np.float64)
    rc = lib().oracle_dsa_rows(_ptr(qi), _ptr(ki), _ptr(wi), _ptr(qn), _ptr(kvn), _ptr(sc), fmt,
                               _ptr(rows), len(rows), Tk, H_I, d_I, H, Dqk, Dv, k, float(sm_scale),
                               _ptr(idx), _ptr(out), nthreads or default_threads())
    assert rc == 0, rc
    return idx, out


def indexer_kl(q_idx, k_idx, w_idx, q, k, sm_scale, idx=None, kv_len=None, nthreads=None):
    """Indexer KL objective (dsa_oracle.c): per-row KL(P || Q) and the gradients of their sum
    with respect to the indexer inputs.  bf16 tensors (or float64 arrays: the _f64 form);
    k is the main attention's keys [B, Tk, Hkv, Dqk]; idx None = every causal key (dense
    warm-up).  Returns (loss [B,Tq], dq_idx, dw_idx, dk_idx [B,Tk,d_I]) as float64."""
    f64 = isinstance(q_idx, np.ndarray) and q_idx.dtype == np.float64
    cv = (lambda x: np.ascontiguousarray(x, dtype=np.float64)) if f64 else (lambda x: _np(x, np.uint16))
    qi, ki, wi, qn, kn = (cv(x) for x in (q_idx, k_idx, w_idx, q, k))
    B, Tq, H_I, d_I = qi.shape
    Tk = ki.shape[1]
    H, Dqk = qn.shape[2], qn.shape[3]
    Hkv = kn.shape[2]
    ix = None if idx is None else _np(idx, np.int32)
    kk = 0 if ix is None else ix.shape[2]
    kl = _kvlen(kv_len, B)
    loss = np.zeros((B, Tq), np.float64)
    dq = np.zeros((B, Tq, H_I, d_I), np.float64)
    dw = np.zeros((B, Tq, H_I), np.float64)
    dk = np.zeros((B, Tk, d_I), np.float64)
    fn = lib().oracle_indexer_kl_f64 if f64 else lib().oracle_indexer_kl
    rc = fn(_ptr(qi), _ptr(ki), _ptr(wi), _ptr(qn), _ptr(kn), _ptr(kl), _ptr(ix), B, Tq, Tk, H_I, d_I, H, Hkv,
            Dqk, kk, float(sm_scale), _ptr(loss), _ptr(dq), _ptr(dw), _ptr(dk), nthreads or default_threads())
    assert rc == 0, rc
    return loss, dq, dw, dk


# ---------- IndexCache F/S reuse ("IndexCache" vLLM feature doc, "How It Works" and
# "Configuration Reference") ----------

def pattern_from_freq(freq: int, n_layers: int) -> str:
    """index_topk_freq = N computes top-k on one layer in N; reading: layers 0, N, 2N, ...
    are the full ones.  N = 1 means every layer computes (the feature is off)."""
    if freq < 1 or n_layers < 1:
        raise ValueError("freq and n_layers must be >= 1")
    return "".join("F" if i % freq == 0 else "S" for i in range(n_layers))


def check_pattern(pattern: str, n_layers: int, cache_prefilled: bool = False) -> None:
    """One character per DSA layer, each F (full) or S (shared); an S layer needs an index
    set computed before it (reading: a leading S is an error unless the caller supplies
    the cache)."""
    if len(pattern) != n_layers:
        raise ValueError("pattern length must equal the number of layers")
    if any(c not in "FS" for c in pattern):
        raise ValueError("pattern characters must be F or S")
    if n_layers and pattern[0] == "S" and not cache_prefilled:
        raise ValueError("a leading S layer has no index set to reuse")


def layer_stack(pattern, layers, k, sm_scale, Dv=None, kv_len=None, index_cache=None, nthreads=None):
    """Run the stack: an F layer computes scores and top-k into the index cache, every
    layer then attends with the cache as it stands (S layers reuse it unchanged).

    `layers` is a list of dicts with q/kv/v/kv_scale and, on F layers, q_idx/k_idx/w_idx.
    Returns (outs, lses, index_sets) with index_sets[l] the indices layer l attended with.
    """
    check_pattern(pattern, len(layers), cache_prefilled=index_cache is not None)
    cache = None if index_cache is None else _np(index_cache, np.int32).copy()
    outs, lses, sets = [], [], []
    for l, (c, L) in enumerate(zip(pattern, layers)):
        if c == "F":
            Tk = L["k_idx"].shape[1]
            s = index_scores(L["q_idx"], L["k_idx"], L["w_idx"], kv_len=kv_len, nthreads=nthreads)
            cache = topk(s, k, kv_len=kv_len, Tk=Tk, nthreads=nthreads)
        o, lse = sparse_attn(L["q"], L["kv"], cache, sm_scale, v=L.get("v"), kv_scale=L.get("kv_scale"),
                             Dv=Dv, nthreads=nthreads)
        outs.append(o)
        lses.append(lse)
        sets.append(cache)
    return outs, lses, sets
