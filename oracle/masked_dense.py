"""Second formulation of the oracle, in NumPy float64: TEST INFRASTRUCTURE ONLY.

The C oracle computes attention by gathering the selected keys.  This module computes
the same quantities the way the pages' portable runtime is described ("scores selectors
and applies masked SDPA", DSV2-Lite IndexCache model card, "Validation and scope"):
dense score and logit matrices over every key, with a mask that keeps only the causal
or selected entries.  Small sizes only (it materialises T x T matrices).
"""
from __future__ import annotations

import numpy as np
import torch


def _f64(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, np.float64)


def index_scores(q_idx, k_idx, w_idx) -> np.ndarray:
    """Dense indexer matrix [B, T, T] with -inf above the diagonal (float64)."""
    q, k, w = _f64(q_idx), _f64(k_idx), _f64(w_idx)
    dots = np.einsum("bthd,bsd->bths", q, k)           # per-head logits for every pair
    scores = np.einsum("bth,bths->bts", w, np.maximum(dots, 0.0))
    T = scores.shape[1]
    causal = np.tril(np.ones((T, k.shape[1]), bool), k=k.shape[1] - T)
    return np.where(causal[None], scores, -np.inf)


def selection_counts(idx, Tk: int) -> np.ndarray:
    """Integer [B, Tq, Tk]: how many entries of query row i's index list name key s.

    A key listed twice is two terms of the softmax sum, as in the gather form, which adds
    one term per index entry."""
    ix = np.asarray(idx)
    B, Tq, k = ix.shape
    c = np.zeros((B, Tq, Tk), np.int64)
    b, t, j = np.nonzero(ix >= 0)
    np.add.at(c, (b, t, ix[b, t, j]), 1)
    return c


def selection_mask(idx, Tk: int) -> np.ndarray:
    """Boolean [B, Tq, Tk]: True where key s is in query row i's index list."""
    return selection_counts(idx, Tk) > 0


def sparse_attn(q, kv, idx, sm_scale, v=None, Dv=None, kv_scale=None):
    """Masked dense attention: softmax over the selected keys only, (out, lse) float64.

    Each key's exponential is weighted by the number of entries that name it, so a
    duplicated entry counts twice, exactly as a sum over the index list would."""
    qd = _f64(q)
    if kv_scale is not None:
        raise NotImplementedError("fp8 rows: decode them first")
    K = _f64(kv)
    V = _f64(v) if v is not None else K[..., :Dv]
    B, Tq, H, _ = qd.shape
    Tk, Hkv = K.shape[1], K.shape[2]
    g = np.arange(H) * Hkv // H
    logits = sm_scale * np.einsum("bthd,bshd->bhts", qd, K[:, :, g, :])
    count = selection_counts(idx, Tk)[:, None, :, :]
    logits = np.where(count > 0, logits, -np.inf)
    m = logits.max(axis=-1, keepdims=True)
    p = count * np.exp(logits - m)
    denom = p.sum(axis=-1, keepdims=True)
    out = np.einsum("bhts,bshd->bthd", p / denom, V[:, :, g, :])
    lse = (m + np.log(denom))[..., 0].transpose(0, 2, 1)
    return out, lse
