"""The C-ABI library on the host: it loads, exports every declared symbol, and its
argument checks reject bad calls before touching the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

import oracle
from tests.conftest import ROOT, golden

import deepseek_sparse_attention_amd as dsa


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.LIB_PATH):
        from deepseek_sparse_attention_amd import build
        build.build()
    return dsa.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dsa_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"dsa_index_scores", "dsa_topk", "dsa_sparse_attn", "dsa_layer_stack"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.dsa_abi_version() == 1


def test_status_strings(L):
    assert L.dsa_status_string(0) == b"DSA_OK"
    assert L.dsa_status_string(4) == b"DSA_ERR_PATTERN"


def test_indexer_argument_checks(L):
    P = ctypes.c_void_p(16)
    assert L.dsa_index_scores(None, P, P, None, 1, 4, 4, 16, 64, P, 4, None) == 1          # NULL
    assert L.dsa_index_scores(P, P, P, None, -1, 4, 4, 16, 64, P, 4, None) == 2            # negative B
    assert L.dsa_index_scores(P, P, P, None, 1, 4, 4, 16, 64, P, 3, None) == 2             # ld < Tk
    assert b"ld must be >= Tk" in L.dsa_last_error()
    assert L.dsa_index_scores(P, P, P, None, 1, 4, 4, 3, 64, P, 4, None) == 3              # H_I
    assert L.dsa_index_scores(P, P, P, None, 1, 4, 4, 16, 48, P, 4, None) == 3             # d_I
    assert L.dsa_index_scores(None, None, None, None, 0, 4, 4, 16, 64, None, 4, None) == 0  # empty batch


def test_topk_argument_checks(L):
    P = ctypes.c_void_p(16)
    assert L.dsa_topk(P, 8, None, 1, 2, 8, 0, P, None, 0, None) == 2          # k = 0
    assert L.dsa_topk(P, 8, None, 1, 2, 8, 4097, P, None, 0, None) == 3       # k too large
    assert L.dsa_topk(None, 8, None, 1, 2, 8, 4, P, None, 0, None) == 1       # NULL scores
    assert L.dsa_topk(P, 8, None, 1, 2, (1 << 24) + 1, 4, P, None, 0, None) == 2  # ld < Tk
    assert L.dsa_topk(None, 8, None, 0, 2, 8, 4, None, None, 0, None) == 0    # empty batch


def test_attention_argument_checks(L):
    P = ctypes.c_void_p(16)
    f = ctypes.c_float
    # MLA shape, fp8 without scale
    assert L.dsa_sparse_attn(P, P, None, None, 1, P, 1, 4, 4, 16, 1, 576, 512, 4, f(0.04), P, None, None, 0, None) == 1
    # unsupported widths
    assert L.dsa_sparse_attn(P, P, None, None, 0, P, 1, 4, 4, 16, 1, 128, 128, 4, f(0.04), P, None, None, 0, None) == 3
    # H not a multiple of Hkv
    assert L.dsa_sparse_attn(P, P, None, P, 0, P, 1, 4, 4, 6, 4, 32, 32, 4, f(0.1), P, None, None, 0, None) == 2
    # non-finite scale
    assert L.dsa_sparse_attn(P, P, None, None, 0, P, 1, 4, 4, 16, 1, 576, 512, 4, f(float("inf")), P, None, None, 0,
                             None) == 2
    # decode shape needs split-key workspace: missing -> DSA_ERR_WORKSPACE
    shp = dsa.Shape(64, 1, 65536, 16, 64, 16, 1, 576, 512, 2048, 0.04, 1, None)
    need = L.dsa_workspace_size(ctypes.byref(shp), dsa.OP_ATTN)
    assert need > 0
    assert L.dsa_sparse_attn(P, P, P, None, 1, P, 64, 1, 65536, 16, 1, 576, 512, 2048, f(0.04), P, None, None, 0,
                             None) == 5
    assert L.dsa_sparse_attn(P, P, P, None, 1, P, 64, 1, 65536, 16, 1, 576, 512, 2048, f(0.04), P, None, P,
                             need - 1, None) == 5
    # unknown kv dtype
    assert L.dsa_sparse_attn(P, P, None, None, 7, P, 1, 4, 4, 16, 1, 576, 512, 4, f(0.04), P, None, None, 0, None) == 2
    # MXFP4 rows: no kv_scale, no separate v, MLA form only; a cache past the 32-bit row
    # offsets (more than 2^32 - 4096 bytes: 13,421,761 rows of 320 bytes) is rejected
    assert L.dsa_sparse_attn(P, P, P, None, 2, P, 1, 4, 4, 16, 1, 576, 512, 4, f(0.04), P, None, None, 0, None) == 3
    assert L.dsa_sparse_attn(P, P, None, P, 2, P, 1, 4, 4, 16, 1, 576, 512, 4, f(0.04), P, None, None, 0, None) == 3
    assert L.dsa_sparse_attn(P, P, None, P, 2, P, 1, 4, 4, 4, 4, 32, 32, 4, f(0.1), P, None, None, 0, None) == 3
    assert L.dsa_sparse_attn(P, P, None, None, 2, P, 1, 4, 13421761, 16, 1, 576, 512, 4, f(0.04), P, None, None, 0,
                             None) == 3
    assert L.dsa_sparse_attn(P, P, None, None, 0, P, 1, 4, 3728302, 16, 1, 576, 512, 4, f(0.04), P, None, None, 0,
                             None) == 3  # bf16: 1152-byte rows


def test_alignment_checks(L):
    P = ctypes.c_void_p(16)   # 16-byte aligned
    U = ctypes.c_void_p(24)   # 8-byte aligned only
    H = ctypes.c_void_p(18)   # 2-byte aligned only
    f = ctypes.c_float
    assert L.dsa_index_scores(U, P, P, None, 1, 4, 4, 16, 64, P, 4, None) == 3    # q_idx
    assert L.dsa_index_scores(P, U, P, None, 1, 4, 4, 16, 64, P, 4, None) == 3    # k_idx
    assert L.dsa_index_scores(P, P, H, None, 1, 4, 4, 16, 64, P, 4, None) == 3    # w_idx, H_I = 16
    assert L.dsa_topk(H, 8, None, 1, 2, 8, 4, P, None, 0, None) == 3              # scores
    assert L.dsa_topk(P, 8, None, 1, 2, 8, 4, H, None, 0, None) == 3              # idx
    mla = (1, 4, 4, 16, 1, 576, 512, 4, f(0.04))
    assert L.dsa_sparse_attn(U, P, None, None, 0, P, *mla, P, None, None, 0, None) == 3   # q
    assert L.dsa_sparse_attn(P, U, None, None, 0, P, *mla, P, None, None, 0, None) == 3   # kv
    assert L.dsa_sparse_attn(P, P, None, None, 0, H, *mla, P, None, None, 0, None) == 3   # idx
    assert L.dsa_sparse_attn(P, P, None, None, 0, P, *mla, U, None, None, 0, None) == 3   # out
    assert b"aligned" in L.dsa_last_error()


def _patterns():
    for line in open(golden("indexcache_patterns.txt")):
        if line.strip() and not line.startswith("#"):
            yield line.split()[1]


def test_pattern_checks_agree_with_the_oracle(L):
    for pat in _patterns():
        dsa.check_pattern(pat)
        oracle.check_pattern(pat, len(pat))
    for bad, n in (("FSX", 3), ("SFF", 3), ("FS", 3), ("FFFF", 3)):
        with pytest.raises(dsa.DSAError):
            dsa.check_pattern(bad, n)
        with pytest.raises(ValueError):
            oracle.check_pattern(bad, n)
    dsa.check_pattern("SFF", prefilled=True)
    for freq in (1, 2, 3, 4, 7):
        for n in (1, 27, 61):
            assert dsa.pattern_from_freq(freq, n) == oracle.pattern_from_freq(freq, n)
    assert dsa.pattern_from_freq(3, 27) == "FSS" * 9
    with pytest.raises(dsa.DSAError):
        dsa.pattern_from_freq(0, 5)


def test_layer_stack_rejects_before_enqueueing(L):
    P = ctypes.c_void_p(16)
    shp = dsa.Shape(1, 64, 64, 16, 64, 16, 1, 576, 512, 32, 0.04, 0, None)
    io = (dsa.LayerIO * 2)()
    io[0] = dsa.LayerIO(None, None, None, 16, 16, None, None, 16, None)  # F layer without indexer inputs
    io[1] = dsa.LayerIO(None, None, None, 16, 16, None, None, 16, None)
    assert L.dsa_layer_stack(b"FS", 2, io, ctypes.byref(shp), P, 0, P, 1 << 30, None) == 1
    assert L.dsa_layer_stack(b"SS", 2, io, ctypes.byref(shp), P, 0, P, 1 << 30, None) == 4
    io[0] = dsa.LayerIO(16, 16, 16, 16, 16, None, None, 16, None)
    need = L.dsa_workspace_size(ctypes.byref(shp), dsa.OP_STACK)
    assert need >= 64 * 64 * 4
    assert L.dsa_layer_stack(b"FS", 2, io, ctypes.byref(shp), P, 0, P, need - 1, None) == 5
    assert L.dsa_layer_stack(b"FS", 2, io, ctypes.byref(shp), None, 0, P, need, None) == 1


def test_stack_chunk_rows_bound_the_score_chunk(L):
    for B, T in ((1, 65536), (1, 16384), (1, 2057), (64, 65536), (1, 100)):
        shp = dsa.Shape(B, T if B == 1 else 1, T, 16, 64, 16, 1, 576, 512, 2048, 0.04, 0, None)
        rows = L.dsa_stack_chunk_rows(ctypes.byref(shp))
        assert 1 <= rows <= max(1, shp.Tq)
        assert B * rows * ((T + 63) // 64 * 64) * 4 <= max(1 << 30, B * ((T + 63) // 64 * 64) * 4)


def test_index_topk_argument_checks(L):
    P = ctypes.c_void_p(16)
    f = ctypes.c_float
    args = lambda **kw: dict(dict(q=P, k=P, w=P, B=1, Tq=4, Tk=4, H_I=16, d_I=64, topk=2, os=f(0.0), idx=P,
                                  ws=P, nb=1 << 20), **kw)

    def call(**kw):
        a = args(**kw)
        return L.dsa_index_topk(a["q"], a["k"], a["w"], None, a["B"], a["Tq"], a["Tk"], a["H_I"], a["d_I"], a["topk"],
                                a["os"], a["idx"], a["ws"], a["nb"], None)

    assert call(q=None) == 1                          # NULL q_idx
    assert call(idx=None) == 1                        # NULL idx
    assert call(topk=0) == 2                          # k = 0
    assert call(topk=4097) == 3                       # k too large
    assert call(H_I=3) == 3                           # H_I
    assert call(B=-1) == 2                            # negative B
    assert call(os=f(float("nan"))) == 2              # oversample
    assert call(ws=None, nb=0) == 5                   # no workspace
    assert call(q=None, k=None, w=None, idx=None, B=0) == 0  # empty batch
    assert call(ws=ctypes.c_void_p(24)) == 3          # unaligned workspace


def test_index_topk_workspace_follows_the_route(L):
    def size(B, Tq, Tk, H_I, k, op):
        shp = dsa.Shape(B, Tq, Tk, H_I, 64, 16, 1, 576, 512, k, 0.04, 0, None)
        return L.dsa_workspace_size(ctypes.byref(shp), op)

    # fused (16 heads, many rows): sample keys (Tk/16 per row), thresholds, counts and 6144
    # candidate slots of 8 bytes per row; nothing of size Tq x Tk
    fused = size(1, 65536, 65536, 16, 2048, dsa.OP_INDEX_TOPK)
    assert 65536 * (4096 * 4 + 6144 * 8) <= fused <= 65536 * (4096 * 4 + 6144 * 8 + 64) + 4096
    # few rows (decode): score chunks, then the split top-k's segment lists (16 segments of
    # 1024 entries of 8 bytes, and a 16-byte word each: list length, theta, largest key)
    lists = 64 * 16 * (1024 * 8 + 16)
    assert size(64, 1, 65536, 16, 2048, dsa.OP_INDEX_TOPK) == 64 * 65536 * 4 + lists
    assert size(64, 1, 65536, 16, 2048, dsa.OP_TOPK) == lists
    # 2 indexer heads: score chunks (at most 1 GiB here)
    assert size(1, 3072, 3072, 2, 512, dsa.OP_INDEX_TOPK) == 3072 * 3072 * 4
    # up to 6144 keys (every row keeps all its keys): score rows too
    assert size(1, 6144, 6144, 16, 2048, dsa.OP_INDEX_TOPK) == 6144 * 6144 * 4
    assert size(1, 6200, 6200, 16, 2048, dsa.OP_INDEX_TOPK) >= 6200 * 6144 * 8
    # the stack holds either route plus attention
    st = size(1, 65536, 65536, 16, 2048, dsa.OP_STACK)
    assert st >= fused and st >= 4096 * 65536 * 4


def test_topk_workspace_sizes_and_checks(L):
    def size(B, Tq, Tk, k):
        shp = dsa.Shape(B, Tq, Tk, 16, 64, 1, 1, 1, 1, k, 1.0, 0, None)
        return L.dsa_workspace_size(ctypes.byref(shp), dsa.OP_TOPK)

    # split only for fewer than 1024 rows of 6145..65536 keys with room for 2k in the lists
    assert size(64, 1, 65536, 2048) == 64 * 16 * (1024 * 8 + 16)
    assert size(3, 40, 65536, 4096) == 120 * 16 * (1024 * 8 + 16)
    assert size(64, 1, 6144, 2048) == 0
    assert size(64, 1, 65537, 2048) == 0
    assert size(1, 1024, 65536, 2048) == 0
    assert size(1, 1, 28672, 2048) == 0 and size(1, 1, 28673, 2048) > 0
    P = ctypes.c_void_p(256)
    need = size(1, 2, 65536, 64)
    assert L.dsa_topk(P, 65536, None, 1, 2, 65536, 64, P, P, need - 1, None) == 5  # small ws
    assert b"topk workspace too small" in L.dsa_last_error()
    assert L.dsa_topk(P, 65536, None, 1, 2, 65536, 64, P, ctypes.c_void_p(264), need, None) == 3  # ws alignment


def test_indexer_kl_argument_checks(L):
    P = ctypes.c_void_p(16)
    f = ctypes.c_float
    kl = lambda *a: L.dsa_indexer_kl(*a[:-1], None, 0, a[-1])  # no workspace
    # MLA-width main attention: unsupported
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 16, 576, 4, f(0.04), P, None, None, None, None) == 3
    # indexer width outside {16,32,64,128}
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 24, 4, 32, 4, f(0.1), P, None, None, None, None) == 3
    # too many keys per row: kk > 4096, or the dense warm-up with Tk > 4096
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 4097, f(0.1), P, None, None, None, None) == 3
    assert kl(P, P, P, P, P, None, None, 1, 4, 5000, 2, 16, 4, 32, 0, f(0.1), P, None, None, None, None) == 3
    # missing loss / inputs; kk < 1 with idx
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 4, f(0.1), None, None, None, None, None) == 1
    assert kl(None, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 4, f(0.1), P, None, None, None, None) == 1
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 0, f(0.1), P, None, None, None, None) == 2
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 4, f(float("nan")), P, None, None, None, None) == 2
    # empty batch without key gradients: nothing to do
    assert kl(None, None, None, None, None, None, None, 0, 4, 8, 2, 16, 4, 32, 4, f(0.1), None, None, None, None,
              None) == 0
    # key gradients need the workspace; 16-byte alignment is not enough
    need = dsa.indexer_kl_workspace_size(1, 4, 8, 2, 16, kk=4)
    assert kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 4, f(0.1), P, None, None, P, None) == 5
    assert L.dsa_indexer_kl(P, P, P, P, P, P, None, 1, 4, 8, 2, 16, 4, 32, 4, f(0.1), P, None, None, P,
                            ctypes.c_void_p(16), need, None) == 3
    # key and entry counts past the 32-bit sort
    assert kl(P, P, P, P, P, P, None, 1 << 16, 1 << 10, 1 << 15, 2, 16, 4, 32, 4, f(0.1), P, None, None, P,
              None) == 3


def test_indexer_kl_workspace_sizes():
    # index lists: every entry's head terms, the two ping-pong (key, entry) arrays, the
    # per-tile digit counts and the per-key offsets
    B, Tq, Tk, H_I, kk = 1, 3072, 3072, 2, 512
    E = B * Tq * kk
    sparse = dsa.indexer_kl_workspace_size(B, Tq, Tk, H_I, 16, kk=kk)
    assert E * H_I * 4 + 4 * E * 4 + (B * Tk + 1) * 4 <= sparse <= E * (H_I * 4 + 16) + 2 ** 20
    # dense warm-up: the head terms of every (row, key) pair, no sort
    dense = dsa.indexer_kl_workspace_size(B, Tq, Tk, H_I, 16)
    assert B * Tq * Tk * H_I * 4 <= dense < B * Tq * Tk * H_I * 4 + 512
    assert dsa.indexer_kl_workspace_size(0, 5, 5, 2, 16) == 0
    assert dsa.indexer_kl_workspace_size(2, 0, 7, 2, 16, kk=3) > 0  # per-key offsets only


def test_paged_argument_checks(L):
    P = ctypes.c_void_p(16)
    f = ctypes.c_float
    good = dsa.PagedKV(16, 47, 64, 100)      # 47 * 64 >= 3000 keys
    bad_page = dsa.PagedKV(16, 47, 48, 100)  # not a power of two
    short = dsa.PagedKV(16, 10, 64, 100)     # 640 < Tk
    no_table = dsa.PagedKV(None, 47, 64, 100)
    huge = dsa.PagedKV(16, 47, 65536, 1 << 16)  # 2^32 rows: past the 32-bit offsets
    idx_call = lambda pg: L.dsa_index_scores_paged(P, P, P, ctypes.byref(pg), None, 1, 4, 3000, 16, 64, P, 3000, None)
    assert idx_call(bad_page) == 3
    assert idx_call(short) == 2
    assert idx_call(no_table) == 1
    assert idx_call(huge) == 3
    assert L.dsa_index_scores_paged(P, P, P, None, None, 1, 4, 3000, 16, 64, P, 3000, None) == 1
    attn = lambda pg, ws, nb: L.dsa_sparse_attn_paged(P, P, P, 1, ctypes.byref(pg), P, None, 4, 1, 3000, 16, 576, 512,
                                                       2048, f(0.04), P, None, ws, nb, None)
    assert attn(bad_page, P, 1 << 30) == 3
    assert attn(good, None, 0) == 5          # workspace: the selected keys' pool rows
    assert L.dsa_sparse_attn_paged(P, P, None, 1, ctypes.byref(good), P, None, 4, 1, 3000, 16, 576, 512, 2048,
                                   f(0.04), P, None, P, 1 << 30, None) == 1  # fp8 pool without scales
    assert L.dsa_sparse_attn_paged(P, P, None, 0, ctypes.byref(good), P, None, 4, 1, 3000, 4, 32, 32, 64,
                                   f(0.1), P, None, P, 1 << 30, None) in (2, 3)  # multi-head form: not paged
    shp = dsa.Shape(4, 1, 3000, 16, 64, 16, 1, 576, 512, 2048, 0.04, 1, None)
    need = L.dsa_workspace_size(ctypes.byref(shp), dsa.OP_ATTN_PAGED)
    assert need >= 4 * 2048 * 4
    assert L.dsa_workspace_size(ctypes.byref(shp), dsa.OP_STACK_PAGED) >= need
