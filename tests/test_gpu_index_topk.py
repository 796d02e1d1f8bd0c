"""GPU parity of the fused indexer -> top-k (dsa_index_topk) through the C ABI.

Its indices must equal, bit for bit, the oracle's top-k run on the score rows the GPU
indexer produces (the same rule the unfused top-k is held to), for rows of every kind:
shorter than k, short enough to keep every key, and long rows that go through the sampled
threshold; and also where the candidate lists fail on purpose (an oversample factor far too
small or too large, or massive score ties) and the exact recomputation takes over.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

dsa = pytest.importorskip("deepseek_sparse_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host(x):
    return x.detach().cpu()


def _fused_route(B, Tq, Tk, H_I, d_I, k):
    # the fused route's workspace holds candidate lists (6144 x 8 bytes per row), the score
    # route's one chunk of Tk-wide fp32 rows; the two sizes tell the routes apart here
    shp = dsa.Shape(B, Tq, Tk, H_I, d_I, 16, 1, 576, 512, k, 0.04, 0, None)
    return dsa.workspace_size(shp, dsa.OP_INDEX_TOPK) >= B * Tq * 6144 * 8


def _check(d, k, kv_len=None, oversample=0.0):
    q, kk, w = (d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx"))
    B, Tq, H_I, d_I = q.shape
    Tk = kk.shape[1]
    assert _fused_route(B, Tq, Tk, H_I, d_I, k)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    got = _host(dsa.index_topk(q, kk, w, k, kv_len=kl, oversample=oversample)).numpy()
    s = dsa.index_scores(q, kk, w, kv_len=kl)
    ref = oracle.topk(_host(s).numpy(), k, kv_len=kv_len, Tk=Tk)
    assert np.array_equal(got, ref)
    # and the unfused GPU route agrees
    assert np.array_equal(got, _host(dsa.topk(s, k, kv_len=kl)).numpy())
    return got


@pytest.mark.parametrize("key,T,k,H_I,d_I", [
    ("D", 7000, 2048, 16, 64),   # rows < k, rows kept whole (<= 6144 keys), sampled rows
    ("B", 8192, 1024, 16, 128),  # the widest indexer keys
    ("B", 7000, 512, 8, 64),     # 8 indexer heads: 16 rows per wave
    ("B", 6500, 64, 16, 32),     # small k: oversample capped at 4
])
def test_index_topk_matches_scores_then_topk(key, T, k, H_I, d_I):
    print(f"index_topk workload {key} T={T} k={k} H_I={H_I} d_I={d_I}", flush=True)
    w = synth.workload(key, T=T, k=k, H_I=H_I, d_I=d_I)
    _check(synth.layer_inputs(w, indexer=True), k)


def test_index_topk_batch_with_ragged_kv_len():
    # two sequences; the second's rows start before position 0 (p < 0: all padding)
    print("index_topk B=2 ragged kv_len", flush=True)
    w = synth.workload("B", B=2, T=7000, k=512)
    got = _check(synth.layer_inputs(w, indexer=True), 512, kv_len=[7000, 1200])
    assert np.all(got[1, :5800] == -1)


def test_index_topk_short_keys_take_the_score_route():
    # up to 6144 keys every row keeps all its keys: the call runs the score kernel + top-k
    print("index_topk short rows", flush=True)
    w = synth.workload("B", T=3000, k=512)
    d = synth.layer_inputs(w, indexer=True)
    assert not _fused_route(1, 3000, 3000, 16, 64, 512)
    q, kk, wi = (d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx"))
    got = _host(dsa.index_topk(q, kk, wi, 512)).numpy()
    ref = oracle.topk(_host(dsa.index_scores(q, kk, wi)).numpy(), 512)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("oversample", [0.05, 40.0])
def test_index_topk_failed_lists_are_recomputed_exactly(oversample):
    # 0.05: every sampled row's list ends shorter than k; 40: every sampled row's list
    # overflows its 6144 slots.  Either way the exact pass must produce the same indices.
    print(f"index_topk forced fallback oversample={oversample}", flush=True)
    w = synth.workload("D", T=9000)
    _check(synth.layer_inputs(w, indexer=True), 2048, oversample=oversample)


def test_index_topk_integer_scores_with_massive_ties():
    # small-integer scores: thousands of keys share the threshold value, lists overflow and
    # ties at the k-th value are resolved by position in the exact pass
    print("index_topk integer scores", flush=True)
    d = synth.integer_indexer_inputs(1, 8000, 16, 64, seed=8101, qk_max=1, w_max=2)
    _check(d, 2048)


def test_layer_stack_fused_and_unfused_agree():
    # 6600 query rows: the stack's 'F' layers take the fused route unless told not to
    print("layer stack fused vs unfused FSF", flush=True)
    w = synth.workload("C", T=6600, k=512, pattern="FSF")
    layers = []
    for l in range(3):
        layers.append({k: (v.to(DEV) if v is not None else None) for k, v in synth.layer_inputs(w, l).items()})
    a = dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=512)
    b = dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=512, unfused=True)
    torch.cuda.synchronize()
    assert torch.equal(a[2], b[2])
    for x, y in zip(a[0], b[0]):
        assert torch.equal(x, y)
    s2 = dsa.index_scores(layers[2]["q_idx"], layers[2]["k_idx"], layers[2]["w_idx"])
    assert np.array_equal(_host(a[2]).numpy(), oracle.topk(_host(s2).numpy(), w.k))


def _decode_lists_check(q, kk, w, k, kv_len, rows):
    # index_topk on one query row per sequence takes the score route; where the held decode
    # indexer builds the split top-k's segment lists itself, the indices must still equal
    # the oracle's top-k on the GPU's score rows (sampled sequences) and, on every row, the
    # one-workgroup top-k of those rows and the segment-kernel route
    B, Tk = q.shape[0], kk.shape[1]
    kl = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    got = dsa.index_topk(q, kk, w, k, kv_len=kl)
    s = dsa.index_scores(q, kk, w, kv_len=kl)
    assert torch.equal(got, dsa.topk(s, k, kv_len=kl, split=False))
    assert torch.equal(got, dsa.topk(s, k, kv_len=kl))
    for b in rows:
        ref = oracle.topk(_host(s[b:b + 1]).numpy(), k, kv_len=[kv_len[b]], Tk=Tk)
        assert np.array_equal(_host(got[b:b + 1]).numpy(), ref), b


@pytest.mark.parametrize("B,Tk,k", [(64, 65536, 2048), (64, 32768, 2048), (256, 8192, 512)])
def test_decode_index_topk_lists_from_the_indexer(B, Tk, k):
    # on 256 CUs: two segments per indexer workgroup at (64, 65536), one at the other two;
    # ragged lengths put some rows' last segments in part of a workgroup, and some rows
    # too short for lists (the merge's one-workgroup path)
    print(f"decode index_topk lists B={B} Tk={Tk} k={k}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(B + Tk + k)
    q = (torch.randn(B, 1, 16, 64, generator=g) / 8).to(torch.bfloat16).to(DEV)
    kk = (torch.randn(B, Tk, 64, generator=g) / 8).to(torch.bfloat16).to(DEV)
    w = torch.randn(B, 1, 16, generator=g).to(torch.bfloat16).to(DEV)
    kv_len = [Tk - (b % 7) * 1111 for b in range(B)]
    kv_len[1] = k + 1
    kv_len[2] = Tk - 4091  # a last segment of 5 keys
    _decode_lists_check(q, kk, w, k, kv_len, rows=(0, 1, 2, 3, B - 1))


def test_decode_index_topk_lists_cannot_decide_or_overflow():
    # scores rising with position put a row's whole top-k in its last segments, so the
    # lists' union above the largest segment threshold holds fewer than k keys (the merge
    # redoes the row); small-integer scores give one value to thousands of keys, so lists
    # overflow.  Half the sequences each.
    print("decode index_topk lists: rising scores and massive ties", flush=True)
    B, Tk, k = 64, 65536, 2048
    d = synth.integer_query_rows_inputs(B, 1, Tk, 16, 64, seed=4242)
    q, kk, w = d["q_idx"].clone(), d["k_idx"].clone(), d["w_idx"].clone()
    ramp = (torch.arange(Tk, dtype=torch.float32) / Tk).to(torch.bfloat16)
    kk[: B // 2] = ramp[None, :, None].expand(B // 2, Tk, 64)
    q[: B // 2] = 1
    w[: B // 2] = 1
    kv_len = [Tk - (b % 3) * 4000 for b in range(B)]
    _decode_lists_check(q.to(DEV), kk.to(DEV), w.to(DEV), k, kv_len, rows=(0, 5, B // 2, B - 1))
