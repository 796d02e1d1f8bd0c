"""GPU parity of the indexer KL objective (dsa_indexer_kl) through the C ABI.

Loss rows and gradients against the oracle (fp64).  Tolerances, from the arithmetic: the
kernel forms logits, softmaxes and KL terms in fp32 (relative rounding ~1e-7 per step,
errors of log P and log Q of up to ~1e-6 each for |log| <= 10) and sums at most 4096
terms, so a loss row is held to 2e-5 + 1e-4 |ref|; each gradient is a sum of at most 4096
fp32 products of G = Q - P (absolute error ~1e-7 of max(P, Q)) with bf16 inputs, held to
1e-4 of its largest reference magnitude (plus 1e-7).  Inputs are scaled so that both
distributions are far from uniform (KL of order 0.1-1), and the ablation card's shape
(indexer 2 x 16, four 32-wide heads, top-512 of 3072) is the main case.
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


def _inputs(w, q_gain, qi_gain):
    d = synth.layer_inputs(w, indexer=True)
    d["q"] = (d["q"].float() * q_gain).to(torch.bfloat16)
    d["q_idx"] = (d["q_idx"].float() * qi_gain).to(torch.bfloat16)
    return d


def _compare(d, scale, idx=None, kv_len=None, check_grads=True):
    args = [d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx", "q", "kv")]
    ix = None if idx is None else torch.from_numpy(idx).to(DEV)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    loss, dq, dw, dk = dsa.indexer_kl(*args, scale, idx=ix, kv_len=kl)
    rl, rdq, rdw, rdk = oracle.indexer_kl(d["q_idx"], d["k_idx"], d["w_idx"], d["q"], d["kv"], scale, idx=idx,
                                          kv_len=kv_len)
    gl = _host(loss).double().numpy()
    assert np.all(np.abs(gl - rl) <= 2e-5 + 1e-4 * np.abs(rl)), np.max(np.abs(gl - rl))
    if check_grads:
        for name, got, ref in (("dq", dq, rdq), ("dw", dw, rdw), ("dk", dk, rdk)):
            g = _host(got).double().numpy()
            err = np.max(np.abs(g - ref))
            assert err <= 1e-4 * np.max(np.abs(ref)) + 1e-7, (name, err, np.max(np.abs(ref)))
    return gl, rl


def test_indexer_kl_ablation_shape_sparse():
    # the ablation card's shape: T=3072, top-512 keys from the indexer's own scores
    print("indexer KL ablation sparse", flush=True)
    w = synth.workload("A")
    d = _inputs(w, q_gain=6.0, qi_gain=3.0)
    s = dsa.index_scores(d["q_idx"].to(DEV), d["k_idx"].to(DEV), d["w_idx"].to(DEV))
    idx = _host(dsa.topk(s, w.k)).numpy()
    gl, rl = _compare(d, w.scale(), idx=idx)
    assert np.mean(rl[0, 600:]) > 0.05  # far from a trivial (near-zero) KL


def test_indexer_kl_dense_warmup_ragged_batch():
    # idx None: every causal key; two sequences of different lengths
    print("indexer KL dense warm-up", flush=True)
    w = synth.workload("A", B=2, T=700)
    d = _inputs(w, q_gain=6.0, qi_gain=3.0)
    _compare(d, w.scale(), idx=None, kv_len=[700, 430])


@pytest.mark.parametrize("H_I,d_I,H", [(16, 64, 16), (8, 128, 4), (4, 32, 1)])
def test_indexer_kl_wider_shapes(H_I, d_I, H):
    print(f"indexer KL H_I={H_I} d_I={d_I} H={H}", flush=True)
    w = synth.workload("A", T=600, k=256, H_I=H_I, d_I=d_I, H=H, Hkv=H)
    d = _inputs(w, q_gain=6.0, qi_gain=2.0)
    rng = np.random.default_rng(H_I + d_I)
    idx = np.full((1, 600, 256), -1, np.int32)
    for t in range(600):
        n = min(t + 1, 256 - (t % 7))  # ragged lists with -1 holes at the end
        idx[0, t, :n] = rng.choice(t + 1, size=n, replace=False)
    idx[0, 5, 0] = -1  # a hole inside a list
    _compare(d, w.scale(), idx=idx)


def test_indexer_kl_empty_rows_and_forward_only():
    print("indexer KL empty rows", flush=True)
    w = synth.workload("A", T=300, k=64)
    d = _inputs(w, q_gain=6.0, qi_gain=3.0)
    s = dsa.index_scores(d["q_idx"].to(DEV), d["k_idx"].to(DEV), d["w_idx"].to(DEV))
    idx = _host(dsa.topk(s, 64)).numpy()
    idx[0, 10:20] = -1  # rows that select nothing
    gl, rl = _compare(d, w.scale(), idx=idx)
    assert np.all(gl[0, 10:20] == 0.0)
    args = [d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx", "q", "kv")]
    loss2, *rest = dsa.indexer_kl(*args, w.scale(), idx=torch.from_numpy(idx).to(DEV), grads=False)
    assert all(r is None for r in rest)
    assert np.array_equal(_host(loss2).numpy(), gl.astype(np.float32))


def test_indexer_kl_key_gradient_is_bit_identical_across_runs():
    # many rows list the same keys (top-512 of 3072, and the dense warm-up's every causal
    # key): dk adds their terms key by key in row order, so repeated calls agree bit for bit
    print("indexer KL determinism", flush=True)
    w = synth.workload("A")
    d = _inputs(w, q_gain=6.0, qi_gain=3.0)
    args = [d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx", "q", "kv")]
    s = dsa.index_scores(*args[:3])
    ix = dsa.topk(s, w.k)
    del s
    for idx in (ix, None):
        runs = [dsa.indexer_kl(*args, w.scale(), idx=idx) for _ in range(3)]
        torch.cuda.synchronize()
        for name, pos in (("loss", 0), ("dq", 1), ("dw", 2), ("dk", 3)):
            a = runs[0][pos].cpu()
            for r in runs[1:]:
                assert torch.equal(a.view(torch.int32), r[pos].cpu().view(torch.int32)), (name, idx is None)


def test_indexer_kl_duplicates_and_two_sequences():
    # two sequences (keys b * Tk + s in the key sort), ragged lengths, lists with repeated
    # keys (each copy is a term of both distributions and of dk) and -1 holes
    print("indexer KL duplicates, B=2", flush=True)
    w = synth.workload("A", B=2, T=520, k=96)
    d = _inputs(w, q_gain=6.0, qi_gain=3.0)
    rng = np.random.default_rng(7)
    kv_len = [520, 301]
    idx = np.full((2, 520, 96), -1, np.int32)
    for b in range(2):
        for t in range(520):
            p = kv_len[b] - 520 + t
            if p < 0:
                continue
            n = min(p + 1, 80)
            idx[b, t, :n] = rng.choice(p + 1, size=n, replace=False)
            if t % 3 == 0:
                idx[b, t, n:n + 5] = idx[b, t, :5]  # five keys listed twice
    _compare(d, w.scale(), idx=idx, kv_len=kv_len)
    # and again, bit for bit
    args = [d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx", "q", "kv")]
    ix = torch.from_numpy(idx).to(DEV)
    kl = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    a = dsa.indexer_kl(*args, w.scale(), idx=ix, kv_len=kl)[3].cpu()
    b_ = dsa.indexer_kl(*args, w.scale(), idx=ix, kv_len=kl)[3].cpu()
    assert torch.equal(a.view(torch.int32), b_.view(torch.int32))


def test_indexer_kl_large_key_sort():
    # 20000 rows of 2048 entries (41M pairs): the key sort takes two 8-bit passes, the
    # first with more than 1024 scan blocks; entries drawn with repeats (early rows list
    # most of their few keys many times)
    print("indexer KL T=20000 k=2048 key sort", flush=True)
    T, kk = 20000, 2048
    w = synth.workload("A", T=T, k=kk, H_I=1, d_I=16, H=1, Hkv=1)
    d = _inputs(w, q_gain=6.0, qi_gain=3.0)
    rng = np.random.default_rng(11)
    u = rng.random((1, T, kk))
    idx = np.floor(u * (np.arange(T)[None, :, None] + 1)).astype(np.int32)
    _compare(d, w.scale(), idx=idx)
