"""The split top-k route (few long rows: per-segment candidate lists, then a merge per row),
through dsa_topk with its workspace, against the oracle bit for bit and against the
one-workgroup route (no workspace).  Cases: lengths around the segment and list edges,
every k, rows whose lists cannot decide (scores rising with position, so the best keys
crowd one segment), lists that overflow on ties, signed zeros, -inf entries, a sink of
boosted keys, and several rows per sequence.  Selection rule: DSV2-Lite IndexCache card,
introduction (causal budget of k keys); ties toward the lower index as in the oracle."""
import numpy as np
import pytest
import torch

import oracle

dsa = pytest.importorskip("deepseek_sparse_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(s_np, k, lens, Tq=1):
    """Rows of the last Tq positions of sequences of length lens[b]; all three routes agree."""
    B, _, T = s_np.shape
    assert dsa.workspace_size(dsa._shape(B, Tq, T, 1, 1, 1, 1, k, 1.0, dsa.KV_BF16), dsa.OP_TOPK) > 0
    s = torch.from_numpy(s_np).to(DEV)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    got = dsa.topk(s, k, kv_len=kl).cpu().numpy()
    one = dsa.topk(s, k, kv_len=kl, split=False).cpu().numpy()
    ref = oracle.topk(s_np, k, kv_len=lens, Tk=T)
    assert np.array_equal(got, ref)
    assert np.array_equal(one, ref)


def test_split_lengths_around_the_edges():
    print("topk split: lengths around segment and list edges", flush=True)
    lens = [6145, 8192, 12288, 28672, 28673, 32767, 32768, 32769, 40961, 61440, 61441, 65535, 65536, 2048, 100, 1]
    rng = np.random.default_rng(5)
    s = rng.standard_normal((len(lens), 1, 65536)).astype(np.float32)
    _check(s, 2048, lens)


@pytest.mark.parametrize("k", [1, 64, 512, 1000, 2048, 4096])
def test_split_every_k(k):
    print(f"topk split: k={k}", flush=True)
    rng = np.random.default_rng(k)
    lens = [65536, 50000, 33000, 20000, 9000, 4097]
    s = (rng.standard_normal((len(lens), 1, 65536)) * 3.0).astype(np.float32)
    _check(s, k, lens)


def test_split_rows_the_lists_cannot_decide():
    # scores rising with position: a row's best keys fill its last segments, beyond the
    # share each segment lists, so the merge takes the whole-row path
    print("topk split: best keys crowded into one segment", flush=True)
    rng = np.random.default_rng(11)
    T = 65536
    pos = np.arange(T, dtype=np.float64)
    s = np.stack([pos * 1e-3 + rng.standard_normal(T) * 0.01, -pos * 1e-3 + rng.standard_normal(T) * 0.01,
                  np.where(pos >= 40000, 5.0, 0.0) + rng.standard_normal(T)])[:, None, :].astype(np.float32)
    _check(s, 2048, [T, T, 60000])


def test_split_ties_overflow_and_signed_zeros():
    print("topk split: ties, signed zeros, -inf", flush=True)
    rng = np.random.default_rng(12)
    T = 65536
    few = rng.integers(0, 4, size=T).astype(np.float32)                   # four values
    same = np.full(T, 1.5, np.float32)                                     # one value
    zeros = np.where(rng.random(T) < 0.5, -0.0, 0.0).astype(np.float32)   # -0 == +0
    zeros[rng.choice(T, 700, replace=False)] = 1.0
    ninf = rng.standard_normal(T).astype(np.float32)
    ninf[rng.random(T) < 0.9] = -np.inf
    lumps = np.round(rng.standard_normal(T) * 4.0).astype(np.float32)     # ~30 values
    s = np.stack([few, same, zeros, ninf, lumps])[:, None, :]
    _check(s, 2048, [T, 50000, T, T, 45000])


def test_split_sink_and_many_rows():
    # boosted first 64 keys (a sink), and several query rows per sequence (Tq = 40)
    print("topk split: sink, 3 sequences x 40 rows", flush=True)
    rng = np.random.default_rng(13)
    T, Tq = 65536, 40
    s = rng.standard_normal((3, Tq, T)).astype(np.float32)
    s[:, :, :64] += 6.0
    _check(s, 2048, [T, 47000, 30000], Tq=Tq)


def test_split_full_decode_shape():
    print("topk split: 64 x 65536, k = 2048", flush=True)
    rng = np.random.default_rng(14)
    s = rng.standard_normal((64, 1, 65536)).astype(np.float32)
    lens = [65536 - 997 * b for b in range(64)]
    _check(s, 2048, lens)
