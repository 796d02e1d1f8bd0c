"""dsa_sparse_attn_noalloc (the entry point for callers that cannot allocate) against
dsa_sparse_attn with a caller workspace, through the C ABI: bit-identical outputs on two
calls in a row (the second smaller, reusing the built-in scratch), shapes that need no
scratch, and every shape's partials within the built-in scratch."""
import numpy as np
import pytest
import torch

import oracle
import synth

dsa = pytest.importorskip("deepseek_sparse_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _decode_case(B, L, k, fmt, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, 576, generator=g)
    q = (torch.randn(B, 1, 16, 576, generator=g) * 4.0).to(torch.bfloat16)
    s = np.random.default_rng(seed).standard_normal((B, 1, L)).astype(np.float32)
    lens = [L - (13 * b) % (L // 2) for b in range(B)]
    idx = torch.from_numpy(oracle.topk(s, k, kv_len=lens, Tk=L))
    if fmt == "fp8":
        codes, sc = synth.fp8_e4m3_rows(x)
        return q, codes.unsqueeze(2), sc, idx
    return q, x.to(torch.bfloat16).unsqueeze(2), None, idx


def _same_as_workspace_call(q, kv, sc, idx):
    q, kv, idx = q.to(DEV), kv.to(DEV), idx.to(DEV)
    sc = None if sc is None else sc.to(DEV)
    a, la = dsa.sparse_attn_noalloc(q, kv, idx, 1.0 / 24, kv_scale=sc, Dv=512)
    b, lb = dsa.sparse_attn(q, kv, idx, 1.0 / 24, kv_scale=sc, Dv=512)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    return a, la


def test_noalloc_attention_equals_workspace_call_twice_then_smaller():
    print("noalloc attention: 64 x 4096 fp8 decode, then 5 x 3000 bf16", flush=True)
    shp = dsa._shape(64, 1, 4096, 16, 1, 576, 512, 2048, 1.0 / 24, dsa.KV_FP8_E4M3)
    need = dsa.workspace_size(shp, dsa.OP_ATTN)
    assert 0 < need <= dsa.noalloc_scratch_bytes()
    q, kv, sc, idx = _decode_case(64, 4096, 2048, "fp8", seed=1)
    out1, lse1 = _same_as_workspace_call(q, kv, sc, idx)
    # the second call is smaller and leaves most of the scratch holding the first's partials
    q2, kv2, sc2, idx2 = _decode_case(5, 3000, 512, "bf16", seed=2)
    out2, lse2 = _same_as_workspace_call(q2, kv2, sc2, idx2)
    ref, rlse = oracle.sparse_attn(q2, kv2, idx2.numpy(), 1.0 / 24, Dv=512)
    err = np.max(np.abs(out2.cpu().double().numpy() - ref))
    assert err <= 2e-2 * np.max(np.abs(ref))
    assert np.max(np.abs(lse2.cpu().double().numpy() - rlse)) <= 1e-3
    # and the first result again, after the smaller call
    again, lagain = dsa.sparse_attn_noalloc(q.to(DEV), kv.to(DEV), idx.to(DEV), 1.0 / 24, kv_scale=sc.to(DEV), Dv=512)
    torch.cuda.synchronize()
    assert torch.equal(again, out1) and torch.equal(lagain, lse1)


def test_noalloc_attention_without_scratch_and_every_shape_fits():
    print("noalloc attention: prefill rows (no scratch), split shapes within the scratch", flush=True)
    w = synth.workload("B", T=300, k=64)
    d = synth.sharp_attention_inputs(w)
    idx = torch.from_numpy(oracle.topk(np.random.default_rng(3).standard_normal((1, 300, 300)).astype(np.float32), 64))
    _same_as_workspace_call(d["q"], d["kv"], None, idx)
    # the key-split planner keeps splits x (row, head group) pairs within 256, so every
    # shape's partials fit the built-in scratch
    lim = dsa.noalloc_scratch_bytes()
    for B in (1, 3, 16, 64, 100, 127, 128, 255, 256, 1000):
        for H in (16, 32, 128):
            for k in (1, 31, 64, 2048, 8192, 65536):
                shp = dsa._shape(B, 1, k, H, 1, 576, 512, k, 1.0 / 24, dsa.KV_BF16)
                assert dsa.workspace_size(shp, dsa.OP_ATTN) <= lim, (B, H, k)
