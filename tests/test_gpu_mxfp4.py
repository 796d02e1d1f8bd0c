"""GPU parity of the MXFP4 latent cache (DSA_KV_MXFP4) through the C ABI.

The kernel decodes each 320-byte row with its block scales while staging it.  The decoded
values (e2m1 times a power of two) are exact in bf16, so attention over MXFP4 rows must
equal, bit for bit, the same call over bf16 rows that hold the decoded values; and the
oracle, which decodes the bytes itself in fp64, within the bf16 path's tolerance (2e-2
absolute on the outputs; on sharp logits also 2e-2 of the largest output and 1e-3 on lse).
Rows carry garbage in the bytes the format ignores, and separate cases give some blocks
scale byte 0 (2^-127: their values are bf16 subnormals).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

dsa = pytest.importorskip("deepseek_sparse_attention_amd")

pytestmark = pytest.mark.gpu
DEV = "cuda"
D = 576
J = np.arange(D // 32)
SCALE_AT = D // 2 + 4 * (J % 8) + J // 8  # byte of block j's scale
IGNORED = sorted(set(range(D // 2, D // 2 + 32)) - set(SCALE_AT.tolist()))
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def _host(x):
    return x.detach().cpu()


def _decode_bf16(rows):
    """MXFP4 rows uint8 [..., 320] -> bf16 [..., 576] with the same values (exact)."""
    r = rows.reshape(-1, rows.shape[-1]).numpy()
    b = r[:, :D // 2].astype(np.int64)
    codes = np.stack([b & 15, b >> 4], axis=-1).reshape(r.shape[0], D)
    e = r[:, SCALE_AT].astype(np.int64)
    vals = E2M1[codes] * np.ldexp(1.0, e - 127).repeat(32, axis=1)
    t = torch.from_numpy(vals).to(torch.float32)
    out = t.to(torch.bfloat16)
    assert torch.equal(out.float(), t)  # exact in bf16, subnormals included
    return out.reshape(*rows.shape[:-1], D)


def _rough(rows, seed, zero_scales=False):
    """Garbage in the ignored bytes; with zero_scales, a few blocks with scale byte 0."""
    g = torch.Generator().manual_seed(seed)
    rows = rows.clone()
    flat = rows.view(-1, rows.shape[-1])
    flat[:, IGNORED] = torch.randint(0, 256, (flat.shape[0], len(IGNORED)), generator=g, dtype=torch.uint8)
    if zero_scales:
        pick = torch.randint(0, flat.shape[0], (max(1, flat.shape[0] // 50),), generator=g)
        flat[pick, int(SCALE_AT[5])] = 0
    return rows


def _run(q, rows, idx, scale, sharp=False):
    """MXFP4 call vs the bf16 twin (bit for bit) and vs the oracle on the raw bytes."""
    ix = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_attn(q.to(DEV), rows.to(DEV), ix, scale, Dv=512)
    out2, lse2 = dsa.sparse_attn(q.to(DEV), _decode_bf16(rows).to(DEV), ix, scale, Dv=512)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    ref, rlse = oracle.sparse_attn(q, rows, idx, scale, Dv=512)
    o = _host(out).double().numpy()
    err = np.max(np.abs(o - ref))
    assert err <= 2e-2, err
    l = _host(lse).double().numpy()
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(l), fin)
    if sharp:
        assert err <= 2e-2 * np.max(np.abs(ref)), (err, np.max(np.abs(ref)))
        assert np.max(np.abs(l[fin] - rlse[fin])) <= 1e-3
    return out, lse


def test_mxfp4_attention_decode_shape():
    # 4 sequences, one query each: the split-key path with its merge kernel; ragged lists
    print("mxfp4 decode shape", flush=True)
    w = synth.workload("E", B=4, T=5000)
    d = synth.decode_layer_inputs(w, 0, kv_format="mxfp4")
    assert d["kv"].shape == (4, 5000, 1, 320) and "kv_scale" not in d
    rows = _rough(d["kv"], 1)
    rng = np.random.default_rng(3)
    idx = np.full((4, 1, 2048), -1, np.int32)
    for b in range(4):
        n = [2048, 1000, 2048, 37][b]
        idx[b, 0, :n] = np.sort(rng.choice(5000, n, replace=False))
    idx[2, 0, 100] = -1  # a hole inside the list: skipped
    _run(d["q"], rows, idx, w.scale())
    _run(d["q"], _rough(d["kv"], 4, zero_scales=True), idx, w.scale())


def test_mxfp4_attention_prefill_shape_sharp():
    # 260 query rows of one sequence (one workgroup per row and 16 heads), sharp logits
    print("mxfp4 prefill shape sharp", flush=True)
    w = synth.workload("B", T=260, k=96)
    g = torch.Generator().manual_seed(12)
    x = torch.randn(1, 260, D, generator=g)
    rows = _rough(synth.mxfp4_rows(x).unsqueeze(2), 2)
    q = (torch.randn(1, 260, 16, D, generator=g) * (4.0 / (24 * w.scale()))).to(torch.bfloat16)
    idx = oracle.topk(np.random.default_rng(1).standard_normal((1, 260, 260)).astype(np.float32), 96)
    _run(q, rows, idx, w.scale(), sharp=True)
    _run(q, _rough(rows, 3, zero_scales=True), idx, w.scale(), sharp=True)


def test_mxfp4_attention_all_codes_and_wide_scales():
    # every code in every position, scale bytes spread over 100..150 (values up to 6 * 2^23)
    print("mxfp4 all codes", flush=True)
    rng = np.random.default_rng(21)
    T = 700
    r = rng.integers(0, 256, size=(1, T, 1, D // 2 + 32)).astype(np.uint8)
    r[..., SCALE_AT] = rng.integers(100, 151, size=(1, T, 1, len(SCALE_AT)))
    rows = torch.from_numpy(r)
    q = (torch.randn(1, 3, 32, D, generator=torch.Generator().manual_seed(5)) * 1e-9).to(torch.bfloat16)
    idx = np.sort(rng.choice(T, size=(1, 3, 200)), axis=-1).astype(np.int32)
    ix = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_attn(q.to(DEV), rows.to(DEV), ix, 0.04, Dv=512)
    out2, lse2 = dsa.sparse_attn(q.to(DEV), _decode_bf16(rows).to(DEV), ix, 0.04, Dv=512)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    ref, rlse = oracle.sparse_attn(q, rows, idx, 0.04, Dv=512)
    o = _host(out).double().numpy()
    assert np.max(np.abs(o - ref)) <= 2e-2 * np.max(np.abs(ref))


def test_mxfp4_paged_attention_matches_dense():
    print("mxfp4 paged", flush=True)
    from tests.test_gpu_paged import _paginate
    w = synth.workload("E", B=4, T=2600)
    lens = [2600, 2100, 777, 2049]
    d = synth.decode_layer_inputs(w, 1, kv_format="mxfp4")
    rows = d["kv"]
    rng = np.random.default_rng(5)
    idx = np.full((4, 1, 2048), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        m = min(2048, n)
        idx[b, 0, :m] = np.sort(rng.choice(n, size=m, replace=False))
    idx_t = torch.from_numpy(idx).to(DEV)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dense_out, dense_lse = dsa.sparse_attn(d["q"].to(DEV), rows.to(DEV), idx_t, w.scale(), Dv=512)
    pool, table, npg = _paginate(rows[:, :, 0], lens, 64, seed=13)
    pg = dsa.paged_kv(table.to(DEV), 64, npg)
    out, lse = dsa.sparse_attn_paged(d["q"].to(DEV), pool.to(DEV), idx_t, w.scale(), pg, 2600, kv_len=kl)
    assert torch.equal(out, dense_out) and torch.equal(lse, dense_lse)
    ref, _ = oracle.sparse_attn(d["q"], rows, idx, w.scale(), Dv=512)
    assert np.max(np.abs(_host(out).double().numpy() - ref)) <= 2e-2


def test_mxfp4_decode_stack_fss():
    # the decode step with MXFP4 latent caches: the F layer's indices feed both S layers
    print("mxfp4 decode FSS", flush=True)
    w = synth.workload("E", B=3, T=3000)
    kcache = synth.decode_indexer_cache(w)
    layers = []
    for l in range(3):
        d = synth.decode_layer_inputs(w, l, kv_format="mxfp4")
        if "q_idx" in d:
            d["k_idx"] = kcache
        layers.append({k: v.to(DEV) for k, v in d.items()})
    kv_len = torch.tensor([3000, 2047, 1024], dtype=torch.int32, device=DEV)
    outs, _, cache = dsa.layer_stack("FSS", layers, 2048, w.scale(), Dv=512, kv_len=kv_len)
    torch.cuda.synchronize()
    s = dsa.index_scores(layers[0]["q_idx"], layers[0]["k_idx"], layers[0]["w_idx"], kv_len=kv_len)
    ref_idx = oracle.topk(_host(s).numpy(), 2048, kv_len=[3000, 2047, 1024], Tk=3000)
    assert np.array_equal(_host(cache).numpy(), ref_idx)
    for l in range(3):
        ref, _ = oracle.sparse_attn(_host(layers[l]["q"]), _host(layers[l]["kv"]), ref_idx, w.scale(), Dv=512)
        assert np.max(np.abs(_host(outs[l]).double().numpy() - ref)) <= 2e-2


def test_mxfp4_binding_rejects_mismatched_rows():
    q = torch.zeros((1, 1, 16, D), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((1, 1, 4), dtype=torch.int32, device=DEV)
    bad = torch.zeros((1, 8, 1, 300), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        dsa.sparse_attn(q, bad, idx, 0.04, Dv=512)
    rows = torch.zeros((1, 8, 1, 320), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):  # a scale given: the rows would have to be e4m3, 576 wide
        dsa.sparse_attn(q, rows, idx, 0.04, Dv=512, kv_scale=torch.ones((1, 8), device=DEV))


def test_mxfp4_nan_scale_poisons_only_the_queries_that_select_it():
    # scale byte 255 is NaN in E8M0: a query that selects that row gets NaN outputs, as in
    # the oracle; a query that does not is unaffected
    print("mxfp4 NaN scale", flush=True)
    g = torch.Generator().manual_seed(31)
    rows = synth.mxfp4_rows(torch.randn(1, 300, D, generator=g)).unsqueeze(2)
    rows[0, 17, 0, int(SCALE_AT[3])] = 255
    q = (torch.randn(1, 2, 16, D, generator=g) * 0.05).to(torch.bfloat16)
    idx = np.full((1, 2, 64), -1, np.int32)
    idx[0, 0, :64] = np.arange(64)       # selects row 17
    idx[0, 1, :64] = np.arange(100, 164)  # does not
    out, lse = dsa.sparse_attn(q.to(DEV), rows.to(DEV), torch.from_numpy(idx).to(DEV), 0.04, Dv=512)
    ref, rlse = oracle.sparse_attn(q, rows, idx, 0.04, Dv=512)
    o, l = _host(out).double().numpy(), _host(lse).double().numpy()
    assert np.all(np.isnan(ref[0, 0])) and np.all(np.isnan(rlse[0, 0]))
    assert np.all(np.isnan(o[0, 0])) and np.all(np.isnan(l[0, 0]))
    assert np.all(np.isfinite(o[0, 1])) and np.max(np.abs(o[0, 1] - ref[0, 1])) <= 2e-2
