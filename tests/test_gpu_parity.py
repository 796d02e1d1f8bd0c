"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same bytes.

Rules (comparison bars):
  * indexer scores: |gpu - ref| <= 1e-2 * M[t,s] with M = sum_j |w_tj| sum_d |q_tjd k_sd|
    (the scale of the terms being summed), and bit-exact on integer-valued inputs where
    every partial sum is exact in fp32;
  * top-k indices: bit-exact against the oracle run on the GPU's own score rows;
  * attention: within 2e-2 absolute given identical indices; on the sharp inputs also
    within 2e-2 * max|ref|, and lse within 1e-3.
Sizes span several tiles and ragged tails while keeping the oracle to seconds.
"""
import math

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


def _magnitude(q_idx, k_idx, w_idx):
    """M[b,t,s] = sum_j |w| * sum_d |q k| (float64 on the GPU)."""
    q, k, w = (x.to(DEV).double().abs() for x in (q_idx, k_idx, w_idx))
    return torch.einsum("bth,bths->bts", w, torch.einsum("bthd,bsd->bths", q, k)).cpu().numpy()


def _causal(B, Tq, Tk, kv_len=None):
    L = np.full(B, Tk) if kv_len is None else np.asarray(kv_len)
    i = np.arange(Tq)[None, :, None]
    s = np.arange(Tk)[None, None, :]
    return s <= (L[:, None, None] - Tq + i)


@pytest.mark.parametrize("H_I,d_I,T", [(16, 64, 333), (2, 16, 517), (1, 16, 100), (4, 32, 200), (8, 128, 130)])
def test_indexer_integer_inputs_bit_exact(H_I, d_I, T):
    print(f"indexer integer H_I={H_I} d_I={d_I} T={T}", flush=True)
    d = synth.integer_indexer_inputs(2, T, H_I, d_I, seed=H_I * 1000 + d_I, qk_max=1, w_max=2)
    ref = oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
    got = _host(dsa.index_scores(*(d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx")))).numpy()
    c = _causal(2, T, T)
    assert np.array_equal(got[c], ref[c])
    assert np.all(np.isneginf(got[~c]))  # written -inf by the library


@pytest.mark.parametrize("d_I", [16, 32, 64, 128])
def test_indexer_few_key_tiles_integer_inputs_bit_exact(d_I):
    # 1 .. 5 key tiles of 32 per wave, with ragged ends: the start and the end of the key
    # pipeline (tiles in flight, the first iterations' waits) on every key width; square
    # causal chunks and single query rows (whose waves split the keys)
    for T in (1, 31, 32, 33, 64, 65, 96, 97, 130, 160):
        print(f"indexer few tiles d_I={d_I} T={T}", flush=True)
        d = synth.integer_indexer_inputs(1, T, 16, d_I, seed=9000 + d_I + T, qk_max=1, w_max=2)
        ref = oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
        got = _host(dsa.index_scores(*(d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx")))).numpy()
        c = _causal(1, T, T)
        assert np.array_equal(got[c], ref[c]), T
        q, w = d["q_idx"][:, -1:].contiguous(), d["w_idx"][:, -1:].contiguous()
        ref1 = oracle.index_scores(q, d["k_idx"], w)
        got1 = _host(dsa.index_scores(q.to(DEV), d["k_idx"].to(DEV), w.to(DEV))).numpy()
        assert np.array_equal(got1, ref1), T


@pytest.mark.parametrize("d_I,Tq,Tk", [(64, 1, 5000), (32, 3, 777), (128, 8, 1500)])
def test_indexer_few_rows_integer_inputs_bit_exact(d_I, Tq, Tk):
    # a few query rows per sequence (decode shapes) take the key-streaming kernel
    print(f"indexer few rows d_I={d_I} Tq={Tq} Tk={Tk}", flush=True)
    d = synth.integer_indexer_inputs(3, Tk, 16, d_I, seed=7000 + d_I, qk_max=1, w_max=2)
    q, w = d["q_idx"][:, -Tq:].contiguous(), d["w_idx"][:, -Tq:].contiguous()
    kv_len = [Tk, Tk - 37, Tq + 5]
    ref = oracle.index_scores(q, d["k_idx"], w, kv_len=kv_len)
    kl = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    got = _host(dsa.index_scores(q.to(DEV), d["k_idx"].to(DEV), w.to(DEV), kv_len=kl)).numpy()
    c = _causal(3, Tq, Tk, kv_len)
    assert np.array_equal(got[c], ref[c])
    assert np.all(np.isneginf(got[~c]))  # written -inf by the library


@pytest.mark.parametrize("B,Tq,Tk", [(520, 1, 8192), (520, 1, 8300), (260, 2, 4000), (260, 2, 4300)])
def test_indexer_one_tile_launch_held_and_flushed_scores(B, Tq, Tk):
    # One query tile per wave (one or two rows per sequence): a wave whose rows x key tiles
    # fit 64 keeps its scores in LDS until its key stream ends, a longer one writes them 1 KB
    # at a time.  On 256 CUs the launch gives each wave 64 tiles at (520, 1, 8192) and 32 at
    # (260, 2, 4000), both held at the limit, and 65 and 34 one past it.  Sampled sequences
    # against the oracle, bit-exact; ragged lengths on some.
    print(f"indexer one-tile launch B={B} Tq={Tq} Tk={Tk}", flush=True)
    d = synth.integer_query_rows_inputs(B, Tq, Tk, 16, 64, seed=B + Tq + Tk)
    kv_len = [Tk - (b % 5) * 97 for b in range(B)]
    kl = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    got = dsa.index_scores(d["q_idx"].to(DEV), d["k_idx"].to(DEV), d["w_idx"].to(DEV), kv_len=kl)
    for b in (0, 1, B // 2 + 3, B - 1):
        ref = oracle.index_scores(d["q_idx"][b:b + 1], d["k_idx"][b:b + 1], d["w_idx"][b:b + 1],
                                  kv_len=[kv_len[b]])
        g = _host(got[b:b + 1]).numpy()
        c = _causal(1, Tq, Tk, [kv_len[b]])
        assert np.array_equal(g[c], ref[c]), b
        assert np.all(np.isneginf(g[~c])), b


@pytest.mark.parametrize("key,T", [("A", 3072), ("B", 2057), ("D", 700)])
def test_indexer_scores_within_tolerance(key, T):
    print(f"indexer workload {key} T={T}", flush=True)
    w = synth.workload(key, T=T)
    d = synth.layer_inputs(w, indexer=True)
    ref = oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
    got = _host(dsa.index_scores(*(d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx")))).numpy()
    M = _magnitude(d["q_idx"], d["k_idx"], d["w_idx"])
    c = _causal(w.B, T, T)
    err = np.abs(got[c].astype(np.float64) - ref[c])
    assert np.all(err <= 1e-2 * M[c])
    # fp32 accumulation is far inside the bar
    assert np.max(err / (M[c] + 1e-30)) < 1e-5


def test_indexer_row_slice_with_kv_len():
    w = synth.workload("B", T=300)
    d = synth.layer_inputs(w, indexer=True)
    full = _host(dsa.index_scores(*(d[x].to(DEV) for x in ("q_idx", "k_idx", "w_idx")))).numpy()
    r0, n = 123, 77
    kv_len = torch.tensor([r0 + n], dtype=torch.int32, device=DEV)
    part = _host(dsa.index_scores(d["q_idx"][:, r0:r0 + n].to(DEV), d["k_idx"].to(DEV),
                                  d["w_idx"][:, r0:r0 + n].to(DEV), kv_len=kv_len)).numpy()
    c = _causal(1, n, 300, [r0 + n])
    assert np.array_equal(part[c], full[:, r0:r0 + n][c])


def _topk_case(scores_np, k, kv_len=None):
    s = torch.from_numpy(scores_np).to(DEV)
    Tk = scores_np.shape[2]
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    got = _host(dsa.topk(s, k, kv_len=kl)).numpy()
    ref = oracle.topk(scores_np, k, kv_len=kv_len, Tk=Tk)
    return got, ref


@pytest.mark.parametrize("k", [1, 7, 64, 512, 2048])
def test_topk_bit_exact_on_random_rows(k):
    print(f"topk random k={k}", flush=True)
    rng = np.random.default_rng(k)
    T = 2600
    s = rng.standard_normal((1, 97, T)).astype(np.float32)
    got, ref = _topk_case(s, k, kv_len=[T])  # the last 97 rows of a length-T sequence
    assert np.array_equal(got, ref)


def test_topk_ties_signed_zeros_and_short_rows():
    rng = np.random.default_rng(5)
    T = 3000
    s = (rng.integers(-2, 3, size=(2, 40, T)).astype(np.float32) * 0.25)
    s[rng.random(s.shape) < 0.3] = 0.0
    s[rng.random(s.shape) < 0.3] *= -1.0
    got, ref = _topk_case(s, 512, kv_len=[T, 1500])
    assert np.array_equal(got, ref)
    # all-equal rows keep the lowest indices; rows shorter than k keep everything
    z = np.zeros((1, 600, 600), np.float32)
    got, ref = _topk_case(z, 256)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("T,k,ties", [(6144, 2048, False), (6144, 4096, False), (5000, 2048, True),
                                      (3073, 3000, True), (4000, 1, False)])
def test_topk_wave_per_row_up_to_6144_keys(T, k, ties):
    # rows of 3073..6144 keys take the wave-per-row kernel's wide instance; ragged lengths,
    # heavy ties (single-value threshold bins far above 64 members) and signed zeros
    print(f"topk wave per row T={T} k={k} ties={ties}", flush=True)
    rng = np.random.default_rng(T + k)
    if ties:
        s = rng.integers(0, 4, size=(2, 60, T)).astype(np.float32)
        z = s == 0
        s[z] = np.where(rng.random(np.count_nonzero(z)) < 0.5, -0.0, 0.0).astype(np.float32)
    else:
        s = rng.standard_normal((2, 60, T)).astype(np.float32)
    got, ref = _topk_case(s, k, kv_len=[T, T - 777])
    assert np.array_equal(got, ref)


def test_topk_threshold_bin_larger_than_candidate_list():
    # >4096 equal scores straddle the threshold: the register fallback path
    rng = np.random.default_rng(8)
    T = 9000
    s = np.zeros((1, 24, T), np.float32)
    s[0, :, ::7] = rng.standard_normal((24, (T + 6) // 7)).astype(np.float32)
    s[0, ::3] *= -1.0  # some rows hold only negatives besides the zeros
    got, ref = _topk_case(s, 2048, kv_len=[T])
    assert np.array_equal(got, ref)


def _sampled_positions(n):
    # the blocks the many-row top-k samples to set its threshold: 256 blocks of 16 positions
    bases = ((np.arange(256) * (n - 16)) // 255) & ~3
    return (bases[:, None] + np.arange(16)[None, :]).ravel()


def test_topk_many_rows_misleading_sample_retries():
    # 1024 rows (the many-row kernel); only the sampled positions carry large scores, so the
    # first threshold keeps far fewer than k keys and the filter must run again
    print("topk many rows, misleading sample", flush=True)
    rng = np.random.default_rng(21)
    Tq, Tk = 1024, 32768
    s = rng.standard_normal((1, Tq, Tk)).astype(np.float32)
    for i in range(Tq):
        n = Tk - Tq + i + 1
        s[0, i, _sampled_positions(n)] += 10.0
    got, ref = _topk_case(s, 2048)
    assert np.array_equal(got, ref)


def test_topk_many_rows_massive_ties_take_the_exact_path():
    # three distinct values (and signed zeros): the candidate list overflows on every try
    print("topk many rows, massive ties", flush=True)
    rng = np.random.default_rng(22)
    Tq, Tk = 1024, 20000
    s = rng.integers(0, 3, size=(1, Tq, Tk)).astype(np.float32)
    s[s == 0] = np.where(rng.random(np.count_nonzero(s == 0)) < 0.5, -0.0, 0.0).astype(np.float32)
    got, ref = _topk_case(s, 2048)
    assert np.array_equal(got, ref)


def test_topk_many_rows_short_and_kept_whole():
    # rows of 1977 .. 3000 keys: shorter than k (all kept) or short enough to keep every key
    print("topk many rows, short rows", flush=True)
    rng = np.random.default_rng(23)
    Tq, Tk = 1024, 3000
    s = rng.standard_normal((1, Tq, Tk)).astype(np.float32)
    got, ref = _topk_case(s, 2048)
    assert np.array_equal(got, ref)


def test_topk_long_rows_from_indexer_scores():
    print("topk on GPU indexer scores (workload D shape, T=9000)", flush=True)
    w = synth.workload("D", T=9000)
    d = synth.layer_inputs(w, indexer=True)
    rows = slice(8900, 9000)
    kv_len = torch.tensor([9000], dtype=torch.int32, device=DEV)
    s = dsa.index_scores(d["q_idx"][:, rows].to(DEV), d["k_idx"].to(DEV), d["w_idx"][:, rows].to(DEV),
                         kv_len=kv_len)
    got = _host(dsa.topk(s, 2048, kv_len=kv_len)).numpy()
    ref = oracle.topk(_host(s).numpy(), 2048, kv_len=[9000], Tk=9000)
    assert np.array_equal(got, ref)


def _attn_compare(q, kv, idx, scale, v=None, kv_scale=None, Dv=None, sharp=False):
    out, lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), scale,
                               v=None if v is None else v.to(DEV),
                               kv_scale=None if kv_scale is None else kv_scale.to(DEV), Dv=Dv)
    ref, rlse = oracle.sparse_attn(q, kv, idx, scale, v=v, kv_scale=kv_scale, Dv=Dv)
    o = _host(out).double().numpy()
    err = np.max(np.abs(o - ref))
    assert err <= 2e-2, err
    if sharp:
        assert err <= 2e-2 * np.max(np.abs(ref)), (err, np.max(np.abs(ref)))
        l = _host(lse).double().numpy()
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(l), fin)
        assert np.max(np.abs(l[fin] - rlse[fin])) <= 1e-3
    return o, ref


@pytest.mark.parametrize("sharp", [False, True])
def test_mla_attention_bf16(sharp):
    w = synth.workload("B", T=260, k=96)
    d = synth.sharp_attention_inputs(w) if sharp else synth.layer_inputs(w, indexer=False)
    s = np.random.default_rng(1).standard_normal((1, 260, 260)).astype(np.float32)
    idx = oracle.topk(s, 96)
    _attn_compare(d["q"], d["kv"], idx, w.scale(), Dv=512, sharp=sharp)


def test_mla_attention_mutated_index_is_detected():
    w = synth.workload("B", T=200, k=40)
    d = synth.sharp_attention_inputs(w)
    s = np.random.default_rng(2).standard_normal((1, 200, 200)).astype(np.float32)
    idx = oracle.topk(s, 40)
    out, _ = dsa.sparse_attn(d["q"].to(DEV), d["kv"].to(DEV), torch.from_numpy(idx).to(DEV), w.scale(), Dv=512)
    bad = idx.copy()
    rows = np.arange(60, 200)
    bad[0, rows, 0] = (bad[0, rows, 0] + 1) % 200  # one wrong key per row
    ref_bad, _ = oracle.sparse_attn(d["q"], d["kv"], bad, w.scale(), Dv=512)
    o = _host(out).double().numpy()
    per_row = np.max(np.abs(o - ref_bad), axis=(2, 3))[0, rows]
    assert np.mean(per_row > 2e-2 * np.max(np.abs(ref_bad))) > 0.5


def test_mla_attention_fp8_decode_shape():
    print("mla fp8 decode", flush=True)
    w = synth.workload("E", B=4, T=5000)
    d = synth.decode_layer_inputs(w, 0)
    rng = np.random.default_rng(3)
    idx = np.full((4, 1, 2048), -1, np.int32)
    for b in range(4):
        n = [2048, 1000, 2048, 37][b]
        idx[b, 0, :n] = np.sort(rng.choice(5000, n, replace=False))
    _attn_compare(d["q"], d["kv"], idx, w.scale(), kv_scale=d["kv_scale"], Dv=512)


def test_mla_attention_sharp_fp8():
    w = synth.workload("E", B=3, T=1200, k=300)
    d = synth.decode_layer_inputs(w, 0)
    g = torch.Generator().manual_seed(9)
    x = torch.randn(3, 1200, 576, generator=g)
    codes, sc = synth.fp8_e4m3_rows(x)
    q = (torch.randn(3, 1, 16, 576, generator=g) * (4.0 / (24 * w.scale()))).to(torch.bfloat16)
    idx = oracle.topk(np.random.default_rng(4).standard_normal((3, 1, 1200)).astype(np.float32), 300,
                      kv_len=[1200, 1200, 700], Tk=1200)
    _attn_compare(q, codes.unsqueeze(2), idx, w.scale(), kv_scale=sc, Dv=512, sharp=True)


@pytest.mark.parametrize("sharp", [False, True])
def test_mha_attention(sharp):
    w = synth.workload("A", T=700, k=128)
    d = synth.sharp_attention_inputs(w) if sharp else synth.layer_inputs(w, indexer=False)
    s = np.random.default_rng(6).standard_normal((1, 700, 700)).astype(np.float32)
    idx = oracle.topk(s, 128)
    _attn_compare(d["q"], d["kv"], idx, w.scale(), v=d["v"], sharp=sharp)


def test_attention_short_rows_equal_dense_causal():
    # rows shorter than k select every key: the result is dense causal attention
    w = synth.workload("B", T=150, k=256)
    d = synth.sharp_attention_inputs(w)
    idx = oracle.topk(np.zeros((1, 150, 150), np.float32), 256)
    out, _ = dsa.sparse_attn(d["q"].to(DEV), d["kv"].to(DEV), torch.from_numpy(idx).to(DEV), w.scale(), Dv=512)
    K = d["kv"].double().expand(-1, -1, 16, -1).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        d["q"].double().permute(0, 2, 1, 3), K, K[..., :512].contiguous(), is_causal=True, scale=w.scale())
    ref = ref.permute(0, 2, 1, 3).numpy()
    o = _host(out).double().numpy()
    assert np.max(np.abs(o - ref)) <= 2e-2 * np.max(np.abs(ref))


def _stack_layers(w, device, sharp=False):
    """Per-layer inputs of a stack; sharp: the attention q / kv of every layer are the
    sharp variant (outputs then depend on which keys a layer attends to)."""
    layers = []
    for l, c in enumerate(w.pattern):
        d = synth.layer_inputs(w, l)
        if sharp:
            d.update({x: synth.sharp_attention_inputs(w, l)[x] for x in ("q", "kv")})
        layers.append({k: (v.to(device) if v is not None else None) for k, v in d.items()})
    return layers


def test_layer_stack_fss_matches_oracle():
    print("layer stack FSSFS", flush=True)
    w = synth.workload("C", T=600, k=128, pattern="FSSFS")
    layers = _stack_layers(w, DEV, sharp=True)
    outs, lses, cache = dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=512)
    torch.cuda.synchronize()
    # F layer 3's indices from the GPU's own scores, bit-exact
    s3 = dsa.index_scores(layers[3]["q_idx"], layers[3]["k_idx"], layers[3]["w_idx"])
    ref_idx = oracle.topk(_host(s3).numpy(), w.k)
    assert np.array_equal(_host(cache).numpy(), ref_idx)
    s0 = dsa.index_scores(layers[0]["q_idx"], layers[0]["k_idx"], layers[0]["w_idx"])
    idx0 = oracle.topk(_host(s0).numpy(), w.k)
    assert not np.array_equal(idx0, ref_idx)
    # every layer on sharp inputs: layers 0-2 attend with layer 0's indices, 3-4 with layer 3's
    for l, ix in ((0, idx0), (1, idx0), (2, idx0), (3, ref_idx), (4, ref_idx)):
        ref, rlse = oracle.sparse_attn(_host(layers[l]["q"]), _host(layers[l]["kv"]), ix, w.scale(), Dv=512)
        err = np.max(np.abs(_host(outs[l]).double().numpy() - ref))
        assert err <= 2e-2 * np.max(np.abs(ref)), (l, err)
        assert np.max(np.abs(_host(lses[l]).double().numpy() - rlse)) <= 1e-3, l
        # a stale index list (the other F layer's) is far outside the bar
        other = ref_idx if ix is idx0 else idx0
        bad, _ = oracle.sparse_attn(_host(layers[l]["q"]), _host(layers[l]["kv"]), other, w.scale(), Dv=512)
        assert np.max(np.abs(_host(outs[l]).double().numpy() - bad)) > 2e-2 * np.max(np.abs(bad)), l


def test_layer_stack_shared_layers_ignore_indexer_inputs_and_reruns_are_bit_identical():
    w = synth.workload("C", T=400, k=64, pattern="FSS")
    layers = _stack_layers(w, DEV)
    a = dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=512)
    poisoned = [dict(L) for L in layers]
    for L in poisoned[1:]:
        nan = lambda shape: torch.full(shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        L["q_idx"], L["k_idx"], L["w_idx"] = nan((1, 400, 16, 64)), nan((1, 400, 64)), nan((1, 400, 16))
    b = dsa.layer_stack(w.pattern, poisoned, w.k, w.scale(), Dv=512)
    c = dsa.layer_stack(w.pattern, layers, w.k, w.scale(), Dv=512)
    for x, y, z in zip(a[0], b[0], c[0]):
        assert torch.equal(x, y) and torch.equal(x, z)
    assert torch.equal(a[2], b[2]) and torch.equal(a[2], c[2])


def test_decode_step_fss_matches_oracle():
    print("decode FSS", flush=True)
    w = synth.workload("E", B=3, T=3000)
    kcache = synth.decode_indexer_cache(w)
    layers = []
    for l in range(3):
        d = synth.decode_layer_inputs(w, l)
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
        ref, _ = oracle.sparse_attn(_host(layers[l]["q"]), _host(layers[l]["kv"]), ref_idx, w.scale(),
                                    kv_scale=_host(layers[l]["kv_scale"]), Dv=512)
        assert np.max(np.abs(_host(outs[l]).double().numpy() - ref)) <= 2e-2


def test_decode_stack_grouped_layers_match_single_calls():
    print("decode grouped layers", flush=True)
    # with few query rows the attention of an 'F' layer and the 'S' layers after it runs in
    # one launch (at most four layers per launch, fewer key splits per layer than a lone
    # call): every layer's output and lse must match a separate dsa_sparse_attn call on the
    # same indices to rounding
    pattern = "FSSSSSF"  # groups of 4 and 2 layers after the first F, then a lone F layer
    w = synth.workload("E", B=3, T=3000, pattern=pattern)
    kcache = synth.decode_indexer_cache(w)
    first = synth.decode_layer_inputs(w, 0)
    layers = []
    for l in range(len(pattern)):
        d = synth.decode_layer_inputs(w, l)
        d["q_idx"], d["w_idx"], d["k_idx"] = first["q_idx"], first["w_idx"], kcache  # both F layers: same indices
        layers.append({k: v.to(DEV) for k, v in d.items()})
    kv_len = torch.tensor([3000, 2047, 1024], dtype=torch.int32, device=DEV)
    outs, lses, cache = dsa.layer_stack(pattern, layers, 2048, w.scale(), Dv=512, kv_len=kv_len)
    torch.cuda.synchronize()
    for l in range(len(pattern)):
        o, lse = dsa.sparse_attn(layers[l]["q"], layers[l]["kv"], cache, w.scale(), kv_scale=layers[l]["kv_scale"],
                                 Dv=512)
        a, b = _host(outs[l]).double().numpy(), _host(o).double().numpy()
        assert np.max(np.abs(a - b)) <= 2.0 ** -7 * np.max(np.abs(b)), l  # rounding: a bf16 ulp at most
        assert np.max(np.abs(_host(lses[l]).double().numpy() - _host(lse).double().numpy())) <= 1e-5, l


def test_prefilled_cache_of_topk_rows_gives_the_same_layers():
    # a stack that starts with 'S' layers on a cache a previous stack wrote: with
    # DSA_CACHE_TOPK_ROWS the attention takes each row's extent from its position, without
    # it every row is scanned; both equal the layers of one stack that computes the cache
    print("prefilled cache of top-k rows", flush=True)
    w = synth.workload("E", B=5, T=3000, pattern="FSS")
    kcache = synth.decode_indexer_cache(w)
    layers = []
    for l in range(3):
        d = synth.decode_layer_inputs(w, l)
        if "q_idx" in d:
            d["k_idx"] = kcache
        layers.append({k: v.to(DEV) for k, v in d.items()})
    kv_len = torch.tensor([3000, 2047, 1024, 2049, 1], dtype=torch.int32, device=DEV)
    outs, lses, cache = dsa.layer_stack("FSS", layers, 2048, w.scale(), Dv=512, kv_len=kv_len)
    for flag in (False, True):
        o2, l2, c2 = dsa.layer_stack("SS", layers[1:], 2048, w.scale(), Dv=512, kv_len=kv_len,
                                     index_cache=cache.clone(), prefilled=True, topk_rows=flag)
        for a, b in zip(o2, outs[1:]):
            assert torch.equal(a, b), flag
        for a, b in zip(l2, lses[1:]):
            assert torch.equal(a, b), flag


def test_empty_batch_and_no_keys():
    q = torch.empty((0, 5, 16, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, 5, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((0, 5, 16), dtype=torch.bfloat16, device=DEV)
    s = dsa.index_scores(q, k, w)
    assert s.shape == (0, 5, 5)
    # kv_len 0: rows have no candidates -> all padding
    s = torch.zeros((1, 4, 10), device=DEV)
    idx = dsa.topk(s, 3, kv_len=torch.zeros(1, dtype=torch.int32, device=DEV))
    assert torch.all(idx == -1)
