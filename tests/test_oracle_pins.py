"""Pins of the CPU oracle to facts other than itself (runs without a GPU).

Each test fixes the oracle against something independent: a value printed on the pages,
a library routine that computes a special case, a closed form, an algebraic identity
that a wrong sign, a dropped term or a transposed operand would break, or brute force
in exact integer arithmetic on tiny inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import masked_dense
from tests.conftest import golden

# ---------------------------------------------------------------- storage formats


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    ref = torch.from_numpy(bits.astype(np.int32).astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(int(b)) for b in bits])
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_to_double(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_fp8_generator_round_trip_is_within_half_ulp():
    x = synth.normal((64, 576), 1.0 / 24, 5)
    codes, scale = synth.fp8_e4m3_rows(x)
    dec = np.array([oracle.e4m3_to_double(c) for c in range(256)])[codes.numpy()] * scale.numpy()[:, None]
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normals, absolute 2^-10*scale below.
    err = np.abs(dec - x.numpy().astype(np.float64))
    bound = np.maximum(np.abs(x.numpy()) * 2.0 ** -4, 2.0 ** -10 * scale.numpy()[:, None])
    assert np.all(err <= bound * 1.0000001)


# OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element values by 3-bit magnitude code
# (sign in bit 3): the spec's table of representable values.
_E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_matches_the_spec_table():
    got = [oracle.e2m1_to_double(c) for c in range(16)]
    assert got[:8] == _E2M1_TABLE
    assert got[8:] == [-v for v in _E2M1_TABLE]
    assert math.copysign(1.0, got[8]) == -1.0  # code 8 is negative zero


def test_e8m0_decode_is_a_power_of_two():
    for e in (0, 1, 100, 126, 127, 128, 200, 254):
        assert oracle.e8m0_to_double(e) == math.ldexp(1.0, e - 127)
    assert math.isnan(oracle.e8m0_to_double(255))


def _decode_table_rows(rows, D):
    """Decode MXFP4 rows [N, D/2+32] with the spec's value table, vectorised."""
    tab = np.array(_E2M1_TABLE + [-v for v in _E2M1_TABLE])
    b = rows[:, :D // 2].astype(np.int64)
    codes = np.stack([b & 15, b >> 4], axis=-1).reshape(rows.shape[0], D)
    j = np.arange(D // 32)
    e = rows[:, D // 2 + 4 * (j % 8) + j // 8].astype(np.int64)
    return tab[codes] * np.ldexp(1.0, e - 127).repeat(32, axis=1)


def test_mxfp4_generator_round_trip_is_nearest_e2m1_value():
    # encoder (synth) and decoder (oracle) are separate code: a layout mistake on either
    # side (nibble order, block or scale position) breaks the round trip.  Each decoded
    # value must be the e2m1 grid point nearest x / X (X = the block's scale) after the
    # clamp to +-6, with X = 2^(floor(log2 amax) - 2).
    x = synth.normal((24, 576), 1.0 / 24, 9)
    x[3, 40] = 0.0
    x[5, 64:96] = 0.0  # an all-zero block
    rows = synth.mxfp4_rows(x).numpy()
    dec = np.stack([oracle.mxfp4_decode_row(r, 576) for r in rows])
    xd = x.numpy().astype(np.float64)
    blk = np.abs(xd).reshape(24, 18, 32).max(-1)
    X = np.where(blk > 0, np.ldexp(1.0, np.floor(np.log2(np.where(blk > 0, blk, 1.0))).astype(int) - 2), 0.0)
    X = X.repeat(32, axis=1)
    nz = X > 0
    v = np.clip(xd[nz] / X[nz], -6.0, 6.0)
    grid = np.array(sorted(set(_E2M1_TABLE + [-t for t in _E2M1_TABLE])))
    dist = np.abs(v[:, None] - grid[None, :])
    got = dec[nz] / X[nz]
    assert np.all(np.isin(got, grid))
    assert np.all(np.abs(got - v) <= dist.min(1) + 1e-12)
    assert np.all(dec[~nz] == 0.0)
    # every block's largest magnitude lands in [4, 6]: the scale is the spec's shared exponent
    amax_code = np.abs(dec / np.where(X > 0, X, 1.0)).reshape(24, 18, 32).max(-1)
    assert np.all((amax_code[blk > 0] >= 4.0) & (amax_code[blk > 0] <= 6.0))


def test_mxfp4_rounding_ties_go_to_the_even_code():
    # values exactly between two e2m1 points (scale 1: block amax 6 -> X = 2^(2-2) = 1)
    x = torch.zeros(1, 32)
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -1.0]
    x[0, :len(ties)] = torch.tensor(ties)
    x[0, 31] = 6.0
    dec = oracle.mxfp4_decode_row(synth.mxfp4_rows(x)[0].numpy(), 32)
    assert list(dec[:len(ties)]) == want and dec[31] == 6.0


def test_mxfp4_rows_equal_the_decoded_bf16_rows():
    # e2m1 values times a power-of-two scale are exact in bf16, so both paths see equal keys;
    # bytes that no block names hold garbage and must be ignored
    rng = np.random.default_rng(7)
    T, D = 24, 576
    rows = rng.integers(0, 256, size=(T, D // 2 + 32)).astype(np.uint8)
    j = np.arange(18)
    rows[:, D // 2 + 4 * (j % 8) + j // 8] = rng.integers(118, 130, size=(T, 18))
    dec = _decode_table_rows(rows, D)
    kv_bf16 = torch.from_numpy(dec).to(torch.float32).to(torch.bfloat16)
    assert np.array_equal(kv_bf16.double().numpy(), dec)
    q = (torch.randn(1, T, 16, D, generator=torch.Generator().manual_seed(3)) * 0.01).to(torch.bfloat16)
    idx = oracle.topk(rng.standard_normal((1, T, T)).astype(np.float32), 8)
    a, la = oracle.sparse_attn(q, rows.reshape(1, T, 1, -1), idx, 0.05, Dv=512)
    b, lb = oracle.sparse_attn(q, kv_bf16.reshape(1, T, 1, D), idx, 0.05, Dv=512)
    assert np.max(np.abs(a - b)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12


# ---------------------------------------------------------------- indexer


def _rand_indexer(B, T, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, T, H, D, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    k = (torch.randn(B, T, D, generator=g) / math.sqrt(D)).to(torch.bfloat16)
    w = torch.randn(B, T, H, generator=g).to(torch.bfloat16)
    return q, k, w


def test_indexer_one_hot_query_reads_back_the_key_coordinate():
    # H=1, w=1, q[t] = e_a(t): I[t,s] = max(0, k[s, a(t)]) for s <= t, -inf after.
    T, D = 37, 16
    g = torch.Generator().manual_seed(3)
    k = torch.randn(1, T, D, generator=g).to(torch.bfloat16)
    a = torch.randint(0, D, (T,), generator=g)
    q = torch.zeros(1, T, 1, D, dtype=torch.bfloat16)
    q[0, torch.arange(T), 0, a] = 1.0
    w = torch.ones(1, T, 1, dtype=torch.bfloat16)
    s = oracle.index_scores(q, k, w)
    kk = k.to(torch.float64).numpy()[0]
    for t in range(T):
        assert np.all(np.isneginf(s[0, t, t + 1:]))
        assert np.array_equal(s[0, t, : t + 1], np.maximum(kk[: t + 1, a[t]], 0.0).astype(np.float32))


def test_indexer_odd_part_is_the_weighted_linear_score():
    # max(0,x) - max(0,-x) = x, so I(q,k,w) - I(q,-k,w) = sum_j w_j q_j.k_s (a plain matmul).
    q, k, w = _rand_indexer(2, 29, 4, 16, 11)
    s_pos = oracle.index_scores(q, k, w).astype(np.float64)
    s_neg = oracle.index_scores(q, -k, w).astype(np.float64)
    lin = torch.einsum("bth,bthd,bsd->bts", w.double(), q.double(), k.double()).numpy()
    even = torch.einsum("bth,bths->bts", w.double(), torch.einsum("bthd,bsd->bths", q.double(), k.double()).abs()).numpy()
    causal = np.tril(np.ones((29, 29), bool))[None].repeat(2, 0)
    s_pos, s_neg = np.where(causal, s_pos, 0.0), np.where(causal, s_neg, 0.0)
    scale = np.abs(even) + np.abs(lin) + 1e-30
    assert np.all(np.abs((s_pos - s_neg) - lin)[causal] <= 2e-7 * scale[causal])
    # and the even part: I(q,k,w) + I(q,-k,w) = sum_j w_j |q_j.k_s|
    assert np.all(np.abs((s_pos + s_neg) - even)[causal] <= 2e-7 * scale[causal])


def test_indexer_is_linear_in_the_head_weights():
    q, k, _ = _rand_indexer(1, 23, 3, 16, 12)
    g = torch.Generator().manual_seed(4)
    w1 = torch.randint(-3, 4, (1, 23, 3), generator=g).to(torch.bfloat16)
    w2 = torch.randint(-3, 4, (1, 23, 3), generator=g).to(torch.bfloat16)
    s1, s2 = oracle.index_scores(q, k, w1), oracle.index_scores(q, k, w2)
    s12 = oracle.index_scores(q, k, (w1.float() + w2.float()).to(torch.bfloat16))
    c = np.isfinite(s12)
    mag = oracle.index_scores(q, k, torch.full_like(w1, 8.0)).astype(np.float64)
    assert np.all(np.abs(s12[c] - (s1[c].astype(np.float64) + s2[c])) <= 1e-6 * (np.abs(mag[c]) + 1e-30))


def test_indexer_head_permutation_and_key_permutation():
    q, k, w = _rand_indexer(1, 40, 5, 16, 13)
    perm = torch.tensor([3, 0, 4, 1, 2])
    s = oracle.index_scores(q, k, w)
    sp = oracle.index_scores(q[:, :, perm], k, w[:, :, perm])
    c = np.isfinite(s)
    assert np.allclose(s[c], sp[c], rtol=1e-6, atol=1e-7)
    # a single query at the last position sees every key: permuting keys permutes its row
    kp = torch.randperm(40, generator=torch.Generator().manual_seed(1))
    last = oracle.index_scores(q[:, -1:], k, w[:, -1:], kv_len=[40])
    lastp = oracle.index_scores(q[:, -1:], k[:, kp], w[:, -1:], kv_len=[40])
    assert np.array_equal(lastp[0, 0], last[0, 0, kp.numpy()])


def test_indexer_integer_inputs_match_exact_integer_brute_force():
    d = synth.integer_indexer_inputs(1, 12, 3, 16, seed=21, qk_max=2, w_max=3)
    s = oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
    q = d["q_idx"].to(torch.int64).tolist()[0]
    k = d["k_idx"].to(torch.int64).tolist()[0]
    w = d["w_idx"].to(torch.int64).tolist()[0]
    for t in range(12):
        for s_ in range(12):
            if s_ > t:
                assert s[0, t, s_] == -np.inf
                continue
            exact = 0
            for j in range(3):
                dot = sum(q[t][j][dd] * k[s_][dd] for dd in range(16))
                exact += w[t][j] * max(dot, 0)
            assert s[0, t, s_] == exact


def test_indexer_row_slices_with_kv_len_match_full_rows():
    q, k, w = _rand_indexer(2, 50, 2, 16, 14)
    full = oracle.index_scores(q, k, w)
    r0, n = 17, 9
    part = oracle.index_scores(q[:, r0:r0 + n], k, w[:, r0:r0 + n], kv_len=[r0 + n, r0 + n])
    assert np.array_equal(part, full[:, r0:r0 + n])


def test_masked_dense_indexer_agrees_with_loop_oracle():
    w_ = synth.workload("A", T=96)
    d = synth.layer_inputs(w_)
    s = oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
    ref = masked_dense.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
    c = np.isfinite(ref)
    assert np.array_equal(np.isfinite(s), c)
    assert np.all(s[c] == ref[c].astype(np.float32))  # same double sum, one rounding


def test_ablation_parameter_count_fixes_one_shared_indexer_key_per_token():
    facts = dict(line.split() for line in open(golden("ablation_params.txt")) if line.strip() and not line.startswith("#"))
    f = {k: int(v) for k, v in facts.items()}
    extra = f["params_total"] - f["params_without_indexers"]
    H, D, hidden, L = f["indexer_heads"], f["indexer_dim"], f["hidden"], f["layers"]
    # the oracle's inputs per token: q_I [H, D], one k_I [D] shared by the heads, w [H]
    w_ = synth.workload("A", T=4)
    d = synth.layer_inputs(w_)
    per_token = d["q_idx"].shape[2] * d["q_idx"].shape[3] + d["k_idx"].shape[2] + d["w_idx"].shape[2]
    assert (d["q_idx"].shape[2], d["q_idx"].shape[3]) == (H, D)
    assert L * hidden * per_token == extra == 32000
    # a key per head would not fit the count
    assert L * hidden * (H * D + H * D + H) != extra


# ---------------------------------------------------------------- top-k


def _row_scores(vals):
    v = np.asarray(vals, np.float32)[None, None, :]
    return v


def test_topk_all_equal_row_keeps_the_lowest_indices():
    T, k = 40, 7
    s = np.zeros((1, T, T), np.float32)
    idx = oracle.topk(s, k)
    for t in range(T):
        n = t + 1
        exp = list(range(min(n, k))) + [-1] * (k - min(n, k))
        assert idx[0, t].tolist() == exp


def test_topk_increasing_row_keeps_the_last_keys():
    T, k = 30, 5
    s = np.tile(np.arange(T, dtype=np.float32), (1, T, 1))
    idx = oracle.topk(s, k)
    for t in range(k, T):
        assert idx[0, t].tolist() == list(range(t - k + 1, t + 1))


def test_topk_short_rows_select_everything_like_dense():
    # "shorter than the top-k ... DSA selects every token" (DSA ablation card, Benchmarks)
    s = np.random.default_rng(0).standard_normal((2, 10, 10)).astype(np.float32)
    idx = oracle.topk(s, 16)
    for b in range(2):
        for t in range(10):
            assert idx[b, t].tolist() == list(range(t + 1)) + [-1] * (16 - t - 1)


def test_topk_signed_zero_ties_follow_index_order():
    row = np.array([-0.0, 0.0, -1.0, 0.5, -0.0, 0.0, 2.0, -0.0], np.float32)
    s = np.tile(row, (1, 8, 1))
    idx = oracle.topk(s, 4, kv_len=[8], Tk=8)
    # the last row sees all 8: 2.0 (6), 0.5 (3), then zeros in index order 0, 1
    assert idx[0, 7].tolist() == [0, 1, 3, 6]


@pytest.mark.parametrize("k", [1, 3, 8, 33])
def test_topk_matches_numpy_lexsort_with_heavy_ties(k):
    rng = np.random.default_rng(k)
    T = 33
    s = rng.integers(-3, 4, size=(2, T, T)).astype(np.float32) * np.float32(0.5)
    s[rng.random(s.shape) < 0.1] *= -1  # signed zeros among the ties
    idx = oracle.topk(s, k)
    for b in range(2):
        for t in range(T):
            n = t + 1
            cand = s[b, t, :n].astype(np.float64)
            order = np.lexsort((np.arange(n), -cand))  # score descending, then index
            sel = np.sort(order[: min(k, n)])
            exp = np.concatenate([sel, -np.ones(k - len(sel), np.int64)])
            assert np.array_equal(idx[b, t], exp)


def test_topk_selected_scores_dominate_unselected():
    rng = np.random.default_rng(7)
    T, k = 300, 64
    s = rng.standard_normal((1, T, T)).astype(np.float32)
    idx = oracle.topk(s, k)
    for t in range(k, T):
        sel = idx[0, t]
        assert len(set(sel.tolist())) == k and np.all(np.diff(sel) > 0) and sel.max() <= t
        rest = np.setdiff1d(np.arange(t + 1), sel)
        assert s[0, t, sel].min() >= s[0, t, rest].max()


def test_topk_prefix_rows_do_not_depend_on_later_tokens():
    # causal negative control: appending tokens must not change earlier rows' selections
    w_ = synth.workload("A", T=160, k=24)
    d = synth.layer_inputs(w_)
    full = oracle.topk(oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"]), 24)
    Tp = 101
    pre = oracle.topk(oracle.index_scores(d["q_idx"][:, :Tp], d["k_idx"][:, :Tp], d["w_idx"][:, :Tp]), 24)
    assert np.array_equal(pre, full[:, :Tp])


# ---------------------------------------------------------------- sparse attention


def _sdpa_causal(q, K, V, scale):
    """torch's scaled_dot_product_attention in float64, causal, heads first."""
    qt = q.double().permute(0, 2, 1, 3)
    kt = K.double().permute(0, 2, 1, 3)
    vt = V.double().permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_attention_with_all_keys_selected_equals_dense_causal_sdpa_mha():
    w_ = synth.workload("A", T=48, k=64)
    d = synth.sharp_attention_inputs(w_)
    idx = oracle.topk(np.zeros((1, 48, 48), np.float32), 64)  # t < k: every causal key
    out, _ = oracle.sparse_attn(d["q"], d["kv"], idx, w_.scale(), v=d["v"])
    ref = _sdpa_causal(d["q"], d["kv"], d["v"], w_.scale())
    assert np.max(np.abs(out - ref)) < 1e-12


def test_attention_with_all_keys_selected_equals_dense_causal_sdpa_mla():
    w_ = synth.workload("B", T=20, k=32, H=4)
    d = synth.sharp_attention_inputs(w_)
    idx = oracle.topk(np.zeros((1, 20, 20), np.float32), 32)
    out, _ = oracle.sparse_attn(d["q"], d["kv"], idx, w_.scale(), Dv=512)
    K = d["kv"].expand(-1, -1, 4, -1)
    ref = _sdpa_causal(d["q"], K, K[..., :512], w_.scale())
    assert np.max(np.abs(out - ref)) < 1e-12


def test_attention_zero_query_is_the_mean_of_selected_rows():
    w_ = synth.workload("A", T=30, k=8)
    d = synth.layer_inputs(w_)
    q = torch.zeros_like(d["q"])
    rng = np.random.default_rng(2)
    idx = np.full((1, 30, 8), -1, np.int32)
    for t in range(30):
        n = rng.integers(1, 9)
        idx[0, t, :n] = np.sort(rng.choice(30, n, replace=False))
    out, lse = oracle.sparse_attn(q, d["kv"], idx, w_.scale(), v=d["v"])
    V = d["v"].double().numpy()
    for t in range(30):
        sel = idx[0, t][idx[0, t] >= 0]
        assert np.allclose(out[0, t], V[0, sel].mean(axis=0), atol=1e-14)
        assert np.allclose(lse[0, t], math.log(len(sel)), atol=1e-14)


def test_attention_single_index_returns_that_value_row():
    w_ = synth.workload("B", T=12, k=4, H=16)
    d = synth.sharp_attention_inputs(w_)
    idx = np.full((1, 12, 4), -1, np.int32)
    pick = np.array([5, 0, 11, 3, 3, 7, 1, 2, 9, 10, 4, 6])
    idx[0, :, 2] = pick
    out, lse = oracle.sparse_attn(d["q"], d["kv"], idx, w_.scale(), Dv=512)
    kv = d["kv"].double().numpy()[0, :, 0]
    q = d["q"].double().numpy()[0]
    for t in range(12):
        assert np.array_equal(out[0, t], np.tile(kv[pick[t], :512], (16, 1)))
        assert np.allclose(lse[0, t], w_.scale() * q[t] @ kv[pick[t]], rtol=1e-13)


def test_masked_dense_attention_agrees_with_gather_oracle():
    for key, H in (("A", 4), ("B", 16)):
        w_ = synth.workload(key, T=64, k=16, H=H)
        d = synth.sharp_attention_inputs(w_)
        s = np.random.default_rng(3).standard_normal((1, 64, 64)).astype(np.float32)
        idx = oracle.topk(s, 16)
        Dv = None if d["v"] is not None else 512
        out, lse = oracle.sparse_attn(d["q"], d["kv"], idx, w_.scale(), v=d["v"], Dv=Dv)
        ref, rlse = masked_dense.sparse_attn(d["q"], d["kv"], idx, w_.scale(), v=d["v"], Dv=Dv)
        assert np.max(np.abs(out - ref)) < 1e-12 and np.max(np.abs(lse - rlse)) < 1e-12


def test_duplicate_entries_count_twice_in_both_forms():
    # an index list that names a key twice puts two terms for it in the softmax sum: with
    # q = 0 every logit is 0, so the output is the entry-weighted mean of the value rows
    # (2 V_a + V_b) / 3 and lse = ln 3; the gather form and the masked-dense form agree
    T, D = 8, 576
    g = torch.Generator().manual_seed(11)
    kv = torch.randn(1, T, 1, D, generator=g).to(torch.bfloat16)
    q = torch.zeros(1, 2, 16, D).to(torch.bfloat16)
    idx = np.array([[[3, 3, 5, -1], [1, 6, 6, 6]]], np.int32)
    V = kv[0, :, 0, :512].double().numpy()
    for out, lse in (oracle.sparse_attn(q, kv, idx, 0.05, Dv=512),
                     masked_dense.sparse_attn(q, kv, idx, 0.05, Dv=512)):
        assert np.allclose(out[0, 0], np.tile((2 * V[3] + V[5]) / 3, (16, 1)), rtol=0, atol=1e-13)
        assert np.allclose(out[0, 1], np.tile((V[1] + 3 * V[6]) / 4, (16, 1)), rtol=0, atol=1e-13)
        assert np.allclose(lse[0, 0], math.log(3), atol=1e-13) and np.allclose(lse[0, 1], math.log(4), atol=1e-13)
    # random sharp inputs with repeated entries: the two forms agree to rounding
    w_ = synth.workload("B", T=48, k=24)
    d = synth.sharp_attention_inputs(w_)
    rng = np.random.default_rng(12)
    idx = np.stack([np.sort(rng.integers(0, t + 1, size=24)) for t in range(48)])[None].astype(np.int32)
    idx[0, ::5, -3:] = -1
    out, lse = oracle.sparse_attn(d["q"], d["kv"], idx, w_.scale(), Dv=512)
    ref, rlse = masked_dense.sparse_attn(d["q"], d["kv"], idx, w_.scale(), Dv=512)
    assert np.max(np.abs(out - ref)) < 1e-12 and np.max(np.abs(lse - rlse)) < 1e-12


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_streamed_rows_equal_scores_topk_attention_composed(fmt):
    # the CPU baseline's row-streaming entry runs scores -> top-k -> attention for single
    # rows of a prefill; it must equal the three separate calls on the whole sequence, rows
    # on both sides of k and the first and last rows included
    T, k = 300, 64
    w_ = synth.workload("B", T=T, k=k)
    d = synth.layer_inputs(w_, 0, indexer=True)
    kv, sc = d["kv"], None
    if fmt == "fp8":
        codes, sc = synth.fp8_e4m3_rows(d["kv"].float()[:, :, 0])
        kv = codes.unsqueeze(2)
    elif fmt == "mxfp4":
        kv = synth.mxfp4_rows(d["kv"].float()[:, :, 0]).unsqueeze(2)
    rows = np.array([0, 1, 62, 63, 64, 65, 150, 298, 299], np.int32)
    idx_s, out_s = oracle.dsa_rows(d["q_idx"], d["k_idx"], d["w_idx"], d["q"], kv, rows, k, w_.scale(),
                                   kv_scale=sc)
    scores = oracle.index_scores(d["q_idx"], d["k_idx"], d["w_idx"])
    idx = oracle.topk(scores, k)
    ref, _ = oracle.sparse_attn(d["q"][:, rows], kv, idx[:, rows], w_.scale(), kv_scale=sc, Dv=512)
    assert np.array_equal(idx_s, idx[0, rows])
    assert np.max(np.abs(out_s - ref[0])) < 1e-12


def test_attention_row_without_valid_entry_and_nan_key():
    # no valid entry: out 0 and lse -inf; a selected NaN key: the sum of exponentials and
    # everything after it is NaN (the -inf rule is for an empty selection only)
    T, D = 6, 576
    g = torch.Generator().manual_seed(2)
    kv = torch.randn(1, T, 1, D, generator=g).to(torch.bfloat16)
    kv[0, 2, 0, 7] = float("nan")
    q = (torch.randn(1, 3, 16, D, generator=g) * 0.05).to(torch.bfloat16)
    idx = np.array([[[-1, -1, -1], [0, 2, 4], [1, 3, -1]]], np.int32)
    out, lse = oracle.sparse_attn(q, kv, idx, 0.04, Dv=512)
    assert np.all(out[0, 0] == 0.0) and np.all(lse[0, 0] == -np.inf)
    assert np.all(np.isnan(out[0, 1])) and np.all(np.isnan(lse[0, 1]))
    assert np.all(np.isfinite(out[0, 2])) and np.all(np.isfinite(lse[0, 2]))


def test_fp8_rows_times_scale_equal_the_decoded_bf16_rows():
    # e4m3 values times a power-of-two scale are exact in bf16, so both paths see equal keys
    rng = np.random.default_rng(5)
    T, D = 24, 576
    codes = rng.integers(0, 256, size=(1, T, 1, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    scale = (2.0 ** rng.integers(-6, 3, size=(1, T))).astype(np.float32)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(scale)[..., None, None]
    kv_bf16 = dec.to(torch.bfloat16)
    assert torch.equal(kv_bf16.float(), dec)
    q = (torch.randn(1, T, 16, D, generator=torch.Generator().manual_seed(1)) * 0.01).to(torch.bfloat16)
    idx = oracle.topk(rng.standard_normal((1, T, T)).astype(np.float32), 8)
    a, la = oracle.sparse_attn(q, codes, idx, 0.05, kv_scale=scale, Dv=512)
    b, lb = oracle.sparse_attn(q, kv_bf16, idx, 0.05, Dv=512)
    assert np.max(np.abs(a - b)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12


# ---------------------------------------------------------------- IndexCache stack


def _patterns():
    rows = []
    for line in open(golden("indexcache_patterns.txt")):
        if line.strip() and not line.startswith("#"):
            name, pat, f, s = line.split()
            rows.append((name, pat, int(f), int(s)))
    return rows


def test_printed_patterns_parse_with_the_printed_shape():
    for name, pat, nf, ns in _patterns():
        oracle.check_pattern(pat, len(pat))
        assert pat.count("F") == nf and pat.count("S") == ns
    assert dict((n, p) for n, p, _, _ in _patterns())["fss_x9"] == "FSS" * 9


def test_pattern_from_freq():
    assert oracle.pattern_from_freq(1, 5) == "FFFFF"
    assert oracle.pattern_from_freq(3, 27) == "FSS" * 9
    assert oracle.pattern_from_freq(4, 61).count("F") == 16
    with pytest.raises(ValueError):
        oracle.check_pattern("FSX", 3)
    with pytest.raises(ValueError):
        oracle.check_pattern("SFF", 3)
    with pytest.raises(ValueError):
        oracle.check_pattern("FS", 3)


def _stack_inputs(pattern, T=40, poison=False):
    w_ = synth.workload("B", T=T, k=8, H=16, pattern=pattern)
    layers = []
    for l, c in enumerate(pattern):
        d = synth.layer_inputs(w_, l, indexer=True)
        if c == "S" and poison:
            for key in ("q_idx", "k_idx", "w_idx"):
                d[key] = torch.full_like(d[key], float("nan"))
        layers.append(d)
    return w_, layers


def test_shared_layers_attend_with_the_full_layers_indices():
    pat = "FSSFS"
    w_, layers = _stack_inputs(pat)
    outs, lses, sets = oracle.layer_stack(pat, layers, 8, w_.scale(), Dv=512)
    assert np.array_equal(sets[1], sets[0]) and np.array_equal(sets[2], sets[0])
    assert np.array_equal(sets[4], sets[3]) and not np.array_equal(sets[3], sets[0])
    for l in (1, 2):
        o, _ = oracle.sparse_attn(layers[l]["q"], layers[l]["kv"], sets[0], w_.scale(), Dv=512)
        assert np.array_equal(o, outs[l])


def test_shared_layers_never_read_their_indexer_inputs():
    pat = "FSS"
    w_, clean = _stack_inputs(pat)
    _, poisoned = _stack_inputs(pat, poison=True)
    a = oracle.layer_stack(pat, clean, 8, w_.scale(), Dv=512)
    b = oracle.layer_stack(pat, poisoned, 8, w_.scale(), Dv=512)
    for x, y in zip(a[0], b[0]):
        assert np.array_equal(x, y)


def test_all_full_stack_equals_independent_layers():
    pat = "FFF"
    w_, layers = _stack_inputs(pat)
    outs, _, sets = oracle.layer_stack(pat, layers, 8, w_.scale(), Dv=512)
    for l in range(3):
        s = oracle.index_scores(layers[l]["q_idx"], layers[l]["k_idx"], layers[l]["w_idx"])
        ix = oracle.topk(s, 8)
        assert np.array_equal(ix, sets[l])
        o, _ = oracle.sparse_attn(layers[l]["q"], layers[l]["kv"], ix, w_.scale(), Dv=512)
        assert np.array_equal(o, outs[l])


# ---------------------------------------------------------------- indexer KL objective


def _kl_inputs(seed, B=2, Tq=3, Tk=9, H_I=2, d_I=4, H=2, Dqk=8, kk=5, margin=0.05):
    """float64 inputs whose indexer dot products all stay at least `margin` away from the
    ReLU's kink (so central differences are smooth)."""
    rng = np.random.default_rng(seed)
    while True:
        qi = rng.standard_normal((B, Tq, H_I, d_I))
        ki = rng.standard_normal((B, Tk, d_I))
        if np.min(np.abs(np.einsum("btjd,bsd->btjs", qi, ki))) > margin:
            break
    wi = rng.standard_normal((B, Tq, H_I))
    q = rng.standard_normal((B, Tq, H, Dqk))
    k = rng.standard_normal((B, Tk, H, Dqk))
    idx = np.full((B, Tq, kk), -1, np.int32)
    for b in range(B):
        for t in range(Tq):
            n = int(rng.integers(1, kk + 1))
            idx[b, t, :n] = rng.choice(Tk, size=n, replace=False)
    return qi, ki, wi, q, k, idx


def test_kl_is_zero_when_the_indexer_reproduces_the_target():
    # one main head, indexer = one head with w = 1, k_I = K and q_I = sm_scale * q, all
    # entries positive (the ReLU passes everything): I_s = z_s, so Q = P, the KL is 0 and so
    # is every gradient
    rng = np.random.default_rng(11)
    B, Tq, Tk, D, scale = 1, 4, 10, 6, 0.3
    q = rng.uniform(0.1, 1.0, (B, Tq, 1, D))
    k = rng.uniform(0.1, 1.0, (B, Tk, 1, D))
    idx = np.array([[[0, 3, 5, 9], [1, 2, -1, -1], [4, -1, 8, 7], [6, 0, 1, 2]]], np.int32)
    loss, dq, dw, dk = oracle.indexer_kl(scale * q, k[:, :, 0], np.ones((B, Tq, 1)), q, k, scale, idx=idx)
    assert np.max(np.abs(loss)) < 1e-14
    assert max(np.max(np.abs(x)) for x in (dq, dw, dk)) < 1e-14
    # and a different indexer gives a positive loss
    loss2, *_ = oracle.indexer_kl(2 * scale * q, k[:, :, 0], np.ones((B, Tq, 1)), q, k, scale, idx=idx)
    assert np.all(loss2[:, [0, 2, 3]] > 1e-6)


def test_kl_two_keys_matches_the_bernoulli_closed_form():
    # two keys, two main heads: P(key 0) = (sigmoid(a0) + sigmoid(a1)) / 2 with a_h the
    # logit difference of head h; Q(key 0) = sigmoid(I_0 - I_1);
    # KL = p log(p/r) + (1-p) log((1-p)/(1-r))
    scale = 0.5
    q = np.zeros((1, 1, 2, 2))
    q[0, 0, 0] = [1.0, 0.0]
    q[0, 0, 1] = [0.0, -2.0]
    k = np.zeros((1, 2, 2, 2))
    k[0, 0, :, :] = [[3.0, 1.0], [3.0, 1.0]]
    k[0, 1, :, :] = [[1.0, 2.0], [1.0, 2.0]]
    qi = np.array([[[[1.0, 0.5]]]])
    ki = np.array([[[2.0, 1.0], [0.5, 3.0]]])
    wi = np.array([[[0.7]]])
    idx = np.array([[[1, 0]]], np.int32)
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    a0 = scale * (3.0 - 1.0)  # head 0: q . K0 - q . K1
    a1 = scale * (-2.0 - (-4.0))
    p = (sig(a0) + sig(a1)) / 2
    r = sig(0.7 * (2.5 - 2.0))
    want = p * math.log(p / r) + (1 - p) * math.log((1 - p) / (1 - r))
    loss, dq, dw, dk = oracle.indexer_kl(qi, ki, wi, q, k, scale, idx=idx)
    assert abs(loss[0, 0] - want) < 1e-14
    # dL/dI_0 = r - p, so dw = (r - p) * (2.5 - 2.0)
    assert abs(dw[0, 0, 0] - (r - p) * 0.5) < 1e-14


def test_kl_gradients_match_central_differences():
    qi, ki, wi, q, k, idx = _kl_inputs(3)
    kv_len = np.array([9, 6], np.int32)
    scale = 0.4
    loss, dq, dw, dk = oracle.indexer_kl(qi, ki, wi, q, k, scale, idx=idx, kv_len=kv_len)
    total = lambda a, b_, c: oracle.indexer_kl(a, b_, c, q, k, scale, idx=idx, kv_len=kv_len)[0].sum()
    h = 1e-6
    for name, x, g in (("q_idx", qi, dq), ("k_idx", ki, dk), ("w_idx", wi, dw)):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            args = {"q_idx": (xp, ki, wi), "k_idx": (qi, xp, wi), "w_idx": (qi, ki, xp)}[name]
            argm = {"q_idx": (xm, ki, wi), "k_idx": (qi, xm, wi), "w_idx": (qi, ki, xm)}[name]
            num[pos] = (total(*args) - total(*argm)) / (2 * h)
        assert np.max(np.abs(num - g)) < 1e-7 * max(1.0, np.max(np.abs(g))), name
    assert np.any(dk != 0) and np.all(loss >= 0)


def test_kl_dense_warmup_equals_every_causal_key_selected():
    qi, ki, wi, q, k, _ = _kl_inputs(4, B=2, Tq=4, Tk=7)
    kv_len = np.array([7, 5], np.int32)
    idx = np.full((2, 4, 7), -1, np.int32)
    for b, L in enumerate(kv_len):
        for t in range(4):
            p = L - 4 + t
            idx[b, t, :p + 1] = np.arange(p + 1)[::-1]  # any order
    a = oracle.indexer_kl(qi, ki, wi, q, k, 0.3, idx=None, kv_len=kv_len)
    b_ = oracle.indexer_kl(qi, ki, wi, q, k, 0.3, idx=idx, kv_len=kv_len)
    for x, y in zip(a, b_):
        assert np.max(np.abs(x - y)) < 1e-13


def test_kl_row_without_keys_and_bf16_entry():
    # a row that selects nothing contributes nothing; the bf16 entry equals the float64 one
    # on the decoded values
    qi, ki, wi, q, k, idx = _kl_inputs(5)
    idx[1, 2, :] = -1
    bf = [torch.from_numpy(x).to(torch.bfloat16) for x in (qi, ki, wi, q, k)]
    a = oracle.indexer_kl(*bf, 0.25, idx=idx)
    b_ = oracle.indexer_kl(*[x.double().numpy() for x in bf], 0.25, idx=idx)
    for x, y in zip(a, b_):
        assert np.array_equal(x, y)
    assert a[0][1, 2] == 0.0 and np.all(a[1][1, 2] == 0.0) and np.all(a[2][1, 2] == 0.0)
