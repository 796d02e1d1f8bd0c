"""GPU checks that make attention and selection parity discriminating, through the C ABI.

  * the score boundary: dsa_index_scores writes every entry of a caller's row (-inf past the
    causal bound and in the padding), whatever the buffer held;
  * the dominant attention instance (bf16 rows, no key split, more keys than the three-
    workgroup schedule takes) on sharp inputs, where a wrong gather moves outputs by O(1),
    and its exact-max recomputation when a late key's logit jumps far above the first ones;
  * duplicate index entries count twice, as in the oracle's gather form;
  * 32 and 64 heads (several 16-head groups per row): resident workgroups walking more
    (row, head group) pairs than they are, on plain lists and on top-k rows, and decode
    rows with key splits;
  * decode equals prefill: a one-query step over a cache of length L gives the indices of
    prefill row L-1 bit for bit, and its outputs within the attention bar ("cached versus
    uncached" logits check, DSV2-Lite-IndexCache-Sparse-1250 card, "Validation and scope");
  * prefix invariance: appending tokens does not change the routes or outputs of earlier
    rows (the causal negative control of the llm-atlas DeepSeek README, "Official chat-
    template sensitivity"), and row slices through kv_len give the rows of the whole call;
  * the grouped decode attention (an 'F' layer and its 'S' layers in one launch, fewer key
    splits per layer than a lone call) against the oracle on sharp fp8 inputs at 64 rows.
Sharp attention outputs are judged by 2e-2 * max|ref| and lse within 1e-3 (besides the
2e-2 absolute rule); indices bit-exact.
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


def _sharp_check(out, lse, ref, rlse, what=""):
    o = _host(out).double().numpy().reshape(ref.shape)
    err = np.max(np.abs(o - ref))
    assert err <= 2e-2, (what, err)
    assert err <= 2e-2 * np.max(np.abs(ref)), (what, err, np.max(np.abs(ref)))
    if lse is not None:
        l = _host(lse).double().numpy().reshape(rlse.shape)
        fin = np.isfinite(rlse)
        assert np.array_equal(np.isfinite(l), fin), what
        assert np.max(np.abs(l[fin] - rlse[fin])) <= 1e-3, what


def _sharp_qkv(Tq, Tk, B=1, seed=0, H=16, D=576, logit_std=4.0, scale=1.0 / 24):
    """q [B,Tq,H,D] and latent rows kv [B,Tk,1,D] ~ N(0,1) (bf16), q scaled so that the
    logits scale * q . k have std ~ logit_std."""
    g = torch.Generator().manual_seed(seed)
    kv = torch.randn(B, Tk, 1, D, generator=g).to(torch.bfloat16)
    qs = logit_std / (math.sqrt(D) * scale)
    q = (torch.randn(B, Tq, H, D, generator=g) * qs).to(torch.bfloat16)
    return q, kv


def _random_index_rows(B, Tq, Tk, k, kv_len, seed):
    s = np.random.default_rng(seed).standard_normal((B, Tq, Tk)).astype(np.float32)
    return oracle.topk(s, k, kv_len=kv_len, Tk=Tk)


# ---------------------------------------------------------------- score boundary

@pytest.mark.parametrize("B,Tq,Tk,ld,lens", [(1, 300, 300, 333, None), (4, 5, 777, 790, [777, 740, 3, 0]),
                                             (2, 1, 4100, 4101, [4100, 1])])
def test_index_scores_writes_every_entry_of_a_garbage_buffer(B, Tq, Tk, ld, lens):
    print(f"score boundary B={B} Tq={Tq} Tk={Tk} ld={ld}", flush=True)
    d = synth.integer_indexer_inputs(B, Tk, 16, 64, seed=Tk + ld, qk_max=1, w_max=2)
    q, w = d["q_idx"][:, -Tq:].contiguous(), d["w_idx"][:, -Tq:].contiguous()
    kl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    buf = torch.full((B, Tq, ld), float("nan"), dtype=torch.float32, device=DEV)
    dsa.index_scores(q.to(DEV), d["k_idx"].to(DEV), w.to(DEV), kv_len=kl, scores=buf, ld=ld)
    got = _host(buf).numpy()
    ref = oracle.index_scores(q, d["k_idx"], w, kv_len=lens, ld=ld)
    L = np.full(B, Tk) if lens is None else np.array(lens)
    vis = np.arange(ld)[None, None, :] <= (L[:, None, None] - Tq + np.arange(Tq)[None, :, None])
    vis &= np.arange(ld)[None, None, :] < Tk
    assert not np.any(np.isnan(got))
    assert np.array_equal(got[vis], ref[vis])
    assert np.all(np.isneginf(got[~vis]))


# ---------------------------------------------------------------- attention

def test_mla_attention_bf16_unsplit_long_sharp():
    # 256 query rows at the end of a 25000-key sequence, k = 2048: bf16 rows, one workgroup
    # per row (no key split) and more keys than the three-workgroup schedule takes, i.e. the
    # kernel instance that serves the long prefill layers
    print("mla attention bf16, unsplit, Tk=25000, sharp", flush=True)
    Tq, Tk, k = 256, 25000, 2048
    q, kv = _sharp_qkv(Tq, Tk, seed=31)
    idx = _random_index_rows(1, Tq, Tk, k, [Tk], seed=32)
    scale = 1.0 / 24
    out, lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), scale, Dv=512)
    ref, rlse = oracle.sparse_attn(q, kv, idx, scale, Dv=512)
    _sharp_check(out, lse, ref, rlse, "unsplit long")
    # one wrong key per row is seen by the same bar: in each of 32 rows the entry with the
    # largest head-0 logit is replaced by a key the row did not select
    n = 32
    bad = idx[:, :n].copy()
    z = torch.einsum("td,tsd->ts", q[0, :n, 0].float(), kv[0, torch.from_numpy(idx[0, :n]).long(), 0].float())
    top = z.argmax(dim=1).numpy()
    for t in range(n):
        unsel = np.setdiff1d(np.arange(Tk - Tq + t + 1), idx[0, t])
        bad[0, t, top[t]] = unsel[t % len(unsel)]
    ref_bad, _ = oracle.sparse_attn(q[:, :n], kv, bad, scale, Dv=512)
    o = _host(out[:, :n]).double().numpy()
    per_row = np.max(np.abs(o - ref_bad), axis=(2, 3))[0]
    assert np.mean(per_row > 2e-2 * np.max(np.abs(ref_bad))) > 0.5


def test_mla_attention_head_groups_and_resident_rows():
    # 32 heads (two 16-head groups per row) over 300 query rows: 600 (row, head group)
    # pairs, more than one launch keeps resident, so workgroups move on from row to row;
    # the plain call walks the pairs front to back, the stack over top-k rows back to front
    print("attention H=32, 300 rows: plain call and stack over top-k rows", flush=True)
    Tq = Tk = 300
    q, kv = _sharp_qkv(Tq, Tk, seed=61, H=32)
    s = np.random.default_rng(62).standard_normal((1, Tq, Tk)).astype(np.float32)
    idx = oracle.topk(s, 96)
    scale = 1.0 / 24
    ref, rlse = oracle.sparse_attn(q, kv, idx, scale, Dv=512)
    out, lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), scale, Dv=512)
    _sharp_check(out, lse, ref, rlse, "plain H=32")
    layer = {"q": q.to(DEV), "kv": kv.to(DEV)}
    cache = torch.from_numpy(idx).to(DEV)
    outs, lses, _ = dsa.layer_stack("S", [layer], 96, scale, Dv=512, index_cache=cache, prefilled=True,
                                    topk_rows=True)
    _sharp_check(outs[0], lses[0], ref, rlse, "stack H=32")
    assert torch.equal(outs[0], out) and torch.equal(lses[0], lse)


def test_mla_attention_64_heads_decode_with_key_splits():
    # 64 heads (four groups) of two decode rows: few workgroups, so the keys are split and
    # the partials merged
    print("attention H=64 decode rows with key splits", flush=True)
    B, L, k = 2, 3000, 2048
    q, kv = _sharp_qkv(1, L, B=B, seed=63, H=64)
    s = np.random.default_rng(64).standard_normal((B, 1, L)).astype(np.float32)
    lens = [L, 2100]
    idx = oracle.topk(s, k, kv_len=lens, Tk=L)
    scale = 1.0 / 24
    assert dsa.workspace_size(dsa._shape(B, 1, L, 64, 1, 576, 512, k, scale, dsa.KV_BF16), dsa.OP_ATTN) > 0
    ref, rlse = oracle.sparse_attn(q, kv, idx, scale, Dv=512)
    out, lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), scale, Dv=512)
    _sharp_check(out, lse, ref, rlse, "decode H=64")


def test_mla_attention_unsplit_logit_jump_beyond_the_first_tiles():
    # the long whole-row kernel takes each head's reference max from its first tile with a
    # valid key and recomputes a row from the exact max when a later key exceeds it by more
    # than 2^64 (base 2): here one key per even row, late in the list, has a logit about
    # 230 (base 2) above the rest for head 0, and the first 20 entries of every third row
    # are missing (the reference then comes from a later tile)
    print("mla attention bf16, unsplit, logit jump", flush=True)
    Tq, Tk, k = 256, 25000, 256
    q, kv = _sharp_qkv(Tq, Tk, seed=51)
    idx = _random_index_rows(1, Tq, Tk, k, [Tk], seed=52)
    idx[0, ::3, :20] = -1
    scale = 1.0 / 24
    for t in range(0, Tq, 2):
        # the jump sits in the 64 rotary columns (K only), so the value rows stay unit-scale
        key = int(idx[0, t, 200])
        q0 = q[0, t, 0, 512:].float()
        kv[0, key, 0, 512:] = (120.0 * q0 / q0.norm()).to(torch.bfloat16)
    # keys may be shared between rows: the oracle sees the same rows
    out, lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), scale, Dv=512)
    ref, rlse = oracle.sparse_attn(q, kv, idx, scale, Dv=512)
    _sharp_check(out, lse, ref, rlse, "logit jump")
    # head 0 of the even rows is the jumping key's value row
    o = _host(out).double().numpy()
    for t in (0, 2, 100):
        v = kv[0, int(idx[0, t, 200]), 0, :512].double().numpy()
        assert np.max(np.abs(o[0, t, 0] - v)) <= 2e-2 * np.max(np.abs(v))


@pytest.mark.parametrize("Tq,B", [(300, 1), (1, 5)])
def test_attention_duplicate_entries_count_twice(Tq, B):
    # an entry repeated in a row is a second term of the softmax sum (prefill rows without
    # key splits, and decode rows with them)
    print(f"attention duplicate entries Tq={Tq} B={B}", flush=True)
    Tk, k = 2500, 256
    q, kv = _sharp_qkv(Tq, Tk, B=B, seed=41)
    rng = np.random.default_rng(42)
    idx = np.stack([np.stack([np.sort(rng.integers(0, Tk, size=k)) for _ in range(Tq)]) for _ in range(B)])
    idx = idx.astype(np.int32)
    idx[:, :, -5:] = idx[:, :, :5]  # sure repeats
    idx[:, ::7, 10:20] = -1
    scale = 1.0 / 24
    out, lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), torch.from_numpy(idx).to(DEV), scale, Dv=512)
    ref, rlse = oracle.sparse_attn(q, kv, idx, scale, Dv=512)
    _sharp_check(out, lse, ref, rlse, "duplicates")


# ---------------------------------------------------------------- decode == prefill

def test_decode_step_equals_prefill_row():
    # integer-valued indexer inputs make every score exact in any summation order (and full
    # of ties), so the decode selection (score kernel + few-row top-k) and the prefill one
    # (fused route) must agree bit for bit; attention on sharp bf16 rows within the bar
    print("decode == prefill row L-1 (T=8192, k=2048)", flush=True)
    T, k = 8192, 2048
    d = synth.integer_indexer_inputs(1, T, 16, 64, seed=77, qk_max=1, w_max=2)
    q, kv = _sharp_qkv(T, T, seed=78)
    scale = 1.0 / 24
    layer = {"q_idx": d["q_idx"].to(DEV), "k_idx": d["k_idx"].to(DEV), "w_idx": d["w_idx"].to(DEV),
             "q": q.to(DEV), "kv": kv.to(DEV)}
    outs, lses, cache = dsa.layer_stack("F", [layer], k, scale, Dv=512)
    Ls = [1, 2048, 2049, 5000, 8192]
    B = len(Ls)
    rows = [L - 1 for L in Ls]
    dec = {"q_idx": layer["q_idx"][0, rows].unsqueeze(1).contiguous(),
           "w_idx": layer["w_idx"][0, rows].unsqueeze(1).contiguous(),
           "k_idx": layer["k_idx"].expand(B, T, 64).contiguous(),
           "q": layer["q"][0, rows].unsqueeze(1).contiguous(),
           "kv": layer["kv"].expand(B, T, 1, 576).contiguous()}
    kl = torch.tensor(Ls, dtype=torch.int32, device=DEV)
    douts, dlses, dcache = dsa.layer_stack("F", [dec], k, scale, Dv=512, kv_len=kl)
    torch.cuda.synchronize()
    pre_idx = _host(cache[0, rows]).numpy()
    assert np.array_equal(_host(dcache[:, 0]).numpy(), pre_idx)
    # and both are the oracle's top-k of the exact scores
    ref_idx = oracle.topk(oracle.index_scores(dec["q_idx"].cpu(), d["k_idx"].expand(B, T, 64).contiguous(),
                                              dec["w_idx"].cpu(), kv_len=Ls), k, kv_len=Ls, Tk=T)
    assert np.array_equal(ref_idx[:, 0], pre_idx)
    ref, rlse = oracle.sparse_attn(q[:, rows], kv, pre_idx[None], scale, Dv=512)
    _sharp_check(douts[0][:, 0], dlses[0][:, 0], ref[0], rlse[0], "decode")
    _sharp_check(outs[0][0, rows], lses[0][0, rows], ref[0], rlse[0], "prefill")
    # decode and prefill outputs differ only by rounding (split keys merge in another order)
    a = _host(douts[0][:, 0]).double().numpy()
    b = _host(outs[0][0, rows]).double().numpy()
    assert np.max(np.abs(a - b)) <= 2e-2 * np.max(np.abs(ref))


# ---------------------------------------------------------------- prefix invariance

def test_prefix_rows_do_not_change_when_tokens_are_appended():
    # the same first 9000 tokens inside a 12000-token sequence: rows < 9000 keep their
    # indices, outputs and lse bit for bit (same kernels, rows independent of later keys)
    print("prefix invariance T'=9000 inside T=12000", flush=True)
    w = synth.workload("D", T=12000)
    full = synth.layer_inputs(w, 0, device=DEV)
    Tp = 9000
    pre = {x: (v[:, :Tp].contiguous() if v is not None else None) for x, v in full.items()}
    outs_f, lses_f, cache_f = dsa.layer_stack("F", [full], w.k, w.scale(), Dv=512)
    outs_p, lses_p, cache_p = dsa.layer_stack("F", [pre], w.k, w.scale(), Dv=512)
    torch.cuda.synchronize()
    assert torch.equal(cache_f[:, :Tp], cache_p)
    assert torch.equal(outs_f[0][:, :Tp], outs_p[0])
    assert torch.equal(lses_f[0][:, :Tp], lses_p[0])
    # row slices through kv_len (a slice [r0, r0 + n) is Tq = n, kv_len = r0 + n) give the
    # rows of the whole call, whatever the slice size
    for n in (500, 4096):  # score-chunk route and fused route
        for r0 in range(0, 12000, n):
            m = min(n, 12000 - r0)
            kl = torch.tensor([r0 + m], dtype=torch.int32, device=DEV)
            part = dsa.index_topk(full["q_idx"][:, r0:r0 + m].contiguous(), full["k_idx"],
                                  full["w_idx"][:, r0:r0 + m].contiguous(), w.k, kv_len=kl)
            assert torch.equal(part, cache_f[:, r0:r0 + m]), (n, r0)


# ---------------------------------------------------------------- grouped decode layers

def test_grouped_decode_layers_at_64_rows_sharp_fp8():
    # 64 decode rows, k = 2048: the three layers of an FSS step run in one attention launch
    # with fewer key splits per layer than a lone call takes (the merge then sums other
    # partials); every layer against the oracle on sharp fp8 rows, and against lone calls
    print("grouped decode layers, 64 rows, sharp fp8", flush=True)
    B, L, k = 64, 4096, 2048
    w = synth.workload("E", B=B, T=L)
    kc = synth.decode_indexer_cache(w, device=DEV)
    scale = w.scale()
    layers = []
    g = torch.Generator().manual_seed(51)
    for l in range(3):
        x = torch.randn(B, L, 576, generator=g)
        codes, sc = synth.fp8_e4m3_rows(x)
        q = (torch.randn(B, 1, 16, 576, generator=g) * (4.0 / (24 * scale))).to(torch.bfloat16)
        d = {"q": q.to(DEV), "kv": codes.unsqueeze(2).to(DEV), "kv_scale": sc.to(DEV)}
        if l == 0:
            f = synth.decode_layer_inputs(synth.workload("E", B=B, T=64), 0, device=DEV)
            d.update(q_idx=f["q_idx"], w_idx=f["w_idx"], k_idx=kc)
        layers.append(d)
    lens = [L - (37 * b) % 1500 for b in range(B)]
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    outs, lses, cache = dsa.layer_stack("FSS", layers, k, scale, Dv=512, kv_len=kl)
    torch.cuda.synchronize()
    idx = _host(cache).numpy()
    s = dsa.index_scores(layers[0]["q_idx"], kc, layers[0]["w_idx"], kv_len=kl)
    assert np.array_equal(idx, oracle.topk(_host(s).numpy(), k, kv_len=lens, Tk=L))
    for l in range(3):
        Ld = layers[l]
        ref, rlse = oracle.sparse_attn(_host(Ld["q"]), _host(Ld["kv"]), idx, scale, kv_scale=_host(Ld["kv_scale"]),
                                       Dv=512)
        _sharp_check(outs[l], lses[l], ref, rlse, f"grouped layer {l}")
        lone, llse = dsa.sparse_attn(Ld["q"], Ld["kv"], cache, scale, kv_scale=Ld["kv_scale"], Dv=512)
        _sharp_check(lone, llse, ref, rlse, f"lone layer {l}")
