"""GPU parity of the paged-cache entry points through the C ABI.

A paged cache holds the same rows as a dense one, scattered over pages of a shared pool
(pages shuffled, unused pages filled with garbage, last pages of a sequence partly filled).
The paged indexer, attention and layer stack must give bit-identical results to the dense
calls on the dense rows (same arithmetic, different addressing), and the dense calls are
held to the oracle by tests/test_gpu_parity.py; the attention is also checked against the
oracle here.
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


def _paginate(dense, lens, page, seed, spare=3):
    """Pool rows and block table for dense [B, L, ...] rows: sequence b's token s goes to
    row table[b, s // page] * page + s % page.  Pages are shuffled; unused pool rows (and the
    tails of last pages) hold garbage; table entries past a sequence's pages hold garbage."""
    g = torch.Generator().manual_seed(seed)
    B, L = dense.shape[0], dense.shape[1]
    max_blocks = (L + page - 1) // page
    need = [(int(n) + page - 1) // page for n in lens]
    num_pages = sum(need) + spare
    perm = torch.randperm(num_pages, generator=g)
    if dense.dtype == torch.uint8:
        pool = torch.randint(0, 256, (num_pages * page,) + tuple(dense.shape[2:]), generator=g, dtype=torch.uint8)
    elif dense.dtype == torch.bfloat16:
        pool = torch.randn((num_pages * page,) + tuple(dense.shape[2:]), generator=g).to(torch.bfloat16)
    else:
        pool = torch.randn((num_pages * page,) + tuple(dense.shape[2:]), generator=g).to(dense.dtype)
    table = torch.randint(-5, num_pages + 5, (B, max_blocks), generator=g, dtype=torch.int32)
    used = 0
    for b in range(B):
        for j in range(need[b]):
            p = int(perm[used])
            used += 1
            table[b, j] = p
            n = min(page, int(lens[b]) - j * page)
            pool[p * page:p * page + n] = dense[b, j * page:j * page + n]
    return pool, table, num_pages


@pytest.mark.parametrize("page,Tq,d_I", [(32, 1, 64), (64, 4, 64), (256, 300, 64), (64, 1, 128)])
def test_paged_indexer_matches_dense(page, Tq, d_I):
    print(f"paged indexer page={page} Tq={Tq} d_I={d_I}", flush=True)
    Tk, B = 3000, 3
    lens = [Tk, Tk - 77, Tq + 500]
    d = synth.integer_indexer_inputs(B, Tk, 16, d_I, seed=page + Tq, qk_max=3, w_max=2)
    q, w = d["q_idx"][:, -Tq:].contiguous(), d["w_idx"][:, -Tq:].contiguous()
    pool, table, npg = _paginate(d["k_idx"], lens, page, seed=page)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dense = _host(dsa.index_scores(q.to(DEV), d["k_idx"].to(DEV), w.to(DEV), kv_len=kl)).numpy()
    bt = table.to(DEV)
    pg = dsa.paged_kv(bt, page, npg)
    paged = _host(dsa.index_scores_paged(q.to(DEV), pool.to(DEV), w.to(DEV), pg, Tk, kv_len=kl)).numpy()
    L = np.array(lens)[:, None, None]
    c = np.arange(Tk)[None, None, :] <= (L - Tq + np.arange(Tq)[None, :, None])
    assert np.array_equal(paged[c], dense[c])
    assert np.all(np.isneginf(paged[~c])) and np.all(np.isneginf(dense[~c]))  # written by the library
    # and the dense scores are the oracle's (integer inputs: exact)
    ref = oracle.index_scores(q, d["k_idx"], w, kv_len=lens)
    assert np.array_equal(dense[c], ref[c])


@pytest.mark.parametrize("fp8", [True, False])
def test_paged_attention_matches_dense_and_oracle(fp8):
    print(f"paged attention fp8={fp8}", flush=True)
    w = synth.workload("E", B=4, T=2600)
    lens = [2600, 2100, 777, 2049]
    layer = synth.decode_layer_inputs(w, 1)
    q, kv, sc = layer["q"], layer["kv"], layer.get("kv_scale")
    if not fp8:  # bf16 latent rows of the same shape
        kv = synth.bf16(synth.normal((4, 2600, 1, 576), 1.0 / 24, seed=777))
        sc = None
    rng = np.random.default_rng(5)
    idx = np.full((4, 1, 2048), -1, dtype=np.int32)
    for b, n in enumerate(lens):
        m = min(2048, n)
        idx[b, 0, :m] = np.sort(rng.choice(n, size=m, replace=False))
    idx_t = torch.from_numpy(idx).to(DEV)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dense_out, dense_lse = dsa.sparse_attn(q.to(DEV), kv.to(DEV), idx_t, w.scale(), Dv=512,
                                           kv_scale=None if sc is None else sc.to(DEV))
    page = 64
    pool, table, npg = _paginate(kv[:, :, 0], lens, page, seed=11)
    pg = dsa.paged_kv(table.to(DEV), page, npg)
    spool = None
    if sc is not None:
        spool, _, _ = _paginate(sc.unsqueeze(-1), lens, page, seed=11)
        spool = spool[:, 0].contiguous()
    out, lse = dsa.sparse_attn_paged(q.to(DEV), pool.to(DEV), idx_t, w.scale(), pg, 2600, kv_len=kl,
                                     kv_scale_pool=None if spool is None else spool.to(DEV))
    assert torch.equal(out, dense_out) and torch.equal(lse, dense_lse)
    ref, ref_lse = oracle.sparse_attn(q, kv, idx, w.scale(), kv_scale=sc, Dv=512)
    assert np.max(np.abs(_host(out).double().numpy() - ref)) <= 2e-2
    assert np.max(np.abs(_host(lse).double().numpy() - ref_lse)) <= 1e-3


def test_paged_decode_stack_matches_dense():
    print("paged decode stack FSS", flush=True)
    w = synth.workload("E", B=3, T=3000)
    lens = [3000, 2047, 1024]
    kcache = synth.decode_indexer_cache(w)
    layers = []
    for l in range(3):
        d = synth.decode_layer_inputs(w, l)
        if "q_idx" in d:
            d["k_idx"] = kcache
        layers.append(d)
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dense_layers = [{k: v.to(DEV) for k, v in L.items()} for L in layers]
    outs, lses, cache = dsa.layer_stack("FSS", dense_layers, 2048, w.scale(), Dv=512, kv_len=kl)
    page = 128
    kpool, table, npg = _paginate(kcache, lens, page, seed=21)
    paged_layers = []
    for L in layers:
        P = {"q": L["q"].to(DEV)}
        if "q_idx" in L:
            P.update(q_idx=L["q_idx"].to(DEV), w_idx=L["w_idx"].to(DEV), k_idx=kpool.to(DEV))
        pool, _, _ = _paginate(L["kv"][:, :, 0], lens, page, seed=21)
        spool, _, _ = _paginate(L["kv_scale"].unsqueeze(-1), lens, page, seed=21)
        P.update(kv=pool.to(DEV), kv_scale=spool[:, 0].contiguous().to(DEV))
        paged_layers.append(P)
    pg = dsa.paged_kv(table.to(DEV), page, npg)
    pouts, plses, pcache = dsa.layer_stack("FSS", paged_layers, 2048, w.scale(), Dv=512, kv_len=kl, pages=pg,
                                           Tk=3000, H_I=16, d_I=64)
    torch.cuda.synchronize()
    assert torch.equal(pcache, cache)
    for a, b in zip(pouts, outs):
        assert torch.equal(a, b)
    for a, b in zip(plses, lses):
        assert torch.equal(a, b)
