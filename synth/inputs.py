"""Seeded synthetic workloads shaped like the pages' DSA workloads.

Every tensor is drawn from its own torch.Generator whose seed is a fixed function of
(base seed, workload id, layer, tensor id), so any single tensor can be regenerated
alone, on the host or on a GPU.  Host and device generators are different streams:
a test generates once and hands the *same bytes* to both the oracle and the library.

Storage formats produced here:
  * bf16: torch's float32 -> bfloat16 conversion (round to nearest even);
  * fp8: OCP e4m3 ("e4m3fn") bytes with one float32 scale per token,
    scale = amax(row)/448 (1 when the row is all zero), values clamped to +-448
    before torch's round-to-nearest-even conversion;
  * MXFP4 (OCP Microscaling Formats v1.0): blocks of 32 values share an E8M0 scale
    2^(floor(log2 amax) - 2) (2 = the largest e2m1 exponent), each value divided by it,
    rounded to the nearest e2m1 value (ties to an even code) and clamped to +-6; rows
    of D/2 + 32 bytes laid out as mxfp4_rows states.

Workloads (sizes from the task's workload list; page facts cited per field):
  A  one DSA layer, multi-head attention, T=3072, k=512, indexer 2 heads x 16
     (DSA ablation model card, model list), 4 heads x 32 RoPE'd Q/K/V.
  B  one MLA-DSA layer, T=2057 (just past k=2048, DSV2-Lite IndexCache model card,
     "Validation and scope"), indexer 16 x 64, 16 MLA heads, 576/512 widths.
  C  27-layer stack, pattern FSS x 9 (same card, intro), T=16384, k=2048.
  D  one MLA-DSA layer at T=65536, k=2048, with a low-rank "sink" on the first 64 keys.
  E  batched decode: 64 sequences x 65536 cached tokens, fp8 latent cache with a
     per-token scale, bf16 indexer key cache, FSS over 3 layers.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import torch

__all__ = [
    "Workload", "WORKLOADS", "workload", "tensor_seed", "normal", "bf16", "fp8_e4m3_rows", "mxfp4_rows",
    "rope_half_split", "layer_inputs", "integer_indexer_inputs", "integer_query_rows_inputs",
    "sharp_attention_inputs",
    "decode_layer_inputs", "decode_indexer_cache",
]


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # workload id mixed into every seed
    seed: int
    B: int
    T: int                   # prefill length, or cache length L for decode
    k: int
    H_I: int
    d_I: int
    H: int
    Hkv: int
    Dqk: int
    Dv: int
    pattern: str = "F"
    mla: bool = True         # V is the first Dv columns of the shared latent row
    rope: bool = False       # multi-head workload: Q/K rotated before bf16 rounding
    sink: bool = False       # low-rank sink direction on the first 64 keys
    decode: bool = False     # one query per sequence at position T-1, fp8 latent cache
    sm_scale: float = field(default=0.0)

    def scale(self) -> float:
        return self.sm_scale if self.sm_scale else 1.0 / math.sqrt(self.Dqk)


WORKLOADS = {
    "A": Workload("mha_t3072_k512", 0, 1337, 1, 3072, 512, 2, 16, 4, 4, 32, 32,
                  mla=False, rope=True),
    "B": Workload("mla_t2057_k2048", 1, 64, 1, 2057, 2048, 16, 64, 16, 1, 576, 512),
    "C": Workload("mla_stack27_fss_t16384_k2048", 2, 64, 1, 16384, 2048, 16, 64, 16, 1, 576, 512,
                  pattern="FSS" * 9),
    "D": Workload("mla_t65536_k2048_sink", 3, 64, 1, 65536, 2048, 16, 64, 16, 1, 576, 512,
                  sink=True),
    "E": Workload("mla_decode_b64_l65536_fp8_fss", 4, 64, 64, 65536, 2048, 16, 64, 16, 1, 576, 512,
                  pattern="FSS", decode=True),
}


def workload(key: str, **overrides) -> Workload:
    """A workload by letter, optionally with fields replaced (e.g. a smaller T for tests)."""
    return replace(WORKLOADS[key], **overrides)


# tensor ids
_T_QI, _T_KI, _T_W, _T_Q, _T_K, _T_V, _T_KV, _T_SINK_I, _T_SINK_L = range(9)


def tensor_seed(w: Workload, layer: int, tid: int, extra: int = 0) -> int:
    """Seed of one tensor: a fixed mix of (base seed, workload, layer, tensor, extra)."""
    return ((((w.seed * 1000003 + w.wid) * 10007 + layer) * 101 + tid) * 65537 + extra) % (1 << 62)


def normal(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def fp8_e4m3_rows(x: torch.Tensor):
    """float32 [..., D] -> (uint8 e4m3 codes [..., D], float32 scale [...])."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-448.0, 448.0)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


# e2m1 magnitudes by 3-bit code, and the midpoints between neighbours
_E2M1_MID = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def mxfp4_rows(x: torch.Tensor) -> torch.Tensor:
    """float32 [..., D] (D a multiple of 32, at most 1024) -> uint8 MXFP4 rows [..., D/2 + 32].

    Block j (values 32j..32j+31): its elements in bytes 16j..16j+15, element 2i in the low
    nibble of byte 16j+i and 2i+1 in the high one (code = sign bit 3, magnitude code
    bits 0..2); its E8M0 scale byte at D/2 + 4*(j % 8) + j // 8; other bytes zero."""
    *lead, D = x.shape
    assert D % 32 == 0 and D <= 1024
    nb = D // 32
    xb = x.reshape(-1, nb, 32).to(torch.float32)
    _, ex = torch.frexp(xb.abs().amax(-1))  # amax = m * 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    e = (ex - 3).clamp(-127, 127)
    y = torch.ldexp(xb, -e.unsqueeze(-1).to(torch.float32))
    mag = y.abs().clamp(max=6.0)
    mid = _E2M1_MID.to(x.device)
    lo, hi = torch.bucketize(mag, mid, right=False), torch.bucketize(mag, mid, right=True)
    m = torch.where(lo % 2 == 0, lo, hi)  # the two differ only on a midpoint: keep the even code
    code = (m | ((y < 0) & (m > 0)).to(m.dtype) << 3).to(torch.uint8)
    out = torch.zeros((xb.shape[0], D // 2 + 32), dtype=torch.uint8, device=x.device)
    out[:, :D // 2] = (code[..., 0::2] | (code[..., 1::2] << 4)).reshape(-1, D // 2)
    j = torch.arange(nb, device=x.device)
    out[:, D // 2 + 4 * (j % 8) + j // 8] = (e + 127).to(torch.uint8)
    return out.reshape(*lead, D // 2 + 32)


def rope_half_split(x: torch.Tensor, pos0: int = 0, base: float = 10000.0) -> torch.Tensor:
    """Standard half-split rotary embedding on the last dim of x [B, T, H, D] (fp32)."""
    B, T, H, D = x.shape
    half = D // 2
    inv = base ** (-torch.arange(half, dtype=torch.float64, device=x.device) / half)
    ang = torch.arange(pos0, pos0 + T, dtype=torch.float64, device=x.device)[:, None] * inv[None, :]
    c = torch.cos(ang).to(torch.float32)[None, :, None, :]
    s = torch.sin(ang).to(torch.float32)[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * c - x2 * s, x1 * s + x2 * c], dim=-1)


def _sink(w: Workload, layer: int, dim: int, tid: int, device):
    u = normal((dim,), 1.0, tensor_seed(w, layer, tid), device)
    return u / u.norm()


def layer_inputs(w: Workload, layer: int = 0, device="cpu", indexer: Optional[bool] = None):
    """Prefill inputs of one layer.

    Returns a dict of torch tensors:
      q_idx bf16 [B,T,H_I,d_I], k_idx bf16 [B,T,d_I], w_idx bf16 [B,T,H_I]  (when indexer)
      q bf16 [B,T,H,Dqk]; kv bf16 [B,T,Hkv,Dqk]; v bf16 [B,T,Hkv,Dv] or None (MLA).
    `indexer` defaults to True on 'F' layers of the workload's pattern.
    """
    assert not w.decode
    B, T = w.B, w.T
    if indexer is None:
        indexer = w.pattern[layer] == "F"
    out = {}
    if indexer:
        sd = 1.0 / math.sqrt(w.d_I)
        q_i = normal((B, T, w.H_I, w.d_I), sd, tensor_seed(w, layer, _T_QI), device)
        k_i = normal((B, T, w.d_I), sd, tensor_seed(w, layer, _T_KI), device)
        if w.sink:
            k_i[:, :64, :] += 4.0 * _sink(w, layer, w.d_I, _T_SINK_I, device)
        out["q_idx"] = bf16(q_i)
        out["k_idx"] = bf16(k_i)
        out["w_idx"] = bf16(normal((B, T, w.H_I), 1.0, tensor_seed(w, layer, _T_W), device))
    sd = 1.0 / math.sqrt(w.Dqk)
    q = normal((B, T, w.H, w.Dqk), sd, tensor_seed(w, layer, _T_Q), device)
    if w.mla:
        kv = normal((B, T, w.Hkv, w.Dqk), sd, tensor_seed(w, layer, _T_KV), device)
        if w.sink:
            kv[:, :64, :, :] += 4.0 * _sink(w, layer, w.Dqk, _T_SINK_L, device)
        out["q"], out["kv"], out["v"] = bf16(q), bf16(kv), None
    else:
        kk = normal((B, T, w.Hkv, w.Dqk), sd, tensor_seed(w, layer, _T_K), device)
        vv = normal((B, T, w.Hkv, w.Dv), 1.0 / math.sqrt(w.Dv), tensor_seed(w, layer, _T_V), device)
        if w.rope:
            q, kk = rope_half_split(q), rope_half_split(kk)
        out["q"], out["kv"], out["v"] = bf16(q), bf16(kk), bf16(vv)
    return out


def integer_indexer_inputs(B, T, H_I, d_I, seed, device="cpu", qk_max=1, w_max=2):
    """Integer-valued indexer inputs (q, k in [-qk_max, qk_max], w in [-w_max, w_max]).

    With d_I * qk_max**2 <= 2**8 and the head sum bounded below 2**24, every product and
    partial sum is an integer exactly representable in fp32, so the score is exact in
    any summation order.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randint(-qk_max, qk_max + 1, (B, T, H_I, d_I), generator=g, device=device)
    k = torch.randint(-qk_max, qk_max + 1, (B, T, d_I), generator=g, device=device)
    wt = torch.randint(-w_max, w_max + 1, (B, T, H_I), generator=g, device=device)
    return {"q_idx": q.to(torch.bfloat16), "k_idx": k.to(torch.bfloat16), "w_idx": wt.to(torch.bfloat16)}


def integer_query_rows_inputs(B, Tq, Tk, H_I, d_I, seed, qk_max=1, w_max=2):
    """Integer-valued indexer inputs with Tq query rows against Tk keys per sequence (the
    few-row shapes of decode, at many sequences or long caches): q [B,Tq,H_I,d_I], k
    [B,Tk,d_I], w [B,Tq,H_I], drawn as int8 on the CPU (cheap at hundreds of MB of keys)."""
    g = torch.Generator()
    g.manual_seed(seed)
    q = torch.randint(-qk_max, qk_max + 1, (B, Tq, H_I, d_I), generator=g, dtype=torch.int8)
    k = torch.randint(-qk_max, qk_max + 1, (B, Tk, d_I), generator=g, dtype=torch.int8)
    wt = torch.randint(-w_max, w_max + 1, (B, Tq, H_I), generator=g, dtype=torch.int8)
    return {"q_idx": q.to(torch.bfloat16), "k_idx": k.to(torch.bfloat16), "w_idx": wt.to(torch.bfloat16)}


def sharp_attention_inputs(w: Workload, layer: int = 0, device="cpu", logit_std: float = 4.0):
    """Q, K/V ~ N(0,1) with Q scaled so the attention logits have std ~ logit_std.

    At the workloads' own scales the softmax over the selected keys is nearly uniform,
    so outputs are close to a mean of V rows; these inputs make each output depend on a
    few keys, so a wrong gather moves it by O(1).
    """
    d = layer_inputs(w, layer, device, indexer=False)
    qs = logit_std / (math.sqrt(w.Dqk) * w.scale())
    g = lambda tid: normal(tuple(d["kv"].shape), 1.0, tensor_seed(w, layer, tid, 7), device)
    d["q"] = bf16(normal(tuple(d["q"].shape), qs, tensor_seed(w, layer, _T_Q, 7), device))
    d["kv"] = bf16(g(_T_KV if w.mla else _T_K))
    if d["v"] is not None:
        d["v"] = bf16(normal(tuple(d["v"].shape), 1.0, tensor_seed(w, layer, _T_V, 7), device))
    return d


def decode_indexer_cache(w: Workload, device="cpu", seqs=None):
    """bf16 indexer key cache [B, L, d_I] of the decode workload (read by F layers)."""
    assert w.decode
    seqs = range(w.B) if seqs is None else seqs
    sd = 1.0 / math.sqrt(w.d_I)
    rows = [bf16(normal((w.T, w.d_I), sd, tensor_seed(w, 0, _T_KI, b), device)) for b in seqs]
    return torch.stack(rows)


def decode_layer_inputs(w: Workload, layer: int, device="cpu", seqs=None, kv_format: str = "fp8"):
    """One decode layer: q bf16 [B,1,H,Dqk], the latent cache as fp8 uint8 [B,L,1,Dqk] + scale
    [B,L] (kv_format "fp8") or MXFP4 rows uint8 [B,L,1,Dqk/2+32] ("mxfp4", drawn from the
    same values), and, on 'F' layers, q_idx bf16 [B,1,H_I,d_I] and w_idx bf16 [B,1,H_I]."""
    assert w.decode
    seqs = list(range(w.B)) if seqs is None else list(seqs)
    sd = 1.0 / math.sqrt(w.Dqk)
    assert kv_format in ("fp8", "mxfp4")
    codes, scales = [], []
    for b in seqs:
        x = normal((w.T, w.Dqk), sd, tensor_seed(w, layer, _T_KV, b), device)
        if kv_format == "fp8":
            c, s = fp8_e4m3_rows(x)
            scales.append(s)
        else:
            c = mxfp4_rows(x)
        codes.append(c)
        del x
    out = {
        "kv": torch.stack(codes).unsqueeze(2),
        "q": torch.stack([bf16(normal((1, w.H, w.Dqk), sd, tensor_seed(w, layer, _T_Q, b), device))
                          for b in seqs]),
    }
    if scales:
        out["kv_scale"] = torch.stack(scales)
    if w.pattern[layer] == "F":
        si = 1.0 / math.sqrt(w.d_I)
        out["q_idx"] = torch.stack([bf16(normal((1, w.H_I, w.d_I), si, tensor_seed(w, layer, _T_QI, b), device))
                                    for b in seqs])
        out["w_idx"] = torch.stack([bf16(normal((1, w.H_I), 1.0, tensor_seed(w, layer, _T_W, b), device))
                                    for b in seqs])
    return out
