"""Seeded synthetic inputs for SAS gated block-sparse attention.

This module only draws random numbers, rounds them to the storage dtype and
arranges them in the documented layouts.  It holds none of the method's
arithmetic (no projection, pooling, normalisation, RoPE, scoring, selection or
attention), so the fp64 oracle and the HIP path can both take their inputs
from it without sharing any computation.

Workload shapes follow the SAS release setup (model card "Checkpoint
configuration" table: 64-token KV blocks, Top-K 31, gate hidden 128, 32,768
training tokens; budgets 1,024/2,048/4,096) on Qwen3 attention shapes.

Random streams: every tensor gets its own torch.Generator seeded from
(seed, workload id, tensor id[, extra ids]) through a splitmix64 mix.  Draws
are fp32 N(0, 1), optionally scaled, then rounded to bf16 with torch's
round-to-nearest-even conversion.  The same seed gives the same values on the
same device type; CPU and GPU streams differ (tests read back whatever values
the device holds, so this never matters for parity).
"""
from __future__ import annotations

import dataclasses
import math

import torch

_M64 = (1 << 64) - 1

# tensor ids of the random streams
TID_Q, TID_K, TID_V, TID_DO, TID_WQ, TID_WK, TID_CTX, TID_BLOCKSCALE, TID_SHARED = range(1, 10)
TID_QGATE, TID_KGCACHE = 10, 11


def _splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & _M64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def stream_seed(*parts: int) -> int:
    """Mix integer ids into one 63-bit seed (order-sensitive)."""
    h = 0x243F6A8885A308D3
    for p in parts:
        h = _splitmix64(h ^ (int(p) & _M64))
    return h & ((1 << 63) - 1)


def generator(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(*parts))
    return g


def normal(shape, *parts: int, device="cpu", scale: float = 1.0,
           dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, scale^2) draws in fp32, then rounded to `dtype` (RNE)."""
    g = generator(device, *parts)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: prefill/training layer or batched decode."""
    name: str
    cfg_id: int
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    dg: int
    topk: int
    block: int = 64
    theta: float = 1.0e6
    eps: float = 1.0e-6
    kind: str = "prefill"          # "prefill" | "train" | "decode"
    skew: str = "none"             # "none" | "lognormal_block" | "shared_dir"
    gate: str = "kv"               # "kv": one gate per KV head; "q": one per query head
    Lmin: int = 0                  # decode context length range (inclusive)
    Lmax: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def NB(self) -> int:
        return -(-self.T // self.block)

    @property
    def Hs(self) -> int:
        """Selection heads: heads that carry one gate each."""
        return self.Hq if self.gate == "q" else self.Hkv

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads (shapes of Qwen3-4B/8B/14B attention layers).
TINY = Workload("tiny_T1024_G2_D64_K3", 1, B=1, T=1024, Hq=2, Hkv=1, D=64, dg=32, topk=3,
                kind="train")
PREFILL_8K = Workload("qwen3_4b_prefill_T8192_K31", 2, B=1, T=8192, Hq=32, Hkv=8, D=128,
                      dg=128, topk=31, kind="prefill")
TRAIN_32K = Workload("qwen3_4b_train_T32768_K31", 3, B=1, T=32768, Hq=32, Hkv=8, D=128,
                     dg=128, topk=31, kind="train")
DECODE_B64 = Workload("qwen3_8b_decode_B64_budget2048", 4, B=64, T=1, Hq=32, Hkv=8, D=128,
                      dg=128, topk=31, kind="decode", Lmin=8192, Lmax=65536)
SKEW_32K = Workload("qwen3_14b_train_T32768_G5_skew", 5, B=1, T=32768, Hq=40, Hkv=8, D=128,
                    dg=128, topk=31, kind="train", skew="lognormal_block")

# The same shape with rankings skewed on purpose: shared per-head directions
# in q and k with a per-block lognormal weight (k = z + s_j u, q = z' + 4 w),
# so that adjacent tokens choose largely the same blocks and a few blocks are
# chosen by many tokens (a per-block scale alone cancels in the gate's Q/K
# normalisation and leaves the rankings uniform).
SKEW5B_32K = SKEW_32K.replace(name="qwen3_14b_train_T32768_G5_shared", skew="shared_dir")

WORKLOADS = {w.name: w for w in (TINY, PREFILL_8K, TRAIN_32K, DECODE_B64, SKEW_32K, SKEW5B_32K)}


def budget_to_topk(budget: int, block: int = 64) -> int:
    """Decode token budget -> historical Top-K (budget counts the current block too)."""
    if budget % block or budget < block:
        raise ValueError("budget must be a positive multiple of the block size")
    return budget // block - 1


def prefill_inputs(w: Workload, seed: int = 0, device="cpu", with_dout: bool = True,
                   dtype=torch.bfloat16) -> dict:
    """q, k, v [B,T,H,D]; router weights Wq [Hkv,G*D,dg] (gate="q": [Hq,D,dg]),
    Wk [Hkv,3D,dg] (N(0,1)/sqrt(fan_in), bf16-representable); RMSNorm weights
    = 1 (fp32); dO [B,T,Hq,D] when requested.

    skew="lognormal_block": every 64-token block j of KV head kappa draws one
    s ~ LogNormal(0, 1) that multiplies all q rows of that head group and all
    k rows of that block.  skew="shared_dir": k = z + s_j * u_kappa and
    q = z' + 4 * w_kappa with shared per-head directions u, w (skews the
    rankings, not only the attention logits).
    """
    B, T, Hq, Hkv, D, dg, G = w.B, w.T, w.Hq, w.Hkv, w.D, w.dg, w.G
    c = w.cfg_id
    if w.skew == "none":
        q = normal((B, T, Hq, D), seed, c, TID_Q, device=device, dtype=dtype)
        k = normal((B, T, Hkv, D), seed, c, TID_K, device=device, dtype=dtype)
    else:
        q32 = normal((B, T, Hq, D), seed, c, TID_Q, device=device, dtype=torch.float32)
        k32 = normal((B, T, Hkv, D), seed, c, TID_K, device=device, dtype=torch.float32)
        NB = w.NB
        g = generator(device, seed, c, TID_BLOCKSCALE)
        s = torch.exp(torch.randn((B, NB, Hkv), generator=g, device=device))
        s_tok = s.repeat_interleave(w.block, dim=1)[:, :T]            # [B,T,Hkv]
        if w.skew == "lognormal_block":
            q32 = (q32.view(B, T, Hkv, G, D) * s_tok[..., None, None]).view(B, T, Hq, D)
            k32 = k32 * s_tok[..., None]
        elif w.skew == "shared_dir":
            g2 = generator(device, seed, c, TID_SHARED)
            u = torch.randn((Hkv, D), generator=g2, device=device)
            wv = torch.randn((Hkv, G * D), generator=g2, device=device)
            k32 = k32 + s_tok[..., None] * u[None, None]
            q32 = (q32.view(B, T, Hkv, G * D) + 4.0 * wv[None, None]).view(B, T, Hq, D)
        else:
            raise ValueError(w.skew)
        q, k = q32.to(dtype), k32.to(dtype)
    v = normal((B, T, Hkv, D), seed, c, TID_V, device=device, dtype=dtype)
    if w.gate == "q":
        wq = normal((Hq, D, dg), seed, c, TID_WQ, device=device,
                    scale=1.0 / math.sqrt(D), dtype=torch.bfloat16)
    else:
        wq = normal((Hkv, G * D, dg), seed, c, TID_WQ, device=device,
                    scale=1.0 / math.sqrt(G * D), dtype=torch.bfloat16)
    wk = normal((Hkv, 3 * D, dg), seed, c, TID_WK, device=device,
                scale=1.0 / math.sqrt(3 * D), dtype=torch.bfloat16)
    out = dict(q=q, k=k, v=v, wq=wq, wk=wk,
               w_qn=torch.ones(dg, device=device, dtype=torch.float32),
               w_kn=torch.ones(dg, device=device, dtype=torch.float32))
    if with_dout:
        out["dout"] = normal((B, T, Hq, D), seed, c, TID_DO, device=device, dtype=dtype)
    return out


def decode_context_lengths(w: Workload, seed: int = 0) -> torch.Tensor:
    """ctx_len[b] ~ U{Lmin..Lmax} (int32, CPU)."""
    g = generator("cpu", seed, w.cfg_id, TID_CTX)
    return torch.randint(w.Lmin, w.Lmax + 1, (w.B,), generator=g, dtype=torch.int32)


def decode_inputs(w: Workload, seed: int = 0, device="cpu", Lmax: int | None = None,
                  ctx_len: torch.Tensor | None = None) -> dict:
    """Batched single-token decode inputs in head-major cache layout.

    q [B,Hq,D] bf16; k_cache, v_cache [B,Hkv,Lmax,D] bf16 ~ N(0,1);
    q_gate [B,Hs,dg] and kg_cache [B,Hkv,NBmax,dg] fp32 ~ N(0,1) (the
    statistics of unit-RMS, norm-preserving-rotated router outputs; decode
    consumes them as given inputs); ctx_len [B] int32.
    """
    Lmax = Lmax or w.Lmax
    NBmax = -(-Lmax // w.block)
    if ctx_len is None:
        ctx_len = decode_context_lengths(w, seed)
    c = w.cfg_id
    return dict(
        q=normal((w.B, w.Hq, w.D), seed, c, TID_Q, device=device),
        q_gate=normal((w.B, w.Hs, w.dg), seed, c, TID_QGATE, device=device,
                      dtype=torch.float32),
        k_cache=normal((w.B, w.Hkv, Lmax, w.D), seed, c, TID_K, device=device),
        v_cache=normal((w.B, w.Hkv, Lmax, w.D), seed, c, TID_V, device=device),
        kg_cache=normal((w.B, w.Hkv, NBmax, w.dg), seed, c, TID_KGCACHE, device=device,
                        dtype=torch.float32),
        ctx_len=ctx_len.to(device=device, dtype=torch.int32),
        Lmax=Lmax, NBmax=NBmax,
    )


TID_SEL, TID_SELLOGG, TID_DLOGG = 12, 13, 14


def random_dlogg(w: Workload, idx: torch.Tensor, seed: int = 0, device="cpu"):
    """An upstream gradient dL/d log g with the structure the gated attention
    gives it: N(0, 1) on the valid slots of each row, less the row's mean over
    them (so each row sums to zero), 0 on pads.  fp32 [B,T,Hkv,S]."""
    idx = idx.to("cpu")
    g = generator("cpu", seed, w.cfg_id, TID_DLOGG)
    v = torch.randn(tuple(idx.shape), generator=g, dtype=torch.float64)
    valid = idx >= 0
    v = torch.where(valid, v, torch.zeros_like(v))
    n = valid.sum(-1, keepdim=True).clamp(min=1)
    v = torch.where(valid, v - v.sum(-1, keepdim=True) / n, torch.zeros_like(v))
    return v.to(torch.float32).to(device)


def random_selection(w: Workload, seed: int = 0, device="cpu", K: int | None = None):
    """A selection with the structure of sas_topk_blocks' output, drawn at
    random (no scoring): for token t of block c, min(K, c) distinct historical
    blocks j < c chosen uniformly, in ascending order, then c, then pads -1;
    log-gates logg ~ N(-log(c + 1), 1) on valid slots, -inf on pads.

    With iid inputs the router's own choices are statistically of this kind
    (adjacent tokens share no more blocks than chance), so this drives the
    attention kernels at full size with inputs that do not depend on the
    router implementation.  Returns idx int32, logg fp32 [B,T,Hs,K+1] (Hs
    selection heads: Hkv, or Hq with one gate per query head).
    """
    K = w.topk if K is None else K
    B, T, H, NB = w.B, w.T, w.Hs, w.NB
    S = K + 1
    g = generator("cpu", seed, w.cfg_id, TID_SEL)
    c = (torch.arange(T) // w.block).view(1, T, 1, 1)
    idx = torch.full((B, T, H, S), -1, dtype=torch.int64)
    if K > 0 and NB > 1:
        keys = torch.rand((B, T, H, NB), generator=g)
        j = torch.arange(NB).view(1, 1, 1, NB)
        keys = torch.where(j < c, keys, torch.full_like(keys, -1.0))
        top = torch.topk(keys, min(K, NB), dim=-1)
        chosen = torch.where(top.values >= 0, top.indices, torch.full_like(top.indices, NB + 1))
        chosen, _ = torch.sort(chosen, dim=-1)
        chosen = torch.where(chosen <= NB, chosen, torch.full_like(chosen, -1))
        idx[..., :chosen.shape[-1]] = chosen
    nsel = torch.minimum(c.expand(B, T, H, 1), torch.tensor(K)).squeeze(-1)   # [B,T,H]
    idx.scatter_(-1, nsel.unsqueeze(-1), c.expand(B, T, H, 1).clone())
    g2 = generator("cpu", seed, w.cfg_id, TID_SELLOGG)
    lg = torch.randn((B, T, H, S), generator=g2) - torch.log(c.float() + 1.0)
    logg = torch.where(idx >= 0, lg, torch.full_like(lg, float("-inf")))
    return idx.to(torch.int32).to(device), logg.to(torch.float32).to(device)
