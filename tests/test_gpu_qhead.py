"""GPU parity of the per-query-head gate variant (SAS_FLAG_GATE_PER_QUERY_HEAD).

Every query head has its own gate query (Qproj [Hq, D, dg] on that head's q),
scores its KV head's gate keys, and keeps its own Top-K selection and
log-gates; the attention of each query head uses its own selection, and
d log g sums over that head alone.  Same bars as the shared-gate tests:
indices bit-exact outside near ties (K-th/(K+1)-th gap < 1e-5), bf16
outputs within 1e-2 max-abs beyond bf16 rounding and 1e-3 raw mean-abs,
router outputs within 1e-4.  Small shapes in full; the 8K prefill shape with
every row's selection and one KV head's attention in full.
"""
import math

import numpy as np
import pytest
import torch

import gated_block_sparse_gate_amd as sas
import synth
from oracle import sas_oracle as O

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
ROUTER_ABS = 1e-4


def bf16_half_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def check(name, gpu, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    a = gpu.detach().float().cpu().numpy().astype(np.float64)
    d = np.abs(a - ref)
    excess = d
    if gpu.dtype == torch.bfloat16:
        excess = np.maximum(0.0, d - bf16_half_ulp(np.maximum(np.abs(ref), np.abs(a))))
    print(f"  {name}: max-abs {d.max():.3e} (beyond bf16 rounding {excess.max():.3e}) "
          f"mean-abs {d.mean():.3e}", flush=True)
    assert excess.max() <= max_abs and d.mean() <= mean_abs, (name, d.max(), excess.max(),
                                                              d.mean())


def W(name, T, Hq, Hkv, D, dg, K, B=1):
    return synth.Workload(name, 96, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, gate="q")


CASES = [
    W("q_g4_ragged", 1000, 8, 2, 128, 128, 7),
    W("q_g5", 700, 10, 2, 128, 128, 5),
    W("q_g2_b2", 300, 4, 2, 64, 64, 2, B=2),
    W("q_short", 50, 4, 1, 128, 128, 3),
    W("q_k0", 400, 4, 2, 64, 32, 0),
    W("q_g8", 260, 8, 1, 128, 128, 3),
]
IDS = [c.name for c in CASES]
_cache = {}


def prepared(w):
    if w.name in _cache:
        return _cache[w.name]
    x = synth.prefill_inputs(w, seed=0, device="cpu")
    x64 = {k: O.as64(v) for k, v in x.items()}
    r = O.route(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"], w.topk,
                w.theta, w.eps)
    sc = 1.0 / math.sqrt(w.D)
    g = O.attn_bwd(x64["q"], x64["k"], x64["v"], x64["dout"], r["idx"], r["logg"], sc)
    out = dict(x=x, x64=x64, r=r, g=g, dev={k: v.cuda() for k, v in x.items()}, scale=sc)
    _cache[w.name] = out
    return out


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_qhead_router_and_topk(w):
    P = prepared(w)
    d, r = P["dev"], P["r"]
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps, per_query_head=True)
    assert tuple(qg.shape) == (w.B, w.T, w.Hq, w.dg)
    idx, logg, lse, probs = sas.topk_blocks(qg, kg, w.topk, w.Hq, w.D, want_probs=True)
    torch.cuda.synchronize()
    check("q_gate", qg, r["qg"], ROUTER_ABS, ROUTER_ABS)
    check("k_gate", kg, r["kg_cur"], ROUTER_ABS, ROUTER_ABS)
    ok = ~r["near_tie"]
    assert (~ok).mean() < 0.01
    np.testing.assert_array_equal(idx.cpu().numpy()[ok], r["idx"][ok])
    fin = np.isfinite(r["logg"]) & ok[..., None]
    assert np.abs(logg.cpu().numpy()[fin] - r["logg"][fin]).max() < ROUTER_ABS
    assert np.abs(lse.cpu().numpy() - r["lse"]).max() < ROUTER_ABS
    assert np.abs(probs.cpu().numpy() - r["probs"]).max() < 1e-5


def _sel(P):
    return (torch.tensor(P["r"]["idx"], dtype=torch.int32).cuda(),
            torch.tensor(P["r"]["logg"], dtype=torch.float32).cuda())


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_qhead_attention_fwd_bwd(w):
    P = prepared(w)
    d, g = P["dev"], P["g"]
    idx, logg = _sel(P)
    o, lse, o32 = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"],
                                      want_f32=True)
    dq, dk, dv, dlogg = sas.sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx, logg,
                                            P["scale"], o_f32=o32)
    torch.cuda.synchronize()
    assert tuple(dlogg.shape) == (w.B, w.T, w.Hq, w.topk + 1)
    check("o", o, g["o"])
    check("o_f32", o32, g["o"])
    check("lse", lse, g["lse"], 1e-3, 1e-4)
    check("dq", dq, g["dq"])
    check("dk", dk, g["dk"])
    check("dv", dv, g["dv"])
    check("dlogg", dlogg, g["dlogg"])
    assert float(dlogg.sum(-1).abs().max()) < 1e-3
    out2 = sas.sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx, logg, P["scale"],
                               o_f32=o32)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv, dlogg), out2):
        assert torch.equal(a, b), "backward not bitwise repeatable"


def test_qhead_router_backward_is_rejected():
    w = CASES[0]
    P = prepared(w)
    d = P["dev"]
    idx, logg = _sel(P)
    d2 = sas.make_dims(w.B, w.T, w.Hq, w.Hkv, w.D, w.dg, w.topk, w.theta, w.eps,
                       flags=sas.FLAG_GATE_PER_QUERY_HEAD)
    lib = sas.load_library()
    import ctypes
    p = ctypes.c_void_p(256)
    st = lib.sas_gate_score_bwd(ctypes.byref(d2), *([p] * 16), None, 0, None)
    assert st == sas.SAS_ERR_UNSUPPORTED


def test_qhead_prefill_8k():
    """The 8K prefill shape with one gate per query head: gate vectors and
    the selection of every row; attention of KV head 5 (its 4 query heads)
    in full and sampled rows of every head, forward and backward."""
    w = synth.PREFILL_8K.replace(name="qwen3_4b_prefill_T8192_K31_qhead", gate="q")
    x = synth.prefill_inputs(w, seed=0, device="cpu")
    x64 = {k: O.as64(v) for k, v in x.items()}
    d = {k: v.cuda() for k, v in x.items()}
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps, per_query_head=True)
    idx, logg, lse_g, _ = sas.topk_blocks(qg, kg, w.topk, w.Hq, w.D)
    torch.cuda.synchronize()
    ra = O.route_all(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"], w.topk,
                     w.theta, w.eps)
    check("q_gate", qg, ra["qg"], ROUTER_ABS, ROUTER_ABS)
    ok = ~ra["near_tie"]
    print(f"  near-tie rows {int((~ok).sum())} of {ok.size}", flush=True)
    assert ok.mean() > 0.99
    bad = (idx.cpu().numpy() != ra["idx"]).any(-1) & ok
    assert not bad.any(), f"{int(bad.sum())} rows differ"
    fin = np.isfinite(ra["logg"]) & ok[..., None]
    assert np.abs(logg.cpu().numpy()[fin] - ra["logg"][fin]).max() < ROUTER_ABS
    # attention on the oracle's selection
    idx_o = torch.tensor(ra["idx"], dtype=torch.int32).cuda()
    logg_o = torch.tensor(ra["logg"], dtype=torch.float32).cuda()
    sc = 1.0 / math.sqrt(w.D)
    o, lse, o32 = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx_o, logg_o, sc, want_f32=True)
    dq, dk, dv, dlogg = sas.sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx_o,
                                            logg_o, sc, o_f32=o32)
    torch.cuda.synchronize()
    kv = 5
    dk_ref = np.zeros((w.T, w.D))
    dv_ref = np.zeros((w.T, w.D))
    for h in range(kv * w.G, (kv + 1) * w.G):
        a = O.attn_head(x64["q"], x64["k"], x64["v"], ra["idx"], ra["logg"], sc, 0, h,
                        dout=x64["dout"])
        check(f"o[h={h}]", o[0, :, h:h + 1], a["o"])
        check(f"dq[h={h}]", dq[0, :, h:h + 1], a["dq"])
        check(f"dlogg[h={h}]", dlogg[0, :, h], a["dlogg"])
        dk_ref += a["dk"]
        dv_ref += a["dv"]
    check(f"dk[kv={kv}]", dk[0, :, kv], dk_ref)
    check(f"dv[kv={kv}]", dv[0, :, kv], dv_ref)
    tok = np.unique(np.concatenate([[0, 63, 64, w.T - 1],
                                    np.random.default_rng(3).choice(w.T, 128, replace=False)]))
    tt = torch.as_tensor(tok, device="cuda")
    ro, _ = O.attn_fwd_rows(x64["q"], x64["k"], x64["v"], ra["idx"], ra["logg"], sc, tokens=tok)
    check("o (sampled rows, all heads)", o[:, tt], ro)
    assert float(dlogg.sum(-1).abs().max()) < 1e-3


DEC = [(3, 8, 2, 128, 128, 7, 5000, [5000, 1, 64]),
       (4, 8, 2, 128, 128, 31, 4200, [65, 4200, 2049, 128]),
       (2, 10, 2, 64, 32, 3, 700, [700, 300]),
       (96, 8, 2, 64, 32, 5, 700,
        [1, 64, 65, 700] + [int(v) for v in np.random.default_rng(5).integers(1, 701, size=92)])]


@pytest.mark.parametrize("case", DEC, ids=[f"qdec{i}" for i in range(len(DEC))])
def test_qhead_decode(case):
    """Decode with one gate per query head (units = (sequence, query head)),
    contiguous and paged caches, against the oracle."""
    B, Hq, Hkv, D, dg, K, Lmax, lens = case
    w = synth.Workload("qdec", 97, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, kind="decode",
                       Lmin=1, Lmax=Lmax, gate="q")
    x = synth.decode_inputs(w, seed=1, device="cpu", ctx_len=torch.tensor(lens, dtype=torch.int32))
    assert tuple(x["q_gate"].shape) == (B, Hq, dg)
    sc = 1.0 / math.sqrt(D)
    ref = O.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], x["kg_cache"], x["ctx_len"],
                   K, sc)
    dv = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in x.items()}
    o, idx, logg = sas.decode(dv["q"], dv["q_gate"], dv["k_cache"], dv["v_cache"],
                              dv["kg_cache"], dv["ctx_len"], K, sc)
    torch.cuda.synchronize()
    ok = ~ref["near_tie"]
    np.testing.assert_array_equal(idx.cpu().numpy()[ok], ref["idx"][ok])
    fin = np.isfinite(ref["logg"]) & ok[..., None]
    assert np.abs(logg.cpu().numpy()[fin] - ref["logg"][fin]).max() < ROUTER_ABS
    check("o", o[torch.from_numpy(ok).cuda()], ref["o"][ok])
    # the same through a paged pool
    NB = x["NBmax"]
    npages = B * NB + 3
    perm = torch.from_numpy(np.random.default_rng(9).permutation(npages)[:B * NB]
                            .astype(np.int32)).view(B, NB).cuda()
    flat = perm.flatten().long()
    Tp = NB * 64

    def pages(c):
        pad = torch.zeros((B, Hkv, Tp, D), dtype=c.dtype, device="cuda")
        pad[:, :, :c.shape[2]] = c
        pool = torch.zeros((npages, Hkv, 64, D), dtype=c.dtype, device="cuda")
        pool[flat] = pad.view(B, Hkv, NB, 64, D).permute(0, 2, 1, 3, 4).reshape(B * NB, Hkv, 64, D)
        return pool

    gpool = torch.zeros((npages, Hkv, dg), dtype=torch.float32, device="cuda")
    gpool[flat] = dv["kg_cache"].permute(0, 2, 1, 3).reshape(B * NB, Hkv, dg)
    o_p, idx_p, _ = sas.decode_paged(dv["q"], dv["q_gate"], pages(dv["k_cache"]),
                                     pages(dv["v_cache"]), gpool, perm, dv["ctx_len"], K, sc)
    torch.cuda.synchronize()
    assert torch.equal(idx_p, idx)
    assert torch.equal(o_p.view(torch.int16), o.view(torch.int16))
