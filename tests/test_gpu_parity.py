"""GPU parity: every libsas call against the fp64 oracle on seeded inputs.

Sizes are small enough for the oracle to finish in seconds while spanning
several 64-token blocks, ragged tails, GQA group sizes 1/2/4/5/8, K = 0 and
K beyond the number of blocks.  Tolerances: selected block indices
bit-exact outside near-tie rows (K-th/(K+1)-th gate-logit gap < 1e-5 in
fp64; exact ties go to the lower index and are compared like any other
row); bf16 outputs and gradients within 1e-2 max-abs beyond the bf16
representation error of the exact value (half a bf16 ulp of the reference,
which alone reaches 1.6e-2 for |x| in [4, 8)) and a raw 1e-3 mean-abs;
fp32 outputs (log-gate gradient, lse) and router outputs within the
stated absolute bounds with no allowance.
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


def W(name, T, Hq, Hkv, D, dg, K, B=1, cfg=90):
    return synth.Workload(name, cfg, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K)


CASES = [
    synth.TINY,
    W("g4_ragged", 1000, 8, 2, 128, 128, 7),
    W("g5", 700, 10, 2, 128, 128, 5),
    W("g1_b2", 300, 2, 2, 64, 64, 2, B=2),
    W("short", 50, 4, 1, 128, 128, 3),
    W("k0", 400, 4, 2, 64, 32, 0),
    W("kbig", 600, 4, 1, 128, 128, 20),
    W("g8", 260, 8, 1, 128, 128, 3),
]
IDS = [c.name for c in CASES]

_cache = {}


def prepared(w, seed=0):
    key = (w.name, seed)
    if key in _cache:
        return _cache[key]
    x = synth.prefill_inputs(w, seed=seed, device="cpu")
    x64 = {k: O.as64(v) for k, v in x.items()}
    r = O.route(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"], w.topk,
                w.theta, w.eps)
    kg_all = O.gate_key(x64["k"], x64["wk"], x64["w_kn"], w.theta, w.eps)
    sc = 1.0 / math.sqrt(w.D)
    g = O.attn_bwd(x64["q"], x64["k"], x64["v"], x64["dout"], r["idx"], r["logg"], sc)
    dev = {k: v.cuda() for k, v in x.items()}
    out = dict(x=x, x64=x64, r=r, kg_all=kg_all, g=g, dev=dev, scale=sc)
    _cache[key] = out
    return out


def bf16_half_ulp(x):
    """Half a bf16 ulp (8 significant bits) at |x|."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def errs(gpu, ref):
    """(raw max-abs, max-abs beyond bf16 representation, raw mean-abs)."""
    a = gpu.detach().float().cpu().numpy().astype(np.float64)
    d = np.abs(a - ref)
    excess = d
    if gpu.dtype == torch.bfloat16:
        excess = np.maximum(0.0, d - bf16_half_ulp(np.maximum(np.abs(ref), np.abs(a))))
    return float(d.max()), float(excess.max()), float(d.mean())


def assert_close(name, gpu, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    """Max-abs beyond the bf16 rounding of the exact value (a bf16 output
    cannot be closer than that), raw mean-abs with no allowance."""
    raw, mx, mn = errs(gpu, ref)
    print(f"  {name}: max-abs {raw:.3e} (beyond bf16 rounding {mx:.3e}) mean-abs {mn:.3e}",
          flush=True)
    assert mx <= max_abs and mn <= mean_abs, (name, raw, mx, mn)


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_gate_score(w):
    P = prepared(w)
    d = P["dev"]
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps)
    torch.cuda.synchronize()
    assert_close("q_gate", qg, P["r"]["qg"], ROUTER_ABS, ROUTER_ABS)
    assert_close("k_gate", kg, P["kg_all"], ROUTER_ABS, ROUTER_ABS)


# (D, dg) pairs the parity shapes above leave out, so that every tiling of
# the gate-key projection (column groups of four waves at dg >= 64, two
# column groups of two row groups at dg = 32) runs with both head sizes;
# ragged last blocks
ROUTER_DIMS = [
    W("d128_dg32", 300, 4, 2, 128, 32, 3),
    W("d128_dg64", 200, 8, 2, 128, 64, 3),
    W("d64_dg128", 260, 4, 1, 64, 128, 3),
]


@pytest.mark.parametrize("w", ROUTER_DIMS, ids=[c.name for c in ROUTER_DIMS])
def test_gate_score_dims(w):
    x = synth.prefill_inputs(w, seed=3, device="cpu", with_dout=False)
    x64 = {k: O.as64(v) for k, v in x.items()}
    r = O.route(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"], w.topk,
                w.theta, w.eps)
    kg_all = O.gate_key(x64["k"], x64["wk"], x64["w_kn"], w.theta, w.eps)
    d = {k: v.cuda() for k, v in x.items()}
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps)
    torch.cuda.synchronize()
    assert_close("q_gate", qg, r["qg"], ROUTER_ABS, ROUTER_ABS)
    assert_close("k_gate", kg, kg_all, ROUTER_ABS, ROUTER_ABS)


def _nontie(r):
    return ~r["near_tie"]


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_topk_on_oracle_gate_vectors(w):
    """Selection numerics alone: the oracle's q_gate / k_gate rounded to fp32."""
    P = prepared(w)
    r = P["r"]
    qg = torch.tensor(np.ascontiguousarray(r["qg"]), dtype=torch.float32).cuda()
    kg = torch.tensor(np.ascontiguousarray(P["kg_all"]), dtype=torch.float32).cuda()
    idx, logg, lse, probs = sas.topk_blocks(qg, kg, w.topk, w.Hq, w.D, want_probs=True)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    ok = _nontie(r)
    print(f"  near-tie rows: {int((~ok).sum())} of {ok.size}")
    assert (~ok).mean() < 0.01
    np.testing.assert_array_equal(gi[ok], r["idx"][ok])
    lg = logg.cpu().numpy().astype(np.float64)
    fin = np.isfinite(r["logg"]) & ok[..., None]
    assert np.all(np.isinf(lg[~np.isfinite(r["logg"])]))
    assert np.abs(lg[fin] - r["logg"][fin]).max() < ROUTER_ABS
    assert np.abs(lse.cpu().numpy() - r["lse"]).max() < ROUTER_ABS
    np.testing.assert_allclose(probs.sum(-1).cpu().numpy(), 1.0, atol=1e-5)
    assert np.abs(probs.cpu().numpy() - r["probs"]).max() < 1e-5


@pytest.mark.parametrize("T", [40000, 60000], ids=["T40000", "T60000"])
def test_topk_long_sequence(T):
    """Sequences of 625 and 938 blocks (up to 15 score registers per lane in
    the selection, score rows of 2.5-3.7 KiB per token in LDS): seeded N(0,1)
    fp32 gate vectors; on sampled tokens the indices must equal the oracle's
    selection outside near ties, and log g and lse must match."""
    K, dg = 31, 128
    g = torch.Generator().manual_seed(T)
    qg = torch.randn((1, T, 1, dg), generator=g)
    kg = torch.randn((1, T, 1, dg), generator=g)
    idx, logg, lse, _ = sas.topk_blocks(qg.cuda(), kg.cuda(), K, 4, 128)
    torch.cuda.synchronize()
    gi, gl, gz = idx.cpu().numpy(), logg.cpu().numpy(), lse.cpu().numpy()
    q64, k64 = qg.double().numpy()[0, :, 0], kg.double().numpy()[0, :, 0]
    bkt = O.block_key_tokens(T)
    rng = np.random.default_rng(T)
    toks = np.unique(np.concatenate([[0, 31, 32, 63, 64, 2047, 2048, T - 33, T - 32, T - 1],
                                     rng.choice(T, 400, replace=False)]))
    near = 0
    for t in toks:
        c = t // 64
        s = O.gate_logits(q64[t], k64[bkt[:c]], k64[t])
        lse_o, lg = O.log_gates(s)
        sel, nt = O.select_blocks(s, K)
        assert abs(gz[0, t, 0] - lse_o) < ROUTER_ABS, t
        if nt:
            near += 1
            continue
        n = len(sel)
        np.testing.assert_array_equal(gi[0, t, 0, :n], sel, err_msg=f"token {t}")
        assert np.all(gi[0, t, 0, n:] == -1)
        assert np.abs(gl[0, t, 0, :n] - lg[sel]).max() < ROUTER_ABS, t
    assert near < len(toks) // 20


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_router_and_topk_chain(w):
    P = prepared(w)
    d = P["dev"]
    r = P["r"]
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps)
    idx, logg, lse, _ = sas.topk_blocks(qg, kg, w.topk, w.Hq, w.D)
    torch.cuda.synchronize()
    ok = _nontie(r)
    gi = idx.cpu().numpy()
    mism = (gi != r["idx"]).any(-1) & ok
    print(f"  index mismatches on non-near-tie rows: {int(mism.sum())}")
    np.testing.assert_array_equal(gi[ok], r["idx"][ok])
    fin = np.isfinite(r["logg"]) & ok[..., None]
    assert np.abs(logg.cpu().numpy()[fin] - r["logg"][fin]).max() < ROUTER_ABS


def _oracle_sel(P):
    r = P["r"]
    idx = torch.tensor(np.ascontiguousarray(r["idx"]), dtype=torch.int32).cuda()
    logg = torch.tensor(np.ascontiguousarray(r["logg"]), dtype=torch.float32).cuda()
    return idx, logg


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_sparse_attn_fwd(w):
    P = prepared(w)
    d = P["dev"]
    idx, logg = _oracle_sel(P)
    o, lse = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"])
    torch.cuda.synchronize()
    assert_close("o", o, P["g"]["o"])
    assert_close("lse", lse, P["g"]["lse"], 1e-3, 1e-4)
    o2, lse2 = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "forward not bitwise repeatable"


@pytest.mark.parametrize("w", CASES[:2], ids=IDS[:2])
def test_sparse_attn_fwd_large_values(w):
    """v scaled by 2^17 (exact in bf16, beyond the fp16 range of the transposed
    copy): the output scales exactly, so o / 2^17 must match the oracle's o."""
    P = prepared(w)
    d = P["dev"]
    idx, logg = _oracle_sel(P)
    big = float(2 ** 17)
    o, lse, o32 = sas.sparse_attn_fwd(d["q"], d["k"], (d["v"].float() * big).to(torch.bfloat16),
                                      idx, logg, P["scale"], want_f32=True)
    torch.cuda.synchronize()
    assert_close("o/2^17", (o.float() / big).to(torch.bfloat16), P["g"]["o"])
    assert_close("o_f32/2^17", o32 / big, P["g"]["o"])
    assert_close("lse", lse, P["g"]["lse"], 1e-3, 1e-4)


@pytest.mark.parametrize("use_f32", [False, True], ids=["o_bf16", "o_f32"])
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_sparse_attn_bwd(w, use_f32):
    """Backward with the fp32 forward output (the training-step path: Delta
    from o before bf16 rounding) and from the bf16 output alone.  Without
    o_f32, Delta carries the bf16 rounding of o times |dout| sqrt(D); that
    error enters dlogg scaled by the slot's attention mass (up to 1) and
    breaks its zero sum, so in that mode only dq, dk, dv are held to the
    bound."""
    P = prepared(w)
    d = P["dev"]
    idx, logg = _oracle_sel(P)
    if use_f32:
        o, lse, o32 = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"],
                                          want_f32=True)
        assert_close("o_f32", o32, P["g"]["o"])
    else:
        o, lse = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"])
        o32 = None
    dq, dk, dv, dlogg = sas.sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx, logg,
                                            P["scale"], o_f32=o32)
    torch.cuda.synchronize()
    g = P["g"]
    assert_close("dq", dq, g["dq"])
    assert_close("dk", dk, g["dk"])
    assert_close("dv", dv, g["dv"])
    if use_f32:
        assert_close("dlogg", dlogg, g["dlogg"])
        # gradient w.r.t. log g sums to zero over each row's selected slots
        assert float(dlogg.sum(-1).abs().max()) < 1e-3
    out2 = sas.sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx, logg, P["scale"],
                               o_f32=o32)
    torch.cuda.synchronize()
    for a, b in zip((dq, dk, dv, dlogg), out2):
        assert torch.equal(a, b), "backward not bitwise repeatable"


@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_gate_score_bwd(w):
    """Router backward from the oracle's selection and its attention dlogg
    (rows summing to zero), against the oracle's chain rule; every output is
    an fp32 gradient held to the bf16-gradient bound.  Bitwise repeatable."""
    P = prepared(w)
    d = P["dev"]
    x64 = P["x64"]
    idx, _ = _oracle_sel(P)
    dl = torch.tensor(np.where(P["r"]["idx"] >= 0, P["g"]["dlogg"], 0.0), dtype=torch.float32)
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps)
    out = sas.gate_score_bwd(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], qg, kg, idx,
                             dl.cuda(), w.theta, w.eps)
    torch.cuda.synchronize()
    ref = O.router_bwd(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"],
                       P["r"]["idx"], O.as64(dl), w.theta, w.eps)
    for name in ("dq", "dk", "dwq", "dwk", "dw_qn", "dw_kn"):
        assert_close(name, out[name], ref[name])
    out2 = sas.gate_score_bwd(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], qg, kg, idx,
                              dl.cuda(), w.theta, w.eps)
    torch.cuda.synchronize()
    for name in out:
        assert torch.equal(out[name], out2[name]), (name, "router backward not repeatable")


@pytest.mark.parametrize("w", CASES[:3], ids=IDS[:3])
def test_gate_score_bwd_nonzero_row_sums(w):
    """A dlogg whose rows do not sum to zero (e.g. from an extra loss on log
    g): the library differentiates sum dlogg * s over the selected logits with
    the row's lse held constant (documented in sas.h), which the oracle's
    router backward computes with lse_term=False; the binding warns."""
    P = prepared(w)
    d = P["dev"]
    x64 = P["x64"]
    idx, _ = _oracle_sel(P)
    rng = np.random.default_rng(17)
    dl = torch.tensor(np.where(P["r"]["idx"] >= 0, rng.standard_normal(P["r"]["idx"].shape), 0.0),
                      dtype=torch.float32)
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps)
    with pytest.warns(UserWarning, match="do not sum to zero"):
        out = sas.gate_score_bwd(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], qg, kg,
                                 idx, dl.cuda(), w.theta, w.eps)
    torch.cuda.synchronize()
    ref = O.router_bwd(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"],
                       P["r"]["idx"], O.as64(dl), w.theta, w.eps, lse_term=False)
    for name in ("dq", "dk", "dwq", "dwk", "dw_qn", "dw_kn"):
        assert_close(name, out[name], ref[name])


def test_outputs_stay_in_bounds():
    """NaN canaries after every output buffer stay untouched."""
    w = CASES[1]
    P = prepared(w)
    d = P["dev"]
    idx, logg = _oracle_sel(P)
    B, T, Hq, D, Hkv, S = w.B, w.T, w.Hq, w.D, w.Hkv, w.topk + 1
    pad = 4096

    def canary(shape, dtype):
        n = int(np.prod(shape))
        buf = torch.full((n + pad,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[:n].view(shape)

    ob, o = canary((B, T, Hq, D), torch.bfloat16)
    lb, lse = canary((B, T, Hq), torch.float32)
    sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"], o=o, lse=lse)
    bufs = [canary((B, T, Hq, D), torch.bfloat16), canary((B, T, Hkv, D), torch.bfloat16),
            canary((B, T, Hkv, D), torch.bfloat16), canary((B, T, Hkv, S), torch.float32)]
    sas.sparse_attn_bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, idx, logg, P["scale"],
                        out=tuple(b[1] for b in bufs))
    torch.cuda.synchronize()
    for b, _ in [(ob, 0), (lb, 0)] + bufs:
        assert torch.isnan(b[-pad:].float()).all()
    for _, v in [(ob, o), (lb, lse)] + bufs:
        assert not torch.isnan(v.float()).any()


# ---------------------------------------------------------------- decode

DEC_CASES = [
    # (B, Hq, Hkv, D, dg, K, Lmax, lengths)
    (3, 8, 2, 128, 128, 7, 5000, [5000, 1, 64]),
    (4, 8, 2, 128, 128, 31, 4200, [65, 4200, 2049, 128]),
    (2, 10, 2, 64, 32, 3, 700, [700, 300]),
    # beyond 1,024 blocks (the selection's long-context path); one visible key
    (2, 2, 1, 64, 32, 5, 70000, [70000, 4161]),
    # budgets 1,024 and 4,096 (K = 15, 63; at K = 63 more than 64 keys pass
    # the lane-maximum bound, so the selection searches all keys)
    (4, 8, 2, 128, 128, 15, 9000, [9000, 1100, 64, 4097]),
    (3, 8, 2, 128, 128, 63, 20000, [20000, 4100, 12000]),
    # 512 units: one workgroup walks all of a unit's slots and writes the
    # output (no split partials); an odd number of two-block passes, one-token
    # and partial current blocks, contexts shorter than the budget
    (128, 8, 4, 64, 32, 5, 700,
     [1, 64, 65, 700] + [int(v) for v in np.random.default_rng(5).integers(1, 701, size=124)]),
    (128, 12, 4, 128, 64, 3, 400,
     [1, 64, 65, 400] + [int(v) for v in np.random.default_rng(6).integers(1, 401, size=124)]),
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[f"dec{i}" for i in range(len(DEC_CASES))])
@pytest.mark.parametrize("apply_gate", [True, False])
def test_decode(case, apply_gate):
    B, Hq, Hkv, D, dg, K, Lmax, lens = case
    w = synth.Workload("dec", 91, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, kind="decode",
                       Lmin=1, Lmax=Lmax)
    x = synth.decode_inputs(w, seed=1, device="cpu", ctx_len=torch.tensor(lens, dtype=torch.int32))
    sc = 1.0 / math.sqrt(D)
    ref = O.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], x["kg_cache"], x["ctx_len"],
                   K, sc, apply_gate=apply_gate)
    dev = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in x.items()}
    o, idx, logg = sas.decode(dev["q"], dev["q_gate"], dev["k_cache"], dev["v_cache"],
                              dev["kg_cache"], dev["ctx_len"], K, sc, apply_gate=apply_gate)
    torch.cuda.synchronize()
    ok = ~ref["near_tie"]
    np.testing.assert_array_equal(idx.cpu().numpy()[ok], ref["idx"][ok])
    fin = np.isfinite(ref["logg"]) & ok[..., None]
    assert np.abs(logg.cpu().numpy()[fin] - ref["logg"][fin]).max() < ROUTER_ABS
    assert_close("o", o, ref["o"])


@pytest.mark.parametrize("case", [DEC_CASES[i] for i in (0, 1, 3, 4)], ids=["dec0", "dec1", "dec3", "dec4"])
def test_decode_bf16_gate_keys(case):
    """Gate-key cache in bf16 (kg_dtype = 1): the oracle scores the same
    bf16 values; selection bit-exact outside near ties, as with fp32 keys."""
    B, Hq, Hkv, D, dg, K, Lmax, lens = case
    w = synth.Workload("dec", 91, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, kind="decode",
                       Lmin=1, Lmax=Lmax)
    x = synth.decode_inputs(w, seed=2, device="cpu", ctx_len=torch.tensor(lens, dtype=torch.int32))
    kg16 = x["kg_cache"].to(torch.bfloat16)
    sc = 1.0 / math.sqrt(D)
    ref = O.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], kg16.float(), x["ctx_len"], K,
                   sc)
    dev = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in x.items()}
    o, idx, logg = sas.decode(dev["q"], dev["q_gate"], dev["k_cache"], dev["v_cache"], kg16.cuda(),
                              dev["ctx_len"], K, sc)
    torch.cuda.synchronize()
    ok = ~ref["near_tie"]
    np.testing.assert_array_equal(idx.cpu().numpy()[ok], ref["idx"][ok])
    fin = np.isfinite(ref["logg"]) & ok[..., None]
    assert np.abs(logg.cpu().numpy()[fin] - ref["logg"][fin]).max() < ROUTER_ABS
    assert_close("o", o, ref["o"])


@pytest.mark.parametrize("case", DEC_CASES, ids=[f"dec{i}" for i in range(len(DEC_CASES))])
def test_decode_paged(case):
    """Paged cache: every (sequence, block) in its own page of a shuffled pool
    (spare pages and every page row past a context filled with NaN, table
    entries past a sequence's blocks pointing outside the pool), with fp32
    and bf16 gate keys: indices bit-exact with the oracle outside near ties
    and outputs within the bound, and, since the arithmetic is the same in the
    same order, bitwise equal to sas_decode's on the contiguous cache."""
    B, Hq, Hkv, D, dg, K, Lmax, lens = case
    w = synth.Workload("dec", 91, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, kind="decode",
                       Lmin=1, Lmax=Lmax)
    x = synth.decode_inputs(w, seed=1, device="cuda", ctx_len=torch.tensor(lens, dtype=torch.int32))
    sc = 1.0 / math.sqrt(D)
    o_c, idx_c, lg_c = sas.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], x["kg_cache"],
                                  x["ctx_len"], K, sc)
    NB = -(-Lmax // 64)
    npages = B * NB + 5
    perm = torch.from_numpy(np.random.default_rng(7).permutation(npages)[:B * NB].astype(np.int32))
    perm = perm.view(B, NB).cuda()
    nan = float("nan")
    kp = torch.full((npages, Hkv, 64, D), nan, dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, nan)
    gp = torch.full((npages, Hkv, dg), nan, dtype=torch.float32, device="cuda")
    # rows at or past each context length stay NaN in the pages
    tok = torch.arange(NB * 64, device="cuda")
    live = (tok[None, :] < x["ctx_len"][:, None].long()).view(B, 1, NB * 64, 1)

    def blocks(c):
        pad = torch.full((B, Hkv, NB * 64, D), nan, dtype=c.dtype, device="cuda")
        pad[:, :, :c.shape[2]] = c
        pad = torch.where(live, pad, torch.full_like(pad, nan))
        return pad.view(B, Hkv, NB, 64, D).permute(0, 2, 1, 3, 4).reshape(B * NB, Hkv, 64, D)

    flat = perm.flatten().long()
    kp[flat] = blocks(x["k_cache"])
    vp[flat] = blocks(x["v_cache"])
    gp[flat] = x["kg_cache"].permute(0, 2, 1, 3).reshape(B * NB, Hkv, dg)
    nblk = (x["ctx_len"].long() - 1) // 64 + 1
    table = torch.where(torch.arange(NB, device="cuda")[None, :] < nblk[:, None], perm,
                        torch.full_like(perm, npages + 3))
    o_p, idx_p, lg_p = sas.decode_paged(x["q"], x["q_gate"], kp, vp, gp, table.contiguous(),
                                        x["ctx_len"], K, sc)
    torch.cuda.synchronize()
    # against the oracle directly (not only against the contiguous path)
    xc = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}
    ref = O.decode(xc["q"], xc["q_gate"], xc["k_cache"], xc["v_cache"], xc["kg_cache"],
                   xc["ctx_len"], K, sc)
    ok = ~ref["near_tie"]
    np.testing.assert_array_equal(idx_p.cpu().numpy()[ok], ref["idx"][ok])
    fin = np.isfinite(ref["logg"]) & ok[..., None]
    assert np.abs(lg_p.cpu().numpy()[fin] - ref["logg"][fin]).max() < ROUTER_ABS
    G = Hq // Hkv
    okh = np.repeat(ok, G, axis=1)
    assert_close("o (paged)", o_p[torch.from_numpy(okh).cuda()], ref["o"][okh])
    assert torch.equal(idx_p, idx_c)
    assert torch.equal(lg_p.nan_to_num(), lg_c.nan_to_num())
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16))
    # the same with bf16 gate keys on both sides
    o_c, idx_c, lg_c = sas.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"],
                                  x["kg_cache"].to(torch.bfloat16), x["ctx_len"], K, sc)
    o_p, idx_p, lg_p = sas.decode_paged(x["q"], x["q_gate"], kp, vp, gp.to(torch.bfloat16),
                                        table.contiguous(), x["ctx_len"], K, sc)
    torch.cuda.synchronize()
    ref = O.decode(xc["q"], xc["q_gate"], xc["k_cache"], xc["v_cache"],
                   xc["kg_cache"].to(torch.bfloat16).float(), xc["ctx_len"], K, sc)
    ok = ~ref["near_tie"]
    np.testing.assert_array_equal(idx_p.cpu().numpy()[ok], ref["idx"][ok])
    okh = np.repeat(ok, G, axis=1)
    assert_close("o (paged, bf16 keys)", o_p[torch.from_numpy(okh).cuda()], ref["o"][okh])
    assert torch.equal(idx_p, idx_c)
    assert torch.equal(lg_p.nan_to_num(), lg_c.nan_to_num())
    assert torch.equal(o_p.view(torch.int16), o_c.view(torch.int16))


@pytest.mark.parametrize("w", CASES[:3], ids=IDS[:3])
@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("kg_dtype", [torch.float32, torch.bfloat16], ids=["kg32", "kg16"])
def test_decode_gate_key(w, paged, kg_dtype):
    """Current-block gate key refreshed from the KV cache after an append:
    for sequences at positions t (block starts, block ends, partial blocks)
    the entry of block t // 64 must equal the oracle's prefill gate key of
    token t; every other entry stays as it was."""
    x = synth.prefill_inputs(w, seed=3, device="cpu", with_dout=False)
    T, Hkv, D, dg = w.T, w.Hkv, w.D, w.dg
    w_kn = 1.0 + 0.25 * torch.randn(dg, generator=torch.Generator().manual_seed(9))
    ts = sorted({0, 1, 63, 64, 65, T // 2, T - 2, T - 1} & set(range(T)))
    B = len(ts)
    ref = O.gate_key(x["k"], x["wk"], w_kn.numpy(), w.theta, w.eps, tokens=ts)[0]  # [n,Hkv,dg]
    NB = -(-T // 64)
    kc = x["k"][0].transpose(0, 1).contiguous()[None].expand(B, -1, -1, -1).contiguous().cuda()
    ctx = torch.tensor([t + 1 for t in ts], dtype=torch.int32, device="cuda")
    wk, wkn = x["wk"].cuda(), w_kn.cuda()
    if not paged:
        kg = torch.full((B, Hkv, NB, dg), 7.0, dtype=kg_dtype, device="cuda")
        sas.decode_gate_key(kc, wk, wkn, ctx, kg, w.theta, w.eps)
        torch.cuda.synchronize()
        got = torch.stack([kg[b, :, t // 64] for b, t in enumerate(ts)]).float().cpu().numpy()
        mask = torch.ones((B, NB), dtype=torch.bool)
        for b, t in enumerate(ts):
            mask[b, t // 64] = False
        rest = kg.permute(0, 2, 1, 3)[mask.cuda()]
    else:
        Tp = NB * 64
        pad = torch.zeros((B, Hkv, Tp, D), dtype=torch.bfloat16, device="cuda")
        pad[:, :, :T] = kc
        npages = B * NB + 3
        perm = torch.from_numpy(np.random.default_rng(8).permutation(npages)[:B * NB]
                                .astype(np.int32)).view(B, NB).cuda()
        pool = torch.zeros((npages, Hkv, 64, D), dtype=torch.bfloat16, device="cuda")
        pool[perm.flatten().long()] = pad.view(B, Hkv, NB, 64, D).permute(0, 2, 1, 3, 4).reshape(
            B * NB, Hkv, 64, D)
        kg = torch.full((npages, Hkv, dg), 7.0, dtype=kg_dtype, device="cuda")
        sas.decode_gate_key(pool, wk, wkn, ctx, kg, w.theta, w.eps, block_table=perm)
        torch.cuda.synchronize()
        pages = [int(perm[b, t // 64]) for b, t in enumerate(ts)]
        got = kg[pages].float().cpu().numpy()
        mask = torch.ones(npages, dtype=torch.bool)
        mask[pages] = False
        rest = kg[mask.cuda()]
    assert bool((rest.float() == 7.0).all()), "entries other than the current blocks changed"
    if kg_dtype == torch.float32:
        assert np.abs(got - ref).max() < ROUTER_ABS
    else:
        r16 = torch.from_numpy(ref).float().to(torch.bfloat16).float().numpy()
        half_ulp = np.abs(r16) * 2.0 ** -8
        assert (np.abs(got - ref) <= half_ulp + ROUTER_ABS).all()


def test_decode_matches_prefill_row():
    """Decode of token L-1 equals the prefill row L-1 computed by the library."""
    w = CASES[1]
    P = prepared(w)
    d = P["dev"]
    qg, kg = sas.gate_score(d["q"], d["k"], d["wq"], d["wk"], d["w_qn"], d["w_kn"], w.topk,
                            w.theta, w.eps)
    idx, logg, _, _ = sas.topk_blocks(qg, kg, w.topk, w.Hq, w.D)
    o, _ = sas.sparse_attn_fwd(d["q"], d["k"], d["v"], idx, logg, P["scale"])
    L = torch.tensor([w.T, 333, 64], dtype=torch.int32)
    B = len(L)
    NBmax = -(-w.T // 64)
    kc = d["k"][0].transpose(0, 1).contiguous()[None].expand(B, -1, -1, -1).contiguous()
    vc = d["v"][0].transpose(0, 1).contiguous()[None].expand(B, -1, -1, -1).contiguous()
    kgc = torch.zeros((B, w.Hkv, NBmax, w.dg), dtype=torch.float32, device="cuda")
    qd = torch.empty((B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    qgd = torch.empty((B, w.Hkv, w.dg), dtype=torch.float32, device="cuda")
    for bi, Lb in enumerate(L.tolist()):
        c = (Lb - 1) // 64
        for j in range(c):
            kgc[bi, :, j] = kg[0, 64 * j + 63]
        kgc[bi, :, c] = kg[0, Lb - 1]
        qd[bi] = d["q"][0, Lb - 1]
        qgd[bi] = qg[0, Lb - 1]
    od, idd, _ = sas.decode(qd, qgd, kc, vc, kgc, L.cuda(), w.topk, P["scale"])
    torch.cuda.synchronize()
    # prefill scores come from fp32 MFMA tiles, decode scores from a differently
    # ordered fp32 reduction: rows the oracle marks near-tie (K-th/(K+1)-th gap
    # < 1e-5) may legitimately differ and are left out, as in the other tests
    G = w.Hq // w.Hkv
    checked = 0
    for bi, Lb in enumerate(L.tolist()):
        for kv in range(w.Hkv):
            if P["r"]["near_tie"][0, Lb - 1, kv]:
                continue
            checked += 1
            assert torch.equal(idd[bi, kv], idx[0, Lb - 1, kv])
            hs = slice(kv * G, (kv + 1) * G)
            diff = (od[bi, hs].float() - o[0, Lb - 1, hs].float()).abs().max().item()
            assert diff <= 1e-2, diff
    assert checked >= len(L) * w.Hkv - 1
