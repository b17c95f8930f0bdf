"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test compares the oracle with a brute force, a closed form, a textbook
special case computed by a library routine (torch SDPA / autograd in fp64),
a finite difference, or numbers printed on the pages.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

from oracle import sas_oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def small_case(T=200, B=1, Hq=4, Hkv=2, D=16, dg=8, K=1, seed=0, theta=1e4, bf16=False):
    w = synth.Workload("pin", 99, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, theta=theta)
    dt = torch.bfloat16 if bf16 else torch.float32
    x = synth.prefill_inputs(w, seed=seed, dtype=dt)
    return w, {k: O.as64(v) for k, v in x.items()}


def sdpa64(q, k, v, mask=None, is_causal=False, scale=None):
    """torch SDPA (math backend, fp64) on [B,T,H,D] numpy inputs, GQA by repeat."""
    G = q.shape[2] // k.shape[2]
    qt = torch.tensor(q).permute(0, 2, 1, 3)
    kt = torch.tensor(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.tensor(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    with sdpa_kernel(SDPBackend.MATH):
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, is_causal=is_causal,
                                           scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# ---------------------------------------------------------------- selection

def test_topk_matches_brute_force_random():
    rng = np.random.default_rng(1)
    for _ in range(300):
        c = int(rng.integers(0, 9))
        K = int(rng.integers(0, 5))
        s = rng.standard_normal(c + 1)
        sel, _ = O.select_blocks(s, K)
        assert sel[-1] == c
        assert sel[:-1] == O.brute_force_topk(list(s[:c]), K)


def test_topk_ties_go_to_lower_index():
    rng = np.random.default_rng(2)
    for _ in range(300):
        c = int(rng.integers(1, 9))
        K = int(rng.integers(1, 5))
        s = rng.integers(-2, 3, size=c + 1).astype(float)   # many exact ties
        sel, near = O.select_blocks(s, K)
        assert sel[:-1] == O.brute_force_topk(list(s[:c]), K)
        if c > K:
            srt = sorted(s[:c], reverse=True)
            assert near == (srt[K - 1] - srt[K] < 1e-5)


def test_topk_degenerate_counts():
    s = np.array([0.3, -1.0, 2.0, 0.1, 5.0])          # c = 4
    assert O.select_blocks(s, 0)[0] == [4]              # K = 0: current only
    assert O.select_blocks(s, 4)[0] == [0, 1, 2, 3, 4]  # K >= c: every block
    assert O.select_blocks(s, 9)[0] == [0, 1, 2, 3, 4]
    assert O.select_blocks(np.array([1.0]), 3)[0] == [0]  # t < 64: one block


# ---------------------------------------------------------------- gates

def test_gates_sum_to_one_and_shift_invariant():
    w, x = small_case(T=300, K=2)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], 2, w.theta, w.eps)
    np.testing.assert_allclose(r["probs"].sum(-1), 1.0, atol=1e-12)
    # log g = s - logsumexp(s) is unchanged by a constant shift of all s
    rng = np.random.default_rng(0)
    for _ in range(20):
        s = rng.standard_normal(int(rng.integers(1, 12)))
        a = O.log_gates(s)[1]
        b = O.log_gates(s + 3.7)[1]
        np.testing.assert_allclose(a, b, atol=1e-12)
        np.testing.assert_allclose(np.exp(a).sum(), 1.0, atol=1e-12)


# ---------------------------------------------------------------- router pieces

def test_rope_is_complex_rotation():
    rng = np.random.default_rng(3)
    dg, theta = 16, 1e6
    x = rng.standard_normal(dg)
    for pos in (0, 1, 63, 4096, 32767):
        z = x[:dg // 2] + 1j * x[dg // 2:]
        f = theta ** (-np.arange(dg // 2) * 2.0 / dg)
        zr = z * np.exp(1j * pos * f)
        want = np.concatenate([zr.real, zr.imag])
        np.testing.assert_allclose(O.rope(x, pos, theta), want, atol=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(4)
    a, b = rng.standard_normal(32), rng.standard_normal(32)
    for m, n in ((5, 2), (1000, 64), (32767, 32704)):
        lhs = O.rope(a, m, 1e6) @ O.rope(b, n, 1e6)
        rhs = O.rope(a, m - n, 1e6) @ b
        assert abs(lhs - rhs) < 1e-9


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 32)) * 3
    y = O.rms_norm(x, np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(-1)), 1.0, atol=1e-12)
    np.testing.assert_allclose(O.rms_norm(4.5 * x, np.ones(32), 0.0), y, atol=1e-12)


def test_pooling_order_and_prefix():
    """[max; min; mean] order and causal prefix pooling, probed through Wk."""
    B, T, Hkv, D, dg = 1, 130, 1, 4, 4
    rng = np.random.default_rng(6)
    k = rng.standard_normal((B, T, Hkv, D))
    for part, fn in ((0, np.max), (1, np.min), (2, np.mean)):
        wk = np.zeros((1, 3 * D, dg))
        wk[0, part * D + 0, 0] = 1.0          # picks channel 0 of one pooled section
        wk[0, part * D + 1, 1] = 1.0
        for t in (0, 5, 63, 64, 100, 129):
            c = t // 64
            p = O.pooled_key(k, t)[0, 0]
            np.testing.assert_allclose(p[part * D:(part + 1) * D],
                                       fn(k[0, 64 * c:t + 1, 0], axis=0), atol=1e-15)
            # through the projection: before norm/rope the first two outputs are
            # the selected channels
            z = p @ wk[0]
            assert z[0] == pytest.approx(fn(k[0, 64 * c:t + 1, 0, 0]))
    # block start: all three sections equal the token's own key
    p = O.pooled_key(k, 64)[0, 0]
    np.testing.assert_allclose(p, np.concatenate([k[0, 64, 0]] * 3), atol=0)


def test_gate_key_is_causal_and_gate_query_is_grouped():
    w, x = small_case(T=150, K=1)
    kg = O.gate_key(x["k"], x["wk"], x["w_kn"], w.theta, w.eps)
    k2 = x["k"].copy()
    k2[:, 100:] += 7.0                          # future of token 99
    kg2 = O.gate_key(k2, x["wk"], x["w_kn"], w.theta, w.eps)
    np.testing.assert_array_equal(kg[:, :100], kg2[:, :100])
    assert not np.allclose(kg[:, 100:], kg2[:, 100:])
    qg = O.gate_query(x["q"], x["wq"], x["w_qn"], w.theta, w.eps)
    q2 = x["q"].copy()
    q2[:, :, 2:] += 1.0                          # heads of group 1 only (G = 2)
    qg2 = O.gate_query(q2, x["wq"], x["w_qn"], w.theta, w.eps)
    np.testing.assert_array_equal(qg[:, :, 0], qg2[:, :, 0])
    assert not np.allclose(qg[:, :, 1], qg2[:, :, 1])


def test_router_parameter_count_matches_model_card():
    """Qproj over the concatenated group + Kproj over [max;min;mean] + two norm
    weights reproduce the released gate sizes (model card checkpoint table)."""
    g = json.load(open(os.path.join(GOLD, "router_param_counts.json")))
    for m in g["models"]:
        n = O.router_param_count(m["Hq"], m["Hkv"], m["D"], m["dg"], m["layers"])
        assert round(n / 1e6, 1) == m["params_M"], m["name"]
        mib = n * 2 / 2 ** 20                  # bf16 storage
        assert m["size_MiB"] - 1.5 <= mib <= m["size_MiB"], (m["name"], mib)
        # rejected alternative: one mean-pooled gate query per KV head
        alt = m["layers"] * (m["Hkv"] * m["D"] * m["dg"] + m["Hkv"] * 3 * m["D"] * m["dg"])
        assert round(alt / 1e6, 1) != m["params_M"]


# ---------------------------------------------------------------- attention forward

def _route(w, x, K):
    return O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, w.theta, w.eps)


def test_uniform_gates_full_topk_is_dense_causal():
    """Wq = 0 -> gate query 0 -> uniform gates; K covering every block ->
    plain causal GQA attention (torch SDPA, is_causal)."""
    w, x = small_case(T=200, Hq=4, Hkv=2, D=16, K=8)
    x["wq"] = np.zeros_like(x["wq"])
    r = _route(w, x, 8)
    sc = 1 / math.sqrt(w.D)
    o_g, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
    o_d, _ = O.attn_fwd_dense(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
    ref = sdpa64(x["q"], x["k"], x["v"], is_causal=True, scale=sc)
    np.testing.assert_allclose(o_g, ref, atol=1e-12)
    np.testing.assert_allclose(o_d, ref, atol=1e-12)


def test_gather_form_matches_sdpa_with_block_bias():
    """General K: SDPA with an additive float mask (log g of the key's block
    when selected and causal, else -inf)."""
    for K, T, G in ((1, 200, 2), (2, 260, 1), (3, 129, 4)):
        w, x = small_case(T=T, Hq=2 * G, Hkv=2, D=16, K=K, seed=K)
        r = _route(w, x, K)
        sc = 1 / math.sqrt(w.D)
        o_g, lse_g = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
        mask = np.full((1, w.Hq, T, T), -np.inf)
        for t in range(T):
            for kv in range(w.Hkv):
                for s_i, j in enumerate(r["idx"][0, t, kv]):
                    if j < 0:
                        continue
                    for tau in range(64 * j, min(64 * j + 64, t + 1)):
                        mask[0, kv * G:(kv + 1) * G, t, tau] = r["logg"][0, t, kv, s_i]
        ref = sdpa64(x["q"], x["k"], x["v"], mask=torch.tensor(mask), scale=sc)
        np.testing.assert_allclose(o_g, ref, atol=1e-12)
        o_d, lse_d = O.attn_fwd_dense(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
        np.testing.assert_allclose(o_d, o_g, atol=1e-12)
        np.testing.assert_allclose(lse_d, lse_g, atol=1e-12)


def test_k0_is_block_diagonal_causal():
    w, x = small_case(T=230, Hq=2, Hkv=1, D=16, K=0)
    r = _route(w, x, 0)
    sc = 1 / math.sqrt(w.D)
    o, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
    t = np.arange(w.T)
    allowed = (t[:, None] // 64 == t[None, :] // 64) & (t[None, :] <= t[:, None])
    mask = torch.tensor(np.where(allowed, 0.0, -np.inf))
    ref = sdpa64(x["q"], x["k"], x["v"], mask=mask, scale=sc)
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_short_sequence_is_plain_causal_and_mha():
    for G in (1, 2):
        w, x = small_case(T=50, Hq=2 * G, Hkv=2, D=16, K=3)
        r = _route(w, x, 3)
        np.testing.assert_allclose(r["logg"][..., 0], 0.0, atol=1e-15)   # g = 1
        sc = 1 / math.sqrt(w.D)
        o, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
        ref = sdpa64(x["q"], x["k"], x["v"], is_causal=True, scale=sc)
        np.testing.assert_allclose(o, ref, atol=1e-12)


def test_gate_bias_shift_on_selected_blocks_cancels():
    """A per-row constant added to every selected slot's log g leaves o unchanged
    (softmax shift invariance; why the gate normaliser cancels inside attention)."""
    w, x = small_case(T=200, K=2)
    r = _route(w, x, 2)
    sc = 1 / math.sqrt(w.D)
    o1, lse1 = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
    shift = np.random.default_rng(0).standard_normal(r["logg"].shape[:-1])[..., None]
    o2, lse2 = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"] + shift, sc)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    G = w.G
    np.testing.assert_allclose(lse2 - lse1, np.repeat(shift[..., 0], G, axis=2), atol=1e-12)


# ---------------------------------------------------------------- backward

def test_backward_matches_torch_autograd():
    for K, G in ((1, 2), (2, 1)):
        w, x = small_case(T=190, Hq=2 * G, Hkv=2, D=16, K=K, seed=10 + K)
        T = w.T
        r = _route(w, x, K)
        sc = 1 / math.sqrt(w.D)
        g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)
        bias = O.dense_bias(r["idx"], r["logg"], T)                # [B,Hkv,T,T]
        qt = torch.tensor(x["q"], requires_grad=True)
        kt = torch.tensor(x["k"], requires_grad=True)
        vt = torch.tensor(x["v"], requires_grad=True)
        mt = torch.tensor(np.repeat(bias, G, axis=1), requires_grad=True)
        with sdpa_kernel(SDPBackend.MATH):
            o = F.scaled_dot_product_attention(
                qt.permute(0, 2, 1, 3),
                kt.permute(0, 2, 1, 3).repeat_interleave(G, 1),
                vt.permute(0, 2, 1, 3).repeat_interleave(G, 1),
                attn_mask=mt, scale=sc).permute(0, 2, 1, 3)
        (o * torch.tensor(x["dout"])).sum().backward()
        np.testing.assert_allclose(g["o"], o.detach().numpy(), atol=1e-12)
        np.testing.assert_allclose(g["dq"], qt.grad.numpy(), atol=1e-11)
        np.testing.assert_allclose(g["dk"], kt.grad.numpy(), atol=1e-11)
        np.testing.assert_allclose(g["dv"], vt.grad.numpy(), atol=1e-11)
        dm = mt.grad.numpy()                                       # [B,Hq,T,T]
        dl = np.zeros_like(g["dlogg"])
        for t in range(T):
            for kv in range(w.Hkv):
                for s_i, j in enumerate(r["idx"][0, t, kv]):
                    if j >= 0:
                        dl[0, t, kv, s_i] = dm[0, kv * G:(kv + 1) * G, t,
                                               64 * j:64 * j + 64].sum()
        np.testing.assert_allclose(g["dlogg"], dl, atol=1e-11)


def test_backward_finite_differences():
    w, x = small_case(T=140, Hq=4, Hkv=2, D=8, K=1, seed=21)
    r = _route(w, x, 1)
    sc = 1 / math.sqrt(w.D)
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)

    def loss(q, k, v, logg):
        o, _ = O.attn_fwd_rows(q, k, v, r["idx"], logg, sc)
        return float((o * x["dout"]).sum())

    rng = np.random.default_rng(7)
    h = 1e-6
    for name, arr_key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("logg", "dlogg")):
        base = dict(q=x["q"], k=x["k"], v=x["v"], logg=r["logg"])
        for _ in range(6):
            a = base[name]
            while True:
                pos = tuple(int(rng.integers(0, s)) for s in a.shape)
                if np.isfinite(a[pos]):
                    break
            p, m = dict(base), dict(base)
            p[name] = a.copy()
            m[name] = a.copy()
            p[name][pos] += h
            m[name][pos] -= h
            fd = (loss(**p) - loss(**m)) / (2 * h)
            an = g[arr_key][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, pos, fd, an)


def test_dlogg_sums_to_zero_over_selected_slots():
    w, x = small_case(T=260, Hq=4, Hkv=2, D=16, K=2, seed=3)
    r = _route(w, x, 2)
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], 1 / 4)
    np.testing.assert_allclose(g["dlogg"].sum(-1), 0.0, atol=1e-12)


def test_gate_logit_gradient_finite_differences():
    """ds (gradient reaching the gate logits s) vs central differences with the
    selection frozen; s enters only through log g = s - lse(s)."""
    w, x = small_case(T=200, Hq=2, Hkv=1, D=8, K=1, seed=5)
    r = _route(w, x, 1)
    sc = 1 / math.sqrt(w.D)
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)
    ds = O.gate_logit_grad(g["dlogg"], r["idx"], r["probs"])
    # selected slots: ds = dlogg because the dlogg sum is zero
    rng = np.random.default_rng(8)
    h = 1e-6
    for _ in range(12):
        t = int(rng.integers(64, w.T))
        c = t // 64
        j = int(rng.integers(0, c + 1))

        def loss(delta):
            s = r["s"][0, t, 0, :c + 1].copy()
            s[j] += delta
            lse, lg = O.log_gates(s)
            logg = r["logg"].copy()
            sel = r["idx"][0, t, 0]
            logg[0, t, 0] = np.where(sel >= 0, lg[np.maximum(sel, 0)], -np.inf)
            o, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], logg, sc, tokens=[t])
            return float((o[0, 0] * x["dout"][0, t]).sum())

        fd = (loss(h) - loss(-h)) / (2 * h)
        assert abs(fd - ds[0, t, 0, j]) < 1e-7, (t, j, fd, ds[0, t, 0, j])


def test_row_and_block_backward_helpers_match_full():
    w, x = small_case(T=200, Hq=4, Hkv=2, D=16, K=2, seed=9)
    r = _route(w, x, 2)
    sc = 1 / math.sqrt(w.D)
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)
    toks = [0, 63, 64, 130, 199]
    dq, dl = O.attn_bwd_rows(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc, toks)
    np.testing.assert_allclose(dq, g["dq"][:, toks], atol=1e-13)
    np.testing.assert_allclose(dl, g["dlogg"][:, toks], atol=1e-13)
    for kv, j in ((0, 0), (1, 1), (1, 3)):
        dk, dv = O.attn_bwd_block(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"],
                                  sc, 0, kv, j)
        hi = min(64 * j + 64, w.T)
        np.testing.assert_allclose(dk, g["dk"][0, 64 * j:hi, kv], atol=1e-13)
        np.testing.assert_allclose(dv, g["dv"][0, 64 * j:hi, kv], atol=1e-13)


# ---------------------------------------------------------------- decode

def test_decode_equals_prefill_last_row():
    w, x = small_case(T=700, B=2, Hq=4, Hkv=2, D=16, dg=8, K=3, seed=4)
    L = np.array([700, 333])
    sc = 1 / math.sqrt(w.D)
    B, Hkv = w.B, w.Hkv
    r = _route(w, x, 3)
    o_pre, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
    NBmax = -(-w.T // 64)
    kg_all = O.gate_key(x["k"], x["wk"], x["w_kn"], w.theta, w.eps)
    q_dec = np.stack([x["q"][b, L[b] - 1] for b in range(B)])
    qg = np.stack([r["qg"][b, L[b] - 1] for b in range(B)])
    kcache = x["k"].transpose(0, 2, 1, 3).copy()
    vcache = x["v"].transpose(0, 2, 1, 3).copy()
    kgc = np.zeros((B, Hkv, NBmax, w.dg))
    for b in range(B):
        c = (L[b] - 1) // 64
        for j in range(c):
            kgc[b, :, j] = kg_all[b, 64 * j + 63]
        kgc[b, :, c] = kg_all[b, L[b] - 1]
    d = O.decode(q_dec, qg, kcache, vcache, kgc, L, 3, sc)
    for b in range(B):
        np.testing.assert_allclose(d["o"][b], o_pre[b, L[b] - 1], atol=1e-12)
        np.testing.assert_array_equal(d["idx"][b], r["idx"][b, L[b] - 1])
        np.testing.assert_allclose(d["logg"][b], r["logg"][b, L[b] - 1], atol=1e-12)
    # selection-only variant = SDPA over the same selected keys with no bias
    d0 = O.decode(q_dec, qg, kcache, vcache, kgc, L, 3, sc, apply_gate=False)
    for b in range(B):
        for kv in range(Hkv):
            taus = np.concatenate([np.arange(64 * j, min(64 * j + 64, L[b]))
                                   for j in d0["idx"][b, kv] if j >= 0])
            Kr = kcache[b, kv, taus]
            Vr = vcache[b, kv, taus]
            for i in range(w.G):
                h = kv * w.G + i
                ref = sdpa64(q_dec[b, h][None, None, None], Kr[None, :, None], Vr[None, :, None],
                             scale=sc)[0, 0, 0]
                np.testing.assert_allclose(d0["o"][b, h], ref, atol=1e-12)


# ---------------------------------------------------------------- router backward

def _router_case(seed=11, T=200, Hq=4, Hkv=2, D=16, dg=8, K=1):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((1, T, Hq, D)), k=rng.standard_normal((1, T, Hkv, D)),
             wq=rng.standard_normal((Hkv, Hq // Hkv * D, dg)) / math.sqrt(Hq // Hkv * D),
             wk=rng.standard_normal((Hkv, 3 * D, dg)) / math.sqrt(3 * D),
             w_qn=1 + 0.2 * rng.standard_normal(dg), w_kn=1 + 0.2 * rng.standard_normal(dg))
    return x, K


def _frozen_logg_loss(x, K, idx, dlogg, theta=1e4, eps=1e-6):
    """L = sum dlogg * log g on the fixed slots idx (selection checked unchanged)."""
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, theta, eps)
    assert np.array_equal(r["idx"], idx), "selection moved under the perturbation"
    s = np.take_along_axis(r["s"], np.maximum(idx, 0), axis=-1)
    logg = s - r["lse"][..., None]
    return float(np.where(idx >= 0, dlogg * logg, 0.0).sum())


@pytest.mark.parametrize("name", ["q", "k", "wq", "wk", "w_qn", "w_kn"])
def test_router_backward_finite_differences(name):
    """Every router gradient vs central differences of L = sum dlogg * log g
    with the selection frozen; dlogg is arbitrary here (its valid slots need
    not sum to zero), so the full gate-logit gradient is exercised."""
    x, K = _router_case()
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, 1e4, 1e-6)
    rng = np.random.default_rng(12)
    dlogg = rng.standard_normal(r["idx"].shape)
    g = O.router_bwd(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], r["idx"], dlogg,
                     1e4, 1e-6)
    grad = {"q": g["dq"], "k": g["dk"], "wq": g["dwq"], "wk": g["dwk"], "w_qn": g["dw_qn"],
            "w_kn": g["dw_kn"]}[name]
    h = 1e-6
    flat = x[name].reshape(-1)
    picks = rng.choice(flat.size, size=min(10, flat.size), replace=False)
    if name == "k":   # include rows that are a channel's max / min of their prefix
        picks = np.concatenate([picks, [0, 5 * x["k"].shape[-1] + 3]])
    for i in picks:
        old = flat[i]
        flat[i] = old + h
        lp = _frozen_logg_loss(x, K, r["idx"], dlogg)
        flat[i] = old - h
        lm = _frozen_logg_loss(x, K, r["idx"], dlogg)
        flat[i] = old
        fd = (lp - lm) / (2 * h)
        an = grad.reshape(-1)[i]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, i, fd, an)


def _frozen_logit_loss(x, K, idx, dlogg, theta=1e4, eps=1e-6):
    """L = sum dlogg * s over the fixed selected slots (no lse term)."""
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, theta, eps)
    assert np.array_equal(r["idx"], idx), "selection moved under the perturbation"
    s = np.take_along_axis(r["s"], np.maximum(idx, 0), axis=-1)
    return float(np.where(idx >= 0, dlogg * s, 0.0).sum())


@pytest.mark.parametrize("name", ["q", "k", "wq", "wk"])
def test_router_backward_without_lse_term_finite_differences(name):
    """lse_term=False: the gradient of sum dlogg * s_selected (what the
    library's router backward computes for any dlogg) vs central differences,
    with a dlogg whose rows do not sum to zero."""
    x, K = _router_case(seed=15)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, 1e4, 1e-6)
    rng = np.random.default_rng(16)
    dlogg = rng.standard_normal(r["idx"].shape)
    g = O.router_bwd(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], r["idx"], dlogg,
                     1e4, 1e-6, lse_term=False)
    grad = {"q": g["dq"], "k": g["dk"], "wq": g["dwq"], "wk": g["dwk"]}[name]
    h = 1e-6
    flat = x[name].reshape(-1)
    for i in rng.choice(flat.size, size=min(10, flat.size), replace=False):
        old = flat[i]
        flat[i] = old + h
        lp = _frozen_logit_loss(x, K, r["idx"], dlogg)
        flat[i] = old - h
        lm = _frozen_logit_loss(x, K, r["idx"], dlogg)
        flat[i] = old
        fd = (lp - lm) / (2 * h)
        an = grad.reshape(-1)[i]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, i, fd, an)


def test_router_backward_zero_sum_dlogg_reaches_selected_logits_only():
    """With dlogg summing to zero over each row's valid slots (what the gated
    attention produces), ds is dlogg on the selected blocks and zero elsewhere."""
    x, K = _router_case(seed=13, T=260, K=2)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, 1e4, 1e-6)
    rng = np.random.default_rng(14)
    d = np.where(r["idx"] >= 0, rng.standard_normal(r["idx"].shape), 0.0)
    nvalid = (r["idx"] >= 0).sum(-1, keepdims=True)
    d = np.where(r["idx"] >= 0, d - d.sum(-1, keepdims=True) / nvalid, 0.0)
    g = O.router_bwd(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], r["idx"], d,
                     1e4, 1e-6)
    want = np.zeros_like(g["ds"])
    for pos in np.ndindex(*r["idx"].shape[:-1]):
        for s_i, j in enumerate(r["idx"][pos]):
            if j >= 0:
                want[pos + (j,)] = d[pos + (s_i,)]
    np.testing.assert_allclose(g["ds"], want, atol=1e-13)


def test_router_backward_pooling_ties_go_to_first_row():
    """bf16 keys tie often; a channel's max / min gradient goes to the first row
    of the prefix that attains it (reading), checked on a hand-made block."""
    k = np.zeros((1, 3, 1, 2))
    k[0, :, 0, 0] = [1.0, 1.0, 0.5]       # max tie at rows 0, 1; min row 2
    k[0, :, 0, 1] = [0.0, -1.0, -1.0]     # max row 0; min tie at rows 1, 2
    _, amax, amin, n = O._pool_with_args(k)
    assert amax[0, 2, 0].tolist() == [0, 0] and amin[0, 2, 0].tolist() == [2, 1]
    assert n.tolist() == [1, 2, 3]


# ------------------------------------------------ whole-sequence evaluations

def test_select_rows_matches_brute_force_with_ties():
    """The many-row selection against the subset brute force, on integer
    scores full of exact ties (ties -> lower index), and its K-th gap."""
    rng = np.random.default_rng(11)
    for _ in range(60):
        c = int(rng.integers(0, 9))
        K = int(rng.integers(0, 6))
        s = rng.integers(-2, 3, size=(7, c)).astype(float)
        sel, gap = O.select_rows(s, K)
        for r in range(7):
            assert list(sel[r]) == O.brute_force_topk(list(s[r]), K)
            full = np.concatenate([s[r], [0.0]])
            assert gap[r] == O.kth_gap(full, K)
            if c > K >= 1:
                srt = sorted(s[r], reverse=True)
                assert gap[r] == srt[K - 1] - srt[K]


@pytest.mark.parametrize("shape", [dict(T=1000, Hq=8, Hkv=2, D=16, dg=8, K=7),
                                   dict(T=700, Hq=10, Hkv=2, D=16, dg=8, K=5),
                                   dict(T=300, B=2, Hq=2, Hkv=2, D=16, dg=8, K=2),
                                   dict(T=400, Hq=4, Hkv=2, D=16, dg=8, K=0),
                                   dict(T=600, Hq=4, Hkv=1, D=16, dg=8, K=20),
                                   dict(T=50, Hq=4, Hkv=1, D=16, dg=8, K=3)])
def test_route_all_matches_route(shape):
    """route_all (every token at once) equals route (token by token)."""
    K = shape.pop("K")
    w, x = small_case(K=K, bf16=True, **shape)
    args = (x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], w.topk, w.theta, w.eps)
    r, ra = O.route(*args), O.route_all(*args)
    np.testing.assert_array_equal(ra["idx"], r["idx"])
    np.testing.assert_array_equal(np.isinf(ra["logg"]), np.isinf(r["logg"]))
    fin = np.isfinite(r["logg"])
    assert np.abs(ra["logg"][fin] - r["logg"][fin]).max() < 1e-12
    assert np.abs(ra["lse"] - r["lse"]).max() < 1e-12
    assert np.abs(ra["qg"] - r["qg"]).max() < 1e-12
    assert np.abs(ra["kg"] - r["kg_cur"]).max() < 1e-12
    np.testing.assert_array_equal(np.isinf(ra["gap"]), np.isinf(r["gap"]))
    g = np.isfinite(r["gap"])
    assert not g.any() or np.abs(ra["gap"][g] - r["gap"][g]).max() < 1e-12
    np.testing.assert_array_equal(ra["near_tie"], r["near_tie"])


@pytest.mark.parametrize("shape", [dict(T=1000, Hq=8, Hkv=2, D=16, dg=8, K=7),
                                   dict(T=700, Hq=10, Hkv=2, D=16, dg=8, K=5),
                                   dict(T=300, B=2, Hq=2, Hkv=2, D=16, dg=8, K=2),
                                   dict(T=130, Hq=4, Hkv=1, D=16, dg=8, K=0)])
def test_attn_head_matches_row_form_and_sdpa(shape):
    """attn_head (all rows of one head, keys grouped per block for dk/dv)
    equals attn_bwd (row by row), and its o equals SDPA with the additive
    block bias (-inf on keys the row did not select)."""
    K = shape.pop("K")
    w, x = small_case(K=K, **shape)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], w.topk, w.theta, w.eps)
    sc = 1.0 / math.sqrt(w.D)
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)
    bias = O.dense_bias(r["idx"], r["logg"], w.T)               # [B,Hkv,T,T]
    G = w.G
    for b in range(w.B):
        for kv in range(w.Hkv):
            a = O.attn_head(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc, b, kv,
                            dout=x["dout"], batch=7)
            hs = slice(kv * G, (kv + 1) * G)
            for name, ref in (("o", g["o"][b, :, hs]), ("lse", g["lse"][b, :, hs]),
                              ("dq", g["dq"][b, :, hs]), ("dlogg", g["dlogg"][b, :, kv]),
                              ("dk", g["dk"][b, :, kv]), ("dv", g["dv"][b, :, kv])):
                assert np.abs(a[name] - ref).max() < 1e-11, name
            mask = torch.tensor(bias[b:b + 1, kv:kv + 1])
            ref_o = sdpa64(x["q"][b:b + 1, :, hs], x["k"][b:b + 1, :, kv:kv + 1],
                           x["v"][b:b + 1, :, kv:kv + 1], mask=mask, scale=sc)
            assert np.abs(a["o"] - ref_o[0]).max() < 1e-11


# ------------------------------------------------ one gate per query head

def _qhead_case(T=260, Hq=4, Hkv=2, D=16, dg=8, K=2, seed=30):
    w = synth.Workload("pin_q", 99, B=1, T=T, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, theta=1e4,
                       gate="q")
    x = synth.prefill_inputs(w, seed=seed, dtype=torch.float32)
    return w, {k: O.as64(v) for k, v in x.items()}


def test_per_query_head_gates_equal_shared_gates_on_split_heads():
    """One gate per query head is the shared-gate method on a problem whose
    every query head has its own copy of its KV head (keys, values, Kproj):
    selection, log-gates, outputs and gradients must agree, with dk, dv the
    sums over the copies."""
    w, x = _qhead_case()
    G = w.G
    sc = 1 / math.sqrt(w.D)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], w.topk, w.theta, w.eps)
    assert r["idx"].shape[2] == w.Hq
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)
    ks, vs = np.repeat(x["k"], G, axis=2), np.repeat(x["v"], G, axis=2)
    wks = np.repeat(x["wk"], G, axis=0)
    r2 = O.route(x["q"], ks, x["wq"], wks, x["w_qn"], x["w_kn"], w.topk, w.theta, w.eps)
    np.testing.assert_array_equal(r["idx"], r2["idx"])
    fin = np.isfinite(r["logg"])
    np.testing.assert_allclose(r["logg"][fin], r2["logg"][fin], atol=1e-12)
    g2 = O.attn_bwd(x["q"], ks, vs, x["dout"], r2["idx"], r2["logg"], sc)
    for name in ("o", "lse", "dq", "dlogg"):
        np.testing.assert_allclose(g[name], g2[name], atol=1e-12, err_msg=name)
    B, T = w.B, w.T
    np.testing.assert_allclose(g["dk"], g2["dk"].reshape(B, T, w.Hkv, G, w.D).sum(3), atol=1e-12)
    np.testing.assert_allclose(g["dv"], g2["dv"].reshape(B, T, w.Hkv, G, w.D).sum(3), atol=1e-12)
    ra = O.route_all(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], w.topk, w.theta,
                     w.eps)
    np.testing.assert_array_equal(ra["idx"], r["idx"])
    for h in range(w.Hq):
        a = O.attn_head(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc, 0, h, dout=x["dout"])
        np.testing.assert_allclose(a["o"], g["o"][0, :, h:h + 1], atol=1e-12)
        np.testing.assert_allclose(a["dlogg"], g["dlogg"][0, :, h], atol=1e-12)


def test_per_query_head_backward_matches_autograd_and_fd():
    """Per-query-head selection: torch fp64 autograd of SDPA with each head's
    own additive block bias, and central differences of the gather form."""
    w, x = _qhead_case(T=190, K=1, seed=31)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], 1, w.theta, w.eps)
    sc = 1 / math.sqrt(w.D)
    g = O.attn_bwd(x["q"], x["k"], x["v"], x["dout"], r["idx"], r["logg"], sc)
    bias = O.dense_bias(r["idx"], r["logg"], w.T)            # [B,Hq,T,T]
    G = w.G
    qt = torch.tensor(x["q"], requires_grad=True)
    kt = torch.tensor(x["k"], requires_grad=True)
    vt = torch.tensor(x["v"], requires_grad=True)
    mt = torch.tensor(bias, requires_grad=True)
    with sdpa_kernel(SDPBackend.MATH):
        o = F.scaled_dot_product_attention(
            qt.permute(0, 2, 1, 3), kt.permute(0, 2, 1, 3).repeat_interleave(G, 1),
            vt.permute(0, 2, 1, 3).repeat_interleave(G, 1), attn_mask=mt,
            scale=sc).permute(0, 2, 1, 3)
    (o * torch.tensor(x["dout"])).sum().backward()
    np.testing.assert_allclose(g["o"], o.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(g["dq"], qt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(g["dk"], kt.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(g["dv"], vt.grad.numpy(), atol=1e-11)
    dm = mt.grad.numpy()
    for t in range(w.T):
        for h in range(w.Hq):
            for s_i, j in enumerate(r["idx"][0, t, h]):
                if j >= 0:
                    assert abs(g["dlogg"][0, t, h, s_i] - dm[0, h, t, 64 * j:64 * j + 64].sum()) < 1e-11
    np.testing.assert_allclose(g["dlogg"].sum(-1), 0.0, atol=1e-12)
    # central differences of L = sum o * dO on log g entries
    rng = np.random.default_rng(32)

    def loss(logg):
        o2, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], logg, sc)
        return float((o2 * x["dout"]).sum())

    for _ in range(6):
        while True:
            pos = tuple(int(rng.integers(0, s)) for s in r["logg"].shape)
            if np.isfinite(r["logg"][pos]):
                break
        p, m = r["logg"].copy(), r["logg"].copy()
        p[pos] += 1e-6
        m[pos] -= 1e-6
        fd = (loss(p) - loss(m)) / 2e-6
        assert abs(fd - g["dlogg"][pos]) <= 1e-6 * max(1.0, abs(fd))


def test_per_query_head_router_parameter_count_matches_model_card():
    """A gate per query head (Qproj Hq x D x dg) has exactly as many weights as
    one per KV head over the concatenated group (Hkv x G*D x dg), so the
    released sizes (model card checkpoint table) do not decide between them."""
    g = json.load(open(os.path.join(GOLD, "router_param_counts.json")))
    for m in g["models"]:
        a = O.router_param_count(m["Hq"], m["Hkv"], m["D"], m["dg"], m["layers"])
        b = O.router_param_count(m["Hq"], m["Hkv"], m["D"], m["dg"], m["layers"],
                                 per_query_head=True)
        assert a == b and round(b / 1e6, 1) == m["params_M"]


def test_per_query_head_decode_equals_prefill_last_row():
    """Decode with one gate per query head equals prefill row L-1."""
    w, x = _qhead_case(T=300, K=2, seed=33)
    r = O.route(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], 2, w.theta, w.eps)
    sc = 1 / math.sqrt(w.D)
    o_pre, _ = O.attn_fwd_rows(x["q"], x["k"], x["v"], r["idx"], r["logg"], sc)
    kg = O.gate_key_all(x["k"], x["wk"], x["w_kn"], w.theta, w.eps)
    L = np.array([300, 130, 64, 1])
    B = len(L)
    NB = -(-w.T // 64)
    kc = np.repeat(x["k"][0].transpose(1, 0, 2)[None], B, axis=0)
    vc = np.repeat(x["v"][0].transpose(1, 0, 2)[None], B, axis=0)
    kgc = np.zeros((B, w.Hkv, NB, w.dg))
    for b, Lb in enumerate(L):
        c = (Lb - 1) // 64
        for j in range(c):
            kgc[b, :, j] = kg[0, 64 * j + 63]
        kgc[b, :, c] = kg[0, Lb - 1]
    d = O.decode(x["q"][0, L - 1], r["qg"][0, L - 1], kc, vc, kgc, L, 2, sc)
    for b, Lb in enumerate(L):
        np.testing.assert_array_equal(d["idx"][b], r["idx"][0, Lb - 1])
        np.testing.assert_allclose(d["o"][b], o_pre[0, Lb - 1], atol=1e-12)
