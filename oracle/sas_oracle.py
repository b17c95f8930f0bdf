"""SAS gated block-sparse attention: plain fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it, and it shares no code with them.

What it computes (citations name the page and the passage):

* SAS, "Simple Attention Sparsification" abstract (arXiv 2609.13141 landing
  page, "The abstract"): a lightweight selector scores context blocks per
  query; Top-K picks historical blocks; the current block is always retained;
  the selector's continuous scores enter the attention softmax as log gates;
  gates are normalised by a softmax that includes the current block.
* GitHub README, intro items (a)/(b): discrete Top-K is kept, and every
  selected block carries a continuous soft gate inside the attention logits,
  so the LM loss has a gradient path to the selector.
* Hugging Face model card, "Checkpoint configuration" table: KV block 64,
  Top-K 31 historical blocks, gate hidden size 128, query projection Qproj,
  key block pooling max + min + average, Q/K normalisation, gate RoPE.
* Chinese usage guide, pitfall 3: the budget caps tokens attended per query,
  not the KV-cache size.

Readings where the pages are silent:
  gate per KV head, gate query = concatenation of the group's G query heads
  [R1]; gate inputs are the attention q/k before any backbone RoPE [R2];
  pooled key = [max; min; mean] channel-wise [R3]; the current block is
  pooled causally over 64c..t, so every query has its own current-block key
  [R4]; RMSNorm with a learnable weight, eps 1e-6 [R5]; rotate-half RoPE,
  inv_freq_i = theta^(-2i/dg), query at position t, block key at 64j [R6];
  bias-free Qproj [R7]; gate logit scale 1/sqrt(dg) [R8]; softmax over all
  candidate blocks 0..c including the current one [R9]; log g added to every
  selected block including the current one [R10]; Top-K over complete
  historical blocks j < c, K_eff = min(K, c) [R11]; ties -> lower index,
  near-tie = K-th/(K+1)-th gap < 1e-5 [R12]; attention scale 1/sqrt(D),
  causal inside the current block [R13]; slots ascending, current block last
  [R14]; budget = 64 (K + 1) [R15]; decode applies log g too (switchable)
  [R16]; partial last block keyed by its last token's prefix key [R19];
  in the router backward a channel's max / min passes its gradient to the
  first row of the prefix that attains it [R21].

Everything is float64 on numpy arrays.  Inputs are the bf16-rounded values
the GPU path consumes (or any float arrays for self-checks).
"""
from __future__ import annotations

import itertools
import math

import numpy as np

BLOCK = 64
NEAR_TIE_GAP = 1e-5


def as64(x) -> np.ndarray:
    """torch tensor or array -> float64 numpy array (copy)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# Router ("lightweight selector"): Qproj, block pooling, Q/K norm, gate RoPE.
# Model card, "Checkpoint configuration" table.
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis, times weight w [R5]."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding over the last axis (size dg) [R6].

    Pair (i, i + dg/2) is rotated by angle pos * theta^(-2i/dg).
    """
    dg = x.shape[-1]
    half = dg // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / dg)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def head_proj(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-head linear map without bias [R7]: out[..., h, :] = x[..., h, :] @ w[h].
    x [B, n, H, F], w [H, F, dg] -> [B, n, H, dg]."""
    return np.matmul(np.moveaxis(x, 2, 0), as64(w)[:, None]).transpose(1, 2, 0, 3)


def gate_query(q, wq, w_qn, theta: float, eps: float, tokens=None) -> np.ndarray:
    """Gate query per (b, t, kappa): RoPE_t(RMSNorm(x_t Wq[kappa]) * w_qn).

    x_t is the concatenation of the group's G query-head vectors [R1, R7].
    q [B,T,Hq,D], wq [Hkv, G*D, dg] -> [B, n, Hkv, dg] for the chosen tokens.
    """
    q = as64(q)
    wq = as64(wq)
    B, T, Hq, D = q.shape
    Hkv = wq.shape[0]
    G = Hq // Hkv
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    x = q[:, tok].reshape(B, len(tok), Hkv, G * D)
    y = head_proj(x, wq)
    y = rms_norm(y, as64(w_qn), eps)
    return rope(y, tok[None, :, None], theta)


def pooled_key(k: np.ndarray, t: int) -> np.ndarray:
    """[max; min; mean] over keys 64c..t of t's block c, channel-wise [R3, R4].

    k [B,T,Hkv,D] -> [B, Hkv, 3D].
    """
    c = t // BLOCK
    R = k[:, BLOCK * c: t + 1]
    return np.concatenate([R.max(axis=1), R.min(axis=1), R.mean(axis=1)], axis=-1)


def gate_key(k, wk, w_kn, theta: float, eps: float, tokens=None) -> np.ndarray:
    """Gate key per (b, t, kappa): RoPE_{64c}(RMSNorm(pool_t Wk[kappa]) * w_kn).

    The key of historical block j is the value at its last token 64j+63.
    k [B,T,Hkv,D], wk [Hkv, 3D, dg] -> [B, n, Hkv, dg].
    """
    k = as64(k)
    wk = as64(wk)
    B, T, Hkv, D = k.shape
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    out = np.empty((B, len(tok), Hkv, wk.shape[2]))
    for n, t in enumerate(tok):
        p = pooled_key(k, int(t))                       # [B, Hkv, 3D]
        z = np.einsum("bkf,kfg->bkg", p, wk)
        z = rms_norm(z, as64(w_kn), eps)
        out[:, n] = rope(z, (int(t) // BLOCK) * BLOCK, theta)
    return out


def block_key_tokens(T: int) -> np.ndarray:
    """Token whose prefix-pooled key represents each block (its last token) [R19]."""
    NB = -(-T // BLOCK)
    return np.minimum(np.arange(NB) * BLOCK + BLOCK - 1, T - 1)


# --------------------------------------------------------------------------
# Candidate softmax and Top-K (abstract: normalised softmax gates calibrate
# history against the always-retained current block; README (a)/(b)).
# --------------------------------------------------------------------------

def gate_logits(qg: np.ndarray, kg_hist: np.ndarray, kg_cur: np.ndarray) -> np.ndarray:
    """s_j = qg . kg_j / sqrt(dg) for historical blocks j < c, then the current block [R8].

    qg [dg], kg_hist [c, dg], kg_cur [dg] -> s [c+1].
    """
    dg = qg.shape[-1]
    return np.concatenate([kg_hist @ qg, [kg_cur @ qg]]) / math.sqrt(dg)


def log_gates(s: np.ndarray):
    """Softmax over all candidates 0..c [R9]: returns (lse, log g)."""
    m = s.max()
    lse = m + math.log(np.exp(s - m).sum())
    return lse, s - lse


def select_blocks(s: np.ndarray, K: int):
    """Top-K historical blocks by score (ties -> lower index) plus the current block.

    s [c+1] (last entry = current block c).  Returns (sel, near_tie): sel is
    ascending with c last [R11, R12, R14]; near_tie flags a K-th/(K+1)-th
    gap below 1e-5.
    """
    c = len(s) - 1
    n = min(K, c)
    order = sorted(range(c), key=lambda j: (-s[j], j))
    sel = sorted(order[:n]) + [c]
    near_tie = bool(K >= 1 and c > K and (s[order[K - 1]] - s[order[K]]) < NEAR_TIE_GAP)
    return sel, near_tie


def kth_gap(s: np.ndarray, K: int) -> float:
    """Gap between the K-th and (K+1)-th largest historical scores of a row
    (s [c+1], current block last); +inf when no historical block is left out
    (c <= K or K = 0).  0 means an exact tie across the selection boundary,
    which the lower-index rule decides [R12]."""
    c = len(s) - 1
    if K < 1 or c <= K:
        return math.inf
    h = np.sort(np.asarray(s[:c]))[::-1]
    return float(h[K - 1] - h[K])


def route(q, k, wq, wk, w_qn, w_kn, K: int, theta: float, eps: float, tokens=None):
    """Router + candidate softmax + selection for the chosen tokens.

    Selection heads Hs = wq.shape[0] (see sel_heads): Hkv with one gate per KV
    head [R1], Hq with one gate per query head; head sg scores the gate keys of
    KV head sg * (Hq / Hs) // G.
    Returns dict with qg [B,n,Hs,dg], kg_cur [B,n,Hkv,dg], idx [B,n,Hs,K+1]
    (pad -1), logg [B,n,Hs,K+1] (pad -inf), lse [B,n,Hs], near_tie, gap
    [B,n,Hs], s [B,n,Hs,NB] (-inf beyond c), probs [B,n,Hs,NB] (0 beyond c).
    """
    q = as64(q)
    k = as64(k)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    Hs = as64(wq).shape[0]
    _, kv_of = sel_heads(Hq, Hkv, Hs)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    NB = -(-T // BLOCK)
    S = K + 1
    qg = gate_query(q, wq, w_qn, theta, eps, tok)
    kg_cur = gate_key(k, wk, w_kn, theta, eps, tok)
    kblk_tok = block_key_tokens(T)
    need = sorted({int(kblk_tok[j]) for t in tok for j in range(int(t) // BLOCK)})
    kblk = {}
    if need:
        kg_need = gate_key(k, wk, w_kn, theta, eps, need)
        for n, t in enumerate(need):
            kblk[t // BLOCK] = kg_need[:, n]
    n_tok = len(tok)
    idx = np.full((B, n_tok, Hs, S), -1, dtype=np.int64)
    logg = np.full((B, n_tok, Hs, S), -np.inf)
    lse = np.zeros((B, n_tok, Hs))
    near = np.zeros((B, n_tok, Hs), dtype=bool)
    gap = np.full((B, n_tok, Hs), np.inf)
    s_dense = np.full((B, n_tok, Hs, NB), -np.inf)
    probs = np.zeros((B, n_tok, Hs, NB))
    for n, t in enumerate(tok):
        c = int(t) // BLOCK
        for b in range(B):
            for sg in range(Hs):
                kv = kv_of(sg)
                hist = (np.stack([kblk[j][b, kv] for j in range(c)]) if c
                        else np.zeros((0, qg.shape[-1])))
                s = gate_logits(qg[b, n, sg], hist, kg_cur[b, n, kv])
                l, lg = log_gates(s)
                sel, nt = select_blocks(s, K)
                idx[b, n, sg, :len(sel)] = sel
                logg[b, n, sg, :len(sel)] = lg[sel]
                lse[b, n, sg] = l
                near[b, n, sg] = nt
                gap[b, n, sg] = kth_gap(s, K)
                s_dense[b, n, sg, :c + 1] = s
                probs[b, n, sg, :c + 1] = np.exp(lg)
    return dict(qg=qg, kg_cur=kg_cur, idx=idx, logg=logg, lse=lse, near_tie=near, gap=gap,
                s=s_dense, probs=probs, tokens=tok)


# --------------------------------------------------------------------------
# Gated sparse attention: log g inside the softmax logits (abstract; README (b)).
# --------------------------------------------------------------------------

def _row_keys(t: int, sel_row: np.ndarray):
    """Key positions of the selected blocks that are <= t, with their slot ids [R13]."""
    taus, slots = [], []
    for s_i, j in enumerate(sel_row):
        j = int(j)
        if j < 0:
            continue
        hi = min(BLOCK * j + BLOCK, t + 1)
        r = np.arange(BLOCK * j, hi)
        taus.append(r)
        slots.append(np.full(len(r), s_i))
    return np.concatenate(taus), np.concatenate(slots)


def sel_heads(Hq: int, Hkv: int, Hs: int):
    """Selection heads: the heads that each carry one gate and one selection.
    With one gate per KV head [R1], Hs = Hkv and selection head sg covers the
    query heads sg*G .. sg*G+G-1; with one gate per query head (the
    alternative reading of "per query"), Hs = Hq and sg covers query head sg
    alone.  Returns (Gs, kv_of): query heads per selection head and the KV head
    (sg * Gs // G) whose keys selection head sg attends."""
    if Hs not in (Hkv, Hq):
        raise ValueError(f"selection heads must be Hkv ({Hkv}) or Hq ({Hq}), got {Hs}")
    G, Gs = Hq // Hkv, Hq // Hs
    return Gs, (lambda sg: sg * Gs // G)


def attn_fwd_rows(q, k, v, idx, logg, scale: float, tokens=None):
    """Gather form: per (b, t, selection head), concatenate the selected blocks' keys.

    l_tau = q.k_tau * scale + logg[slot(tau)];  o = softmax(l) V;  lse = logsumexp(l).
    idx/logg are [B, T, Hs, S] (full token axis; Hs selection heads, see
    sel_heads).  Returns o [B,n,Hq,D], lse [B,n,Hq] for the chosen tokens.
    """
    q, k, v, logg = as64(q), as64(k), as64(v), as64(logg)
    idx = np.asarray(idx)
    B, T, Hq, D = q.shape
    Hkv, Hs = k.shape[2], idx.shape[2]
    Gs, kv_of = sel_heads(Hq, Hkv, Hs)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    o = np.zeros((B, len(tok), Hq, D))
    lse = np.zeros((B, len(tok), Hq))
    for n, t in enumerate(tok):
        t = int(t)
        for b in range(B):
            for sg in range(Hs):
                kv = kv_of(sg)
                taus, slots = _row_keys(t, idx[b, t, sg])
                Kr, Vr = k[b, taus, kv], v[b, taus, kv]
                bias = logg[b, t, sg, slots]
                hs = slice(sg * Gs, (sg + 1) * Gs)
                Q = q[b, t, hs]                                # [Gs, D]
                L = Q @ Kr.T * scale + bias                    # [Gs, n]
                m = L.max(axis=1, keepdims=True)
                P = np.exp(L - m)
                l = P.sum(axis=1, keepdims=True)
                o[b, n, hs] = (P / l) @ Vr
                lse[b, n, hs] = (m + np.log(l))[:, 0]
    return o, lse


def dense_bias(idx, logg, T: int) -> np.ndarray:
    """Dense-masked form: bias [B, Hs, T, T] (per selection head) = logg of the
    key's block when the block is selected by the query and tau <= t, else -inf."""
    idx = np.asarray(idx)
    logg = as64(logg)
    B, _, Hs, S = idx.shape
    bias = np.full((B, Hs, T, T), -np.inf)
    for b in range(B):
        for t in range(T):
            for sg in range(Hs):
                for s_i in range(S):
                    j = int(idx[b, t, sg, s_i])
                    if j < 0:
                        continue
                    hi = min(BLOCK * j + BLOCK, t + 1)
                    bias[b, sg, t, BLOCK * j:hi] = logg[b, t, sg, s_i]
    return bias


def attn_fwd_dense(q, k, v, idx, logg, scale: float):
    """Dense-masked form: full T x T logits per head plus the block bias, row softmax."""
    q, k, v = as64(q), as64(k), as64(v)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    Gs, _ = sel_heads(Hq, Hkv, np.asarray(idx).shape[2])
    bias = dense_bias(idx, logg, T)
    o = np.zeros_like(q)
    lse = np.zeros((B, T, Hq))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            L = q[b, :, h] @ k[b, :, kv].T * scale + bias[b, h // Gs]
            m = L.max(axis=1, keepdims=True)
            P = np.exp(L - m)
            l = P.sum(axis=1, keepdims=True)
            o[b, :, h] = (P / l) @ v[b, :, kv]
            lse[b, :, h] = (m + np.log(l))[:, 0]
    return o, lse


def attn_bwd(q, k, v, dout, idx, logg, scale: float, tokens=None):
    """Backward of the gather form for all rows (small T), or for the query
    rows of the chosen tokens only (dk, dv then hold those rows' contributions).

    dP = dO.v;  Delta = dO.o;  dS = P (dP - Delta);
    dq = scale sum dS k;  dk += scale dS q;  dv += P dO;
    dlogg[slot] = sum over the selection head's query heads and the block's
    keys of dS (README (b): the gradient reaching the selector through log g).
    Returns dict(o, lse, dq, dk, dv, dlogg [B,T,Hs,S]).
    """
    q, k, v, dout, logg = as64(q), as64(k), as64(v), as64(dout), as64(logg)
    idx = np.asarray(idx)
    B, T, Hq, D = q.shape
    Hkv, Hs = k.shape[2], idx.shape[2]
    Gs, kv_of = sel_heads(Hq, Hkv, Hs)
    S = idx.shape[-1]
    o = np.zeros_like(q)
    lse = np.zeros((B, T, Hq))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlogg = np.zeros((B, T, Hs, S))
    tok = range(T) if tokens is None else [int(t) for t in tokens]
    for b in range(B):
        for t in tok:
            for sg in range(Hs):
                kv = kv_of(sg)
                taus, slots = _row_keys(t, idx[b, t, sg])
                Kr, Vr = k[b, taus, kv], v[b, taus, kv]
                bias = logg[b, t, sg, slots]
                hs = slice(sg * Gs, (sg + 1) * Gs)
                Q, dO = q[b, t, hs], dout[b, t, hs]
                L = Q @ Kr.T * scale + bias
                m = L.max(axis=1, keepdims=True)
                E = np.exp(L - m)
                l = E.sum(axis=1, keepdims=True)
                P = E / l
                O = P @ Vr
                o[b, t, hs] = O
                lse[b, t, hs] = (m + np.log(l))[:, 0]
                dP = dO @ Vr.T
                delta = (dO * O).sum(axis=1, keepdims=True)
                dS = P * (dP - delta)                       # [G, n]
                dq[b, t, hs] = scale * dS @ Kr
                np.add.at(dk[b, :, kv], taus, scale * dS.T @ Q)
                np.add.at(dv[b, :, kv], taus, P.T @ dO)
                np.add.at(dlogg[b, t, sg], slots, dS.sum(axis=0))
    pad = idx < 0
    dlogg[pad] = 0.0
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, dlogg=dlogg)


def attn_bwd_rows(q, k, v, dout, idx, logg, scale: float, tokens):
    """dq [B,n,Hq,D] and dlogg [B,n,Hs,S] for chosen query tokens (gather form)."""
    q, k, v, dout, logg = as64(q), as64(k), as64(v), as64(dout), as64(logg)
    idx = np.asarray(idx)
    B, T, Hq, D = q.shape
    Hkv, Hs = k.shape[2], idx.shape[2]
    Gs, kv_of = sel_heads(Hq, Hkv, Hs)
    S = idx.shape[-1]
    tok = np.asarray(tokens)
    dq = np.zeros((B, len(tok), Hq, D))
    dlogg = np.zeros((B, len(tok), Hs, S))
    for n, t in enumerate(tok):
        t = int(t)
        for b in range(B):
            for sg in range(Hs):
                kv = kv_of(sg)
                taus, slots = _row_keys(t, idx[b, t, sg])
                Kr, Vr = k[b, taus, kv], v[b, taus, kv]
                hs = slice(sg * Gs, (sg + 1) * Gs)
                Q, dO = q[b, t, hs], dout[b, t, hs]
                L = Q @ Kr.T * scale + logg[b, t, sg, slots]
                P = np.exp(L - L.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                O = P @ Vr
                dS = P * (dO @ Vr.T - (dO * O).sum(axis=1, keepdims=True))
                dq[b, n, hs] = scale * dS @ Kr
                np.add.at(dlogg[b, n, sg], slots, dS.sum(axis=0))
    return dq, dlogg


def attn_bwd_block(q, k, v, dout, idx, logg, scale: float, b: int, kv: int, j: int):
    """dk, dv [64, D] of KV block j of head kv (batch b): sums over every query
    row, of every selection head attending kv, that selected block j (its P
    needs that row's full softmax)."""
    q, k, v, dout, logg = as64(q), as64(k), as64(v), as64(dout), as64(logg)
    idx = np.asarray(idx)
    B, T, Hq, D = q.shape
    Hkv, Hs = k.shape[2], idx.shape[2]
    Gs, kv_of = sel_heads(Hq, Hkv, Hs)
    lo, hi = BLOCK * j, min(BLOCK * j + BLOCK, T)
    dk = np.zeros((hi - lo, D))
    dv = np.zeros((hi - lo, D))
    rows = [(sg, int(t)) for sg in range(Hs) if kv_of(sg) == kv
            for t in np.nonzero((idx[b, :, sg, :] == j).any(axis=1))[0]]
    for sg, t in rows:
        taus, slots = _row_keys(t, idx[b, t, sg])
        Kr, Vr = k[b, taus, kv], v[b, taus, kv]
        hs = slice(sg * Gs, (sg + 1) * Gs)
        Q, dO = q[b, t, hs], dout[b, t, hs]
        L = Q @ Kr.T * scale + logg[b, t, sg, slots]
        P = np.exp(L - L.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        O = P @ Vr
        dS = P * (dO @ Vr.T - (dO * O).sum(axis=1, keepdims=True))
        inb = (taus >= lo) & (taus < hi)
        tb = taus[inb] - lo
        np.add.at(dk, tb, scale * dS[:, inb].T @ Q)
        np.add.at(dv, tb, P[:, inb].T @ dO)
    return dk, dv


# --------------------------------------------------------------------------
# Whole-sequence evaluation of the same definitions, for full-size checks:
# the router and selection of every token, and the gather-form attention
# (forward and backward) of every query row of one KV head.  Each restates
# the per-row definitions above with the rows of a query block (router) or a
# batch of tokens (attention) stacked along a leading axis; nothing is
# reordered inside a row.  Pinned against route() and attn_bwd() on small
# shapes.
# --------------------------------------------------------------------------

def gate_key_all(k, wk, w_kn, theta: float, eps: float) -> np.ndarray:
    """gate_key() of every token at once: the causal prefix [max; min; mean]
    of each token's block [R3, R4], Kproj, RMSNorm, RoPE at 64c [R6].
    k [B,T,Hkv,D], wk [Hkv,3D,dg] -> [B,T,Hkv,dg]."""
    k = as64(k)
    B, T, Hkv, D = k.shape
    NB = -(-T // BLOCK)
    kp = np.zeros((B, NB * BLOCK, Hkv, D))
    kp[:, :T] = k
    kb = kp.reshape(B, NB, BLOCK, Hkv, D)
    n = np.arange(1, BLOCK + 1, dtype=np.float64)[None, None, :, None, None]
    pool = np.concatenate([np.maximum.accumulate(kb, axis=2), np.minimum.accumulate(kb, axis=2),
                           np.cumsum(kb, axis=2) / n], axis=-1)
    pool = pool.reshape(B, NB * BLOCK, Hkv, 3 * D)[:, :T]
    z = rms_norm(head_proj(pool, wk), as64(w_kn), eps)
    tok = np.arange(T)
    return rope(z, ((tok // BLOCK) * BLOCK)[None, :, None], theta)


def select_rows(s_hist: np.ndarray, K: int):
    """select_blocks() for many rows with the same c at once: s_hist [m, c]
    historical scores -> (sel [m, min(K, c)] ascending block ids, gap [m]
    K-th/(K+1)-th gap or +inf).  A stable sort on -s keeps equal scores in
    ascending block order, so ties go to the lower index [R11, R12]."""
    m, c = s_hist.shape
    n = min(K, c)
    order = np.argsort(-s_hist, axis=1, kind="stable")
    sel = np.sort(order[:, :n], axis=1)
    gap = np.full(m, np.inf)
    if K >= 1 and c > K:
        srt = np.take_along_axis(s_hist, order, axis=1)
        gap = srt[:, K - 1] - srt[:, K]
    return sel, gap


def route_all(q, k, wq, wk, w_qn, w_kn, K: int, theta: float, eps: float):
    """route() for every token: gate vectors, candidate softmax and Top-K.

    Selection heads Hs = wq.shape[0] (Hkv: one gate per KV head [R1]); head
    sg scores the gate keys of KV head sg * (Hq / Hs) // G.  Historical blocks
    are ranked by a stable sort on -s, which keeps equal scores in ascending
    block order (ties -> lower index [R12]).
    Returns qg [B,T,Hs,dg], kg [B,T,Hkv,dg], idx, logg [B,T,Hs,K+1],
    lse, gap [B,T,Hs] (K-th/(K+1)-th gap, +inf when nothing is left out),
    near_tie [B,T,Hs].
    """
    q, k = as64(q), as64(k)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    Hs = as64(wq).shape[0]
    _, kv_of = sel_heads(Hq, Hkv, Hs)
    S = K + 1
    qg = gate_query(q, wq, w_qn, theta, eps)
    kg = gate_key_all(k, wk, w_kn, theta, eps)
    kblk = kg[:, block_key_tokens(T)]                       # [B,NB,Hkv,dg]
    rdg = math.sqrt(qg.shape[-1])
    idx = np.full((B, T, Hs, S), -1, dtype=np.int64)
    logg = np.full((B, T, Hs, S), -np.inf)
    lse = np.zeros((B, T, Hs))
    gap = np.full((B, T, Hs), np.inf)
    NB = -(-T // BLOCK)
    for c in range(NB):
        t0, t1 = BLOCK * c, min(BLOCK * c + BLOCK, T)
        n = min(K, c)
        for b in range(B):
            for sg in range(Hs):
                kv = kv_of(sg)
                Q = qg[b, t0:t1, sg]                                   # [m, dg]
                s = np.concatenate([Q @ kblk[b, :c, kv].T,
                                    (Q * kg[b, t0:t1, kv]).sum(-1, keepdims=True)], axis=1) / rdg
                m = s.max(axis=1, keepdims=True)
                l = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
                sel, gp = select_rows(s[:, :c], K)
                idx[b, t0:t1, sg, :n] = sel
                idx[b, t0:t1, sg, n] = c
                logg[b, t0:t1, sg, :n] = np.take_along_axis(s, sel, axis=1) - l[:, None]
                logg[b, t0:t1, sg, n] = s[:, c] - l
                lse[b, t0:t1, sg] = l
                gap[b, t0:t1, sg] = gp
    return dict(qg=qg, kg=kg, idx=idx, logg=logg, lse=lse, gap=gap,
                near_tie=gap < NEAR_TIE_GAP)


def attn_head(q, k, v, idx, logg, scale: float, b: int, sg: int, dout=None, batch: int = 32):
    """Gather-form attention of every query row of selection head sg (batch b).

    Selection heads Hs = idx.shape[2]; sg covers query heads sg*Gs ..
    (sg+1)*Gs - 1 (Gs = Hq/Hs) and KV head sg*Gs // G.  Per token t: the keys
    of its selected blocks with tau <= t [R13], l = q.k * scale + logg[slot]
    [R10], P = softmax(l), o = P V, lse = logsumexp(l); with dout, the
    backward of attn_bwd(): Delta = dO.o, dS = P (dO.v - Delta),
    dq = scale dS K, dlogg[slot] = sum over the heads and the block's keys of
    dS.  dk, dv of the KV head are the sums over every row that selected a
    key's block (rows of this selection head only; with one gate per KV head
    that is all of them): per key block j, the rows that chose j, with P taken
    from each row's lse.
    Returns dict with o [T,Gs,D], lse [T,Gs] and, with dout, dq [T,Gs,D],
    dlogg [T,S], dk, dv [T,D].
    """
    import torch

    f64 = torch.float64
    q, k, v = (torch.as_tensor(as64(x)) for x in (q, k, v))
    lg_all = torch.as_tensor(as64(logg))
    idx = torch.as_tensor(np.asarray(idx)).long()
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    Hs, S = idx.shape[2], idx.shape[3]
    G, Gs = Hq // Hkv, Hq // Hs
    kv = sg * Gs // G
    hs = slice(sg * Gs, (sg + 1) * Gs)
    NB = -(-T // BLOCK)
    Kb = torch.zeros((NB * BLOCK, D), dtype=f64)
    Vb = torch.zeros((NB * BLOCK, D), dtype=f64)
    Kb[:T], Vb[:T] = k[b, :, kv], v[b, :, kv]
    Kb, Vb = Kb.view(NB, BLOCK, D), Vb.view(NB, BLOCK, D)
    Qh = q[b, :, hs]                                           # [T,Gs,D]
    lg = lg_all[b, :, sg]                                      # [T,S]
    sel_all = idx[b, :, sg]
    tok = torch.arange(T)
    valid_all = (sel_all >= 0) & (sel_all <= (tok // BLOCK)[:, None])
    o = torch.zeros((T, Gs, D), dtype=f64)
    lse = torch.zeros((T, Gs), dtype=f64)
    if dout is not None:
        dO_all = torch.as_tensor(as64(dout))[b, :, hs]
        dq = torch.zeros((T, Gs, D), dtype=f64)
        dlogg = torch.zeros((T, S), dtype=f64)
        delta = torch.zeros((T, Gs), dtype=f64)
    ar = torch.arange(BLOCK)
    # rows: per batch of tokens, the selected blocks gathered and concatenated
    for t0 in range(0, T, batch):
        ts = tok[t0:min(T, t0 + batch)]
        n = len(ts)
        valid = valid_all[ts]
        j = torch.where(valid, sel_all[ts], torch.zeros_like(sel_all[ts]))
        Kg = Kb[j].view(n, S * BLOCK, D)
        Vg = Vb[j].view(n, S * BLOCK, D)
        tau = (j[..., None] * BLOCK + ar).view(n, S * BLOCK)
        mask = (valid[..., None] & (tau.view(n, S, BLOCK) <= ts[:, None, None])).view(n, 1, S * BLOCK)
        bias = lg[ts].repeat_interleave(BLOCK, dim=1)[:, None, :]     # [n,1,S*64]
        Q = Qh[ts]
        L = torch.bmm(Q, Kg.transpose(1, 2)) * scale + bias
        L = torch.where(mask, L, torch.full_like(L, -math.inf))
        m = L.amax(dim=2, keepdim=True)
        E = torch.exp(L - m)
        lsum = E.sum(dim=2, keepdim=True)
        P = E / lsum
        O = torch.bmm(P, Vg)
        o[ts] = O
        lse[ts] = (m + torch.log(lsum))[..., 0]
        if dout is None:
            continue
        dO = dO_all[ts]
        dP = torch.bmm(dO, Vg.transpose(1, 2))
        dlt = (dO * O).sum(-1)
        dS = P * (dP - dlt[..., None])
        dq[ts] = scale * torch.bmm(dS, Kg)
        per_slot = dS.sum(dim=1).view(n, S, BLOCK).sum(-1)
        dlogg[ts] = torch.where(valid, per_slot, torch.zeros_like(per_slot))
        delta[ts] = dlt
    out = dict(o=o.numpy(), lse=lse.numpy())
    if dout is None:
        return out
    # keys: per block j, the rows (token, head) whose selection holds j
    dkb = torch.zeros((NB, BLOCK, D), dtype=f64)
    dvb = torch.zeros((NB, BLOCK, D), dtype=f64)
    tt, ss = torch.nonzero(valid_all, as_tuple=True)
    jj = sel_all[tt, ss]
    order = torch.argsort(jj, stable=True)
    tt, ss, jj = tt[order], ss[order], jj[order]
    bounds = torch.searchsorted(jj, torch.arange(NB + 1))
    for jb in range(NB):
        lo, hi = int(bounds[jb]), int(bounds[jb + 1])
        if lo == hi:
            continue
        rt, rs = tt[lo:hi], ss[lo:hi]
        QR = Qh[rt].reshape(-1, D)                                 # [m*Gs, D]
        dOR = dO_all[rt].reshape(-1, D)
        trow = rt.repeat_interleave(Gs)
        bias = lg[rt, rs].repeat_interleave(Gs)
        Sm = QR @ Kb[jb].T * scale + bias[:, None]
        keep = (jb * BLOCK + ar)[None, :] <= trow[:, None]
        P = torch.where(keep, torch.exp(Sm - lse[rt].reshape(-1)[:, None]), torch.zeros_like(Sm))
        dvb[jb] = P.T @ dOR
        dS = P * (dOR @ Vb[jb].T - delta[rt].reshape(-1)[:, None])
        dkb[jb] = scale * dS.T @ QR
    out.update(dq=dq.numpy(), dlogg=dlogg.numpy(),
               dk=dkb.view(NB * BLOCK, D)[:T].numpy(), dv=dvb.view(NB * BLOCK, D)[:T].numpy())
    return out


def gate_logit_grad(dlogg, idx, probs) -> np.ndarray:
    """Gradient reaching the gate logits s through log g = s - lse(s) [R18]:
    ds_j = dlogg_j [j selected] - g_j * sum over selected i of dlogg_i, for j <= c.

    dlogg, idx [..., S]; probs [..., NB] (0 beyond c) -> ds [..., NB].
    """
    dlogg = as64(dlogg)
    idx = np.asarray(idx)
    probs = as64(probs)
    valid = idx >= 0
    dl = np.where(valid, dlogg, 0.0)
    tot = dl.sum(axis=-1)
    ds = np.zeros(probs.shape)
    lead = np.indices(idx.shape[:-1])                         # row coordinates
    pos = tuple(np.broadcast_to(c[..., None], idx.shape) for c in lead)
    np.add.at(ds, pos + (np.where(valid, idx, 0),), dl)      # pads add 0 at block 0
    ds -= probs * tot[..., None]
    return ds


# --------------------------------------------------------------------------
# Router backward: the gradient that reaches the selector through log g
# (README intro (b): the gates give the LM loss a path to the selector; model
# card "Checkpoint configuration" table for the router's layers).  Chain rule
# through the gate logits, the gate RoPE, the Q/K RMSNorm, the projections and
# the max + min + average pooling, with the selection held fixed.
# --------------------------------------------------------------------------

def _rms_norm_bwd(y: np.ndarray, w: np.ndarray, eps: float, dn: np.ndarray):
    """n = y * r * w with r = (mean(y^2) + eps)^(-1/2) over the last axis [R5].

    Returns (dy, per-element contribution to dw) for upstream gradient dn:
    dn/dy_k = r u_k - r^3 y_k mean(u * y), u = dn * w;  dn/dw = dn * y * r.
    """
    r = 1.0 / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps)
    u = dn * w
    dy = r * u - r ** 3 * y * np.mean(u * y, axis=-1, keepdims=True)
    return dy, dn * y * r


def _pool_with_args(k: np.ndarray):
    """Causal prefix [max; min; mean] of every token's block [R3, R4], plus the
    row that holds each channel's max and min (the first such row on ties)
    and the number of pooled rows [R21].

    k [B,T,Hkv,D] -> p [B,T,Hkv,3D], amax, amin [B,T,Hkv,D] (token ids), n [T].
    Walks the 64 positions of every block at once.
    """
    B, T, H, D = k.shape
    NB = -(-T // BLOCK)
    kp = np.zeros((B, NB * BLOCK, H, D))
    kp[:, :T] = k
    kb = kp.reshape(B, NB, BLOCK, H, D)
    pool = np.empty((B, NB, BLOCK, H, 3 * D))
    amax = np.empty((B, NB, BLOCK, H, D), dtype=np.int64)
    amin = np.empty((B, NB, BLOCK, H, D), dtype=np.int64)
    for r in range(BLOCK):
        v = kb[:, :, r]
        if r == 0:
            mx, mn, sm = v.copy(), v.copy(), v.copy()
            ax = np.zeros(v.shape, dtype=np.int64)
            an = np.zeros(v.shape, dtype=np.int64)
        else:
            up, dn = v > mx, v < mn                           # strict: ties keep the first row
            mx, ax = np.where(up, v, mx), np.where(up, r, ax)
            mn, an = np.where(dn, v, mn), np.where(dn, r, an)
            sm = sm + v
        pool[:, :, r] = np.concatenate([mx, mn, sm / (r + 1)], axis=-1)
        amax[:, :, r], amin[:, :, r] = ax, an
    base = (np.arange(NB) * BLOCK)[None, :, None, None, None]
    tok = np.arange(T)
    n = tok - (tok // BLOCK) * BLOCK + 1
    return (pool.reshape(B, NB * BLOCK, H, 3 * D)[:, :T],
            (amax + base).reshape(B, NB * BLOCK, H, D)[:, :T],
            (amin + base).reshape(B, NB * BLOCK, H, D)[:, :T], n)


def router_bwd(q, k, wq, wk, w_qn, w_kn, idx, dlogg, theta: float, eps: float, heads=None,
               lse_term: bool = True):
    """Gradient of L = sum over (b, t, kappa, valid slot) of dlogg * log g with
    the selection idx held fixed, with respect to the router's inputs and
    weights [R1-R9, R18, R21].

    q [B,T,Hq,D], k [B,T,Hkv,D], wq [Hkv,G*D,dg], wk [Hkv,3D,dg], w_qn, w_kn
    [dg]; idx, dlogg [B,T,Hkv,S].  heads: the KV heads to take (default all);
    the outputs then cover those heads only (dq: their query heads), and
    dw_qn, dw_kn their share of the sums.  Returns dq, dk, dwq, dwk, dw_qn,
    dw_kn, and the intermediate gradients dqg, dkg with respect to the gate
    query and the per-token gate key [B,T,H,dg], and ds [B,T,H,NB] with
    respect to the gate logits.  lse_term=False differentiates
    L = sum dlogg * s over the selected logits instead (the row's lse held
    constant): ds = dlogg on the selected blocks, 0 elsewhere, which equals the
    full gradient whenever each row's dlogg sums to zero [R18].
    """
    q, k, wq, wk = as64(q), as64(k), as64(wq), as64(wk)
    w_qn, w_kn = as64(w_qn), as64(w_kn)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if as64(wq).shape[0] != Hkv:
        raise ValueError("router_bwd covers one gate per KV head")
    heads = np.arange(Hkv) if heads is None else np.asarray(heads)
    H = len(heads)
    idx = np.asarray(idx)[:, :, heads]
    dlogg = np.where(idx >= 0, as64(dlogg)[:, :, heads], 0.0)
    wq, wk = wq[heads], wk[heads]
    dg = wq.shape[2]
    NB = -(-T // BLOCK)
    tok = np.arange(T)
    cblk = tok // BLOCK
    kt = block_key_tokens(T)
    sq = math.sqrt(dg)
    # forward values the chain rule needs
    x = q.reshape(B, T, Hkv, G * D)[:, :, heads]
    y = np.einsum("btkf,kfg->btkg", x, wq)
    qg = rope(rms_norm(y, w_qn, eps), tok[None, :, None], theta)
    p, amax, amin, npool = _pool_with_args(k[:, :, heads])
    z = np.einsum("btkf,kfg->btkg", p, wk)
    kg = rope(rms_norm(z, w_kn, eps), (cblk * BLOCK)[None, :, None], theta)
    kblk = kg[:, kt]                                          # [B, NB, H, dg]
    # gate logits over the candidates 0..c of every row, probabilities, ds
    hist = (np.arange(NB)[None, :] < cblk[:, None])[None, :, None, :]   # [1, T, 1, NB]
    ccol = np.broadcast_to(cblk[None, :, None, None], (B, T, H, 1))
    s = np.where(hist, np.einsum("btkg,bjkg->btkj", qg, kblk) / sq, -np.inf)
    np.put_along_axis(s, ccol, (np.einsum("btkg,btkg->btk", qg, kg) / sq)[..., None], axis=-1)
    probs = np.exp(s - s.max(axis=-1, keepdims=True))
    probs /= probs.sum(axis=-1, keepdims=True)
    ds = gate_logit_grad(dlogg, idx, probs if lse_term else np.zeros_like(probs))
    ds_hist = np.where(hist, ds, 0.0)
    ds_cur = np.take_along_axis(ds, ccol, axis=-1)[..., 0]
    # s -> gate query and gate keys
    dqg = (np.einsum("btkj,bjkg->btkg", ds_hist, kblk) + ds_cur[..., None] * kg) / sq
    dkg = ds_cur[..., None] * qg / sq
    dkg[:, kt] += np.einsum("btkj,btkg->bjkg", ds_hist, qg) / sq
    # RoPE is a rotation: its transpose rotates by the opposite angle
    dy, dwq_n = _rms_norm_bwd(y, w_qn, eps, rope(dqg, -tok[None, :, None], theta))
    dz, dwk_n = _rms_norm_bwd(z, w_kn, eps, rope(dkg, -(cblk * BLOCK)[None, :, None], theta))
    dwq = np.einsum("btkf,btkg->kfg", x, dy)
    dwk = np.einsum("btkf,btkg->kfg", p, dz)
    dq = np.einsum("btkg,kfg->btkf", dy, wq).reshape(B, T, H * G, D)
    dp = np.einsum("btkg,kfg->btkf", dz, wk)                 # [B,T,H,3D]
    # pooling: max / min pass the gradient to their row, mean to every row of
    # the prefix (a suffix sum over each block)
    dk = np.zeros((B, T, H, D))
    ib = np.broadcast_to(np.arange(B)[:, None, None, None], amax.shape)
    ih = np.broadcast_to(np.arange(H)[None, None, :, None], amax.shape)
    idd = np.broadcast_to(np.arange(D)[None, None, None, :], amax.shape)
    np.add.at(dk, (ib, amax, ih, idd), dp[..., :D])
    np.add.at(dk, (ib, amin, ih, idd), dp[..., D:2 * D])
    mean_g = np.zeros((B, NB * BLOCK, H, D))
    mean_g[:, :T] = dp[..., 2 * D:] / npool[None, :, None, None]
    mb = mean_g.reshape(B, NB, BLOCK, H, D)
    suffix = np.flip(np.cumsum(np.flip(mb, axis=2), axis=2), axis=2)
    dk += suffix.reshape(B, NB * BLOCK, H, D)[:, :T]
    return dict(dq=dq, dk=dk, dwq=dwq, dwk=dwk, dw_qn=dwq_n.sum(axis=(0, 1, 2)),
                dw_kn=dwk_n.sum(axis=(0, 1, 2)), dqg=dqg, dkg=dkg, ds=ds)


# --------------------------------------------------------------------------
# Budgeted single-token decode (model card: sparse decode budget 1,024 /
# 2,048 / 4,096 tokens; usage guide pitfall 3: the budget bounds attended
# tokens per query, not the cache).
# --------------------------------------------------------------------------

def decode(q, q_gate, k_cache, v_cache, kg_cache, ctx_len, K: int, scale: float,
           apply_gate: bool = True, units=None):
    """One decode step per sequence.

    q [B,Hq,D]; q_gate [B,Hs,dg] (Hs selection heads, see sel_heads);
    k_cache, v_cache [B,Hkv,Lmax,D]; kg_cache [B,Hkv,NBmax,dg] (entry c =
    current block's prefix-pooled key); ctx_len [B] counts the new token (at
    position L-1).
    Returns o [B,Hq,D], idx, logg [B,Hs,K+1], near_tie, gap [B,Hs] for the
    chosen (b, selection head) units (others left zero / -1).
    apply_gate=False is the selection-only variant [R16].
    """
    q, q_gate = as64(q), as64(q_gate)
    ctx = np.asarray(ctx_len.cpu() if hasattr(ctx_len, "cpu") else ctx_len)
    B, Hq, D = q.shape
    Hs = q_gate.shape[1]
    Hkv = k_cache.shape[1]
    Gs, kv_of = sel_heads(Hq, Hkv, Hs)
    S = K + 1
    o = np.zeros((B, Hq, D))
    idx = np.full((B, Hs, S), -1, dtype=np.int64)
    logg = np.full((B, Hs, S), -np.inf)
    near = np.zeros((B, Hs), dtype=bool)
    gap = np.full((B, Hs), np.inf)
    if units is None:
        units = [(b, sg) for b in range(B) for sg in range(Hs)]
    for b, sg in units:
        kv = kv_of(sg)
        L = int(ctx[b])
        t = L - 1
        c = t // BLOCK
        kg = as64(kg_cache[b, kv, :c + 1])
        s = gate_logits(q_gate[b, sg], kg[:c], kg[c])
        _, lg = log_gates(s)
        sel, nt = select_blocks(s, K)
        idx[b, sg, :len(sel)] = sel
        logg[b, sg, :len(sel)] = lg[sel]
        near[b, sg] = nt
        gap[b, sg] = kth_gap(s, K)
        taus, slots = _row_keys(t, np.array(sel))
        Kr = as64(k_cache[b, kv, taus])
        Vr = as64(v_cache[b, kv, taus])
        bias = lg[np.array(sel)][slots] if apply_gate else np.zeros(len(taus))
        hs = slice(sg * Gs, (sg + 1) * Gs)
        Q = q[b, hs]
        Lg = Q @ Kr.T * scale + bias
        P = np.exp(Lg - Lg.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        o[b, hs] = P @ Vr
    return dict(o=o, idx=idx, logg=logg, near_tie=near, gap=gap)


# --------------------------------------------------------------------------
# Router size (model card, "Released checkpoints" table).
# --------------------------------------------------------------------------

def router_param_count(Hq: int, Hkv: int, D: int, dg: int, layers: int,
                       norm_weights: bool = True, per_query_head: bool = False) -> int:
    """Per layer: Qproj Hkv x (G*D) x dg (one gate per KV head) or Hq x D x dg
    (one gate per query head), Kproj Hkv x 3D x dg over [max;min;mean], plus
    the two dg-wide RMSNorm weights."""
    G = Hq // Hkv
    qproj = Hq * D * dg if per_query_head else Hkv * G * D * dg
    per = qproj + Hkv * 3 * D * dg + (2 * dg if norm_weights else 0)
    return per * layers


def brute_force_topk(s_hist, K: int):
    """Tiny-input reference: the K-subset of historical blocks with the largest
    score sum; among equal sums the lexicographically smallest ascending subset."""
    c = len(s_hist)
    n = min(K, c)
    best, best_key = None, None
    for comb in itertools.combinations(range(c), n):
        key = (-sum(s_hist[j] for j in comb), comb)
        if best_key is None or key < best_key:
            best, best_key = comb, key
    return list(best)
