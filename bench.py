"""Benchmark of the SAS gated block-sparse attention hot path on one MI355X.

One step = one training-layer pass of the whole prefill path on the 32K
workload (Qwen3-4B attention shape: B=1, T=32768, 32 query / 8 KV heads,
head dim 128, gate hidden 128, KV block 64, Top-31 + current block):
gate router -> candidate softmax + Top-K -> sparse attention forward ->
sparse attention backward (dQ, dK, dV, d log g).  The budgeted decode
(64 sequences, Qwen3-8B shape, contexts U[8192, 65536], budget 2048) is
timed in the same run and reported in the "decode" object, and the router
backward (gradients of the gate router from the step's d log g) in the
"router_bwd" object; neither is part of the step time.

value = effective fwd+bwd attention FLOPs / whole-step time, where the
effective FLOPs count 4*D (forward) + 10*D (backward) per attended
(query head, key) pair; router and selection time is inside the step time.

Prints ONE JSON line.  Inputs are synthetic, seeded, resident in HBM before
the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 (vector and MFMA)


def attended_pairs(T: int, K: int, block: int = 64) -> int:
    """Sum over query tokens t of attended keys n_t = 64 min(K, c) + (t mod 64) + 1."""
    tot = 0
    for t in range(T):
        c = t // block
        tot += block * min(K, c) + (t - block * c) + 1
    return tot


def decode_bytes(ctx_len, Hkv, D, dg, K, G, block=64):
    """Algorithmic bytes of one decode step: selected K/V blocks (only keys < L),
    the c+1 gate keys per (sequence, KV head), q, q_gate and o."""
    kv = 0
    gk = 0
    for L in ctx_len:
        c = (L - 1) // block
        n_cur = L - block * c
        kv += (block * min(K, c) + n_cur) * D * 2 * 2 * Hkv
        gk += (c + 1) * dg * 4 * Hkv
    B = len(ctx_len)
    small = B * Hkv * (G * D * 2 * 2 + dg * 4)
    return kv, gk, small


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str, src_hash: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
    (profiles/traffic.json), only if taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(kernel_key)
        if e and e.get("source_hash") == src_hash:
            return e.get("bytes_per_launch")
    except Exception:
        return None
    return None


COPY_BYTES = 1 << 30          # the calibration copy (--copy-calib)
# sources each kernel's behaviour depends on (besides the shared headers): a
# profile taken on other sources is stale and not reported.  The forward and
# dQ walks also depend on the staging order walk_order.h makes for them.
KERNEL_SOURCES = {"sparse_fwd_kernel": ("attn_fwd.hip", "walk_order.hip", "walk_order.h"),
                  "dkdv_kernel": ("attn_bwd.hip",),
                  "dq_kernel": ("attn_bwd.hip", "walk_order.h"),
                  "walk_order_kernel": ("walk_order.hip", "walk_order.h"),
                  "bwd_prep_kernel": ("attn_bwd.hip", "walk_order.h"),
                  "topk_kernel": ("topk.hip",),
                  "gate_query_kernel": ("router.hip",), "gate_key_kernel": ("router.hip",),
                  "decode_attn_kernel": ("decode.hip",),
                  # fp32 gate keys (the bench also runs the bf16-key variant)
                  "decode_score_kernel<128, false>": ("decode.hip",),
                  "decode_topk_kernel": ("decode.hip",), "decode_merge_kernel": ("decode.hip",),
                  "sas_decode": ("decode.hip",)}
for _k in ("gbwd_key_kernel", "gbwd_query_kernel", "gbwd_blockkey_kernel", "gbwd_wsum_kernel",
           "gbwd_rows_kernel", "gbwd_reduce_kernel", "gbwd_colsum_kernel",
           "gbwd_blockkey_sum_kernel", "sas_gate_score_bwd"):
    KERNEL_SOURCES[_k] = ("router_bwd.hip",)
SHARED_HEADERS = ("sas_device.h", "sas_kernels.h", "bwd_index.h")
# kernels whose HBM traffic the counter summary records
TRAFFIC_KERNELS = tuple(k for k in KERNEL_SOURCES if not k.startswith("sas_")
                        and k not in ("gate_query_kernel", "gate_key_kernel"))


def kernel_hash(key: str) -> str:
    csrc = os.path.join(ROOT, "gated_block_sparse_gate_amd", "csrc")
    return source_hash([os.path.join(csrc, f) for f in KERNEL_SOURCES[key] + SHARED_HEADERS])


def summarize_pmc(fetch_dir: str, write_dir: str, out_json: str):
    """HBM traffic per launch from two rocprofv3 --pmc runs of this script with
    --copy-calib (one with FETCH_SIZE, one with WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by what it reads for the 1 GiB device-to-device
    copy (rocclr copyBuffer) of the same run, so bytes = counter * 1 GiB /
    counter(copy).  Writes profiles/traffic.json keyed by kernel, with the
    hash of the kernel's source so stale entries are ignored."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    res, lines = {}, []
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        copies = [v for k, l in vals.items() if "copyBuffer" in k for v in l
                  if v * 1024 >= COPY_BYTES // 2]
        if not copies:
            raise SystemExit(f"no calibration copy found in {d}")
        ref = sum(copies) / len(copies)
        factor = COPY_BYTES / ref
        lines.append(f"{counter}: calibration copy of {COPY_BYTES} B reads {ref:.0f} KiB "
                     f"per dispatch -> factor {factor:.4f} B per KiB")
        for key in TRAFFIC_KERNELS:
            # the key as a whole name ("::topk_kernel" is not inside
            # "::decode_topk_kernel")
            l = [v for k, ll in vals.items() if k.startswith(key) or ("::" + key) in k
                 for v in ll]
            if not l:
                continue
            avg = sum(l) / len(l)
            e = res.setdefault(key, {})
            e[counter.lower() + "_kib_per_dispatch"] = round(avg, 1)
            e[counter.lower() + "_bytes"] = round(avg * factor)
            e["dispatches"] = len(l)
    for key, e in res.items():
        e["bytes_per_launch"] = e.get("fetch_size_bytes", 0) + e.get("write_size_bytes", 0)
        e["source_hash"] = kernel_hash(key)
        lines.append(f"{key}: fetch {e.get('fetch_size_bytes', 0) / 1e9:.3f} GB + write "
                     f"{e.get('write_size_bytes', 0) / 1e9:.3f} GB per launch "
                     f"({e['dispatches']} dispatches)")
    # one router-backward call: its kernels' bytes per dispatch times their
    # dispatches, per call (gbwd_key_kernel runs once per call)
    gb = [k for k in res if k.startswith("gbwd_")]
    if "gbwd_key_kernel" in res:
        calls = res["gbwd_key_kernel"]["dispatches"]
        res["sas_gate_score_bwd"] = {
            "bytes_per_launch": round(sum(res[k]["bytes_per_launch"] * res[k]["dispatches"]
                                          for k in gb) / calls),
            "kernels": sorted(gb),
            "source_hash": kernel_hash("sas_gate_score_bwd")}
        lines.append(f"sas_gate_score_bwd: {res['sas_gate_score_bwd']['bytes_per_launch'] / 1e9:.3f}"
                     f" GB per call ({' + '.join(sorted(gb))})")
    # the decode step as a whole: each of its kernels runs once per step
    dec = [k for k in res if k.startswith("decode_")]
    if dec:
        res["sas_decode"] = {
            "bytes_per_launch": sum(res[k]["bytes_per_launch"] for k in dec),
            "kernels": sorted(dec),
            "source_hash": kernel_hash("sas_decode")}
        lines.append(f"sas_decode: {res['sas_decode']['bytes_per_launch'] / 1e9:.3f} GB per step "
                     f"({' + '.join(sorted(dec))})")
    json.dump(res, open(out_json, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def selection_stats(idx: torch.Tensor, block: int = 64) -> dict:
    """Locality statistics of a selection idx [B,T,H,S] (pads -1; the last
    valid slot is the current block): mean overlap of the historical blocks
    of adjacent tokens (|A & B| / |A|, tokens of the same block), mean size of
    the union of historical blocks over groups of 16 consecutive tokens, and
    the share of all historical selections that go to the top 5 % of blocks
    (per head).  Counting only; no scores are involved."""
    import torch
    idx = idx.to("cpu").long()
    B, T, H, S = idx.shape
    NB = -(-T // block)
    c = (torch.arange(T) // block).view(1, T, 1, 1)
    hist = (idx >= 0) & (idx < c)
    onehot = torch.zeros((B, T, H, NB + 1), dtype=torch.bool)
    onehot.scatter_(-1, torch.where(hist, idx, torch.full_like(idx, NB)), True)
    onehot = onehot[..., :NB]
    a, b_ = onehot[:, :-1], onehot[:, 1:]
    same = (torch.arange(T - 1) // block == torch.arange(1, T) // block).view(1, T - 1, 1)
    na = a.sum(-1).float()
    keep = same & (na > 0)
    overlap = ((a & b_).sum(-1).float() / na.clamp(min=1))[keep].mean().item()
    G16 = T // 16
    union = onehot[:, :G16 * 16].view(B, G16, 16, H, NB).any(2).sum(-1).float().mean().item()
    cnt = onehot.sum(1).float()                                   # [B,H,NB]
    top = max(1, NB // 20)
    share = (cnt.sort(-1, descending=True).values[..., :top].sum(-1) /
             cnt.sum(-1).clamp(min=1)).mean().item()
    return dict(adjacent_overlap=round(overlap, 4), union16=round(union, 2),
                top5pct_share=round(share, 4))


def assert_sound(sas, what: str, **tensors):
    """Exit non-zero (printing no metric) if an attention kernel abandoned a
    ring wait since the last check or any given output holds NaN / Inf."""
    import torch
    fault = sas.take_device_fault()
    bad = [n for n, t in tensors.items() if not bool(torch.isfinite(t.float()).all())]
    if fault or bad:
        print(f"bench.py: {what}: device fault flag {fault}, non-finite outputs {bad}; "
              "no result reported", file=sys.stderr, flush=True)
        sys.exit(3)


def time_layer(sas, w, K: int, seed: int, steps: int, warmup: int, backward: bool = True,
               stats: bool = False) -> dict:
    """One prefill / training layer of workload w at Top-K K, inputs resident
    in HBM: gate router -> Top-K -> sparse attention forward (with the fp32
    output when the backward follows) -> backward.  Returns ms per step,
    per-stage ms, effective TFLOP/s (4 D forward + 10 D backward per attended
    pair) and, with stats, the locality of the router's selection."""
    import torch
    import synth

    dev = torch.device("cuda:0")
    x = synth.prefill_inputs(w, seed=seed, device=dev, with_dout=backward)
    B, T, Hq, Hkv, D, dg = w.B, w.T, w.Hq, w.Hkv, w.D, w.dg
    Hs, S = w.Hs, K + 1
    pq = w.gate == "q"
    flags = sas.FLAG_GATE_PER_QUERY_HEAD if pq else 0
    d = sas.make_dims(B, T, Hq, Hkv, D, dg, K, w.theta, w.eps, flags=flags)
    ws_gate = torch.empty(sas.workspace_size(sas.OP_GATE_SCORE, d), dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(sas.workspace_size(sas.OP_FWD, d), dtype=torch.uint8, device=dev)
    ws_bwd = (torch.empty(sas.workspace_size(sas.OP_BWD, d), dtype=torch.uint8, device=dev)
              if backward else None)
    f32 = dict(dtype=torch.float32, device=dev)
    qg = torch.empty((B, T, Hs, dg), **f32)
    kg = torch.empty((B, T, Hkv, dg), **f32)
    idx = torch.empty((B, T, Hs, S), dtype=torch.int32, device=dev)
    logg = torch.empty((B, T, Hs, S), **f32)
    glse = torch.empty((B, T, Hs), **f32)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, T, Hq), **f32)
    o32 = torch.empty((B, T, Hq, D), **f32) if backward else None
    if backward:
        dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
        dlogg = torch.empty_like(logg)
    sc = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        sas.gate_score(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, w.theta, w.eps,
                       q_gate=qg, k_gate=kg, workspace=ws_gate, per_query_head=pq)
        if ev:
            ev[1].record(stream)
        sas.topk_blocks(qg, kg, K, Hq, D, out=(idx, logg, glse))
        if ev:
            ev[2].record(stream)
        sas.sparse_attn_fwd(x["q"], x["k"], x["v"], idx, logg, sc, o=o, lse=lse, o_f32=o32,
                            workspace=ws_fwd)
        if ev:
            ev[3].record(stream)
        if backward:
            sas.sparse_attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, sc,
                                workspace=ws_bwd, out=(dq, dk, dv, dlogg), o_f32=o32)
        if ev:
            ev[4].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    outs = dict(o=o, lse=lse)
    if backward:
        outs.update(o_f32=o32, dq=dq, dk=dk, dv=dv, dlogg=dlogg)
    assert_sound(sas, f"{w.name} K={K}", **outs)
    ms = t0.elapsed_time(t1) / steps
    st = [sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps for i in range(4)]
    pairs = attended_pairs(T, K) * Hq * B
    fl_f, fl_b = 4.0 * D * pairs, (10.0 * D * pairs if backward else 0.0)
    res = {"workload": w.name, "gate": "per_query_head" if pq else "per_kv_head", "topk": K,
           "budget": 64 * (K + 1), "Hq": Hq, "Hkv": Hkv, "T": T,
           "ms_per_step": round(ms, 4),
           "stages_ms": {"gate_score": round(st[0], 4), "topk": round(st[1], 4),
                         "fwd": round(st[2], 4), "bwd": round(st[3], 4)},
           "tflops": round((fl_f + fl_b) / (ms * 1e-3) / 1e12, 2),
           "fwd_tflops": round(fl_f / (st[2] * 1e-3) / 1e12, 2),
           "frac_of_peak": round((fl_f + fl_b) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    if backward:
        res["bwd_tflops"] = round(fl_b / (st[3] * 1e-3) / 1e12, 2)
    if stats:
        res["selection"] = selection_stats(idx)
    return res


def time_decode_budget(sas, wd, K: int, seed: int, steps: int) -> dict:
    """Cold decode step (a 1 GiB read between steps evicts the cache) at
    Top-K K (budget 64 (K + 1)) on the batched decode workload."""
    import torch
    import synth

    dev = torch.device("cuda:0")
    xd = synth.decode_inputs(wd, seed=seed, device=dev)
    od = torch.empty((wd.B, wd.Hq, wd.D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(sas.decode_workspace_size(sas.DecodeDims(
        wd.B, wd.Hq, wd.Hkv, wd.D, wd.dg, 64, K, xd["Lmax"], xd["NBmax"], 1)),
        dtype=torch.uint8, device=dev)
    sc = 1.0 / math.sqrt(wd.D)

    def dstep():
        sas.decode(xd["q"], xd["q_gate"], xd["k_cache"], xd["v_cache"], xd["kg_cache"],
                   xd["ctx_len"], K, sc, want_idx=False, workspace=ws, out=(od, None, None))

    for _ in range(3):
        dstep()
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    cold = []
    for _ in range(steps):
        flush.sum()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        dstep()
        a1.record(stream)
        torch.cuda.synchronize()
        cold.append(a0.elapsed_time(a1) * 1e3)
    assert_sound(sas, f"decode K={K}", o=od)
    cold.sort()
    us = cold[len(cold) // 2]
    kvb, gkb, smb = decode_bytes(xd["ctx_len"].cpu().tolist(), wd.Hkv, wd.D, wd.dg, K, wd.G)
    tot = kvb + gkb + smb
    return {"budget": 64 * (K + 1), "topk": K, "us_per_step_cold": round(us, 2),
            "algorithmic_bytes": tot, "GBps_cold": round(tot / (us * 1e-6) / 1e9, 1),
            "KV_GBps_cold": round(kvb / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(tot / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


COUNTER_KERNELS = ("sparse_fwd_kernel", "dkdv_kernel", "dq_kernel", "topk_kernel",
                   "walk_order_kernel", "bwd_prep_kernel", "gate_query_kernel", "gate_key_kernel")


def summarize_counters(dirs, out_json: str):
    """Per-kernel averages (per dispatch) of every counter found in rocprofv3
    --pmc runs (one directory per pass) for the attention, Top-K and router
    kernels, with derived figures: executed MFMA FLOPs (the MOPS counters
    count 512 FLOPs each), MFMA busy share of the SIMD cycles, L2 hit rate,
    and the bytes behind the L1 -> L2 requests (128-byte lines).  Written to
    profiles/counters.json with each kernel's source hash."""
    import csv
    import glob

    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                k = next((n for n in COUNTER_KERNELS if ("::" + n) in r["Kernel_Name"]), None)
                if k is None:
                    continue
                vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                    float(r["Counter_Value"]))
    res, lines = {}, []
    for k, cs in vals.items():
        e = {c: sum(v) / len(v) for c, v in cs.items()}
        mops = sum(e.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16",
                                           "SQ_INSTS_VALU_MFMA_MOPS_F16",
                                           "SQ_INSTS_VALU_MFMA_MOPS_F32"))
        d = {"counters_per_dispatch": {c: round(v, 1) for c, v in e.items()},
             "dispatches": max(len(v) for v in cs.values())}
        if mops:
            d["executed_mfma_flops"] = mops * 512
        if e.get("GRBM_GUI_ACTIVE") and "SQ_VALU_MFMA_BUSY_CYCLES" in e:
            # GRBM_GUI_ACTIVE comes summed over the 8 XCDs; 1024 SIMDs
            d["mfma_busy_frac"] = e["SQ_VALU_MFMA_BUSY_CYCLES"] / (e["GRBM_GUI_ACTIVE"] / 8 * 1024)
        if e.get("TCC_REQ_sum"):
            d["l2_hit_rate"] = e.get("TCC_HIT_sum", 0.0) / e["TCC_REQ_sum"]
        if "TCP_TCC_READ_REQ_sum" in e:
            d["l1_to_l2_read_bytes"] = e["TCP_TCC_READ_REQ_sum"] * 128
        d["source_hash"] = kernel_hash(k)
        res[k] = d
        lines.append(f"{k}: " + ", ".join(f"{n} {d[n]:.4g}" for n in
                                          ("executed_mfma_flops", "mfma_busy_frac", "l2_hit_rate",
                                           "l1_to_l2_read_bytes") if n in d))
    json.dump(res, open(out_json, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def load_counters(kernel_key: str, src_hash: str):
    """Counter figures of profiles/counters.json for a kernel, if taken on
    the current kernel source."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        e = json.load(open(p)).get(kernel_key)
    except Exception:
        return None
    if not e or e.get("source_hash") != src_hash:
        return None
    return {k: e[k] for k in ("executed_mfma_flops", "mfma_busy_frac", "l2_hit_rate",
                              "l1_to_l2_read_bytes") if k in e}


def cpu_baseline(seed: int, n_tokens: int):
    """The fp64 oracle, as it stands, on a bounded sample of the 32K workload:
    forward + backward of every query head for n_tokens query tokens spread
    over the sequence (all 8 KV heads), with BLAS and torch on the host's
    cores (OMP_NUM_THREADS if set, else every core)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import sas_oracle as O

    w = synth.TRAIN_32K
    x = synth.prefill_inputs(w, seed=seed, device="cpu")
    x64 = {k: O.as64(v) for k, v in x.items()}
    T = w.T
    toks = np.unique(np.linspace(64 * (w.topk + 2), T - 1, n_tokens).astype(int))
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    with threadpool_limits(limits=cores):
        torch.set_num_threads(cores)
        r = O.route(x64["q"], x64["k"], x64["wq"], x64["wk"], x64["w_qn"], x64["w_kn"], w.topk,
                    w.theta, w.eps, tokens=toks)
        S = w.topk + 1
        idx = np.full((w.B, T, w.Hkv, S), -1, dtype=np.int64)
        logg = np.full((w.B, T, w.Hkv, S), -np.inf)
        idx[:, toks] = r["idx"]
        logg[:, toks] = r["logg"]
        sc = 1.0 / math.sqrt(w.D)
        t0 = time.perf_counter()
        O.attn_bwd(x64["q"], x64["k"], x64["v"], x64["dout"], idx, logg, sc, tokens=toks)
        dt = time.perf_counter() - t0
    flops = 0
    for t in toks:
        c = t // 64
        n = 64 * min(w.topk, c) + (t - 64 * c) + 1
        flops += 14 * w.D * n * w.Hq
    return dict(value=float(round(flops / dt / 1e12, 6)), unit="TFLOP/s", cores=cores,
                kind="oracle",
                sample=f"{len(toks)} query tokens x {w.Hq} heads of the 32K training layer, "
                       f"fp64 forward+backward (numpy, {cores} BLAS threads), {dt:.1f} s",
                seconds=round(dt, 2))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--cpu-tokens", type=int, default=600)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-router-bwd", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 8K, G=5 budget-sweep, per-query-head and decode-budget timings")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for traffic)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/counters.json from rocprofv3 --pmc runs and exit")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, os.path.join(ROOT, "profiles", "counters.json"))
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the path shards over batch x KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_block_sparse_gate_amd as sas
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sas.load_library()

    # ------------------------------------------------------------ training layer
    w = synth.TRAIN_32K
    x = synth.prefill_inputs(w, seed=args.seed, device=dev)
    B, T, Hq, Hkv, D, dg, K = w.B, w.T, w.Hq, w.Hkv, w.D, w.dg, w.topk
    S = K + 1
    NB = w.NB
    scale = 1.0 / math.sqrt(D)
    d = sas.make_dims(B, T, Hq, Hkv, D, dg, K, w.theta, w.eps)
    ws_gate = torch.empty(sas.workspace_size(sas.OP_GATE_SCORE, d), dtype=torch.uint8, device=dev)
    ws_bwd = torch.empty(sas.workspace_size(sas.OP_BWD, d), dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(sas.workspace_size(sas.OP_FWD, d), dtype=torch.uint8, device=dev)
    qg = torch.empty((B, T, Hkv, dg), dtype=torch.float32, device=dev)
    kg = torch.empty_like(qg)
    idx = torch.empty((B, T, Hkv, S), dtype=torch.int32, device=dev)
    logg = torch.empty((B, T, Hkv, S), dtype=torch.float32, device=dev)
    glse = torch.empty((B, T, Hkv), dtype=torch.float32, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device=dev)
    o32 = torch.empty((B, T, Hq, D), dtype=torch.float32, device=dev)
    dq = torch.empty_like(x["q"])
    dk = torch.empty_like(x["k"])
    dv = torch.empty_like(x["v"])
    dlogg = torch.empty_like(logg)
    stream = torch.cuda.current_stream(dev)

    ev = None
    fev = bev = None

    def step(record=False):
        if record:
            ev[0].record(stream)
        sas.gate_score(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], K, w.theta, w.eps,
                       q_gate=qg, k_gate=kg, workspace=ws_gate)
        if record:
            ev[1].record(stream)
        sas.topk_blocks(qg, kg, K, Hq, D, out=(idx, logg, glse))
        if record:
            ev[2].record(stream)
            sas.set_timing_events(fev)       # stage boundaries inside the calls
        sas.sparse_attn_fwd(x["q"], x["k"], x["v"], idx, logg, scale, o=o, lse=lse, o_f32=o32,
                            workspace=ws_fwd)
        if record:
            ev[3].record(stream)
            sas.set_timing_events(bev)
        sas.sparse_attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg, scale,
                            workspace=ws_bwd, out=(dq, dk, dv, dlogg), o_f32=o32)
        if record:
            ev[4].record(stream)
            sas.set_timing_events(None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.warmup > 0:           # with no warm-up the outputs are not written yet
        assert_sound(sas, "warm-up", o=o, o_f32=o32, dq=dq, dk=dk, dv=dv, dlogg=dlogg)
    stage_ms = [0.0] * 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    bevs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in [e for l in fevs + bevs for e in l]:
        e.record(stream)                    # create the events before the timed region
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        ev, fev, bev = evs[i], fevs[i], bevs[i]
        step(record=True)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # A ring wait in the attention kernels that gives up ends the kernel
    # early with NaN outputs, which would time as a faster step: refuse to
    # report a number unless no wait gave up and every output is finite.
    assert_sound(sas, "training step", o=o, lse=lse, o_f32=o32, dq=dq, dk=dk, dv=dv,
                 dlogg=dlogg, logg_valid=logg[idx >= 0])
    for i in range(args.steps):
        for s_ in range(4):
            stage_ms[s_] += evs[i][s_].elapsed_time(evs[i][s_ + 1]) / args.steps
    ms_per_step = total_ms / args.steps

    def avg_ms(lst, a, b):
        return sum(l[a].elapsed_time(l[b]) for l in lst) / len(lst)

    kern_ms = {"sparse_fwd_kernel": avg_ms(fevs, 1, 2),
               "walk_order+transpose_v": avg_ms(fevs, 0, 1),
               "bwd_delta+csr+walk_order": avg_ms(bevs, 0, 1), "dkdv_kernel": avg_ms(bevs, 1, 2),
               "dq_kernel": avg_ms(bevs, 2, 3)}

    if args.copy_calib:
        src_c = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst_c = torch.empty_like(src_c)
        for _ in range(3):
            dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    pairs = attended_pairs(T, K) * Hq * B
    fwd_flops = 4.0 * D * pairs
    bwd_flops = 10.0 * D * pairs
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = fwd_flops / (stage_ms[2] * 1e-3) / 1e12
    bwd_tflops = bwd_flops / (stage_ms[3] * 1e-3) / 1e12
    attn_tflops = (fwd_flops + bwd_flops) / ((stage_ms[2] + stage_ms[3]) * 1e-3) / 1e12

    # algorithmic FLOPs per launch: the contractions each kernel must perform,
    # 2 D per attended (query head, key) pair each: forward S and PV (4 D);
    # dK/dV kernel S, dP, dV, dK (8 D; it also writes dS); dQ kernel dQ = dS K
    # (2 D, reading dS)
    kflops = {"sparse_fwd_kernel": 4.0 * D * pairs, "dkdv_kernel": 8.0 * D * pairs,
              "dq_kernel": 2.0 * D * pairs}
    kernels = {}
    for kname, fl in kflops.items():
        ms = kern_ms[kname]
        kernels[kname] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                          "frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    dom = max(kflops, key=lambda k: kern_ms[k])
    dom_tf = kflops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    dom_hash = kernel_hash(dom)
    roofline = {
        "kernel": dom,
        "bound": "mfma",
        "achieved": round(dom_tf, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
        "traffic": load_traffic(dom, dom_hash),
        "algorithmic_flops_per_launch": kflops[dom],
        "launch_ms": round(kern_ms[dom], 4),
    }
    cnt = load_counters(dom, dom_hash)
    if cnt:
        # executed MFMA work (masked tile rows and the hi + lo halves of the
        # fp32-accurate products included) against the algorithmic FLOPs
        roofline["counters"] = dict(cnt, executed_over_algorithmic=round(
            cnt["executed_mfma_flops"] / kflops[dom], 3)) if "executed_mfma_flops" in cnt else cnt
    for kname in kflops:
        c = load_counters(kname, kernel_hash(kname))
        if c:
            kernels[kname]["counters"] = c

    out = {
        "metric": "sparse-attn fwd+bwd TFLOP/s @32K (% MFMA peak); decode KV GB/s @budget 2048",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 q/k/v/dO, N(0,1)/sqrt(fan_in) bf16 router weights)",
        "config": {"workload": w.name, "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "D": D, "dg": dg,
                   "block": 64, "topk": K, "parallelism": "single GPU"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "stages_ms": {"gate_score": round(stage_ms[0], 4), "topk": round(stage_ms[1], 4),
                      "fwd": round(stage_ms[2], 4), "bwd": round(stage_ms[3], 4)},
        "attn_fwd_tflops": round(fwd_tflops, 2),
        "attn_bwd_tflops": round(bwd_tflops, 2),
        "attn_fwd_bwd_tflops": round(attn_tflops, 2),
        "effective_pairs_per_head": attended_pairs(T, K),
        "roofline": roofline,
        "kernels": kernels,
        "other_ms": {k: round(v, 4) for k, v in kern_ms.items() if k not in kflops},
    }

    # ------------------------------------------------------------ router backward
    # (reported beside the step, not inside it): gradients of the router from
    # the step's dlogg with its selection fixed
    if not args.no_router_bwd:
        gws = torch.empty(sas.workspace_size(sas.OP_GATE_BWD, d), dtype=torch.uint8, device=dev)
        for _ in range(2):
            gout = sas.gate_score_bwd(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], qg,
                                      kg, idx, dlogg, w.theta, w.eps, workspace=gws)
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nrb = 5
        r0.record(stream)
        for _ in range(nrb):
            sas.gate_score_bwd(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], qg, kg, idx,
                               dlogg, w.theta, w.eps, workspace=gws, check_row_sums=False)
        r1.record(stream)
        torch.cuda.synchronize()
        rb_ms = r0.elapsed_time(r1) / nrb
        G = Hq // Hkv
        rows = B * T
        # algorithmic bytes: q, k, q_gate, k_gate, idx, dlogg read once; dq, dk
        # (fp32) written once; weights negligible
        rb_bytes = (rows * Hq * D * 2 + rows * Hkv * D * 2 + 2 * rows * Hkv * dg * 4
                    + 2 * rows * Hkv * S * 4 + rows * Hq * D * 4 + rows * Hkv * D * 4)
        # contractions (2 flops per multiply-add): projections recomputed
        # (x Wq, p Wk), dx = dy Wq^T, dp = dz Wk^T, dWq = x^T dy, dWk = p^T dz,
        # and the gate-logit gradients onto q_gate / the keys (2 S dg per row)
        rb_flops = 2.0 * rows * Hkv * dg * (3 * G * D + 3 * 3 * D + 2 * S)
        t_hbm = rb_bytes / (PEAK_HBM_GBS * 1e9)
        t_mfma = rb_flops / (PEAK_FP32_TFLOPS * 1e12)
        rb_traffic = load_traffic("sas_gate_score_bwd", kernel_hash("sas_gate_score_bwd"))
        out["router_bwd"] = {
            "workload": w.name, "ms": round(rb_ms, 4),
            "algorithmic_bytes": rb_bytes, "algorithmic_flops": rb_flops,
            "GBps": round(rb_bytes / (rb_ms * 1e-3) / 1e9, 1),
            "tflops": round(rb_flops / (rb_ms * 1e-3) / 1e12, 2),
            "roofline": ({"bound": "mfma", "achieved": round(rb_flops / (rb_ms * 1e-3) / 1e12, 2),
                          "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(t_mfma / (rb_ms * 1e-3), 4), "traffic": rb_traffic}
                         if t_mfma >= t_hbm else
                         {"bound": "hbm", "achieved": round(rb_bytes / (rb_ms * 1e-3) / 1e9, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": round(t_hbm / (rb_ms * 1e-3), 4), "traffic": rb_traffic}),
        }
        del gws, gout

    # ------------------------------------------------------------ decode
    if not args.no_decode:
        del x, qg, kg, idx, logg, glse, o, o32, lse, dq, dk, dv, dlogg, ws_gate, ws_bwd, ws_fwd
        torch.cuda.empty_cache()
        wd = synth.DECODE_B64
        xd = synth.decode_inputs(wd, seed=args.seed, device=dev)
        Kd = wd.topk
        od = torch.empty((wd.B, wd.Hq, wd.D), dtype=torch.bfloat16, device=dev)
        ws_d = torch.empty(sas.decode_workspace_size(sas.DecodeDims(
            wd.B, wd.Hq, wd.Hkv, wd.D, wd.dg, 64, Kd, xd["Lmax"], xd["NBmax"], 1)),
            dtype=torch.uint8, device=dev)
        scd = 1.0 / math.sqrt(wd.D)

        def dstep():
            sas.decode(xd["q"], xd["q_gate"], xd["k_cache"], xd["v_cache"], xd["kg_cache"],
                       xd["ctx_len"], Kd, scd, apply_gate=True, want_idx=False,
                       workspace=ws_d, out=(od, None, None))

        for _ in range(3):
            dstep()
        torch.cuda.synchronize()
        # warm: back-to-back steps
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.decode_steps):
            dstep()
        e1.record(stream)
        torch.cuda.synchronize()
        warm_us = e0.elapsed_time(e1) / args.decode_steps * 1e3
        assert_sound(sas, "decode (contiguous, warm)", o=od)
        # cold: read 1 GiB between steps so no selected block or gate key is
        # cached (a read leaves no dirty lines whose write-back would compete
        # with the step, as a 1 GiB write would)
        flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        cold = []
        for _ in range(args.decode_steps):
            flush.sum()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            dstep()
            a1.record(stream)
            torch.cuda.synchronize()
            cold.append(a0.elapsed_time(a1) * 1e3)
        cold.sort()
        cold_us = cold[len(cold) // 2]
        assert_sound(sas, "decode (contiguous, cold)", o=od)
        # the same step over a paged cache: every (sequence, block) in its own
        # page of a shuffled pool, through sas_decode_paged
        NBd = xd["NBmax"]
        npages = wd.B * NBd
        gen = torch.Generator().manual_seed(args.seed + 11)
        perm = torch.randperm(npages, generator=gen).to(torch.int32).view(wd.B, NBd).to(dev)
        flat = perm.flatten().long()

        def paged(c):
            pool = torch.empty((npages, wd.Hkv, 64, wd.D), dtype=c.dtype, device=dev)
            pool[flat] = c.view(wd.B, wd.Hkv, NBd, 64, wd.D).permute(0, 2, 1, 3, 4).reshape(
                npages, wd.Hkv, 64, wd.D)
            return pool

        kpool, vpool = paged(xd["k_cache"]), paged(xd["v_cache"])
        gpool = torch.empty((npages, wd.Hkv, wd.dg), dtype=torch.float32, device=dev)
        gpool[flat] = xd["kg_cache"].permute(0, 2, 1, 3).reshape(npages, wd.Hkv, wd.dg)

        def dstep_paged():
            sas.decode_paged(xd["q"], xd["q_gate"], kpool, vpool, gpool, perm, xd["ctx_len"], Kd,
                             scd, apply_gate=True, want_idx=False, workspace=ws_d,
                             out=(od, None, None))

        for _ in range(3):
            dstep_paged()
        cold_p = []
        for _ in range(args.decode_steps):
            flush.sum()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            dstep_paged()
            a1.record(stream)
            torch.cuda.synchronize()
            cold_p.append(a0.elapsed_time(a1) * 1e3)
        cold_p.sort()
        cold_paged_us = cold_p[len(cold_p) // 2]
        assert_sound(sas, "decode (paged)", o=od)
        del kpool, vpool, gpool
        # the contiguous step with the gate-key cache in bf16 (kg_dtype = 1)
        kg16 = xd["kg_cache"].to(torch.bfloat16)

        def dstep_kg16():
            sas.decode(xd["q"], xd["q_gate"], xd["k_cache"], xd["v_cache"], kg16, xd["ctx_len"],
                       Kd, scd, apply_gate=True, want_idx=False, workspace=ws_d,
                       out=(od, None, None))

        for _ in range(3):
            dstep_kg16()
        cold_b = []
        for _ in range(args.decode_steps):
            flush.sum()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            dstep_kg16()
            a1.record(stream)
            torch.cuda.synchronize()
            cold_b.append(a0.elapsed_time(a1) * 1e3)
        cold_b.sort()
        cold_kg16_us = cold_b[len(cold_b) // 2]
        assert_sound(sas, "decode (bf16 gate keys)", o=od)
        del kg16
        lens = xd["ctx_len"].cpu().tolist()
        kvb, gkb, smb = decode_bytes(lens, wd.Hkv, wd.D, wd.dg, Kd, wd.G)
        tot = kvb + gkb + smb
        dec_hash = kernel_hash("sas_decode")
        out["decode"] = {
            "workload": wd.name, "B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "D": wd.D, "dg": wd.dg,
            "budget": 64 * (Kd + 1), "ctx_len_range": [wd.Lmin, wd.Lmax],
            "us_per_step_cold": round(cold_us, 2), "us_per_step_warm": round(warm_us, 2),
            "us_per_step_cold_paged": round(cold_paged_us, 2),
            "us_per_step_cold_kg_bf16": round(cold_kg16_us, 2),
            "algorithmic_bytes": tot, "kv_bytes": kvb, "gate_key_bytes": gkb,
            "GBps_cold": round(tot / (cold_us * 1e-6) / 1e9, 1),
            "KV_GBps_cold": round(kvb / (cold_us * 1e-6) / 1e9, 1),
            "GBps_warm": round(tot / (warm_us * 1e-6) / 1e9, 1),
            "roofline": {"kernel": "sas_decode (score + select + attention)",
                         "bound": "hbm", "achieved": round(tot / (cold_us * 1e-6) / 1e9, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(tot / (cold_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                         "traffic": load_traffic("sas_decode", dec_hash)},
        }
    # ------------------------------------------------------------ other configurations
    # (reported beside the headline, not part of it): the 8K prefill layer
    # (router + Top-K + forward); the Qwen3-14B-shaped G = 5 layer at budgets
    # 1,024 / 2,048 / 4,096 for both skew recipes, with the locality of the
    # router's selections; the 32K training layer with one gate per query
    # head; decode at budgets 1,024 and 4,096
    if not args.no_configs:
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        cfg = {"prefill_8k": time_layer(sas, synth.PREFILL_8K, synth.PREFILL_8K.topk, args.seed,
                                        steps=10, warmup=3, backward=False)}
        skew = []
        for w5 in (synth.SKEW_32K, synth.SKEW5B_32K):
            for K5 in (15, 31, 63):
                skew.append(time_layer(sas, w5.replace(topk=K5), K5, args.seed, steps=3,
                                       warmup=1, stats=True))
                gc.collect()
                torch.cuda.empty_cache()
        cfg["g5_32k_budgets"] = skew
        wq = synth.TRAIN_32K.replace(name=synth.TRAIN_32K.name + "_per_query_head_gates", gate="q")
        cfg["train_32k_per_query_head"] = time_layer(sas, wq, wq.topk, args.seed, steps=3,
                                                     warmup=1, stats=True)
        gc.collect()
        torch.cuda.empty_cache()
        if "decode" in out:
            out["decode"]["other_budgets"] = [
                time_decode_budget(sas, synth.DECODE_B64, K4, args.seed, args.decode_steps)
                for K4 in (15, 63)]
        out["configs"] = cfg
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.seed, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
