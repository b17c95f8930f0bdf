"""HIP graph capture of the library calls: the training chain (router, Top-K,
forward, backward) and a decode step are captured into one graph each,
replayed three times with eager work between the replays (the outputs are
cleared, other kernels run), and every replay is compared bit-exactly with
the eager run.  The calls enqueue kernels only, and every
kernel is deterministic, so the replays must reproduce the eager outputs
exactly."""
import pytest
import torch

import gated_block_sparse_gate_amd as sas
import synth

pytestmark = pytest.mark.gpu

W = synth.Workload("graph_g4", 95, B=1, T=1000, Hq=8, Hkv=2, D=128, dg=128, topk=7, kind="train")


def _chain(x, ws, outs):
    qg, kg, idx, logg, glse, o, lse, o32, dq, dk, dv, dlogg = outs
    sas.gate_score(x["q"], x["k"], x["wq"], x["wk"], x["w_qn"], x["w_kn"], W.topk, W.theta, W.eps,
                   q_gate=qg, k_gate=kg, workspace=ws["gate"])
    sas.topk_blocks(qg, kg, W.topk, W.Hq, W.D, out=(idx, logg, glse))
    sas.sparse_attn_fwd(x["q"], x["k"], x["v"], idx, logg, o=o, lse=lse, o_f32=o32,
                        workspace=ws["fwd"])
    sas.sparse_attn_bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, idx, logg,
                        workspace=ws["bwd"], out=(dq, dk, dv, dlogg), o_f32=o32)


def test_training_chain_graph_replays_match_eager():
    x = synth.prefill_inputs(W, seed=0, device="cuda")
    B, T, Hq, Hkv, D, dg, S = W.B, W.T, W.Hq, W.Hkv, W.D, W.dg, W.topk + 1
    d = sas.make_dims(B, T, Hq, Hkv, D, dg, W.topk)
    ws = {n: torch.empty(max(1, sas.workspace_size(op, d)), dtype=torch.uint8, device="cuda")
          for n, op in (("gate", sas.OP_GATE_SCORE), ("fwd", sas.OP_FWD), ("bwd", sas.OP_BWD))}
    f32, i32, bf = torch.float32, torch.int32, torch.bfloat16
    outs = [torch.empty(B, T, Hkv, dg, dtype=f32, device="cuda"),
            torch.empty(B, T, Hkv, dg, dtype=f32, device="cuda"),
            torch.empty(B, T, Hkv, S, dtype=i32, device="cuda"),
            torch.empty(B, T, Hkv, S, dtype=f32, device="cuda"),
            torch.empty(B, T, Hkv, dtype=f32, device="cuda"),
            torch.empty(B, T, Hq, D, dtype=bf, device="cuda"),
            torch.empty(B, T, Hq, dtype=f32, device="cuda"),
            torch.empty(B, T, Hq, D, dtype=f32, device="cuda"),
            torch.empty(B, T, Hq, D, dtype=bf, device="cuda"),
            torch.empty(B, T, Hkv, D, dtype=bf, device="cuda"),
            torch.empty(B, T, Hkv, D, dtype=bf, device="cuda"),
            torch.empty(B, T, Hkv, S, dtype=f32, device="cuda")]
    names = ["q_gate", "k_gate", "idx", "logg", "gate_lse", "o", "lse", "o_f32", "dq", "dk", "dv",
             "dlogg"]
    print("graph capture: eager reference", flush=True)
    _chain(x, ws, outs)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert sas.take_device_fault() == 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream's side, as torch asks
        _chain(x, ws, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("graph capture: capturing", flush=True)
    with torch.cuda.graph(g):
        _chain(x, ws, outs)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: the outputs cleared, unrelated kernels
        for t in outs:
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").square().sum()
        torch.cuda.synchronize()
        print(f"graph capture: replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert sas.take_device_fault() == 0
        for n, a, b in zip(names, outs, ref):
            assert torch.equal(a, b), (rep, n)
        assert torch.isfinite(junk)


def test_decode_graph_replays_match_eager():
    wd = synth.Workload("graph_dec", 96, B=4, T=1, Hq=8, Hkv=2, D=128, dg=128, topk=15,
                        kind="decode", Lmin=300, Lmax=3000)
    x = synth.decode_inputs(wd, seed=0, device="cuda")
    print("graph capture: decode eager reference", flush=True)
    o_ref, idx_ref, _ = sas.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], x["kg_cache"],
                                   x["ctx_len"], wd.topk)
    torch.cuda.synchronize()
    d = sas.DecodeDims(wd.B, wd.Hq, wd.Hkv, wd.D, wd.dg, 64, wd.topk, x["k_cache"].shape[2],
                       x["kg_cache"].shape[2], 1)
    ws = torch.empty(max(1, sas.decode_workspace_size(d)), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(o_ref)
    idx = torch.empty_like(idx_ref)
    logg = torch.empty(idx_ref.shape, dtype=torch.float32, device="cuda")

    def step():
        sas.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], x["kg_cache"], x["ctx_len"],
                   wd.topk, workspace=ws, out=(o, idx, logg))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        o.zero_()
        idx.zero_()
        torch.cuda.synchronize()
        print(f"graph capture: decode replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(idx, idx_ref), rep
