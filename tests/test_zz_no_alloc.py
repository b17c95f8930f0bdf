"""sas_decode_noalloc (fixed per-device scratch, no workspace argument)
against sas_decode (caller workspace) through the C ABI: two calls in a row
on the same GPU, the second with a smaller batch, shorter contexts and a
different budget, so the second call reuses scratch that still holds the
first call's contents.  The same kernels run on the same inputs, so indices
and outputs must be bitwise equal (stronger than the parity bar: indices
bit-exact, outputs within 1e-2 / 1e-3); the outputs are also checked against
the oracle.  Dimensions needing more scratch than the fixed size are
rejected before any launch."""
import math

import numpy as np
import pytest
import torch

import gated_block_sparse_gate_amd as sas
import synth
from oracle import sas_oracle as O

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, D, dg, K, Lmax, seed):
    w = synth.Workload("noalloc", 94, B=B, T=1, Hq=Hq, Hkv=Hkv, D=D, dg=dg, topk=K, kind="decode",
                       Lmin=1, Lmax=Lmax)
    lens = torch.randint(1, Lmax + 1, (B,), generator=torch.Generator().manual_seed(seed),
                         dtype=torch.int32)
    lens[0] = Lmax
    return synth.decode_inputs(w, seed=seed, device="cpu", ctx_len=lens)


@pytest.mark.parametrize("kg_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_decode_matches_workspace_decode(kg_dtype):
    calls = [(48, 16, 4, 128, 128, 31, 9000, 1), (5, 8, 2, 64, 32, 15, 3000, 2)]
    for B, Hq, Hkv, D, dg, K, Lmax, seed in calls:
        x = _inputs(B, Hq, Hkv, D, dg, K, Lmax, seed)
        d = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in x.items()}
        kg = d["kg_cache"].to(kg_dtype)
        sc = 1.0 / math.sqrt(D)
        print(f"[noalloc] B={B} Hq={Hq} Hkv={Hkv} D={D} K={K} Lmax={Lmax} kg={kg_dtype}",
              flush=True)
        o_n, i_n, l_n = sas.decode_noalloc(d["q"], d["q_gate"], d["k_cache"], d["v_cache"], kg,
                                           d["ctx_len"], K, sc)
        o_w, i_w, l_w = sas.decode(d["q"], d["q_gate"], d["k_cache"], d["v_cache"], kg,
                                   d["ctx_len"], K, sc)
        torch.cuda.synchronize()
        assert torch.equal(i_n, i_w)
        assert torch.equal(l_n.nan_to_num(), l_w.nan_to_num())
        assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
        ref = O.decode(x["q"], x["q_gate"], x["k_cache"], x["v_cache"], kg.float().cpu(),
                       x["ctx_len"], K, sc)
        ok = ~ref["near_tie"]
        np.testing.assert_array_equal(i_n.cpu().numpy()[ok], ref["idx"][ok])
        okh = np.repeat(ok, Hq // Hkv, axis=1)
        err = np.abs(o_n.float().cpu().numpy()[okh] - ref["o"][okh])
        assert err.max() < 2e-2 and err.mean() < 1e-3


def test_noalloc_decode_rejects_oversized_dims():
    """B = 512 sequences x 8 KV heads at Lmax = 262144 need 64 MiB of scores:
    SAS_ERR_WORKSPACE, nothing launched (the pointers are never read)."""
    B, Hq, Hkv, D, dg, K, Lmax = 512, 32, 8, 128, 128, 31, 262144
    d = sas.DecodeDims(B, Hq, Hkv, D, dg, 64, K, Lmax, Lmax // 64, 1, 0)
    assert sas.decode_workspace_size(d) > 16 << 20
    lib = sas.load_library()
    import ctypes
    p = ctypes.c_void_p(256)
    st = lib.sas_decode_noalloc(ctypes.byref(d), p, p, p, p, p, p, ctypes.c_float(0.1), p, None,
                                None, None)
    assert st == sas.SAS_ERR_WORKSPACE
    assert b"16777216" in lib.sas_last_error()
