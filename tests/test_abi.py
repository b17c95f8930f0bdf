"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

import gated_block_sparse_gate_amd as sas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sas.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sas.LIB_PATH),
                                reason="libsas.so not built (run __graft_entry__.build())")


def declared_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:sas_status|int|size_t|const char\*)\s+(sas_\w+)\s*\(",
                                 txt, re.M)))


def test_header_declares_the_five_calls_and_helpers():
    names = declared_functions()
    for n in ("sas_gate_score", "sas_topk_blocks", "sas_sparse_attn_fwd", "sas_sparse_attn_bwd",
              "sas_decode", "sas_workspace_size", "sas_last_error", "sas_version"):
        assert n in names
    assert set(names) == set(sas.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = sas.load_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert sas.version() == 1


def test_nm_shows_c_linkage():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sas.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (sas_\w+)", out))
    assert set(declared_functions()) <= exported


def _dims(**kw):
    base = dict(B=1, T=1024, Hq=8, Hkv=2, D=128, dg=128, topk=31)
    base.update(kw)
    return sas.make_dims(**base)


@pytest.mark.parametrize("bad,code", [
    (dict(D=96), sas.SAS_ERR_UNSUPPORTED),
    (dict(dg=48), sas.SAS_ERR_UNSUPPORTED),
    (dict(Hq=6, Hkv=4), sas.SAS_ERR_INVALID),
    (dict(Hq=18, Hkv=2), sas.SAS_ERR_UNSUPPORTED),
    (dict(topk=-1), sas.SAS_ERR_INVALID),
    (dict(topk=64), sas.SAS_ERR_UNSUPPORTED),
    (dict(T=0), sas.SAS_ERR_INVALID),
    (dict(T=65537), sas.SAS_ERR_UNSUPPORTED),
    (dict(block=32), sas.SAS_ERR_UNSUPPORTED),
])
def test_invalid_dims_rejected(bad, code):
    lib = sas.load_library()
    d = _dims(**bad)
    assert lib.sas_workspace_size(sas.OP_BWD, ctypes.byref(d)) == ctypes.c_size_t(-1).value
    # a call with these dims fails validation before touching any pointer
    st = lib.sas_sparse_attn_fwd(ctypes.byref(d), *([ctypes.c_void_p(16)] * 5),
                                 ctypes.c_float(0.1), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                 None, None, 0, None)
    assert st == code
    assert lib.sas_last_error()


def test_null_and_misaligned_pointers_rejected():
    lib = sas.load_library()
    d = _dims()
    p = ctypes.c_void_p(4096)
    st = lib.sas_sparse_attn_fwd(ctypes.byref(d), p, p, None, p, p, ctypes.c_float(0.1), p, p,
                                 None, None, 0, None)
    assert st == sas.SAS_ERR_INVALID
    assert b"'v'" in lib.sas_last_error()
    st = lib.sas_sparse_attn_fwd(ctypes.byref(d), p, p, ctypes.c_void_p(4098), p, p,
                                 ctypes.c_float(0.1), p, p, None, None, 0, None)
    assert st == sas.SAS_ERR_INVALID
    assert b"aligned" in lib.sas_last_error()
    st = lib.sas_sparse_attn_fwd(None, p, p, p, p, p, ctypes.c_float(0.1), p, p, None, None, 0,
                                 None)
    assert st == sas.SAS_ERR_INVALID
    st = lib.sas_sparse_attn_fwd(ctypes.byref(d), p, p, p, p, p, ctypes.c_float(float("nan")), p,
                                 p, None, None, 0, None)
    assert st == sas.SAS_ERR_INVALID


def test_workspace_checks():
    lib = sas.load_library()
    d = _dims(T=4096)
    need = sas.workspace_size(sas.OP_BWD, d)
    assert need > 0
    # fp16 transposed v, per-block |v| maxima (64 blocks), per-head scales, and the
    # staging orders (2 heads x 74 groups of 56 tokens x 72 uint16); 256-byte aligned
    order = 2 * 74 * 72 * 2
    assert sas.workspace_size(sas.OP_WALK_ORDER, d) == order
    assert sas.workspace_size(sas.OP_FWD, d) == (1 * 2 * 128 * 4096 * 2 + 512 + 256
                                                 + (order + 255) // 256 * 256)
    assert sas.workspace_size(sas.OP_TOPK, d) == 0
    p = ctypes.c_void_p(4096)
    args = [p] * 9 + [ctypes.c_float(0.1)] + [p] * 4
    st = lib.sas_sparse_attn_bwd(ctypes.byref(d), *args, None, need, None)
    assert st == sas.SAS_ERR_WORKSPACE
    st = lib.sas_sparse_attn_bwd(ctypes.byref(d), *args, p, need - 1, None)
    assert st == sas.SAS_ERR_WORKSPACE
    g = sas.workspace_size(sas.OP_GATE_SCORE, d)
    st = lib.sas_gate_score(ctypes.byref(d), *([p] * 8), p, g - 1, None)
    assert st == sas.SAS_ERR_WORKSPACE


def test_walk_order_validation():
    """sas_walk_order rejects bad dims, null / unaligned pointers and a short
    order buffer before launching anything."""
    lib = sas.load_library()
    d = _dims(T=4096)
    need = sas.workspace_size(sas.OP_WALK_ORDER, d)
    p = ctypes.c_void_p(4096)
    assert lib.sas_walk_order(ctypes.byref(d), None, p, need, None) == sas.SAS_ERR_INVALID
    assert b"'idx'" in lib.sas_last_error()
    assert lib.sas_walk_order(ctypes.byref(d), p, ctypes.c_void_p(4098), need, None) == \
        sas.SAS_ERR_INVALID
    assert lib.sas_walk_order(ctypes.byref(d), p, p, need - 1, None) == sas.SAS_ERR_INVALID
    assert b"too small" in lib.sas_last_error()
    bad = _dims(T=4096, D=96)
    assert lib.sas_walk_order(ctypes.byref(bad), p, p, need, None) == sas.SAS_ERR_UNSUPPORTED
    # per-query-head gates: Hq selection heads of 64-token groups (TPT = 16)
    pq = _dims(T=4096, flags=sas.FLAG_GATE_PER_QUERY_HEAD)
    assert sas.workspace_size(sas.OP_WALK_ORDER, pq) == 8 * 64 * 72 * 2


def test_decode_dims_validation():
    lib = sas.load_library()
    good = sas.DecodeDims(64, 32, 8, 128, 128, 64, 31, 65536, 1024, 1)
    assert sas.decode_workspace_size(good) > 0
    bad = sas.DecodeDims(64, 32, 8, 128, 128, 64, 31, 65536, 1000, 1)   # NBmax mismatch
    assert lib.sas_decode_workspace_size(ctypes.byref(bad)) == ctypes.c_size_t(-1).value
    bad2 = sas.DecodeDims(64, 32, 8, 128, 128, 64, 31, 65536, 1024, 2)  # apply_gate
    assert lib.sas_decode_workspace_size(ctypes.byref(bad2)) == ctypes.c_size_t(-1).value


def test_budget_mapping():
    assert [sas.budget_to_topk(b) for b in (1024, 2048, 4096)] == [15, 31, 63]
    with pytest.raises(ValueError):
        sas.budget_to_topk(1000)


def test_compute_calls_fail_loudly_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    q = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sas.sparse_attn_fwd(q, q[:, :, :1], q[:, :, :1], torch.zeros(1, 64, 1, 4, dtype=torch.int32),
                            torch.zeros(1, 64, 1, 4))
