"""The no-allocation plan upload (zz_plan_upload_static) through the C ABI.

It binds a plan to the library's own per-GPU workspace instead of a
caller-allocated one; every kernel then reads the same tables, so the results
must equal those of a plan uploaded into a caller's buffer bit for bit.  Two
uploads in a row (the second plan smaller) check that the shared workspace is
rewritten, and that the first plan is refused once its tables are gone."""
import ctypes

import pytest

import synthetic
from zz_testlib import Case

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")

ZZ_OK, ZZ_ERR_WORKSPACE, ZZ_ERR_STATE = 0, 5, 7


def static_upload(plan):
    """Call the C entry point directly (no binding code in between)."""
    L = zz.lib()
    f = L.zz_plan_upload_static
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int32
    import torch
    return int(f(plan.handle, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))


def run_path(plan, case):
    """Forward + backward through the ring driver, all outputs fp32."""
    o_acc, lse = zz.ring_attention_fwd(plan, case.qz, case.kz, case.vz)
    o_zz = zz.finalize_fwd(plan, o_acc)
    dq, dk, dv = zz.ring_attention_bwd(plan, case.qz, case.kz, case.vz, o_zz, case.doz, lse)
    return o_acc, lse, dq, dk, dv


def same_plan_args(case):
    return (case.cu, case.cp, case.hq, case.hkv, case.d, case.dtype)


def test_static_upload_equals_caller_workspace_twice_then_refuses_stale_plan():
    import torch
    big = Case((128, 256, 64), 2, 4, 2, 128, "bf16", 11, with_do=True)
    small = Case((48, 16), 2, 2, 1, 64, "bf16", 12, with_do=True)

    # first call: the larger workload
    want_big = run_path(big.plan, big)
    p_big = zz.Plan(*same_plan_args(big))           # host plan only, not uploaded
    assert static_upload(p_big) == ZZ_OK
    got_big = run_path(p_big, big)
    torch.cuda.synchronize()
    for a, b in zip(want_big, got_big):
        assert torch.equal(a, b)

    # second call, smaller input: the same workspace is rewritten
    want_small = run_path(small.plan, small)
    p_small = zz.Plan(*same_plan_args(small))
    assert p_small.workspace_bytes() < p_big.workspace_bytes()
    assert static_upload(p_small) == ZZ_OK
    got_small = run_path(p_small, small)
    torch.cuda.synchronize()
    for a, b in zip(want_small, got_small):
        assert torch.equal(a, b)

    # the first plan's tables were overwritten: its calls are refused
    with pytest.raises(zz.ZZError, match="static workspace"):
        zz.ring_attention_fwd(p_big, big.qz, big.kz, big.vz)
    # uploading it again makes it usable again (and stales the small plan)
    assert static_upload(p_big) == ZZ_OK
    again = run_path(p_big, big)
    torch.cuda.synchronize()
    for a, b in zip(want_big, again):
        assert torch.equal(a, b)
    with pytest.raises(zz.ZZError, match="static workspace"):
        zz.ring_attention_fwd(p_small, small.qz, small.kz, small.vz)


STATIC_WORKSPACE_BYTES = 96 << 20   # the maximum include/zz.h states


def test_static_upload_rejects_a_plan_larger_than_the_static_workspace():
    L = zz.lib()
    # one 262144-token sequence at CP 16: tile tables of about 324 MiB
    p = zz.Plan([0, 262144], 16, 64, 8, 128, "bf16")
    assert p.workspace_bytes() > STATIC_WORKSPACE_BYTES
    assert static_upload(p) == ZZ_ERR_WORKSPACE
    assert b"static workspace" in L.zz_last_error()
    # the largest workload here (131072 tokens, CP 16) fits
    assert zz.Plan([0, 131072], 16, 64, 8, 128, "bf16").workspace_bytes() <= STATIC_WORKSPACE_BYTES
