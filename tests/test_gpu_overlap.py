"""Buffer-overlap checks of the C ABI on a GPU-bound plan: a call whose written
buffer overlaps another of its buffers is rejected on the host with
ZZ_ERR_ARG naming the two, before anything is launched (the sentinel outputs
stay untouched); buffers that are only read may share memory."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")

ERR_ARG = 1
LENGTHS, CP, HQ, HKV, D = [64, 128], 2, 4, 2, 64


def _p(t, byte_offset=0):
    return ctypes.c_void_p(t.data_ptr() + byte_offset)


def _rejected(rc, names):
    assert rc == ERR_ARG
    msg = zz.lib().zz_last_error().decode()
    assert msg.startswith("buffers overlap") and all(n in msg for n in names), msg


@pytest.fixture(scope="module")
def env():
    import torch

    cu = [0]
    for n in LENGTHS:
        cu.append(cu[-1] + n)
    plan = zz.Plan(cu, CP, HQ, HKV, D, "bf16", device="cuda")
    T = cu[-1]
    g = torch.Generator(device="cpu").manual_seed(5)
    mk = lambda h: torch.randn((T, h, D), generator=g).to(torch.bfloat16).cuda()
    return plan, T, mk(HQ), mk(HKV), mk(HKV), mk(HQ)


def test_forward_step_rejects_overlapping_outputs(env):
    import torch

    plan, T, q, k, v, _ = env
    L = zz.lib()
    o = torch.full((T, HQ, D), 7.0, device="cuda")
    # the LSE buffer placed inside the O accumulator
    rc = L.zz_varlen_ring_step_fwd(plan.handle, zz.ALL_RANKS, 0, _p(q), _p(k), _p(v), _p(o), _p(o, 4096), 0, None)
    _rejected(rc, ("o_acc", "lse_acc"))
    # the O accumulator over the query buffer
    lse = torch.empty((HQ, T), device="cuda")
    rc = L.zz_varlen_ring_step_fwd(plan.handle, zz.ALL_RANKS, 0, _p(q), _p(k), _p(v), _p(q), _p(lse), 0, None)
    _rejected(rc, ("o_acc", "q_zz"))
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


def test_read_only_buffers_may_share_memory(env):
    import torch

    plan, T, q, k, _, _ = env
    # K passed as V too: both only read
    o1, l1 = zz.ring_attention_fwd(plan, q, k, k)
    o2, l2 = zz.ring_attention_fwd(plan, q, k, k.clone())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_backward_rejects_overlapping_accumulators(env):
    import torch

    plan, T, q, k, v, do = env
    L = zz.lib()
    lse = torch.zeros((HQ, T), device="cuda")
    delta = torch.zeros((HQ, T), device="cuda")
    dq = torch.full((T, HQ, D), 3.0, device="cuda")
    dkv = torch.full((T, HKV, D), 3.0, device="cuda")
    dv = torch.full((T, HKV, D), 3.0, device="cuda")
    # dK and dV accumulators in one buffer
    rc = L.zz_varlen_ring_step_bwd(plan.handle, zz.ALL_RANKS, 0, _p(q), _p(k), _p(v), _p(do), _p(lse), _p(delta),
                                   _p(dq), _p(dkv), _p(dkv), 0, None)
    _rejected(rc, ("dk_acc", "dv_acc"))
    rc = L.zz_varlen_ring_step_bwd_dkv(plan.handle, zz.ALL_RANKS, 0, _p(q), _p(k), _p(v), _p(do), _p(lse),
                                       _p(delta), _p(dkv), _p(dkv, 256), 0, None)
    _rejected(rc, ("dk_acc", "dv_acc"))
    # dQ accumulator over the delta buffer
    rc = L.zz_varlen_ring_step_bwd_dq(plan.handle, zz.ALL_RANKS, 0, _p(q), _p(k), _p(v), _p(do), _p(lse),
                                      _p(delta), _p(delta), 0, None)
    _rejected(rc, ("dq_acc", "delta"))
    rc = L.zz_varlen_gathered_bwd(plan.handle, zz.ALL_RANKS, _p(q), _p(k), _p(v), _p(do), _p(lse), _p(delta),
                                  _p(dq), _p(dq, 1024), _p(dv), None)
    _rejected(rc, ("dq", "dk"))
    torch.cuda.synchronize()
    assert bool((dq == 3.0).all()) and bool((dkv == 3.0).all()) and bool((dv == 3.0).all())


def test_finalize_permute_and_merge_reject_overlap(env):
    import torch

    plan, T, q, _, _, _ = env
    L = zz.lib()
    acc = torch.full((T, HQ, D), 2.0, device="cuda")
    kv_acc = torch.full((T, HKV, D), 2.0, device="cuda")
    out_q = torch.zeros((T, HQ, D), dtype=torch.bfloat16, device="cuda")
    out_kv = torch.zeros((T, HKV, D), dtype=torch.bfloat16, device="cuda")
    # in-place cast: the bf16 output inside the fp32 accumulator
    _rejected(L.zz_finalize_fwd(plan.handle, _p(acc), _p(acc, 64), 0, None), ("o_out", "o_acc"))
    _rejected(L.zz_finalize_bwd(plan.handle, _p(acc), _p(kv_acc), _p(kv_acc), _p(out_q), _p(out_kv), _p(out_kv),
                                0, None), ("dk_out", "dv_out"))
    row_bytes = HQ * D * 2
    _rejected(L.zz_zigzag_permute(plan.handle, _p(q), _p(q, row_bytes), row_bytes, None), ("x_zz", "x_packed"))
    lse = torch.zeros((HQ, T), device="cuda")
    _rejected(L.zz_lse_merge(_p(acc), _p(lse), _p(acc, 1024), _p(lse), T, HQ, D, None), ("o_acc", "o_part"))
    torch.cuda.synchronize()
    assert bool((acc == 2.0).all()) and bool((out_q == 0).all()) and bool((out_kv == 0).all())
