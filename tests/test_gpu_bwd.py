"""GPU parity of the backward ring steps against the CPU oracle."""
import numpy as np
import pytest

import oracle
import synthetic
from zz_testlib import TOL, Case, check_grad, max_abs, to_np

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")


def gpu_backward(case):
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    o_zz = zz.finalize_fwd(case.plan, o_acc, unpermute=False)
    dq, dk, dv = zz.ring_attention_bwd(case.plan, case.qz, case.kz, case.vz, o_zz, case.doz, lse)
    # back to packed order (fp32)
    return [to_np(x)[case.dst] for x in (dq, dk, dv)]


def check_grads(case, tol, q_scale=1.0):
    got = gpu_backward(case)
    want = oracle.attn_bwd(case.q, case.k, case.v, case.do, case.cu, case.scale)
    tag = "%s cp=%d hq=%d hkv=%d d=%d q_scale=%g" % (case.lengths, case.cp, case.hq, case.hkv, case.d, q_scale)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        check_grad(name, g, w, tol, q_scale, tag)


@pytest.mark.parametrize("lengths,cp,hq,hkv,d", [
    ((96, 64, 96), 2, 2, 2, 32),
    ((8, 24, 16), 4, 4, 2, 64),
    ((40, 24), 1, 2, 1, 32),
    ((200, 56), 2, 4, 2, 32),
    ((64, 192), 2, 2, 1, 128),       # fp32 head_dim 128: 32-row dK/dV query tiles, 32-key dQ tiles
    ((36, 12, 60, 96), 3, 4, 2, 64),  # CP not a power of two
    ((64, 128, 320), 32, 2, 1, 32),   # CP 32
])
def test_backward_fp32(lengths, cp, hq, hkv, d):
    case = Case(lengths, cp, hq, hkv, d, "f32", 21, with_do=True)
    check_grads(case, TOL["f32"])


@pytest.mark.parametrize("lengths,cp,hq,hkv,d,q_scale", [
    ((128, 256, 64), 2, 4, 2, 128, 1.0),
    ((16, 48, 528, 8), 4, 8, 1, 128, 1.0),
    ((512,), 4, 8, 1, 128, 4.0),
    ((96, 160, 8), 2, 4, 2, 64, 1.0),    # head_dim 64
    ((40, 24, 200), 2, 2, 2, 32, 2.0),   # head_dim 32, MHA
    ((36, 12, 60, 96), 3, 8, 2, 128, 1.0),  # CP not a power of two, GQA 4:1
    ((72, 24), 1, 4, 1, 64, 2.0),        # one rank (only the diagonal step), GQA 4:1
])
def test_backward_bf16(lengths, cp, hq, hkv, d, q_scale):
    case = Case(lengths, cp, hq, hkv, d, "bf16", 23, with_do=True, q_scale=q_scale)
    check_grads(case, TOL["bf16"], q_scale)


def test_backward_c2_full():
    """The c2 packing (8192 tokens in 5 documents, 16/16 heads, head_dim 128,
    CP 4; dO drawn after Q, K, V): every element of dQ, dK and dV against
    the oracle's backward, at the flat gate."""
    w = synthetic.WORKLOADS["c2"]
    case = Case(tuple(synthetic.lengths_for(w)), w.cp, w.hq, w.hkv, w.d, w.dtype, w.seed, with_do=True)
    check_grads(case, TOL["bf16"])


def test_backward_with_dq_on_a_second_stream_is_bitwise_equal():
    import torch
    case = Case((64, 320, 128, 96), 4, 4, 2, 128, "bf16", 7, with_do=True)
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    o_zz = zz.finalize_fwd(case.plan, o_acc)
    one = zz.ring_attention_bwd(case.plan, case.qz, case.kz, case.vz, o_zz, case.doz, lse)
    side = torch.cuda.Stream()
    for _ in range(2):   # the second call reuses the side stream after the first finished
        two = zz.ring_attention_bwd(case.plan, case.qz, case.kz, case.vz, o_zz, case.doz, lse, dq_stream=side)
        torch.cuda.synchronize()
        for a, b in zip(one, two):
            assert torch.equal(a, b)


def test_backward_per_rank_equals_all_ranks():
    import torch
    case = Case((128, 256, 64), 2, 4, 2, 128, "bf16", 3, with_do=True)
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    o_zz = zz.finalize_fwd(case.plan, o_acc)
    delta = zz.bwd_preprocess(case.plan, o_zz, case.doz)
    outs = []
    for mode in ("all", "per_rank", "split"):
        dq = torch.zeros((case.T, case.hq, case.d), device="cuda")
        dk = torch.zeros((case.T, case.hkv, case.d), device="cuda")
        dv = torch.zeros_like(dk)
        for s in range(case.cp):
            ranks = range(case.cp) if mode == "per_rank" else [zz.ALL_RANKS]
            for r in ranks:
                if mode == "split":   # the two kernels of a step through their own entry points
                    zz.varlen_ring_step_bwd_dq(case.plan, r, s, case.qz, case.kz, case.vz, case.doz, lse,
                                               delta, dq, accumulate=True)
                    zz.varlen_ring_step_bwd_dkv(case.plan, r, s, case.qz, case.kz, case.vz, case.doz, lse,
                                                delta, dk, dv, accumulate=True)
                else:
                    zz.varlen_ring_step_bwd(case.plan, r, s, case.qz, case.kz, case.vz, case.doz, lse, delta,
                                            dq, dk, dv, accumulate=True)
        outs.append((dq, dk, dv))
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a, b)
    # overwrite on step 0 (it touches every row) equals zero-fill + accumulate
    dq2, dk2, dv2 = zz.ring_attention_bwd(case.plan, case.qz, case.kz, case.vz, o_zz, case.doz, lse)
    for a, b in zip(outs[0], (dq2, dk2, dv2)):
        assert torch.equal(a, b)


def test_bwd_preprocess_is_rowsum():
    import torch
    case = Case((64, 192), 2, 4, 2, 128, "bf16", 8, with_do=True)
    o = synthetic.randn_qkv(99, case.T, case.hq, case.hkv, case.d, "bf16")[0].cuda()
    delta = zz.bwd_preprocess(case.plan, o, case.doz)
    want = (o.double() * case.doz.double()).sum(-1).T.contiguous()
    assert max_abs(to_np(delta), want.cpu().numpy()) < 1e-4


def test_finalize_bwd_casts_and_unpermutes():
    import torch
    case = Case((64, 192), 2, 4, 2, 128, "bf16", 8)
    g = torch.Generator(device="cuda").manual_seed(0)
    dq = torch.randn((case.T, case.hq, case.d), device="cuda", generator=g)
    dk = torch.randn((case.T, case.hkv, case.d), device="cuda", generator=g)
    dv = torch.randn((case.T, case.hkv, case.d), device="cuda", generator=g)
    a, b, c = zz.finalize_bwd(case.plan, dq, dk, dv, unpermute=True)
    for x, y in ((a, dq), (b, dk), (c, dv)):
        assert torch.equal(x, zz.zigzag_unpermute(case.plan, y.to(torch.bfloat16)))
