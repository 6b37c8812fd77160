"""GPU parity of the forward path (zigzag permute, ring steps, merge,
finalize) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
import synthetic
from zz_testlib import TOL, Case, max_abs, rel_l2, to_np

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")


def oracle_packed_fwd(case):
    return oracle.attn_fwd(case.q, case.k, case.v, case.cu, case.scale)


# ------------------------------------------------------------------ permutation

@pytest.mark.parametrize("lengths,cp,h,d,dtype", [
    ((96, 64, 96), 2, 2, 32, "f32"),
    ((8, 24, 16), 4, 3, 64, "bf16"),
    (tuple(synthetic.lengths_for(synthetic.WORKLOADS["c2"])), 4, 16, 128, "bf16"),
    ((2, 2, 4), 1, 1, 32, "f32"),
    # wide rows (16-byte vectors per row 640, 1024, 768): the permute's
    # eight-deep loop with and without a tail
    ((64, 192, 128), 4, 40, 128, "bf16"),
    ((96, 32), 2, 64, 128, "bf16"),
    ((48, 16), 2, 24, 128, "f32"),
])
def test_permute_unpermute_bit_exact(lengths, cp, h, d, dtype):
    import torch
    cu = synthetic.make_cu_seqlens(lengths)
    T = int(cu[-1])
    plan = zz.Plan(cu, cp, h, h, d, dtype, device="cuda")
    x = synthetic.randn_qkv(3, T, h, h, d, dtype)[0]
    xz = zz.zigzag_permute(plan, x.cuda())
    want = oracle.permute(x.view(torch.int16 if dtype == "bf16" else torch.int32).numpy(), cu, cp)
    got = xz.cpu().view(torch.int16 if dtype == "bf16" else torch.int32).numpy()
    assert np.array_equal(got, want)
    back = zz.zigzag_unpermute(plan, xz)
    assert torch.equal(back.cpu(), x)


@pytest.mark.parametrize("hq,dtype", [(4, "bf16"), (40, "bf16"), (64, "bf16"), (24, "f32")])
def test_finalize_fwd_casts_and_unpermutes_bit_exact(hq, dtype):
    """fp32 rows -> plan dtype by round-to-nearest-even (torch's cast), in
    zigzag or packed order; hq 40/64 at head_dim 128 make rows of 1280/2048
    four-float vectors (the cast kernel's unrolled loop and its tail)."""
    import torch
    cu = synthetic.make_cu_seqlens((64, 192, 128))
    plan = zz.Plan(cu, 4, hq, 1, 128, dtype, device="cuda")
    o = torch.randn((plan.total, hq, 128), generator=torch.Generator().manual_seed(6)).cuda()
    want = o.to(plan.torch_dtype)
    assert torch.equal(zz.finalize_fwd(plan, o, unpermute=False), want)
    assert torch.equal(zz.finalize_fwd(plan, o, unpermute=True), zz.zigzag_unpermute(plan, want))


# ------------------------------------------------------------------ masks

@pytest.mark.parametrize("lengths,cp,bm,bn", [
    ((96, 64, 96), 2, 128, 64), ((96, 64, 96), 2, 16, 8), ((8, 24, 16), 4, 4, 3),
    ((6, 6, 12), 3, 1, 1), ((192, 64), 2, 128, 64),
])
def test_debug_mask_bit_exact_all_passes(lengths, cp, bm, bn):
    cu = synthetic.make_cu_seqlens(lengths)
    plan = zz.Plan(cu, cp, 2, 2, 32, "f32", bm, bn, device="cuda")
    for r in range(cp):
        for s in range(cp):
            want = oracle.step_mask(cu, cp, r, s)
            for pass_ in (zz.PASS_FWD, zz.PASS_BWD_DQ, zz.PASS_BWD_DKV):
                got = zz.debug_mask(plan, pass_, r, s).cpu().numpy()
                assert np.array_equal(got, want), (pass_, r, s)


def test_debug_mask_c2_bit_exact():
    w = synthetic.WORKLOADS["c2"]
    cu = synthetic.cu_seqlens_for(w)
    plan = zz.Plan(cu, w.cp, 2, 2, 128, "bf16", device="cuda")
    for r in range(w.cp):
        for s in range(w.cp):
            want = oracle.step_mask(cu, w.cp, r, s)
            got = zz.debug_mask(plan, zz.PASS_FWD, r, s).cpu().numpy()
            assert np.array_equal(got, want), (r, s)


# ------------------------------------------------------------------ ring steps

def check_step_partials(case, tol):
    import torch
    n = case.T // case.cp
    qz, kz, vz = (oracle.permute(x.float().numpy(), case.cu, case.cp) for x in (case.q, case.k, case.v))
    for r in range(case.cp):
        for s in range(case.cp):
            o = torch.full((case.T, case.hq, case.d), 7.0, device="cuda")
            lse = torch.full((case.hq, case.T), 7.0, device="cuda")
            zz.varlen_ring_step_fwd(case.plan, r, s, case.qz, case.kz, case.vz, o, lse, merge=False)
            ow = oracle.ring_step_fwd(qz, kz, vz, case.cu, case.cp, r, s, case.scale)
            og, lg = to_np(o)[r * n:(r + 1) * n], to_np(lse)[:, r * n:(r + 1) * n]
            empty = np.isinf(ow[1])
            assert np.array_equal(np.isinf(lg), empty), (r, s)
            assert np.all(og.transpose(1, 0, 2)[empty] == 0.0)
            assert max_abs(og, ow[0]) < tol["abs"], (r, s)
            assert max_abs(lg[~empty], ow[1][~empty]) < tol["lse"], (r, s)
            # other ranks' rows are untouched
            rest = np.ones(case.T, bool); rest[r * n:(r + 1) * n] = False
            assert np.all(to_np(o)[rest] == 7.0) and np.all(to_np(lse)[:, rest] == 7.0)


def test_step_partials_c1_fp32():
    w = synthetic.WORKLOADS["c1"]
    case = Case(synthetic.lengths_for(w), w.cp, w.hq, w.hkv, w.d, w.dtype, w.seed)
    check_step_partials(case, TOL["f32"])


@pytest.mark.parametrize("lengths,cp,hq,hkv,d,dtype,bm,bn", [
    ((8, 24, 16), 4, 4, 2, 64, "f32", 128, 64),
    ((8, 24, 16), 4, 4, 2, 64, "f32", 3, 5),
    ((96, 320, 64), 2, 4, 1, 128, "bf16", 128, 64),
    ((96, 320, 64), 2, 2, 2, 128, "bf16", 48, 40),
])
def test_step_partials_small(lengths, cp, hq, hkv, d, dtype, bm, bn):
    case = Case(lengths, cp, hq, hkv, d, dtype, 5, bm=bm, bn=bn)
    check_step_partials(case, TOL[dtype])


def run_forward(case, rank=zz.ALL_RANKS):
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz, rank=rank)
    out = zz.finalize_fwd(case.plan, o_acc, unpermute=True)
    return o_acc, lse, out


def check_full(case, o_acc, lse, out, tol):
    ow, lw = oracle_packed_fwd(case)
    n_o = to_np(o_acc)[case.dst]            # back to packed order
    n_l = to_np(lse)[:, case.dst]
    assert max_abs(n_o, ow) < tol["abs"]
    assert rel_l2(n_o, ow) < tol["rel"]
    assert max_abs(n_l, lw) < tol["lse"]
    fo = to_np(out)
    assert max_abs(fo, ow) < tol["abs"]
    assert rel_l2(fo, ow) < tol["rel"]


def test_forward_c1_fp32_full():
    w = synthetic.WORKLOADS["c1"]
    case = Case(synthetic.lengths_for(w), w.cp, w.hq, w.hkv, w.d, w.dtype, w.seed)
    check_full(case, *run_forward(case), TOL["f32"])


@pytest.mark.parametrize("lengths,cp,hq,hkv,d,dtype,q_scale", [
    ((128, 256, 64), 2, 4, 2, 128, "bf16", 1.0),
    ((128, 256, 64), 2, 4, 2, 128, "bf16", 8.0),       # sharp softmax: the rescale path
    ((16, 48, 528, 8), 4, 8, 1, 128, "bf16", 1.0),     # ragged tiles, GQA 8:1
    ((40, 24), 1, 2, 2, 64, "f32", 1.0),               # one rank
    ((40, 24), 2, 2, 2, 32, "bf16", 1.0),
    ((512,), 4, 2, 2, 64, "f32", 4.0),
    ((64, 192), 2, 2, 1, 128, "f32", 1.0),            # fp32 head_dim 128 (128 KB of LDS)
    ((200, 56), 2, 4, 4, 64, "bf16", 1.0),            # bf16 head_dim 64, MHA
    ((36, 12, 60, 96), 3, 4, 2, 64, "f32", 1.0),      # CP not a power of two
    ((96, 36, 150), 3, 4, 2, 128, "bf16", 1.0),
    ((96, 36, 150), 3, 8, 2, 128, "bf16", 2.0),       # GQA 4:1
    ((72, 24), 1, 4, 1, 64, "bf16", 1.0),             # one rank, GQA 4:1
    ((64, 128, 320), 32, 2, 1, 32, "f32", 1.0),       # CP 32: one- and two-row chunks, 1024 rank-steps
])
def test_forward_small_full(lengths, cp, hq, hkv, d, dtype, q_scale):
    case = Case(lengths, cp, hq, hkv, d, dtype, 9, q_scale=q_scale)
    check_full(case, *run_forward(case), TOL[dtype])


def test_forward_c2_full():
    w = synthetic.WORKLOADS["c2"]
    case = Case(synthetic.lengths_for(w), w.cp, w.hq, w.hkv, w.d, w.dtype, w.seed)
    check_full(case, *run_forward(case), TOL["bf16"])


def test_per_rank_launches_equal_all_ranks_launch():
    import torch
    case = Case((96, 320, 64), 2, 4, 2, 128, "bf16", 4)
    a_o, a_l, _ = run_forward(case)
    b_o, b_l, _ = run_forward(case, rank=0)
    c_o, c_l = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz, rank=1, o_acc=b_o, lse=b_l)
    assert torch.equal(a_o, c_o) and torch.equal(a_l, c_l)


def test_fused_merge_equals_partial_then_lse_merge_bitwise():
    import torch
    case = Case((96, 320, 64), 2, 4, 2, 128, "bf16", 6)
    n = case.T
    o1 = torch.empty((n, case.hq, case.d), device="cuda")
    l1 = torch.empty((case.hq, n), device="cuda")
    zz.varlen_ring_step_fwd(case.plan, zz.ALL_RANKS, 0, case.qz, case.kz, case.vz, o1, l1, merge=False)
    o2, l2 = o1.clone(), l1.clone()
    # fused: step 1 merged in place
    zz.varlen_ring_step_fwd(case.plan, zz.ALL_RANKS, 1, case.qz, case.kz, case.vz, o1, l1, merge=True)
    # unfused: step 1 partial, then the standalone merge
    op = torch.empty_like(o2)
    lp = torch.empty_like(l2)
    zz.varlen_ring_step_fwd(case.plan, zz.ALL_RANKS, 1, case.qz, case.kz, case.vz, op, lp, merge=False)
    zz.lse_merge(o2, l2, op, lp)
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


def test_lse_merge_matches_oracle():
    import torch
    g = torch.Generator().manual_seed(1)
    rows, heads, d = 257, 3, 64
    oa = torch.randn(rows, heads, d, generator=g)
    ob = torch.randn(rows, heads, d, generator=g)
    la = torch.randn(heads, rows, generator=g) * 3
    lb = torch.randn(heads, rows, generator=g) * 3
    la[0, :10] = float("-inf"); oa[:10, 0] = 0
    lb[1, 5:20] = float("-inf"); ob[5:20, 1] = 0
    la[2, 30:40] = float("-inf"); lb[2, 30:40] = float("-inf"); oa[30:40, 2] = 0; ob[30:40, 2] = 0
    wo, wl = oracle.lse_merge(oa.double().numpy(), la.double().numpy(), ob.double().numpy(), lb.double().numpy())
    go, gl = oa.cuda(), la.cuda()
    zz.lse_merge(go, gl, ob.cuda(), lb.cuda())
    gl_np = to_np(gl)
    assert np.array_equal(np.isinf(gl_np), np.isinf(wl))
    fin = ~np.isinf(wl)
    assert max_abs(gl_np[fin], wl[fin]) < 2e-6
    assert max_abs(to_np(go), wo) < 2e-6


def test_finalize_rounds_like_torch():
    import torch
    case = Case((96, 320, 64), 2, 4, 2, 128, "bf16", 2)
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    zig = zz.finalize_fwd(case.plan, o_acc, unpermute=False)
    assert torch.equal(zig, o_acc.to(torch.bfloat16))
    packed = zz.finalize_fwd(case.plan, o_acc, unpermute=True)
    assert torch.equal(packed, zz.zigzag_unpermute(case.plan, zig))


def test_unreordered_tokens_fail_parity():
    """MaxText PR #1133: load-balanced CP attention needs the tokens reordered;
    feeding the packed order straight in must give wrong results."""
    case = Case((128, 256, 64), 2, 4, 2, 128, "bf16", 9)
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qg, case.kg, case.vg)   # not permuted
    out = to_np(zz.finalize_fwd(case.plan, o_acc, unpermute=False))
    ow, _ = oracle_packed_fwd(case)
    assert max_abs(out, ow) > 10 * TOL["bf16"]["abs"]


def test_constant_value_gives_constant_output():
    case = Case((16, 48, 528, 8), 4, 8, 2, 128, "bf16", 1, const_v=0.625)
    o_acc, lse = zz.ring_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    # weights enter P.V rounded to bf16 while the row sum is fp32: a relative
    # error of at most about 2^-9 on short rows
    assert max_abs(to_np(o_acc), 0.625) < 0.625 * 2.0 ** -8
