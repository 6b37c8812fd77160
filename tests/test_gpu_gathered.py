"""GPU parity of the gathered forward (every rank's queries against all K/V
shards in one launch, no step partials or merges) against the CPU oracle,
through the C ABI."""
import numpy as np
import pytest

import oracle
import synthetic
from zz_testlib import TOL, Case, check_grad, max_abs, rel_l2, to_np

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")


def check_against_oracle(case, o, lse, tol):
    want_o, want_lse = oracle.attn_fwd(case.q, case.k, case.v, case.cu, case.scale)
    got_o = to_np(o)[case.dst]
    got_lse = to_np(lse)[:, case.dst]
    assert max_abs(got_o, want_o) < tol["abs"], max_abs(got_o, want_o)
    assert rel_l2(got_o, want_o) < tol["rel"], rel_l2(got_o, want_o)
    assert max_abs(got_lse, want_lse) < tol["lse"], max_abs(got_lse, want_lse)


@pytest.mark.parametrize("lengths,cp,hq,hkv,d,dtype,bm,bn", [
    ((96, 64, 96), 2, 2, 2, 32, "f32", 128, 64),
    ((96, 64, 96), 2, 2, 2, 32, "f32", 16, 8),
    ((8, 24, 16), 4, 4, 2, 64, "f32", 4, 3),
    ((128, 256, 64), 2, 4, 2, 128, "bf16", 128, 64),
    ((16, 48, 528, 8), 4, 8, 1, 128, "bf16", 128, 64),
    (tuple(synthetic.lengths_for(synthetic.WORKLOADS["c2"])), 4, 16, 16, 128, "bf16", 128, 64),
])
def test_gathered_forward_matches_oracle(lengths, cp, hq, hkv, d, dtype, bm, bn):
    case = Case(lengths, cp, hq, hkv, d, dtype, 31, bm=bm, bn=bn)
    o, lse = zz.gathered_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    check_against_oracle(case, o, lse, TOL[dtype])


def test_gathered_forward_per_rank_equals_all_ranks():
    import torch
    case = Case((16, 48, 528, 8), 4, 8, 1, 128, "bf16", 5)
    o_all, lse_all = zz.gathered_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    o = torch.full_like(o_all, 3.0)
    lse = torch.full_like(lse_all, 3.0)
    for r in range(case.cp):
        zz.varlen_gathered_fwd(case.plan, r, case.qz, case.kz, case.vz, o, lse)
    assert torch.equal(o, o_all) and torch.equal(lse, lse_all)


def test_gathered_forward_sharp_softmax():
    """Q x 4: sharp softmax rows exercise the running-maximum moves."""
    case = Case((512,), 4, 8, 1, 128, "bf16", 7, q_scale=4.0)
    o, lse = zz.gathered_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    check_against_oracle(case, o, lse, TOL["bf16"])


def test_gathered_forward_c4_full_size():
    """c4 (65536 tokens, 15 documents, GQA 64/8, CP 8): sampled rows against
    the oracle, and every row against the merged ring forward (same tiles,
    other grouping: equal up to rounding order)."""
    import torch
    w = synthetic.WORKLOADS["c4"]
    cu = synthetic.cu_seqlens_for(w)
    q, k, v = synthetic.randn_qkv(w.seed, w.total, w.hq, w.hkv, w.d, w.dtype)
    plan = zz.Plan(cu, w.cp, w.hq, w.hkv, w.d, w.dtype, device="cuda")
    qz, kz, vz = (zz.zigzag_permute(plan, x.cuda()) for x in (q, k, v))
    o, lse = zz.gathered_attention_fwd(plan, qz, kz, vz)
    o_ring, lse_ring = zz.ring_attention_fwd(plan, qz, kz, vz)
    # P is rounded to bf16 against different running maxima in the two
    # groupings, so O agrees to the bf16 gate, LSE (fp32 sums) much closer.
    assert float((o - o_ring).abs().max()) < TOL["bf16"]["abs"]
    assert rel_l2(to_np(o), to_np(o_ring)) < TOL["bf16"]["rel"]
    assert float((lse - lse_ring).abs().max()) < 1e-4
    rng = np.random.default_rng(41)
    rows = np.sort(rng.integers(0, w.total, size=512)).astype(np.int64)
    heads = rng.integers(0, w.hq, size=len(rows)).astype(np.int32)
    want_o, want_lse = oracle.attn_fwd_rows(q, k, v, cu, w.scale, rows, heads)
    dst = plan.zigzag_dst()
    zr, hd = torch.as_tensor(dst[rows], device="cuda"), torch.as_tensor(heads, device="cuda", dtype=torch.int64)
    got_o = o[zr, hd].cpu().numpy()
    got_lse = lse[hd, zr].cpu().numpy()
    assert max_abs(got_o, want_o) < TOL["bf16"]["abs"]
    assert rel_l2(got_o, want_o) < TOL["bf16"]["rel"]
    assert max_abs(got_lse, want_lse) < TOL["bf16"]["lse"]


# ------------------------------------------------------------------ backward

def gathered_grads(case):
    o, lse = zz.gathered_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    o_zz = zz.finalize_fwd(case.plan, o)
    dq, dk, dv = zz.gathered_attention_bwd(case.plan, case.qz, case.kz, case.vz, o_zz, case.doz, lse)
    return [to_np(x)[case.dst] for x in (dq, dk, dv)]


@pytest.mark.parametrize("lengths,cp,hq,hkv,d,dtype", [
    ((96, 64, 96), 2, 2, 2, 32, "f32"),
    ((8, 24, 16), 4, 4, 2, 64, "f32"),
    ((200, 56), 2, 4, 2, 32, "f32"),
    ((128, 256, 64), 2, 4, 2, 128, "bf16"),
    ((16, 48, 528, 8), 4, 8, 1, 128, "bf16"),
    ((96, 160, 8), 2, 4, 2, 64, "bf16"),
])
def test_gathered_backward_matches_oracle(lengths, cp, hq, hkv, d, dtype):
    case = Case(lengths, cp, hq, hkv, d, dtype, 37, with_do=True)
    got = gathered_grads(case)
    want = oracle.attn_bwd(case.q, case.k, case.v, case.do, case.cu, case.scale)
    tag = "gathered %s cp=%d hq=%d hkv=%d d=%d %s" % (lengths, cp, hq, hkv, d, dtype)
    for name, g, w in zip(("dq", "dk", "dv"), got, want):
        check_grad(name, g, w, TOL[dtype], 1.0, tag)


def test_gathered_backward_per_rank_equals_all_ranks():
    import torch
    case = Case((16, 48, 528, 8), 4, 8, 1, 128, "bf16", 9, with_do=True)
    o, lse = zz.gathered_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    o_zz = zz.finalize_fwd(case.plan, o)
    delta = zz.bwd_preprocess(case.plan, o_zz, case.doz)
    outs = []
    for ranks in ([zz.ALL_RANKS], list(range(case.cp))):
        dq = torch.full((case.T, case.hq, case.d), 5.0, device="cuda")
        dk = torch.full((case.T, case.hkv, case.d), 5.0, device="cuda")
        dv = torch.full_like(dk, 5.0)
        for r in ranks:
            zz.varlen_gathered_bwd(case.plan, r, case.qz, case.kz, case.vz, case.doz, lse, delta, dq, dk, dv)
        outs.append((dq, dk, dv))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_gathered_backward_c4_full_size_equals_ring():
    """c4 at full size: the gathered backward against the sum of the ring
    steps (same tiles grouped per item instead of per step)."""
    import torch
    w = synthetic.WORKLOADS["c4"]
    cu = synthetic.cu_seqlens_for(w)
    q, k, v, do = synthetic.randn_qkv(w.seed, w.total, w.hq, w.hkv, w.d, w.dtype, with_do=True)
    plan = zz.Plan(cu, w.cp, w.hq, w.hkv, w.d, w.dtype, device="cuda")
    qz, kz, vz, doz = (zz.zigzag_permute(plan, x.cuda()) for x in (q, k, v, do))
    o_acc, lse = zz.ring_attention_fwd(plan, qz, kz, vz)
    o_zz = zz.finalize_fwd(plan, o_acc)
    ring = zz.ring_attention_bwd(plan, qz, kz, vz, o_zz, doz, lse)
    gath = zz.gathered_attention_bwd(plan, qz, kz, vz, o_zz, doz, lse)
    for name, a, b in zip(("dq", "dk", "dv"), gath, ring):
        scale = max(1.0, float(b.abs().max()))
        # both sum the same fp32 tile products, in a different order
        assert float((a - b).abs().max()) < 1e-3 * scale, name
        assert rel_l2(to_np(a), to_np(b)) < 1e-4, name
