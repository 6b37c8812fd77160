"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (all simulated ranks of a step in one launch, step 0 writing, later
steps merging in the kernel epilogue).

At these sizes the oracle checks sampled outputs it can compute one by one
(O, LSE and dQ rows), and properties that hold at any size check the rest:
closed forms on special inputs and exact gradient identities."""
import math

import numpy as np
import pytest

import oracle
import synthetic
from zz_testlib import TOL, max_abs, rel_l2, to_np

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")

TOL_BF16 = TOL["bf16"]


def setup(name, zero_q=False, zero_k=False, with_do=False):
    import torch
    w = synthetic.WORKLOADS[name]
    cu = synthetic.cu_seqlens_for(w)
    T = w.total
    q, k, v, *rest = synthetic.randn_qkv(w.seed, T, w.hq, w.hkv, w.d, w.dtype, with_do=with_do)
    if zero_q:
        q = torch.zeros_like(q)
    if zero_k:
        k = torch.zeros_like(k)
    plan = zz.Plan(cu, w.cp, w.hq, w.hkv, w.d, w.dtype, device="cuda")
    qz, kz, vz = (zz.zigzag_permute(plan, x.cuda()) for x in (q, k, v))
    doz = zz.zigzag_permute(plan, rest[0].cuda()) if with_do else None
    return w, cu, plan, (q, k, v, rest[0] if with_do else None), (qz, kz, vz, doz)


def sample_rows(cu, cp, n_random, hq, seed):
    """Rows at every zigzag chunk edge of every sequence, plus random rows,
    each with a random head."""
    rng = np.random.default_rng(seed)
    rows = set()
    for i in range(len(cu) - 1):
        L = int(cu[i + 1] - cu[i])
        c = L // (2 * cp)
        for x in range(2 * cp):
            rows.add(int(cu[i]) + x * c)
            rows.add(int(cu[i]) + x * c + c - 1)
    rows.update(int(r) for r in rng.integers(0, int(cu[-1]), size=n_random))
    rows = np.array(sorted(rows), dtype=np.int64)
    heads = rng.integers(0, hq, size=len(rows)).astype(np.int32)
    return rows, heads


def forward(plan, qz, kz, vz):
    o_acc, lse = zz.ring_attention_fwd(plan, qz, kz, vz)
    out = zz.finalize_fwd(plan, o_acc, unpermute=True)
    return o_acc, lse, out


@pytest.mark.parametrize("name,n_random", [("c3", 1024), ("c4", 768), ("c5", 384)])
def test_forward_sampled_rows_full_size(name, n_random):
    w, cu, plan, (q, k, v, _), (qz, kz, vz, _) = setup(name)
    o_acc, lse, out = forward(plan, qz, kz, vz)
    rows, heads = sample_rows(cu, w.cp, n_random, w.hq, w.seed)
    ow, lw = oracle.attn_fwd_rows(q, k, v, cu, w.scale, rows, heads)
    dst = plan.zigzag_dst()
    zrows = dst[rows]
    og = o_acc[zrows, heads].float().cpu().numpy()
    lg = lse[heads, zrows].float().cpu().numpy()
    fo = out[rows, heads].float().cpu().numpy()
    assert max_abs(og, ow) < TOL_BF16["abs"]
    assert rel_l2(og, ow) < TOL_BF16["rel"]
    assert max_abs(lg, lw) < TOL_BF16["lse"]
    assert max_abs(fo, ow) < TOL_BF16["abs"]


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_forward_zero_query_closed_form_full_size(name):
    """Q = 0: O is the running mean of V within each sequence and LSE is the
    log of the number of visible keys, at every row of every head."""
    import torch
    w, cu, plan, (q, k, v, _), (qz, kz, vz, _) = setup(name, zero_q=True)
    o_acc, lse, _ = forward(plan, qz, kz, vz)
    dst = torch.as_tensor(plan.zigzag_dst(), device="cuda")
    vd = v.cuda().double()
    G = w.hq // w.hkv
    worst_o = worst_l = 0.0
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        n = torch.arange(1, b - a + 1, device="cuda", dtype=torch.float64)
        mean = torch.cumsum(vd[a:b], dim=0) / n[:, None, None]            # [L,hkv,d]
        og = o_acc[dst[a:b]].double()                                       # [L,hq,d]
        worst_o = max(worst_o, float((og - mean.repeat_interleave(G, dim=1)).abs().max()))
        lg = lse[:, dst[a:b]].double()
        worst_l = max(worst_l, float((lg - torch.log(n)[None, :]).abs().max()))
    assert worst_o < 2e-3        # averages of bf16 values: rounding of the weights only
    assert worst_l < 1e-4


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_backward_sampled_dq_rows(name):
    """c4: 65536 tokens packed from 15 documents (document mask), GQA 64/8;
    c5: one 131072-token sequence, GQA 64/8."""
    w, cu, plan, (q, k, v, do), (qz, kz, vz, doz) = setup(name, with_do=True)
    o_acc, lse, _ = forward(plan, qz, kz, vz)
    o_zz = zz.finalize_fwd(plan, o_acc)
    dq, dk, dv = zz.ring_attention_bwd(plan, qz, kz, vz, o_zz, doz, lse)
    rows, heads = sample_rows(cu, w.cp, 192, w.hq, 55)
    want = oracle.attn_bwd_dq_rows(q, k, v, do, cu, w.scale, rows, heads)
    dst = plan.zigzag_dst()
    got = dq[dst[rows], heads].float().cpu().numpy()
    gate = TOL_BF16["abs"] * max(1.0, float(np.abs(want).max()))
    assert max_abs(got, want) < gate
    assert rel_l2(got, want) < TOL_BF16["rel"]


@pytest.mark.parametrize("name", ["c4", "c5"])
def test_backward_gradient_identities(name):
    """Exact identities of the attention gradient, per key/value group (they
    hold per document, hence also summed over a packed batch):
    sum_k dK_k = 0;  sum_k dV_k = sum over the group's heads of sum_q dO_q;
    sum over heads of <Q, dQ> = <K, dK>."""
    import torch
    w, cu, plan, (q, k, v, do), (qz, kz, vz, doz) = setup(name, with_do=True)
    o_acc, lse, _ = forward(plan, qz, kz, vz)
    o_zz = zz.finalize_fwd(plan, o_acc)
    dq, dk, dv = zz.ring_attention_bwd(plan, qz, kz, vz, o_zz, doz, lse)
    G = w.hq // w.hkv
    dkd, dvd, dqd = dk.double(), dv.double(), dq.double()
    sum_dk = dkd.sum(0)                                      # [hkv,d]
    assert float(sum_dk.abs().max()) < 1e-3 * float(dkd.abs().sum(0).max())
    sum_do = doz.double().sum(0).view(w.hkv, G, w.d).sum(1)  # [hkv,d]
    assert float((dvd.sum(0) - sum_do).abs().max()) < 1e-3 * float(sum_do.abs().max() + 1.0)
    qdq = (qz.double() * dqd).sum(dim=(0, 2)).view(w.hkv, G).sum(1)
    kdk = (kz.double() * dkd).sum(dim=(0, 2))
    # Both sides are sums of about 1e9 products that cancel to ~1e2; dQ and dK
    # are formed by different kernels from independently rounded bf16 dS, so
    # the identity holds to rounding noise, not to fp32 accuracy.
    assert float((qdq - kdk).abs().max()) < 1e-2 * float(kdk.abs().max() + 1.0)


def test_backward_c5_zero_key_closed_form():
    """K = 0: every visible key has weight 1/n, so dQ = 0 exactly and
    dV_k = sum over later rows q and the group's heads of dO_q / n_q."""
    import torch
    w, cu, plan, (q, k, v, do), (qz, kz, vz, doz) = setup("c5", zero_k=True, with_do=True)
    o_acc, lse, _ = forward(plan, qz, kz, vz)
    o_zz = zz.finalize_fwd(plan, o_acc)
    dq, dk, dv = zz.ring_attention_bwd(plan, qz, kz, vz, o_zz, doz, lse)
    assert float(dq.abs().max()) == 0.0
    G = w.hq // w.hkv
    T = w.total
    n = torch.arange(1, T + 1, device="cuda", dtype=torch.float64)
    contrib = do.cuda().double().view(T, w.hkv, G, w.d).sum(2) / n[:, None, None]
    want = torch.flip(torch.cumsum(torch.flip(contrib, [0]), 0), [0])      # packed order
    dst = torch.as_tensor(plan.zigzag_dst(), device="cuda")
    got = dv[dst].double()
    err = float((got - want).abs().max())
    assert err < 2e-3 * max(1.0, float(want.abs().max()))


def test_backward_c4_one_head_full():
    """Document-masked backward at full size (65536 tokens, 15 documents):
    with dO zero for every query head but one, that head's dQ and its
    group's dK, dV are the one-head gradients, compared in full against the
    oracle's backward of that head alone."""
    import torch
    w, cu, plan, (q, k, v, do), (qz, kz, vz, doz) = setup("c4", with_do=True)
    G = w.hq // w.hkv
    h = w.hq - 3
    g = h // G
    keep = torch.zeros((1, w.hq, 1), dtype=doz.dtype, device=doz.device)
    keep[0, h, 0] = 1
    doz = doz * keep
    do_h = do[:, h:h + 1]
    o_acc, lse, _ = forward(plan, qz, kz, vz)
    o_zz = zz.finalize_fwd(plan, o_acc)
    dq, dk, dv = zz.ring_attention_bwd(plan, qz, kz, vz, o_zz, doz, lse)
    want = oracle.attn_bwd(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], do_h, cu, w.scale)
    dst = torch.as_tensor(plan.zigzag_dst(), device="cuda")
    got = (dq[dst][:, h], dk[dst][:, g], dv[dst][:, g])
    for nm, gt, wt in zip(("dq", "dk", "dv"), got, want):
        gt = gt.float().cpu().numpy()
        wt = wt[:, 0]
        gate = TOL_BF16["abs"] * max(1.0, float(np.abs(wt).max()))
        assert max_abs(gt, wt) < gate, (nm, max_abs(gt, wt), gate)
        assert rel_l2(gt, wt) < TOL_BF16["rel"], (nm, rel_l2(gt, wt))
    # the other query heads of the group contribute nothing, the other
    # groups nothing at all
    others = [x for x in range(w.hkv) if x != g]
    assert float(dk[:, others].abs().max()) == 0.0 and float(dv[:, others].abs().max()) == 0.0


def test_debug_mask_c3_sampled_steps():
    w = synthetic.WORKLOADS["c3"]
    cu = synthetic.cu_seqlens_for(w)
    plan = zz.Plan(cu, w.cp, 2, 1, 128, "bf16", device="cuda")
    for r, s in [(0, 0), (3, 1), (7, 7), (5, 6)]:
        want = oracle.step_mask(cu, w.cp, r, s)
        for pass_ in (zz.PASS_FWD, zz.PASS_BWD_DQ, zz.PASS_BWD_DKV):
            got = zz.debug_mask(plan, pass_, r, s).cpu().numpy()
            assert np.array_equal(got, want), (pass_, r, s)
