"""GPU parity at the full workload sizes, in the launch configuration bench.py
times (all simulated ranks of a step in one launch, step 0 writing, later
steps merging in the kernel epilogue).

At these sizes the oracle checks outputs it can compute one by one: sampled
O / LSE rows (at least 4096 (row, head) pairs, every zigzag chunk's first and
last row among them) and one whole query head of the forward, sampled dQ rows,
and sampled dK / dV key rows.  Properties that hold at any size check the
rest: closed forms on special inputs and exact gradient identities.  Every
gate on N(0,1) inputs is the flat one (max-abs 2e-2, bf16)."""
import functools

import numpy as np
import pytest

import oracle
import synthetic
from zz_testlib import TOL, check_grad, max_abs, progress, rel_l2, to_np

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")

TOL_BF16 = TOL["bf16"]


class Setup:
    """One workload's seeded inputs: fp32 numpy copies for the oracle (exact
    upcasts of the bf16 values) and zigzag-layout device tensors."""

    def __init__(self, name, zero_q=False, zero_k=False, with_do=False):
        import torch
        w = synthetic.WORKLOADS[name]
        self.w = w
        self.cu = synthetic.cu_seqlens_for(w)
        t = synthetic.randn_qkv(w.seed, w.total, w.hq, w.hkv, w.d, w.dtype, with_do=with_do)
        q, k, v = t[0], t[1], t[2]
        if zero_q:
            q = torch.zeros_like(q)
        if zero_k:
            k = torch.zeros_like(k)
        self.plan = zz.Plan(self.cu, w.cp, w.hq, w.hkv, w.d, w.dtype, device="cuda")
        self.qz, self.kz, self.vz = (zz.zigzag_permute(self.plan, x.cuda()) for x in (q, k, v))
        self.doz = zz.zigzag_permute(self.plan, t[3].cuda()) if with_do else None
        self.q, self.k, self.v = (x.float().numpy() for x in (q, k, v))
        self.do = t[3].float().numpy() if with_do else None
        self.dst = self.plan.zigzag_dst()

    def forward(self):
        o_acc, lse = zz.ring_attention_fwd(self.plan, self.qz, self.kz, self.vz)
        out = zz.finalize_fwd(self.plan, o_acc, unpermute=True)
        return o_acc, lse, out

    def backward(self, doz=None):
        o_acc, lse, _ = self.forward()
        o_zz = zz.finalize_fwd(self.plan, o_acc)
        return zz.ring_attention_bwd(self.plan, self.qz, self.kz, self.vz, o_zz,
                                     self.doz if doz is None else doz, lse)


@functools.lru_cache(maxsize=8)
def setup(name, zero_q=False, zero_k=False, with_do=False):
    return Setup(name, zero_q, zero_k, with_do)


@pytest.fixture(scope="module", autouse=True)
def _release_inputs():
    yield
    head_reference.cache_clear()
    setup.cache_clear()


@functools.lru_cache(maxsize=16)
def head_reference(name, head):
    """The oracle's forward of every row of one query head: o [T, d] float64,
    lse [T].  Computed in row chunks of equal work, printing progress, since
    at c5 it is 4.4 TFLOP of CPU work."""
    s = setup(name, with_do=name != "c3")
    T = s.w.total
    cost = np.empty(T, dtype=np.float64)
    for i in range(len(s.cu) - 1):
        a, b = int(s.cu[i]), int(s.cu[i + 1])
        cost[a:b] = np.arange(1, b - a + 1)
    cum = np.cumsum(cost)
    nchunk = 24
    edges = np.searchsorted(cum, cum[-1] * np.arange(1, nchunk) / nchunk)
    bounds = [0] + [int(e) for e in edges] + [T]
    o = np.empty((T, s.w.d), dtype=np.float64)
    lse = np.empty(T, dtype=np.float64)
    for c in range(nchunk):
        a, b = bounds[c], bounds[c + 1]
        if b <= a:
            continue
        rows = np.arange(a, b, dtype=np.int64)
        o[a:b], lse[a:b] = oracle.attn_fwd_rows(s.q, s.k, s.v, s.cu, s.w.scale, rows,
                                                np.full(b - a, head, dtype=np.int32))
        progress("oracle %s head %d: rows %d..%d done (%d/%d)" % (name, head, a, b, c + 1, nchunk))
    return o, lse


def row_stats(name, heads, do):
    """LSE and D = <dO, O> tables [hq, T] (packed rows) for the given heads,
    from the oracle's own forward of each head; other heads' entries are NaN."""
    s = setup(name, with_do=True)
    lse = np.full((s.w.hq, s.w.total), np.nan)
    dsum = np.full((s.w.hq, s.w.total), np.nan)
    for h in heads:
        o, l = head_reference(name, h)
        lse[h] = l
        dsum[h] = (o * do[:, h].astype(np.float64)).sum(-1)
    return lse, dsum


def chunk_edges(cu, cp):
    """First and last row of every zigzag chunk of every sequence (packed rows)."""
    rows = set()
    for i in range(len(cu) - 1):
        c = int(cu[i + 1] - cu[i]) // (2 * cp)
        for x in range(2 * cp):
            rows.add(int(cu[i]) + x * c)
            rows.add(int(cu[i]) + x * c + c - 1)
    return rows


def sample_rows(cu, cp, n_total, heads, seed):
    """At least n_total rows: every chunk edge plus uniform random rows, each
    with a head drawn from `heads`."""
    rng = np.random.default_rng(seed)
    rows = chunk_edges(cu, cp)
    while len(rows) < n_total:
        rows.update(int(r) for r in rng.integers(0, int(cu[-1]), size=n_total - len(rows)))
    rows = np.array(sorted(rows), dtype=np.int64)
    hs = np.asarray(heads)[rng.integers(0, len(heads), size=len(rows))].astype(np.int32)
    return rows, hs


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_forward_sampled_rows_full_size(name):
    """4096 (row, head) pairs over every head, every chunk edge included."""
    s = setup(name, with_do=name != "c3")
    w = s.w
    o_acc, lse, out = s.forward()
    rows, heads = sample_rows(s.cu, w.cp, 4096, range(w.hq), w.seed)
    ow, lw = oracle.attn_fwd_rows(s.q, s.k, s.v, s.cu, w.scale, rows, heads)
    zrows = s.dst[rows]
    og = o_acc[zrows, heads].float().cpu().numpy()
    lg = lse[heads, zrows].float().cpu().numpy()
    fo = out[rows, heads].float().cpu().numpy()
    print("parity %s fwd rows=%d: o max_abs=%.3e lse max_abs=%.3e out max_abs=%.3e"
          % (name, len(rows), max_abs(og, ow), max_abs(lg, lw), max_abs(fo, ow)), flush=True)
    assert len(rows) >= 4096
    assert max_abs(og, ow) < TOL_BF16["abs"]
    assert rel_l2(og, ow) < TOL_BF16["rel"]
    assert max_abs(lg, lw) < TOL_BF16["lse"]
    assert max_abs(fo, ow) < TOL_BF16["abs"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,head", [("c3", 29), ("c4", 45), ("c5", 61)])
def test_forward_one_full_head_full_size(name, head):
    """Every row of one query head against the oracle (c5: 4.4 TFLOP of
    oracle work, the largest CPU job of the suite; its result also serves
    the c5 backward check below)."""
    s = setup(name, with_do=name != "c3")
    o_acc, lse, out = s.forward()
    ow, lw = head_reference(name, head)
    og = o_acc[:, head].float().cpu().numpy()[s.dst]
    lg = lse[head].float().cpu().numpy()[s.dst]
    fo = out[:, head].float().cpu().numpy()
    print("parity %s fwd head %d: o max_abs=%.3e rel_l2=%.3e lse max_abs=%.3e"
          % (name, head, max_abs(og, ow), rel_l2(og, ow), max_abs(lg, lw)), flush=True)
    assert max_abs(og, ow) < TOL_BF16["abs"]
    assert rel_l2(og, ow) < TOL_BF16["rel"]
    assert max_abs(lg, lw) < TOL_BF16["lse"]
    assert max_abs(fo, ow) < TOL_BF16["abs"]
    assert rel_l2(fo, ow) < TOL_BF16["rel"]


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_forward_zero_query_closed_form_full_size(name):
    """Q = 0: O is the running mean of V within each sequence and LSE is the
    log of the number of visible keys, at every row of every head."""
    import torch
    s = setup(name, zero_q=True)
    w = s.w
    o_acc, lse, _ = s.forward()
    dst = torch.as_tensor(s.dst, device="cuda")
    vd = torch.as_tensor(s.v, device="cuda").double()
    G = w.hq // w.hkv
    worst_o = worst_l = 0.0
    cu = s.cu
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


# ----------------------------------------------------------------- backward

@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_backward_sampled_dq_rows(name):
    """c3: one 32768-token sequence, GQA 32/8 (its own configuration is
    forward-only; dO drawn after Q, K, V as for c5); c4: 65536 tokens packed
    from 15 documents (document mask), GQA 64/8; c5: one 131072-token
    sequence, GQA 64/8.  512 (row, head) pairs."""
    s = setup(name, with_do=True)
    w = s.w
    dq, dk, dv = s.backward()
    rows, heads = sample_rows(s.cu, w.cp, 512, range(w.hq), 55)
    want = oracle.attn_bwd_dq_rows(s.q, s.k, s.v, s.do, s.cu, w.scale, rows, heads)
    got = dq[s.dst[rows], heads].float().cpu().numpy()
    check_grad("dq", got, want, TOL_BF16, 1.0, "%s sampled rows=%d" % (name, len(rows)))


@pytest.mark.timeout(900)
def test_backward_c4_sampled_dkv_rows():
    """c4 with dO on every head: 512 key rows of one key/value group (every
    chunk edge of every document included), each summed over the group's 8
    query heads and all later rows of its document."""
    s = setup("c4", with_do=True)
    w = s.w
    g = 5
    G = w.hq // w.hkv
    dq, dk, dv = s.backward()
    rows, _ = sample_rows(s.cu, w.cp, 512, [0], 57)
    kvh = np.full(len(rows), g, dtype=np.int32)
    stats = row_stats("c4", range(g * G, (g + 1) * G), s.do)
    wk, wv = oracle.attn_bwd_dkv_rows(s.q, s.k, s.v, s.do, s.cu, w.scale, rows, kvh, row_stats=stats)
    zr = s.dst[rows]
    tag = "c4 group %d key rows=%d" % (g, len(rows))
    check_grad("dk", dk[zr, g].float().cpu().numpy(), wk, TOL_BF16, 1.0, tag)
    check_grad("dv", dv[zr, g].float().cpu().numpy(), wv, TOL_BF16, 1.0, tag)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,h", [("c3", 29), ("c5", 61)])
def test_backward_one_head_sampled_rows(name, h):
    """c5 (the benchmarked configuration) and c3 with dO zero on every query
    head but one: that head's group gets its dK, dV from that head alone.
    Compared: 512 key rows of dK and dV (every chunk's first and last row
    included) and 512 dQ rows of the head; every other head's dQ and every
    other group's dK, dV must be exactly zero."""
    import torch
    s = setup(name, with_do=True)
    w = s.w
    G = w.hq // w.hkv
    g = h // G
    keep = torch.zeros((1, w.hq, 1), dtype=s.doz.dtype, device=s.doz.device)
    keep[0, h, 0] = 1
    doz = s.doz * keep
    do = np.zeros_like(s.do)
    do[:, h] = s.do[:, h]
    dq, dk, dv = s.backward(doz)
    rows, _ = sample_rows(s.cu, w.cp, 512, [0], 59)
    kvh = np.full(len(rows), g, dtype=np.int32)
    wk, wv = oracle.attn_bwd_dkv_rows(s.q, s.k, s.v, do, s.cu, w.scale, rows, kvh, heads_on=[h],
                                      row_stats=row_stats(name, [h], do))
    zr = s.dst[rows]
    tag = "%s head %d key rows=%d" % (name, h, len(rows))
    check_grad("dk", dk[zr, g].float().cpu().numpy(), wk, TOL_BF16, 1.0, tag)
    check_grad("dv", dv[zr, g].float().cpu().numpy(), wv, TOL_BF16, 1.0, tag)
    qrows, _ = sample_rows(s.cu, w.cp, 512, [0], 61)
    wq = oracle.attn_bwd_dq_rows(s.q, s.k, s.v, do, s.cu, w.scale, qrows,
                                 np.full(len(qrows), h, dtype=np.int32))
    check_grad("dq", dq[s.dst[qrows], h].float().cpu().numpy(), wq, TOL_BF16, 1.0,
               "%s head %d rows=%d" % (name, h, len(qrows)))
    others_q = [x for x in range(w.hq) if x != h]
    others_kv = [x for x in range(w.hkv) if x != g]
    assert float(dq[:, others_q].abs().max()) == 0.0
    assert float(dk[:, others_kv].abs().max()) == 0.0 and float(dv[:, others_kv].abs().max()) == 0.0


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_backward_gradient_identities(name):
    """Exact identities of the attention gradient, per key/value group (they
    hold per document, hence also summed over a packed batch):
    sum_k dK_k = 0;  sum_k dV_k = sum over the group's heads of sum_q dO_q;
    sum over heads of <Q, dQ> = <K, dK>."""
    s = setup(name, with_do=True)
    w = s.w
    dq, dk, dv = s.backward()
    G = w.hq // w.hkv
    dkd, dvd, dqd = dk.double(), dv.double(), dq.double()
    sum_dk = dkd.sum(0)                                      # [hkv,d]
    assert float(sum_dk.abs().max()) < 1e-3 * float(dkd.abs().sum(0).max())
    sum_do = s.doz.double().sum(0).view(w.hkv, G, w.d).sum(1)  # [hkv,d]
    assert float((dvd.sum(0) - sum_do).abs().max()) < 1e-3 * float(sum_do.abs().max() + 1.0)
    qdq = (s.qz.double() * dqd).sum(dim=(0, 2)).view(w.hkv, G).sum(1)
    kdk = (s.kz.double() * dkd).sum(dim=(0, 2))
    # Both sides are sums of about 1e9 products that cancel to ~1e2; dQ and dK
    # are formed by different kernels from independently rounded bf16 dS, so
    # the identity holds to rounding noise, not to fp32 accuracy.
    assert float((qdq - kdk).abs().max()) < 1e-2 * float(kdk.abs().max() + 1.0)


def test_backward_c5_zero_key_closed_form():
    """K = 0: every visible key has weight 1/n, so dQ = 0 exactly and
    dV_k = sum over later rows q and the group's heads of dO_q / n_q."""
    import torch
    s = setup("c5", zero_k=True, with_do=True)
    w = s.w
    dq, dk, dv = s.backward()
    assert float(dq.abs().max()) == 0.0
    G = w.hq // w.hkv
    T = w.total
    n = torch.arange(1, T + 1, device="cuda", dtype=torch.float64)
    contrib = torch.as_tensor(s.do, device="cuda").double().view(T, w.hkv, G, w.d).sum(2) / n[:, None, None]
    want = torch.flip(torch.cumsum(torch.flip(contrib, [0]), 0), [0])      # packed order
    dst = torch.as_tensor(s.dst, device="cuda")
    got = dv[dst].double()
    err = float((got - want).abs().max())
    print("parity c5 K=0 dv: max_abs=%.3e max|ref|=%.3g" % (err, float(want.abs().max())), flush=True)
    # exact weights 1/n_q rounded once to bf16: tighter than the flat gate
    assert err < 2e-3 * max(1.0, float(want.abs().max()))


def test_backward_c4_one_head_full():
    """Document-masked backward at full size (65536 tokens, 15 documents):
    with dO zero for every query head but one, that head's dQ and its
    group's dK, dV are the one-head gradients, compared in full against the
    oracle's backward of that head alone."""
    import torch
    s = setup("c4", with_do=True)
    w = s.w
    G = w.hq // w.hkv
    h = w.hq - 3
    g = h // G
    keep = torch.zeros((1, w.hq, 1), dtype=s.doz.dtype, device=s.doz.device)
    keep[0, h, 0] = 1
    dq, dk, dv = s.backward(s.doz * keep)
    want = oracle.attn_bwd(s.q[:, h:h + 1], s.k[:, g:g + 1], s.v[:, g:g + 1], s.do[:, h:h + 1], s.cu,
                           w.scale)
    dst = torch.as_tensor(s.dst, device="cuda")
    got = (dq[dst][:, h], dk[dst][:, g], dv[dst][:, g])
    for nm, gt, wt in zip(("dq", "dk", "dv"), got, want):
        check_grad(nm, gt.float().cpu().numpy(), wt[:, 0], TOL_BF16, 1.0, "c4 one head %d" % h)
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
