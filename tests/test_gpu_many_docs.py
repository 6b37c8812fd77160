"""GPU parity on a packing of many short documents around one long one: a
hundred-odd work items per rank whose chunks are a few rows long (one-row
chunks included), ragged tiles everywhere, next to long key walks.  This is
the mix the MiniMax-01 issue #6 discussion ("Question about varlen ring
attention") worries about for packed data; here it stresses the planner's
item and tile bookkeeping against the oracle."""
import numpy as np
import pytest

import oracle
import synthetic
from test_gpu_bwd import check_grads
from test_gpu_fwd import check_full, run_forward
from zz_testlib import TOL, Case

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")

CP = 4


def many_lengths(seed: int):
    # one 2048-token document plus short ones (8 to 400 tokens, multiples of
    # 2*CP, log-uniform), shuffled so the long one sits inside the packing
    short = synthetic.lengths_loguniform(seed, 6144, 8, 400, 2 * CP)
    lengths = short + [2048, 2 * CP, 2 * CP, 4 * CP]   # one-row and two-row chunks too
    rng = np.random.default_rng(seed)
    rng.shuffle(lengths)
    return [int(x) for x in lengths]


@pytest.mark.parametrize("d", [64, 128])
def test_forward_many_documents(d):
    lengths = many_lengths(31)
    assert len(lengths) > 50 and min(lengths) == 2 * CP
    case = Case(lengths, CP, 4, 2, d, "bf16", 31)
    check_full(case, *run_forward(case), TOL["bf16"])


def test_backward_many_documents():
    case = Case(many_lengths(32), CP, 4, 2, 128, "bf16", 32, with_do=True)
    check_grads(case, TOL["bf16"])


def test_gathered_matches_ring_many_documents():
    case = Case(many_lengths(33), CP, 4, 2, 128, "bf16", 33)
    o_ring, lse_ring, _ = run_forward(case)
    o_g, lse_g = zz.gathered_attention_fwd(case.plan, case.qz, case.kz, case.vz)
    ow, lw = oracle.attn_fwd(case.q, case.k, case.v, case.cu, case.scale)
    for o, l in ((o_ring, lse_ring), (o_g, lse_g)):
        n_o = o.cpu().numpy()[case.dst]
        n_l = l.cpu().numpy()[:, case.dst]
        assert float(np.abs(n_o - ow).max()) < TOL["bf16"]["abs"]
        assert float(np.abs(n_l - lw).max()) < TOL["bf16"]["lse"]


def test_debug_mask_many_documents_sampled_steps():
    lengths = many_lengths(34)
    cu = synthetic.make_cu_seqlens(lengths)
    plan = zz.Plan(cu, CP, 2, 2, 32, "f32", device="cuda")
    for r, s in ((0, 0), (3, 0), (1, 2), (2, 1), (0, 3)):
        want = oracle.step_mask(cu, CP, r, s)
        for pass_ in (zz.PASS_FWD, zz.PASS_BWD_DQ, zz.PASS_BWD_DKV):
            got = zz.debug_mask(plan, pass_, r, s).cpu().numpy()
            assert np.array_equal(got, want), (pass_, r, s)
