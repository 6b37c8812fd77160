"""The ring step captured in a HIP graph: every library call launches on
torch's current stream with no allocation or memset of its own, so a whole
forward + backward step is capturable.  Replays are checked bit for bit
against the eager step, with eager work and synchronisations between the
replays, on every replay."""
import pytest

from zz_testlib import Case

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")


def test_graph_replays_match_eager_step():
    import torch

    case = Case((128, 256, 64, 16), 2, 4, 2, 128, "bf16", 41, with_do=True)
    plan, T, hq, hkv, d = case.plan, case.T, case.hq, case.hkv, case.d
    dev = case.qz.device
    f32, bf = torch.float32, torch.bfloat16
    o_acc = torch.empty((T, hq, d), dtype=f32, device=dev)
    lse = torch.empty((hq, T), dtype=f32, device=dev)
    o_zz = torch.empty((T, hq, d), dtype=bf, device=dev)
    delta = torch.empty((hq, T), dtype=f32, device=dev)
    dq_acc = torch.empty((T, hq, d), dtype=f32, device=dev)
    dk_acc = torch.empty((T, hkv, d), dtype=f32, device=dev)
    dv_acc = torch.empty((T, hkv, d), dtype=f32, device=dev)
    grads = (torch.empty((T, hq, d), dtype=bf, device=dev), torch.empty((T, hkv, d), dtype=bf, device=dev),
             torch.empty((T, hkv, d), dtype=bf, device=dev))

    def step():
        for s in range(case.cp):
            zz.varlen_ring_step_fwd(plan, zz.ALL_RANKS, s, case.qz, case.kz, case.vz, o_acc, lse, merge=s > 0)
        zz.finalize_fwd(plan, o_acc, unpermute=False, out=o_zz)
        zz.bwd_preprocess(plan, o_zz, case.doz, delta)
        for s in range(case.cp):
            zz.varlen_ring_step_bwd(plan, zz.ALL_RANKS, s, case.qz, case.kz, case.vz, case.doz, lse, delta,
                                    dq_acc, dk_acc, dv_acc, accumulate=s > 0)
        zz.finalize_bwd(plan, dq_acc, dk_acc, dv_acc, unpermute=False, out=grads)

    outs = [o_zz, lse, *grads]
    step()
    torch.cuda.synchronize()
    want = [x.clone() for x in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()

    other = torch.zeros_like(case.qz)
    for rep in range(4):
        for x in outs:
            x.fill_(float("nan"))
        # the program's own eager work between replays
        zz.zigzag_permute(plan, case.qg, other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(outs, want)):
            assert torch.equal(x, y), (rep, i)
        assert torch.equal(other, case.qz)
