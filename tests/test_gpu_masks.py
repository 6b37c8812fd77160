"""The masks the three attention kernels apply inside their tiles, read back
from their outputs and compared bit for bit with the oracle's step masks
(causal within a sequence, no attention across packed sequences).

The tile lists are pinned elsewhere (zz_debug_mask); these tests pin the
in-register masking of partial (diagonal) and ragged tiles itself.  Inputs
are chosen so that every output element is an exact small integer:
 * forward: Q = 0 gives every visible key weight exactly 1; with V row k =
   the unit vector of k's index in its shard, O * exp(LSE) is the row's
   visible-key indicator;
 * dK/dV: Q = 0 and LSE = 0 give P = 1 on visible pairs and 0 elsewhere; with
   dO row q = the unit vector of q's index in its rank, dV of key k is its
   visible-query indicator (summed over the query heads of the group);
 * dQ: the same P, dO = V = the first unit vector and delta = 0 give dS = P;
   with K row k = the unit vector of k's index in its shard, dQ / scale is the
   row's visible-key indicator.
Each needs rows per rank <= head_dim (one unit vector per row or key)."""
import math

import numpy as np
import pytest

import oracle
import synthetic

pytestmark = pytest.mark.gpu

zz = pytest.importorskip("zigzag_ring_attention_amd")

SHAPES = [
    # lengths, cp, head_dim, dtype, forward tile (bm, bn)
    ((96, 64, 96), 2, 128, "bf16", 128, 64),   # 128 rows per rank, partial 128x64 tiles
    ((512,), 4, 128, "bf16", 128, 64),         # one sequence, 64-row chunks
    ((36, 12, 60, 96), 3, 128, "bf16", 48, 40),  # CP not a power of two, ragged tiles
    ((8, 24, 16), 4, 64, "bf16", 3, 5),        # 12 rows per rank, tiny tiles
    ((16, 48), 2, 32, "f32", 128, 64),         # fp32 path
    ((40, 8, 16), 2, 32, "bf16", 16, 8),
]


def unit_rows(T, n, d, heads, dtype):
    """[T, heads, d]: zigzag row z is the unit vector of z's index in its rank (z % n)."""
    import torch
    x = torch.zeros((T, heads, d), dtype=torch.float32)
    z = torch.arange(T)
    x[z, :, z % n] = 1.0
    return x.to(dtype).cuda()


def tdtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@pytest.mark.parametrize("lengths,cp,d,dtype,bm,bn", SHAPES)
def test_forward_kernel_mask_is_the_step_mask(lengths, cp, d, dtype, bm, bn):
    import torch
    cu = synthetic.make_cu_seqlens(lengths)
    T = int(cu[-1])
    n = T // cp
    assert n <= d
    hq, hkv = 2, 1
    plan = zz.Plan(cu, cp, hq, hkv, d, dtype, bm, bn, device="cuda")
    q = torch.zeros((T, hq, d), dtype=tdtype(dtype), device="cuda")
    k = torch.randn((T, hkv, d), generator=torch.Generator().manual_seed(3)).to(tdtype(dtype)).cuda()
    v = unit_rows(T, n, d, hkv, tdtype(dtype))
    for r in range(cp):
        for s in range(cp):
            o = torch.full((T, hq, d), 7.0, device="cuda")
            lse = torch.full((hq, T), 7.0, device="cuda")
            zz.varlen_ring_step_fwd(plan, r, s, q, k, v, o, lse, merge=False)
            want = oracle.step_mask(cu, cp, r, s)
            rows = slice(r * n, (r + 1) * n)
            for h in range(hq):
                w = o[rows, h, :n].double() * torch.exp(lse[h, rows].double())[:, None]
                got = torch.round(w).to(torch.uint8).cpu().numpy()
                assert float((w - torch.round(w)).abs().max()) < 1e-3
                assert np.array_equal(got, want), (r, s, h)


@pytest.mark.parametrize("lengths,cp,d,dtype,bm,bn", SHAPES)
def test_backward_kernel_masks_are_the_step_mask(lengths, cp, d, dtype, bm, bn):
    import torch
    cu = synthetic.make_cu_seqlens(lengths)
    T = int(cu[-1])
    n = T // cp
    assert n <= d
    hq, hkv = 2, 1
    G = hq // hkv
    scale = 1.0 / math.sqrt(d)
    dt = tdtype(dtype)
    plan = zz.Plan(cu, cp, hq, hkv, d, dtype, bm, bn, device="cuda")
    q = torch.zeros((T, hq, d), dtype=dt, device="cuda")
    lse = torch.zeros((hq, T), device="cuda")
    delta = torch.zeros((hq, T), device="cuda")
    # dK/dV: random K, V (their values do not reach dV when P is 0 or 1),
    # one-hot dO over the rank's query rows
    k_rand = torch.randn((T, hkv, d), generator=torch.Generator().manual_seed(4)).to(dt).cuda()
    v_rand = torch.randn((T, hkv, d), generator=torch.Generator().manual_seed(5)).to(dt).cuda()
    do_unit = unit_rows(T, n, d, hq, dt)
    # dQ: one-hot K over the shard's keys, dO = V = first unit vector
    k_unit = unit_rows(T, n, d, hkv, dt)
    e0 = torch.zeros((T, 1, d), dtype=dt, device="cuda")
    e0[:, :, 0] = 1
    v_e0, do_e0 = e0.expand(T, hkv, d).contiguous(), e0.expand(T, hq, d).contiguous()
    for r in range(cp):
        for s in range(cp):
            want = oracle.step_mask(cu, cp, r, s)           # [query of rank r, key of shard j]
            j = (r - s) % cp
            dk = torch.full((T, hkv, d), 7.0, device="cuda")
            dv = torch.full((T, hkv, d), 7.0, device="cuda")
            zz.varlen_ring_step_bwd_dkv(plan, r, s, q, k_rand, v_rand, do_unit, lse, delta, dk, dv,
                                        accumulate=False)
            keys = slice(j * n, (j + 1) * n)
            # dV[k, 0, e] = sum over the group's heads of [query e sees key k];
            # a key no query of the step sees is not touched (keeps 7.0)
            seen = want.any(axis=0)
            dvk = dv[keys, 0, :n].double().cpu().numpy()
            assert np.all(dvk[~seen] == 7.0), ("dkv untouched", r, s)
            w = dvk[seen] / G
            assert np.abs(w - np.round(w)).max(initial=0.0) < 1e-3
            assert np.array_equal(np.round(w).astype(np.uint8), want.T[seen]), ("dkv", r, s)
            dq = torch.full((T, hq, d), 7.0, device="cuda")
            zz.varlen_ring_step_bwd_dq(plan, r, s, q, k_unit, v_e0, do_e0, lse, delta, dq, accumulate=False)
            rows = slice(r * n, (r + 1) * n)
            sees = want.any(axis=1)
            for h in range(hq):
                dqh = dq[rows, h, :n].double().cpu().numpy()
                assert np.all(dqh[~sees] == 7.0), ("dq untouched", r, s, h)
                w = dqh[sees] / scale
                assert np.abs(w - np.round(w)).max(initial=0.0) < 1e-3
                assert np.array_equal(np.round(w).astype(np.uint8), want[sees]), ("dq", r, s, h)
