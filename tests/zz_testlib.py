"""Helpers shared by the GPU parity tests: seeded inputs on the device,
zigzag-layout copies, comparison metrics.  Holds no attention arithmetic."""
from __future__ import annotations

import numpy as np

import synthetic


class Case:
    """One seeded workload: CPU inputs (the oracle's copy) and device tensors."""

    def __init__(self, lengths, cp, hq, hkv, d, dtype, seed, with_do=False, q_scale=1.0,
                 bm=128, bn=64, zero_q=False, zero_k=False, const_v=None):
        import torch
        import zigzag_ring_attention_amd as zz
        self.lengths = list(lengths)
        self.cu = synthetic.make_cu_seqlens(self.lengths)
        self.T = int(self.cu[-1])
        self.cp, self.hq, self.hkv, self.d, self.dtype = cp, hq, hkv, d, dtype
        self.scale = 1.0 / float(np.sqrt(d))
        t = synthetic.randn_qkv(seed, self.T, hq, hkv, d, dtype, with_do=with_do, q_scale=q_scale)
        q, k, v = t[0], t[1], t[2]
        if zero_q:
            q = torch.zeros_like(q)
        if zero_k:
            k = torch.zeros_like(k)
        if const_v is not None:
            v = torch.full_like(v, const_v)
        self.q, self.k, self.v = q, k, v
        self.do = t[3] if with_do else None
        self.plan = zz.Plan(self.cu, cp, hq, hkv, d, dtype, bm, bn, device="cuda")
        self.qg, self.kg, self.vg = (x.cuda() for x in (q, k, v))
        self.qz = zz.zigzag_permute(self.plan, self.qg)
        self.kz = zz.zigzag_permute(self.plan, self.kg)
        self.vz = zz.zigzag_permute(self.plan, self.vg)
        self.doz = zz.zigzag_permute(self.plan, self.do.cuda()) if with_do else None
        self.dst = self.plan.zigzag_dst()


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.abs(a - b).max()) if a.size else 0.0


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.linalg.norm(b))
    return float(np.linalg.norm(a - b)) / den if den > 0 else float(np.linalg.norm(a - b))


# Tolerances: max-abs on outputs and gradients; LSE and relative-L2 gates on top.
TOL = {
    "f32": dict(abs=1e-5, lse=1e-5, rel=1e-5),
    "bf16": dict(abs=2e-2, lse=1e-3, rel=1e-2),
}


def to_np(t):
    return t.detach().float().cpu().numpy()
