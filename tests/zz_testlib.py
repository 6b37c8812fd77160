"""Helpers shared by the GPU parity tests: seeded inputs on the device,
zigzag-layout copies, comparison metrics.  Holds no attention arithmetic."""
from __future__ import annotations

import numpy as np

import synthetic

_capture = None   # pytest's capture manager (set by conftest.py)


def set_capture_manager(capman) -> None:
    global _capture
    _capture = capman


def progress(msg: str) -> None:
    """Print a progress line past pytest's output capture, so a test that
    runs the oracle for minutes keeps writing to the terminal (or log)."""
    if _capture is None:
        print(msg, flush=True)
        return
    with _capture.global_and_fixture_disabled():
        print(msg, flush=True)


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
# ``grad_rel`` applies only to the sharp-softmax stress inputs (see grad_gate).
TOL = {
    "f32": dict(abs=1e-5, lse=1e-5, rel=1e-5, grad_rel=2.0 ** -22),
    "bf16": dict(abs=2e-2, lse=1e-3, rel=1e-2, grad_rel=2.0 ** -7),
}


def grad_gate(tol, want, q_scale: float = 1.0) -> float:
    """Max-abs gate of a gradient tensor.

    Inputs drawn N(0,1) (q_scale == 1) get the flat gate: 2e-2 in bf16, 1e-5
    in fp32.  The stress inputs whose queries are scaled by q_scale > 1 (sharp
    softmax rows) get max(flat, grad_rel * max|want|): every gradient element
    is a sum of products one factor of which (P for dV, dS for dQ and dK) is
    rounded to the operand type once, with relative error at most the unit
    roundoff u (2^-8 for bf16, 2^-24 for fp32).  A sharp row concentrates the
    sum in a few terms of the size of the result, so the error approaches
    u * |result| per rounding; grad_rel = 2u allows the two roundings a term
    can carry (its dS and the P it was formed from)."""
    flat = tol["abs"]
    if q_scale == 1.0:
        return flat
    return max(flat, tol["grad_rel"] * float(np.abs(np.asarray(want)).max()))


def check_grad(name, got, want, tol, q_scale: float = 1.0, case: str = ""):
    """Gate one gradient tensor and print its measured errors."""
    gate = grad_gate(tol, want, q_scale)
    err, rel = max_abs(got, want), rel_l2(got, want)
    print("parity %s %s: max_abs=%.3e (gate %.1e) rel_l2=%.3e (gate %.0e) max|ref|=%.3g"
          % (case, name, err, gate, rel, tol["rel"], float(np.abs(np.asarray(want)).max())), flush=True)
    assert err < gate, (case, name, err, gate)
    assert rel < tol["rel"], (case, name, rel)


def to_np(t):
    return t.detach().float().cpu().numpy()
