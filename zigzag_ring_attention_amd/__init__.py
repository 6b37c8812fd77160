"""zigzag_ring_attention_amd -- zigzag varlen ring attention on AMD MI355X (gfx950).

Thin ctypes binding over ``libzz.so`` (C ABI in ``include/zz.h``).  PyTorch
only provides device memory and the current stream; every step of the
attention runs in the library's HIP kernels.  There is no fallback: if the
library is not built, importing the binding's entry points raises.

Layouts follow the C ABI: packed token-major tensors ``[T, H, d]``, zigzag
layout = the same shape reordered rank-major, LSE / delta fp32 ``[Hq, T]``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Plan", "ZZError", "PASS_FWD", "PASS_BWD_DQ", "PASS_BWD_DKV", "ALL_RANKS", "ALL_STEPS",
    "lib", "zigzag_permute", "zigzag_unpermute", "varlen_ring_step_fwd", "lse_merge",
    "finalize_fwd", "bwd_preprocess", "varlen_ring_step_bwd", "varlen_ring_step_bwd_dkv",
    "varlen_ring_step_bwd_dq", "finalize_bwd", "debug_mask",
    "ring_attention_fwd", "ring_attention_bwd", "library_path",
    "varlen_gathered_fwd", "gathered_attention_fwd", "varlen_gathered_bwd", "gathered_attention_bwd",
]

PASS_FWD, PASS_BWD_DQ, PASS_BWD_DKV = 0, 1, 2
ALL_RANKS = -1
ALL_STEPS = -1
F32, BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# The library built in-tree next to this file; there is no other search path.
_LIB_PATH = os.path.join(_HERE, "libzz.so")
_lib = None


class ZZError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libzz.so (built by ``python -m zigzag_ring_attention_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ZZError("libzz.so is not built; run `python -m zigzag_ring_attention_amd.build` "
                      "(or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "zz_status_str": ([i32], ctypes.c_char_p),
        "zz_last_error": ([], ctypes.c_char_p),
        "zz_plan_create": ([P, i32, i32, i32, i32, i32, i32, i32, i32, P], i32),
        "zz_plan_destroy": ([P], None),
        "zz_plan_workspace_bytes": ([P], sz),
        "zz_plan_upload": ([P, P, sz, P], i32),
        "zz_plan_upload_static": ([P, P], i32),
        "zz_plan_shape": ([P, P, P, P, P, P, P, P], i32),
        "zz_plan_local_cu_seqlens": ([P, P], i32),
        "zz_plan_zigzag_dst": ([P, P], i32),
        "zz_plan_tile_shape": ([P, i32, P, P], i32),
        "zz_plan_tiles": ([P, i32, i32, i32, P, i64, P], i32),
        "zz_plan_gathered_tiles": ([P, i32, i32, P, i64, P], i32),
        "zz_plan_pair_counts": ([P, i32, i32, i32, P, P], i32),
        "zz_plan_rank_useful_pairs": ([P, P], i32),
        "zz_zigzag_permute": ([P, P, P, i64, P], i32),
        "zz_zigzag_unpermute": ([P, P, P, i64, P], i32),
        "zz_varlen_ring_step_fwd": ([P, i32, i32, P, P, P, P, P, i32, P], i32),
        "zz_varlen_gathered_fwd": ([P, i32, P, P, P, P, P, P], i32),
        "zz_varlen_gathered_bwd": ([P, i32, P, P, P, P, P, P, P, P, P, P], i32),
        "zz_lse_merge": ([P, P, P, P, i64, i32, i32, P], i32),
        "zz_finalize_fwd": ([P, P, P, i32, P], i32),
        "zz_bwd_preprocess": ([P, P, P, P, P], i32),
        "zz_varlen_ring_step_bwd": ([P, i32, i32, P, P, P, P, P, P, P, P, P, i32, P], i32),
        "zz_varlen_ring_step_bwd_dkv": ([P, i32, i32, P, P, P, P, P, P, P, P, i32, P], i32),
        "zz_varlen_ring_step_bwd_dq": ([P, i32, i32, P, P, P, P, P, P, P, i32, P], i32),
        "zz_finalize_bwd": ([P, P, P, P, P, P, P, i32, P], i32),
        "zz_debug_mask": ([P, i32, i32, i32, P, P], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != 0:
        L = lib()
        raise ZZError("%s failed: %s (%s)" % (what, L.zz_status_str(rc).decode(),
                                               L.zz_last_error().decode()))


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    if not t.is_cuda:
        raise ZZError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ZZError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """Host plan of one packed batch plus its device workspace.

    ``cu_seqlens``: packed sequence boundaries (every length a multiple of
    2*cp).  ``bm``/``bn``: forward tile (query rows x keys).
    """

    def __init__(self, cu_seqlens: Sequence[int], cp: int, hq: int, hkv: int, head_dim: int,
                 dtype: str = "bf16", bm: int = 128, bn: int = 64, device=None):
        L = lib()
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
        self.cu_seqlens = cu.copy()
        self.nseq = len(cu) - 1
        self.cp, self.hq, self.hkv, self.d = int(cp), int(hq), int(hkv), int(head_dim)
        self.dtype = dtype
        dt = {"f32": F32, "bf16": BF16}[dtype]
        h = ctypes.c_void_p()
        _check(L.zz_plan_create(cu.ctypes.data_as(ctypes.c_void_p), self.nseq, self.cp, self.hq,
                                self.hkv, self.d, dt, int(bm), int(bn), ctypes.byref(h)),
               "zz_plan_create")
        self._h = h
        self.total = int(cu[-1])
        self.rows_per_rank = self.total // self.cp
        self.workspace = None
        if device is not None:
            self.upload(device)

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.zz_plan_destroy(h)
            self._h = None

    @property
    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def workspace_bytes(self) -> int:
        return int(lib().zz_plan_workspace_bytes(self._h))

    def upload(self, device="cuda"):
        import torch
        n = self.workspace_bytes()
        self.workspace = torch.empty(n, dtype=torch.uint8, device=device)
        _check(lib().zz_plan_upload(self._h, _ptr(self.workspace), n, _stream()), "zz_plan_upload")
        return self

    def upload_static(self):
        """Bind the plan to the library's own per-GPU workspace (no device
        allocation); another plan uploaded this way on the GPU makes this one
        stale until it is uploaded again."""
        _check(lib().zz_plan_upload_static(self._h, _stream()), "zz_plan_upload_static")
        self.workspace = None
        return self

    def local_cu_seqlens(self) -> np.ndarray:
        out = np.empty(self.nseq + 1, dtype=np.int32)
        _check(lib().zz_plan_local_cu_seqlens(self._h, out.ctypes.data_as(ctypes.c_void_p)),
               "zz_plan_local_cu_seqlens")
        return out

    def zigzag_dst(self) -> np.ndarray:
        out = np.empty(self.total, dtype=np.int64)
        _check(lib().zz_plan_zigzag_dst(self._h, out.ctypes.data_as(ctypes.c_void_p)), "zz_plan_zigzag_dst")
        return out

    def tile_shape(self, pass_: int = PASS_FWD):
        bm, bn = ctypes.c_int32(), ctypes.c_int32()
        _check(lib().zz_plan_tile_shape(self._h, pass_, ctypes.byref(bm), ctypes.byref(bn)), "zz_plan_tile_shape")
        return bm.value, bn.value

    def tiles(self, rank: int, step: int, pass_: int = PASS_FWD) -> np.ndarray:
        L = lib()
        n = ctypes.c_int64()
        rc = L.zz_plan_tiles(self._h, pass_, rank, step, None, 0, ctypes.byref(n))
        if rc not in (0, 5):
            _check(rc, "zz_plan_tiles")
        out = np.empty((max(n.value, 1), 5), dtype=np.int32)
        _check(L.zz_plan_tiles(self._h, pass_, rank, step, out.ctypes.data_as(ctypes.c_void_p),
                               n.value, ctypes.byref(n)), "zz_plan_tiles")
        return out[: n.value]

    def gathered_tiles(self, owner: int, pass_: int = PASS_FWD) -> np.ndarray:
        """Tiles of the all-gather form for rank (or, for the dK/dV pass,
        shard) `owner`: [n, 5] (q0, q1, k0, k1, kind) in global zigzag rows."""
        L = lib()
        n = ctypes.c_int64()
        rc = L.zz_plan_gathered_tiles(self._h, pass_, owner, None, 0, ctypes.byref(n))
        if rc not in (0, 5):
            _check(rc, "zz_plan_gathered_tiles")
        out = np.empty((max(n.value, 1), 5), dtype=np.int32)
        _check(L.zz_plan_gathered_tiles(self._h, pass_, owner, out.ctypes.data_as(ctypes.c_void_p),
                                        n.value, ctypes.byref(n)), "zz_plan_gathered_tiles")
        return out[: n.value]

    def pair_counts(self, rank: int = ALL_RANKS, step: int = ALL_STEPS, pass_: int = PASS_FWD):
        u, i = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().zz_plan_pair_counts(self._h, pass_, rank, step, ctypes.byref(u), ctypes.byref(i)),
               "zz_plan_pair_counts")
        return u.value, i.value

    def rank_useful_pairs(self) -> np.ndarray:
        """Visible (query, key) pairs per head of each rank over the whole ring: int64 [cp]."""
        out = np.empty(self.cp, dtype=np.int64)
        _check(lib().zz_plan_rank_useful_pairs(self._h, out.ctypes.data_as(ctypes.c_void_p)),
               "zz_plan_rank_useful_pairs")
        return out


# ----------------------------------------------------------------- device ops

def zigzag_permute(plan: Plan, x, out=None, stream=None):
    import torch
    out = torch.empty_like(x) if out is None else out
    if x.shape[0] != plan.total or out.shape != x.shape:
        raise ZZError("permute: expected [T, ...] with T=%d" % plan.total)
    row_bytes = x[0].numel() * x.element_size()
    _check(lib().zz_zigzag_permute(plan.handle, _ptr(x), _ptr(out), row_bytes, _stream(stream)),
           "zz_zigzag_permute")
    return out


def zigzag_unpermute(plan: Plan, x_zz, out=None, stream=None):
    import torch
    out = torch.empty_like(x_zz) if out is None else out
    if x_zz.shape[0] != plan.total or out.shape != x_zz.shape:
        raise ZZError("unpermute: expected [T, ...] with T=%d" % plan.total)
    row_bytes = x_zz[0].numel() * x_zz.element_size()
    _check(lib().zz_zigzag_unpermute(plan.handle, _ptr(x_zz), _ptr(out), row_bytes, _stream(stream)),
           "zz_zigzag_unpermute")
    return out


def _check_qkv(plan: Plan, q, k, v):
    import torch
    T = plan.total
    if tuple(q.shape) != (T, plan.hq, plan.d) or tuple(k.shape) != (T, plan.hkv, plan.d) \
            or tuple(v.shape) != (T, plan.hkv, plan.d):
        raise ZZError("q/k/v shapes must be [T,hq,d] / [T,hkv,d]")
    for t in (q, k, v):
        if t.dtype != plan.torch_dtype:
            raise ZZError("q/k/v dtype must be %s" % plan.dtype)


def _check_acc(plan: Plan, o, lse):
    import torch
    if o.dtype != torch.float32 or tuple(o.shape) != (plan.total, plan.hq, plan.d):
        raise ZZError("o_acc must be fp32 [T,hq,d]")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (plan.hq, plan.total):
        raise ZZError("lse must be fp32 [hq,T]")


def varlen_ring_step_fwd(plan: Plan, rank: int, step: int, q_zz, k_zz, v_zz, o_acc, lse_acc,
                         merge: bool, stream=None):
    _check_qkv(plan, q_zz, k_zz, v_zz)
    _check_acc(plan, o_acc, lse_acc)
    _check(lib().zz_varlen_ring_step_fwd(plan.handle, rank, step, _ptr(q_zz), _ptr(k_zz), _ptr(v_zz),
                                         _ptr(o_acc), _ptr(lse_acc), 1 if merge else 0, _stream(stream)),
           "zz_varlen_ring_step_fwd")


def varlen_gathered_fwd(plan: Plan, rank: int, q_zz, k_zz, v_zz, o, lse, stream=None):
    """Forward of rank `rank` (or ALL_RANKS) against every shard in one launch:
    writes the normalized O (fp32 [T,hq,d]) and LSE (fp32 [hq,T]) of its rows."""
    _check_qkv(plan, q_zz, k_zz, v_zz)
    _check_acc(plan, o, lse)
    _check(lib().zz_varlen_gathered_fwd(plan.handle, rank, _ptr(q_zz), _ptr(k_zz), _ptr(v_zz), _ptr(o),
                                        _ptr(lse), _stream(stream)), "zz_varlen_gathered_fwd")


def gathered_attention_fwd(plan: Plan, q_zz, k_zz, v_zz, rank: int = ALL_RANKS, o=None, lse=None, stream=None):
    """The all-gather alternative to the ring forward: every rank's queries
    against all K/V at once.  Returns (o fp32 [T,hq,d], lse fp32 [hq,T])."""
    import torch
    dev = q_zz.device
    o = torch.empty((plan.total, plan.hq, plan.d), dtype=torch.float32, device=dev) if o is None else o
    lse = torch.empty((plan.hq, plan.total), dtype=torch.float32, device=dev) if lse is None else lse
    varlen_gathered_fwd(plan, rank, q_zz, k_zz, v_zz, o, lse, stream)
    return o, lse


def varlen_gathered_bwd(plan: Plan, rank: int, q_zz, k_zz, v_zz, do_zz, lse, delta, dq, dk, dv,
                        stream=None):
    """Backward of the gathered form: dq rows of `rank` and dk/dv rows of its
    shard (or every rank) against all the other side's rows, written in one
    launch per kernel."""
    _check_qkv(plan, q_zz, k_zz, v_zz)
    _check(lib().zz_varlen_gathered_bwd(plan.handle, rank, _ptr(q_zz), _ptr(k_zz), _ptr(v_zz), _ptr(do_zz),
                                        _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream)),
           "zz_varlen_gathered_bwd")


def gathered_attention_bwd(plan: Plan, q_zz, k_zz, v_zz, o_zz, do_zz, lse, stream=None):
    """Backward of the gathered form from the forward output O and its LSE.
    Returns (dq fp32 [T,hq,d], dk, dv fp32 [T,hkv,d]) in the zigzag layout."""
    import torch
    dev = q_zz.device
    delta = bwd_preprocess(plan, o_zz, do_zz, stream=stream)
    dq = torch.empty((plan.total, plan.hq, plan.d), dtype=torch.float32, device=dev)
    dk = torch.empty((plan.total, plan.hkv, plan.d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    varlen_gathered_bwd(plan, ALL_RANKS, q_zz, k_zz, v_zz, do_zz, lse, delta, dq, dk, dv, stream)
    return dq, dk, dv


def lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    import torch
    rows, heads, d = o_acc.shape
    for t in (o_acc, lse_acc, o_part, lse_part):
        if t.dtype != torch.float32:
            raise ZZError("lse_merge: fp32 tensors required")
    if o_part.shape != o_acc.shape or tuple(lse_acc.shape) != (heads, rows) or lse_part.shape != lse_acc.shape:
        raise ZZError("lse_merge: o [rows,heads,d], lse [heads,rows]")
    _check(lib().zz_lse_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), rows, heads, d,
                              _stream(stream)), "zz_lse_merge")


def finalize_fwd(plan: Plan, o_acc, unpermute: bool = False, out=None, stream=None):
    import torch
    out = torch.empty(o_acc.shape, dtype=plan.torch_dtype, device=o_acc.device) if out is None else out
    _check(lib().zz_finalize_fwd(plan.handle, _ptr(o_acc), _ptr(out), 1 if unpermute else 0, _stream(stream)),
           "zz_finalize_fwd")
    return out


def bwd_preprocess(plan: Plan, o_zz, do_zz, delta=None, stream=None):
    import torch
    delta = torch.empty((plan.hq, plan.total), dtype=torch.float32, device=o_zz.device) if delta is None else delta
    if o_zz.dtype != plan.torch_dtype or do_zz.dtype != plan.torch_dtype:
        raise ZZError("bwd_preprocess: O and dO must be %s" % plan.dtype)
    _check(lib().zz_bwd_preprocess(plan.handle, _ptr(o_zz), _ptr(do_zz), _ptr(delta), _stream(stream)),
           "zz_bwd_preprocess")
    return delta


def varlen_ring_step_bwd(plan: Plan, rank: int, step: int, q_zz, k_zz, v_zz, do_zz, lse, delta,
                         dq_acc, dk_acc, dv_acc, accumulate: bool = True, stream=None):
    _check_qkv(plan, q_zz, k_zz, v_zz)
    _check(lib().zz_varlen_ring_step_bwd(plan.handle, rank, step, _ptr(q_zz), _ptr(k_zz), _ptr(v_zz),
                                         _ptr(do_zz), _ptr(lse), _ptr(delta), _ptr(dq_acc), _ptr(dk_acc),
                                         _ptr(dv_acc), 1 if accumulate else 0, _stream(stream)),
           "zz_varlen_ring_step_bwd")


def varlen_ring_step_bwd_dkv(plan: Plan, rank: int, step: int, q_zz, k_zz, v_zz, do_zz, lse, delta,
                             dk_acc, dv_acc, accumulate: bool = True, stream=None):
    _check_qkv(plan, q_zz, k_zz, v_zz)
    _check(lib().zz_varlen_ring_step_bwd_dkv(plan.handle, rank, step, _ptr(q_zz), _ptr(k_zz), _ptr(v_zz),
                                             _ptr(do_zz), _ptr(lse), _ptr(delta), _ptr(dk_acc), _ptr(dv_acc),
                                             1 if accumulate else 0, _stream(stream)),
           "zz_varlen_ring_step_bwd_dkv")


def varlen_ring_step_bwd_dq(plan: Plan, rank: int, step: int, q_zz, k_zz, v_zz, do_zz, lse, delta,
                            dq_acc, accumulate: bool = True, stream=None):
    _check_qkv(plan, q_zz, k_zz, v_zz)
    _check(lib().zz_varlen_ring_step_bwd_dq(plan.handle, rank, step, _ptr(q_zz), _ptr(k_zz), _ptr(v_zz),
                                            _ptr(do_zz), _ptr(lse), _ptr(delta), _ptr(dq_acc),
                                            1 if accumulate else 0, _stream(stream)),
           "zz_varlen_ring_step_bwd_dq")


def finalize_bwd(plan: Plan, dq_acc, dk_acc, dv_acc, unpermute: bool = False, out=None, stream=None):
    import torch
    if out is not None:
        dq, dk, dv = out
    else:
        dq = torch.empty(dq_acc.shape, dtype=plan.torch_dtype, device=dq_acc.device)
        dk = torch.empty(dk_acc.shape, dtype=plan.torch_dtype, device=dk_acc.device)
        dv = torch.empty(dv_acc.shape, dtype=plan.torch_dtype, device=dv_acc.device)
    _check(lib().zz_finalize_bwd(plan.handle, _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _ptr(dq), _ptr(dk),
                                 _ptr(dv), 1 if unpermute else 0, _stream(stream)), "zz_finalize_bwd")
    return dq, dk, dv


def debug_mask(plan: Plan, pass_: int, rank: int, step: int, stream=None):
    import torch
    n = plan.rows_per_rank
    m = torch.empty((n, n), dtype=torch.uint8, device="cuda")
    _check(lib().zz_debug_mask(plan.handle, pass_, rank, step, _ptr(m), _stream(stream)), "zz_debug_mask")
    return m


# ----------------------------------------------------------------- ring driver

def ring_attention_fwd(plan: Plan, q_zz, k_zz, v_zz, rank: int = ALL_RANKS, o_acc=None, lse=None,
                       stream=None):
    """All ring steps of the forward on zigzag-layout tensors.  Step 0 (the
    diagonal shard) writes the partial, later steps merge into it.  Returns
    (o_acc fp32 [T,hq,d], lse fp32 [hq,T])."""
    import torch
    dev = q_zz.device
    o_acc = torch.empty((plan.total, plan.hq, plan.d), dtype=torch.float32, device=dev) if o_acc is None else o_acc
    lse = torch.empty((plan.hq, plan.total), dtype=torch.float32, device=dev) if lse is None else lse
    ranks = range(plan.cp) if rank == ALL_RANKS else [rank]
    for s in range(plan.cp):
        if rank == ALL_RANKS:
            varlen_ring_step_fwd(plan, ALL_RANKS, s, q_zz, k_zz, v_zz, o_acc, lse, s > 0, stream)
        else:
            for r in ranks:
                varlen_ring_step_fwd(plan, r, s, q_zz, k_zz, v_zz, o_acc, lse, s > 0, stream)
    return o_acc, lse


def ring_attention_bwd(plan: Plan, q_zz, k_zz, v_zz, o_zz, do_zz, lse, stream=None, dq_stream=None):
    """All ring steps of the backward.  Step 0 (the diagonal shard, which
    touches every row) overwrites, later steps accumulate.  Returns fp32
    (dq, dk, dv) in zigzag layout.

    dq_stream: optional second stream for the dQ launches (the dK/dV and dQ
    launches of a step write disjoint buffers); it waits for `stream` after
    the pre-pass and `stream` waits for it at the end, so the results are the
    same bits.  It pays off when a step's launches are only a few rounds of
    workgroups (packings of short documents); with one long sequence the
    concurrent grids run slower than one stream."""
    import torch
    dev = q_zz.device
    base = stream if stream is not None else torch.cuda.current_stream()
    delta = bwd_preprocess(plan, o_zz, do_zz, stream=base)
    dq = torch.empty((plan.total, plan.hq, plan.d), dtype=torch.float32, device=dev)
    dk = torch.empty((plan.total, plan.hkv, plan.d), dtype=torch.float32, device=dev)
    dv = torch.empty((plan.total, plan.hkv, plan.d), dtype=torch.float32, device=dev)
    if dq_stream is None:
        for s in range(plan.cp):
            varlen_ring_step_bwd(plan, ALL_RANKS, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dq, dk, dv,
                                 accumulate=s > 0, stream=base)
        return dq, dk, dv
    dq_stream.wait_stream(base)
    dq.record_stream(dq_stream)      # allocated here, used on the side stream
    delta.record_stream(dq_stream)
    for s in range(plan.cp):
        varlen_ring_step_bwd_dkv(plan, ALL_RANKS, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dk, dv,
                                 accumulate=s > 0, stream=base)
        varlen_ring_step_bwd_dq(plan, ALL_RANKS, s, q_zz, k_zz, v_zz, do_zz, lse, delta, dq,
                                accumulate=s > 0, stream=dq_stream)
    base.wait_stream(dq_stream)
    return dq, dk, dv
