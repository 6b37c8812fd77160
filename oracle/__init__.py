"""CPU oracle for zigzag varlen ring attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library never calls it, and it
imports nothing from ``zigzag_ring_attention_amd``.

All arithmetic happens in ``oracle.c`` in double precision, one query row at a
time, straight from the definitions (see the header of ``oracle.c`` for the
passages each function follows).  This module only marshals numpy arrays.

Every function has a pin that does not go through the oracle itself; see
``tests/test_oracle_pins.py``.  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=False)
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
            L.oracle_check_lengths.argtypes = [P, i32, i32]
            L.oracle_zigzag_dst.argtypes = [P, i32, i32, P]
            L.oracle_attn_fwd.argtypes = [P, P, P, P, i32, i32, i32, i32, f64, P, P]
            L.oracle_attn_fwd_rows.argtypes = [P, P, P, P, i32, i32, i32, i32, f64, P, P, i64, P, P]
            L.oracle_masked_attn.argtypes = [P, P, P, P, i64, i64, i32, i32, i32, f64, P, P]
            L.oracle_step_mask.argtypes = [P, i32, i32, i32, i32, P]
            L.oracle_ring_step_fwd.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, P, P]
            L.oracle_lse_merge.argtypes = [P, P, P, P, i64, i32, i32]
            L.oracle_attn_bwd.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, P, P, P]
            L.oracle_attn_bwd_dq_rows.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, P, P, i64, P]
            L.oracle_attn_bwd_dkv_rows.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, P, P, i64, P,
                                                   P, P, P, P]
            L.oracle_tiles.argtypes = [P, i32, i32, i32, i32, i32, i32, P, i64, P]
            L.oracle_rank_pairs.argtypes = [P, i32, i32, P]
            L.oracle_num_threads.argtypes = []
            _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    """Accept torch tensors (any float dtype, exact upcast) or numpy arrays."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.float32)


def _cu(cu) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cu), dtype=np.int32)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def check_lengths(cu, cp: int) -> bool:
    cu = _cu(cu)
    return lib().oracle_check_lengths(_p(cu), len(cu) - 1, cp) == 0


def zigzag_dst(cu, cp: int) -> np.ndarray:
    """dst[p] = zigzag row of packed token p."""
    cu = _cu(cu)
    out = np.empty(int(cu[-1]), dtype=np.int64)
    if lib().oracle_zigzag_dst(_p(cu), len(cu) - 1, cp, _p(out)) != 0:
        raise ValueError("every length must be a positive multiple of 2*cp")
    return out


def permute(x, cu, cp: int):
    """Packed [T, ...] -> zigzag rank-major layout (row p goes to dst[p])."""
    dst = zigzag_dst(cu, cp)
    y = np.empty_like(np.asarray(x))
    y[dst] = np.asarray(x)
    return y


def unpermute(y, cu, cp: int):
    dst = zigzag_dst(cu, cp)
    return np.asarray(y)[dst]


def attn_fwd(q, k, v, cu, scale: float):
    """Packed attention. Returns o [T,hq,d] float64, lse [hq,T] float64."""
    q, k, v, cu = _f32(q), _f32(k), _f32(v), _cu(cu)
    T, hq, d = q.shape
    hkv = k.shape[1]
    o = np.empty((T, hq, d), dtype=np.float64)
    lse = np.empty((hq, T), dtype=np.float64)
    lib().oracle_attn_fwd(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, hq, hkv, d, scale, _p(o), _p(lse))
    return o, lse


def attn_fwd_rows(q, k, v, cu, scale: float, rows, heads):
    """Attention for the given (packed row, head) pairs: o [n,d], lse [n]."""
    q, k, v, cu = _f32(q), _f32(k), _f32(v), _cu(cu)
    T, hq, d = q.shape
    hkv = k.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    n = len(rows)
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    lib().oracle_attn_fwd_rows(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, hq, hkv, d, scale,
                               _p(rows), _p(heads), n, _p(o), _p(lse))
    return o, lse


def masked_attn(q, k, v, mask, scale: float):
    """q [tq,hq,d], k/v [tk,hkv,d], mask [tq,tk] bool -> o [tq,hq,d], lse [hq,tq]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    tq, hq, d = q.shape
    tk, hkv = k.shape[0], k.shape[1]
    o = np.empty((tq, hq, d), dtype=np.float64)
    lse = np.empty((hq, tq), dtype=np.float64)
    lib().oracle_masked_attn(_p(q), _p(k), _p(v), _p(mask), tq, tk, hq, hkv, d, scale, _p(o), _p(lse))
    return o, lse


def step_mask(cu, cp: int, rank: int, step: int) -> np.ndarray:
    cu = _cu(cu)
    n = int(cu[-1]) // cp
    m = np.empty((n, n), dtype=np.uint8)
    if lib().oracle_step_mask(_p(cu), len(cu) - 1, cp, rank, step, _p(m)) != 0:
        raise ValueError("bad step-mask arguments")
    return m


def ring_step_fwd(q_zz, k_zz, v_zz, cu, cp: int, rank: int, step: int, scale: float):
    """Partial (o [T/cp,hq,d], lse [hq,T/cp]) of ring step (rank, step)."""
    q, k, v, cu = _f32(q_zz), _f32(k_zz), _f32(v_zz), _cu(cu)
    T, hq, d = q.shape
    hkv = k.shape[1]
    n = T // cp
    o = np.empty((n, hq, d), dtype=np.float64)
    lse = np.empty((hq, n), dtype=np.float64)
    rc = lib().oracle_ring_step_fwd(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, cp, rank, step, hq,
                                    hkv, d, scale, _p(o), _p(lse))
    if rc != 0:
        raise ValueError("bad ring-step arguments")
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Return the merge of two partials (inputs untouched).  o [rows,heads,d], lse [heads,rows]."""
    o = np.array(o_a, dtype=np.float64, order="C", copy=True)
    lse = np.array(lse_a, dtype=np.float64, order="C", copy=True)
    ob = np.ascontiguousarray(o_b, dtype=np.float64)
    lb = np.ascontiguousarray(lse_b, dtype=np.float64)
    rows, heads, d = o.shape
    lib().oracle_lse_merge(_p(o), _p(lse), _p(ob), _p(lb), rows, heads, d)
    return o, lse


def attn_bwd(q, k, v, dout, cu, scale: float):
    """Gradients (dq [T,hq,d], dk [T,hkv,d], dv [T,hkv,d]) in float64."""
    q, k, v, do, cu = _f32(q), _f32(k), _f32(v), _f32(dout), _cu(cu)
    T, hq, d = q.shape
    hkv = k.shape[1]
    dq = np.empty((T, hq, d), dtype=np.float64)
    dk = np.empty((T, hkv, d), dtype=np.float64)
    dv = np.empty((T, hkv, d), dtype=np.float64)
    lib().oracle_attn_bwd(_p(q), _p(k), _p(v), _p(do), _p(cu), len(cu) - 1, hq, hkv, d, scale,
                          _p(dq), _p(dk), _p(dv))
    return dq, dk, dv


def attn_bwd_dq_rows(q, k, v, dout, cu, scale: float, rows, heads):
    q, k, v, do, cu = _f32(q), _f32(k), _f32(v), _f32(dout), _cu(cu)
    T, hq, d = q.shape
    hkv = k.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    n = len(rows)
    dq = np.empty((n, d), dtype=np.float64)
    lib().oracle_attn_bwd_dq_rows(_p(q), _p(k), _p(v), _p(do), _p(cu), len(cu) - 1, hq, hkv, d,
                                  scale, _p(rows), _p(heads), n, _p(dq))
    return dq


def attn_bwd_dkv_rows(q, k, v, dout, cu, scale: float, rows, kv_heads, heads_on=None, row_stats=None):
    """dK, dV for the given (packed key row, key/value head) pairs: dk [n,d], dv [n,d].

    ``heads_on``: query heads to sum over (default: all).  Pass a subset only
    when dO is identically zero on every other head of the selected groups;
    those heads contribute exactly zero and their row statistics are then not
    computed.  ``row_stats``: optional (lse, dsum), float64 [hq, T] in packed
    rows, each needed row's LSE and D = <dO_q, O_q> from this oracle's own
    forward (``attn_fwd_rows``); without it they are computed here."""
    q, k, v, do, cu = _f32(q), _f32(k), _f32(v), _f32(dout), _cu(cu)
    T, hq, d = q.shape
    hkv = k.shape[1]
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    kv_heads = np.ascontiguousarray(kv_heads, dtype=np.int32)
    n = len(rows)
    on = None
    if heads_on is not None:
        on = np.zeros(hq, dtype=np.int32)
        on[np.asarray(list(heads_on), dtype=np.int64)] = 1
    lse = dsum = None
    if row_stats is not None:
        lse = np.ascontiguousarray(row_stats[0], dtype=np.float64)
        dsum = np.ascontiguousarray(row_stats[1], dtype=np.float64)
        if lse.shape != (hq, T) or dsum.shape != (hq, T):
            raise ValueError("row_stats must be two float64 [hq, T] tables")
    dk = np.empty((n, d), dtype=np.float64)
    dv = np.empty((n, d), dtype=np.float64)
    lib().oracle_attn_bwd_dkv_rows(_p(q), _p(k), _p(v), _p(do), _p(cu), len(cu) - 1, hq, hkv, d,
                                   scale, _p(rows), _p(kv_heads), n,
                                   _p(on) if on is not None else None,
                                   _p(lse) if lse is not None else None,
                                   _p(dsum) if dsum is not None else None, _p(dk), _p(dv))
    return dk, dv


def tiles(cu, cp: int, rank: int, step: int, bm: int, bn: int) -> np.ndarray:
    """Visible tiles of a ring step, int32 [n,5] = (q0, q1, k0, k1, kind)."""
    cu = _cu(cu)
    cap = 1 << 16
    while True:
        out = np.empty((cap, 5), dtype=np.int32)
        n = ctypes.c_int64(0)
        rc = lib().oracle_tiles(_p(cu), len(cu) - 1, cp, rank, step, bm, bn, _p(out), cap,
                                ctypes.byref(n))
        if rc == -2:
            cap = int(n.value)
            continue
        if rc != 0:
            raise ValueError("bad tile arguments")
        return out[: n.value].copy()


def rank_pairs(cu, cp: int) -> np.ndarray:
    cu = _cu(cu)
    out = np.empty(cp, dtype=np.int64)
    if lib().oracle_rank_pairs(_p(cu), len(cu) - 1, cp, _p(out)) != 0:
        raise ValueError("bad lengths")
    return out
