"""Host-side tests of libzz (no GPU): the C ABI loads and exports every
declared symbol, the planner validates its inputs, and its zigzag map, tile
lists and pair counts equal the oracle's brute-force results bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synthetic

zz = pytest.importorskip("zigzag_ring_attention_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "zz.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(zz_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(zz.library_path())
    syms = header_symbols()
    assert len(syms) >= 20
    missing = [s for s in syms if not hasattr(L, s)]
    assert not missing, missing


def test_status_strings():
    L = zz.lib()
    for s in range(8):
        assert L.zz_status_str(s)
    assert L.zz_status_str(0) == b"ok"


@pytest.mark.parametrize("kw,msg", [
    (dict(cu=[0, 10], cp=2), "multiple of 2*cp"),
    (dict(cu=[0, 16, 16], cp=2), "strictly increasing"),
    (dict(cu=[1, 17], cp=2), "cu_seqlens[0]"),
    (dict(cu=[0, 16], cp=0), "cp"),
    (dict(cu=[0, 16], cp=2, hq=3, hkv=2), "multiple of hkv"),
    (dict(cu=[0, 16], cp=2, d=48), "head_dim"),
    (dict(cu=[0, 16], cp=2, bm=129), "tile"),
    (dict(cu=[0, 16], cp=2, bn=0), "tile"),
])
def test_plan_rejects_bad_arguments(kw, msg):
    args = dict(cu=[0, 16], cp=2, hq=2, hkv=2, d=32, bm=128, bn=64)
    args.update(kw)
    with pytest.raises(zz.ZZError, match=re.escape(msg)):
        zz.Plan(args["cu"], args["cp"], args["hq"], args["hkv"], args["d"], "f32", args["bm"], args["bn"])


def test_device_calls_need_upload():
    p = zz.Plan([0, 16], 2, 2, 2, 32, "f32")
    L = zz.lib()
    rc = L.zz_varlen_ring_step_fwd(p.handle, 0, 0, ctypes.c_void_p(16), ctypes.c_void_p(16),
                                   ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 0, None)
    assert rc == 7   # ZZ_ERR_STATE: nothing is launched before the plan is bound to a workspace


def test_bad_rank_step_and_merge_flag_are_rejected_before_launch():
    p = zz.Plan([0, 16], 2, 2, 2, 32, "f32")
    L = zz.lib()
    # tiles: rank / step out of range
    n = ctypes.c_int64()
    assert L.zz_plan_tiles(p.handle, 0, 2, 0, None, 0, ctypes.byref(n)) == 1
    assert L.zz_plan_tiles(p.handle, 0, 0, -1, None, 0, ctypes.byref(n)) == 1
    assert L.zz_plan_tiles(p.handle, 3, 0, 0, None, 0, ctypes.byref(n)) == 1
    # merge needs aligned, non-null pointers
    assert L.zz_lse_merge(None, None, None, None, 4, 1, 8, None) == 1
    assert L.zz_lse_merge(ctypes.c_void_p(8), ctypes.c_void_p(16), ctypes.c_void_p(16),
                          ctypes.c_void_p(16), 4, 1, 8, None) == 4
    # a written buffer overlapping another one of the call is rejected before
    # any launch (o: 4 rows x 1 head x 8 = 128 bytes; lse: 16 bytes)
    base = 1 << 20
    rc = L.zz_lse_merge(ctypes.c_void_p(base), ctypes.c_void_p(base + 4096), ctypes.c_void_p(base + 64),
                        ctypes.c_void_p(base + 8192), 4, 1, 8, None)
    assert rc == 1 and L.zz_last_error().decode() == "buffers overlap: o_acc and o_part"
    rc = L.zz_lse_merge(ctypes.c_void_p(base), ctypes.c_void_p(base + 112), ctypes.c_void_p(base + 4096),
                        ctypes.c_void_p(base + 8192), 4, 1, 8, None)
    assert rc == 1 and L.zz_last_error().decode() == "buffers overlap: o_acc and lse_acc"


WORK = {
    "c1": (synthetic.lengths_for(synthetic.WORKLOADS["c1"]), 2),
    "c2": (synthetic.lengths_for(synthetic.WORKLOADS["c2"]), 4),
    "tiny_a": ([8, 24, 16], 4),
    "tiny_b": ([6, 6, 12], 3),
    "tiny_c": ([2, 4, 2], 1),
    "tiny_d": ([64, 32, 96], 2),
}


@pytest.mark.parametrize("name", list(WORK))
def test_zigzag_map_and_local_cu_match_oracle(name):
    lengths, cp = WORK[name]
    cu = synthetic.make_cu_seqlens(lengths)
    p = zz.Plan(cu, cp, 2, 1, 32, "f32")
    assert np.array_equal(p.zigzag_dst(), oracle.zigzag_dst(cu, cp))
    assert np.array_equal(p.local_cu_seqlens(), cu // cp)


@pytest.mark.parametrize("name,bm,bn", [
    ("c1", 128, 64), ("c1", 16, 16), ("c1", 7, 5), ("c2", 128, 64),
    ("tiny_a", 4, 2), ("tiny_b", 1, 1), ("tiny_c", 3, 3), ("tiny_d", 32, 64),
])
def test_forward_tiles_match_oracle_bit_exact(name, bm, bn):
    lengths, cp = WORK[name]
    cu = synthetic.make_cu_seqlens(lengths)
    p = zz.Plan(cu, cp, 2, 2, 32, "f32", bm, bn)
    for r in range(cp):
        for s in range(cp):
            got = p.tiles(r, s, zz.PASS_FWD)
            want = oracle.tiles(cu, cp, r, s, bm, bn)
            assert np.array_equal(got, want), (r, s)


@pytest.mark.parametrize("name", ["c1", "c2", "tiny_a", "tiny_b", "tiny_d"])
def test_backward_tiles_match_oracle_bit_exact(name):
    lengths, cp = WORK[name]
    cu = synthetic.make_cu_seqlens(lengths)
    p = zz.Plan(cu, cp, 4, 2, 64, "bf16")
    for pass_ in (zz.PASS_BWD_DQ, zz.PASS_BWD_DKV):
        bm, bn = p.tile_shape(pass_)
        for r in range(cp):
            for s in range(cp):
                assert np.array_equal(p.tiles(r, s, pass_), oracle.tiles(cu, cp, r, s, bm, bn)), (pass_, r, s)


@pytest.mark.parametrize("name", list(WORK))
def test_pair_counts_balanced_and_exact(name):
    lengths, cp = WORK[name]
    cu = synthetic.make_cu_seqlens(lengths)
    L = np.array(lengths, dtype=np.int64)
    per_rank = int((L * (L + 1)).sum() // (2 * cp))
    p = zz.Plan(cu, cp, 2, 2, 32, "f32", 16, 16)
    for pass_ in (zz.PASS_FWD, zz.PASS_BWD_DQ, zz.PASS_BWD_DKV):
        issued = []
        for r in range(cp):
            u, i = p.pair_counts(r, zz.ALL_STEPS, pass_)
            assert u == per_rank
            assert i >= u
            issued.append(i)
        # chunk-aligned tiles: every rank also issues the same work
        assert len(set(issued)) == 1
    # per step, the useful pairs equal the oracle's visible-pair count
    for r in range(cp):
        for s in range(cp):
            u, _ = p.pair_counts(r, s)
            assert u == int(oracle.step_mask(cu, cp, r, s).sum())


def test_rank_pairs_oracle_agrees_with_plan():
    lengths, cp = WORK["c2"]
    cu = synthetic.make_cu_seqlens(lengths)
    p = zz.Plan(cu, cp, 2, 2, 32, "f32")
    want = oracle.rank_pairs(cu, cp)
    got = np.array([p.pair_counts(r)[0] for r in range(cp)])
    assert np.array_equal(got, want)
    assert np.array_equal(p.rank_useful_pairs(), want)


def test_contiguous_split_would_be_unbalanced():
    """What zigzag fixes: with a plain contiguous split, the last rank holds
    the latest tokens and does most of the causal work (MiniMax-01 issue #6;
    ring-attention-pytorch issue #20)."""
    for cp, want in ((2, 1.5), (4, 1.75), (8, 1.875)):
        L = 2 * cp * 512
        work = []
        for r in range(cp):
            a = np.arange(r * L // cp, (r + 1) * L // cp)
            work.append(int((a + 1).sum()))
        ratio = max(work) / np.mean(work)
        assert abs(ratio - want) < 2e-3
        p = zz.Plan([0, L], cp, 1, 1, 32, "f32")
        zzw = [p.pair_counts(r)[0] for r in range(cp)]
        assert max(zzw) == min(zzw)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_gathered_tiles_are_the_union_of_ring_steps(name):
    """The all-gather walks list exactly the tiles of the ring steps (pinned
    above against the oracle), moved to global zigzag rows: rank r's queries
    against every shard j = (r - s) mod cp, and shard j's keys against every
    rank r = (j + s) mod cp."""
    w = synthetic.WORKLOADS[name]
    cu = synthetic.cu_seqlens_for(w)
    plan = zz.Plan(cu, w.cp, w.hq, w.hkv, w.d, w.dtype)
    n = plan.total // w.cp
    for pass_ in (zz.PASS_FWD, zz.PASS_BWD_DQ, zz.PASS_BWD_DKV):
        for owner in range(w.cp):
            parts = []
            for s in range(w.cp):
                r, j = ((owner + s) % w.cp, owner) if pass_ == zz.PASS_BWD_DKV else (owner, (owner - s) % w.cp)
                t = plan.tiles(r, s, pass_).astype(np.int64)
                t[:, 0:2] += r * n
                t[:, 2:4] += j * n
                parts.append(t)
            want = np.concatenate(parts)
            want = want[np.lexsort((want[:, 2], want[:, 0]))]
            got = plan.gathered_tiles(owner, pass_)
            assert np.array_equal(got, want), (pass_, owner)
