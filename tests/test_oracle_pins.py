"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each test ties one oracle function to a fact the pages or the mathematics fix:
the hand-derived worked examples of the zigzag split, the split written with
torch's chunk/cat, torch's own attention routine in float64, a dense -inf bias
matrix, closed forms on special inputs, finite differences, and exact counts.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "zigzag_extract_local.txt")


# ---------------------------------------------------------------- helpers

def split_like_extract_local(x: torch.Tensor, rank: int, world: int) -> torch.Tensor:
    """The rows a rank keeps under the zigzag split that ring-attention-pytorch
    issue #20 ("Zigzag attention support?") describes: with 2*world equal
    chunks of c rows, rank r holds chunk r and then chunk 2*world-1-r, i.e. the
    row indices [r*c, (r+1)*c) followed by [(2*world-1-r)*c, (2*world-r)*c)."""
    c = x.shape[0] // (2 * world)
    mirror = 2 * world - 1 - rank
    idx = torch.cat([torch.arange(rank * c, (rank + 1) * c), torch.arange(mirror * c, (mirror + 1) * c)])
    return x.index_select(0, idx)


def packed_split(lengths, world):
    """Per-sequence split, ranks stacked one after the other: the packed token
    id found at every zigzag row."""
    ids = torch.arange(sum(lengths))
    seqs = ids.split(list(lengths))
    rows = []
    for r in range(world):
        for s in seqs:
            rows.append(split_like_extract_local(s, r, world))
    return torch.cat(rows).numpy()


def torch_reference_fwd(q, k, v, lengths, scale):
    """float64 attention per sequence with torch's SDPA (causal), GQA by
    repeating K/V heads over contiguous groups.  Returns o [T,hq,d], lse [hq,T]."""
    q = torch.as_tensor(q, dtype=torch.float64)
    k = torch.as_tensor(k, dtype=torch.float64)
    v = torch.as_tensor(v, dtype=torch.float64)
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    outs, lses = [], []
    start = 0
    for L in lengths:
        qs = q[start:start + L].transpose(0, 1)                      # [hq,L,d]
        ks = k[start:start + L].repeat_interleave(G, dim=1).transpose(0, 1)
        vs = v[start:start + L].repeat_interleave(G, dim=1).transpose(0, 1)
        o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, is_causal=True, scale=scale)
        s = (qs @ ks.transpose(1, 2)) * scale
        s = s.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        lses.append(torch.logsumexp(s, dim=-1))                     # [hq,L]
        outs.append(o.transpose(0, 1))
        start += L
    return torch.cat(outs).numpy(), torch.cat(lses, dim=1).numpy()


def dense_bias_fwd(q, k, v, lengths, scale):
    """Brute force with a dense T x T additive bias: 0 where a key is visible,
    -inf across packed examples and above the diagonal (EasyDeL issue #129:
    packed examples must not see each other, done with a -inf bias)."""
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    T, hq, d = q.shape
    G = hq // k.shape[1]
    seg = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.arange(T)
    bias = np.where((seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None]), 0.0, -np.inf)
    o = np.empty_like(q)
    lse = np.empty((hq, T))
    for h in range(hq):
        s = q[:, h, :] @ k[:, h // G, :].T * scale + bias
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        o[:, h, :] = (e @ v[:, h // G, :]) / e.sum(axis=1, keepdims=True)
        lse[h] = m[:, 0] + np.log(e.sum(axis=1))
    return o, lse


def rand_inputs(seed, lengths, hq, hkv, d, with_do=False):
    T = sum(lengths)
    return synthetic.randn_qkv(seed, T, hq, hkv, d, "f32", with_do=with_do)


# ---------------------------------------------------------------- zigzag map

def test_zigzag_golden_examples():
    n = 0
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = dict(kv.split("=") for kv in line.split())
        lengths = [int(x) for x in f["lengths"].split(",")]
        world, rank = int(f["world"]), int(f["rank"])
        want = [int(x) for x in f["tokens"].split(",")]
        cu = synthetic.make_cu_seqlens(lengths)
        dst = oracle.zigzag_dst(cu, world)
        T = sum(lengths)
        src = np.empty(T, dtype=np.int64)
        src[dst] = np.arange(T)
        per = T // world
        assert list(src[rank * per:(rank + 1) * per]) == want, line
        n += 1
    assert n >= 9


@pytest.mark.parametrize("world", [1, 2, 3, 4, 8, 16])
def test_zigzag_single_sequence_is_extract_local(world):
    T = 2 * world * 7
    dst = oracle.zigzag_dst([0, T], world)
    src = np.empty(T, dtype=np.int64)
    src[dst] = np.arange(T)
    ids = torch.arange(T)
    want = torch.cat([split_like_extract_local(ids, r, world) for r in range(world)]).numpy()
    assert np.array_equal(src, want)


@pytest.mark.parametrize("seed", range(12))
def test_zigzag_packed_is_per_sequence_split(seed):
    rng = np.random.default_rng(seed)
    world = int(rng.choice([1, 2, 3, 4, 8]))
    lengths = synthetic.random_lengths(seed, 6, 5, world)
    cu = synthetic.make_cu_seqlens(lengths)
    dst = oracle.zigzag_dst(cu, world)
    T = sum(lengths)
    assert sorted(dst.tolist()) == list(range(T))            # bijection
    src = np.empty(T, dtype=np.int64)
    src[dst] = np.arange(T)
    assert np.array_equal(src, packed_split(lengths, world))
    x = rng.standard_normal((T, 3)).astype(np.float32)
    assert np.array_equal(oracle.unpermute(oracle.permute(x, cu, world), cu, world), x)
    if world == 1:
        assert np.array_equal(dst, np.arange(T))


def test_zigzag_rejects_bad_lengths():
    assert not oracle.check_lengths([0, 12], 4)
    assert not oracle.check_lengths([0, 16, 16], 4)
    assert oracle.check_lengths([0, 16, 24], 2)
    with pytest.raises(ValueError):
        oracle.zigzag_dst([0, 10], 2)


# ---------------------------------------------------------------- forward

@pytest.mark.parametrize("lengths,hq,hkv,d", [
    ((96, 64, 96), 2, 2, 32),
    ((8, 24, 16), 4, 2, 16),
    ((40,), 8, 1, 8),
    ((4, 4, 12, 20), 3, 3, 5),
])
def test_fwd_matches_torch_sdpa(lengths, hq, hkv, d):
    q, k, v = rand_inputs(11, lengths, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.attn_fwd(q, k, v, synthetic.make_cu_seqlens(lengths), scale)
    o_ref, lse_ref = torch_reference_fwd(q, k, v, lengths, scale)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_fwd_matches_dense_bias(seed):
    lengths = synthetic.random_lengths(seed, 5, 6, 2)
    q, k, v = rand_inputs(seed, lengths, 4, 2, 8)
    o, lse = oracle.attn_fwd(q, k, v, synthetic.make_cu_seqlens(lengths), 0.3)
    o_ref, lse_ref = dense_bias_fwd(q, k, v, lengths, 0.3)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - lse_ref).max() < 1e-12


def test_fwd_zero_query_closed_form():
    """Q = 0: every visible key gets the same weight, so O is the running mean
    of V over the sequence so far and LSE = ln(number of visible keys)."""
    lengths = [12, 20, 8]
    _, k, v = rand_inputs(3, lengths, 4, 2, 6)
    q = torch.zeros((sum(lengths), 4, 6))
    o, lse = oracle.attn_fwd(q, k, v, synthetic.make_cu_seqlens(lengths), 0.5)
    vv = v.double().numpy()
    start = 0
    for L in lengths:
        n = np.arange(1, L + 1)
        mean = np.cumsum(vv[start:start + L], axis=0) / n[:, None, None]      # [L,hkv,d]
        for h in range(4):
            assert np.abs(o[start:start + L, h] - mean[:, h // 2]).max() < 1e-12
            assert np.abs(lse[h, start:start + L] - np.log(n)).max() < 1e-12
        start += L


def test_fwd_constant_value_and_shift():
    lengths = [16, 8]
    q, k, v = rand_inputs(5, lengths, 2, 1, 4)
    cu = synthetic.make_cu_seqlens(lengths)
    o, lse = oracle.attn_fwd(q, k, torch.full_like(v, 1.75), cu, 0.5)
    assert np.abs(o - 1.75).max() < 1e-12
    # adding u to every key adds scale*<q,u> to every score of a row:
    # O is unchanged and LSE moves by exactly that amount.
    # keys rounded to bf16 and small entries zeroed, so k + u is exact in fp32
    k = synthetic.round_bf16(k)
    k[k.abs() < 2.0 ** -10] = 0.0
    u = torch.tensor([0.5, -1.0, 2.0, 0.25])
    assert torch.equal((k + u).double(), k.double() + u.double())
    o0, l0 = oracle.attn_fwd(q, k, v, cu, 0.5)
    o1, l1 = oracle.attn_fwd(q, k + u, v, cu, 0.5)
    shift = 0.5 * (q.double() @ u.double()).numpy().T            # [hq,T]
    assert np.abs(o1 - o0).max() < 1e-12
    assert np.abs(l1 - l0 - shift).max() < 1e-12


def test_fwd_rows_equal_full():
    lengths = [24, 40]
    q, k, v = rand_inputs(7, lengths, 4, 2, 8)
    cu = synthetic.make_cu_seqlens(lengths)
    o, lse = oracle.attn_fwd(q, k, v, cu, 0.35)
    rows = np.array([0, 5, 23, 24, 63, 40])
    heads = np.array([0, 3, 1, 2, 3, 0])
    orows, lrows = oracle.attn_fwd_rows(q, k, v, cu, 0.35, rows, heads)
    assert np.array_equal(orows, o[rows, heads])
    assert np.array_equal(lrows, lse[heads, rows])


# ---------------------------------------------------------------- ring steps and merge

def test_lse_merge_closed_forms():
    rng = np.random.default_rng(0)
    oa = rng.standard_normal((3, 2, 4)); ob = rng.standard_normal((3, 2, 4))
    a = rng.standard_normal((2, 3))
    o, l = oracle.lse_merge(oa, a, ob, a)           # equal weights: the mean
    assert np.abs(o - 0.5 * (oa + ob)).max() < 1e-14
    assert np.abs(l - (a + math.log(2.0))).max() < 1e-14
    ninf = np.full((2, 3), -np.inf)
    o, l = oracle.lse_merge(oa, a, np.zeros_like(ob), ninf)     # identity element
    assert np.array_equal(o, oa) and np.array_equal(l, a)
    o, l = oracle.lse_merge(np.zeros_like(oa), ninf, np.zeros_like(ob), ninf)
    assert np.all(o == 0) and np.all(l == -np.inf)
    # weights e^a : e^b = 1 : 3
    b = a + math.log(3.0)
    o, l = oracle.lse_merge(oa, a, ob, b)
    assert np.abs(o - (0.25 * oa + 0.75 * ob)).max() < 1e-14
    assert np.abs(l - (a + math.log(4.0))).max() < 1e-14


@pytest.mark.parametrize("seed", range(3))
def test_merge_over_random_key_partitions_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    lengths = synthetic.random_lengths(seed, 4, 5, 2)
    T = sum(lengths)
    q, k, v = rand_inputs(seed, lengths, 4, 2, 8)
    seg = np.repeat(np.arange(len(lengths)), lengths)
    pos = np.arange(T)
    full = (seg[:, None] == seg[None, :]) & (pos[None, :] <= pos[:, None])
    o_ref, l_ref = oracle.masked_attn(q, k, v, full, 0.4)
    parts = rng.integers(0, 4, size=T)     # key -> part; some parts may be empty for a row
    o = np.zeros_like(o_ref)
    lse = np.full_like(l_ref, -np.inf)
    for p in rng.permutation(4):
        op, lp = oracle.masked_attn(q, k, v, full & (parts[None, :] == p), 0.4)
        o, lse = oracle.lse_merge(o, lse, op, lp)
    assert np.abs(o - o_ref).max() < 1e-12
    assert np.abs(lse - l_ref).max() < 1e-12
    o2, l2 = oracle.attn_fwd(q, k, v, synthetic.make_cu_seqlens(lengths), 0.4)
    assert np.abs(o_ref - o2).max() < 1e-12 and np.abs(l_ref - l2).max() < 1e-12


@pytest.mark.parametrize("name_or_lengths,cp", [("c1", 2), ((8, 24, 16), 4), ((48,), 3), ((6, 6, 12), 3)])
def test_ring_steps_merge_to_full_attention(name_or_lengths, cp):
    if isinstance(name_or_lengths, str):
        w = synthetic.WORKLOADS[name_or_lengths]
        lengths, hq, hkv, d = synthetic.lengths_for(w), w.hq, w.hkv, w.d
    else:
        lengths, hq, hkv, d = list(name_or_lengths), 4, 2, 8
    cu = synthetic.make_cu_seqlens(lengths)
    T = sum(lengths)
    q, k, v = rand_inputs(2, lengths, hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    qz, kz, vz = (oracle.permute(x.numpy(), cu, cp) for x in (q, k, v))
    o_full, l_full = oracle.attn_fwd(q, k, v, cu, scale)
    dst = oracle.zigzag_dst(cu, cp)
    n = T // cp
    rng = np.random.default_rng(cp)
    for r in range(cp):
        o = np.zeros((n, hq, d)); lse = np.full((hq, n), -np.inf)
        for s in rng.permutation(cp):
            op, lp = oracle.ring_step_fwd(qz, kz, vz, cu, cp, r, int(s), scale)
            o, lse = oracle.lse_merge(o, lse, op, lp)
        rows = np.nonzero((dst >= r * n) & (dst < (r + 1) * n))[0]       # packed rows of rank r
        loc = dst[rows] - r * n
        assert np.abs(o[loc] - o_full[rows]).max() < 1e-12
        assert np.abs(lse[:, loc] - l_full[:, rows]).max() < 1e-12


def test_step_mask_from_positions():
    lengths = [8, 24, 16]
    cp = 4
    cu = synthetic.make_cu_seqlens(lengths)
    src = packed_split(lengths, cp)          # pinned to extract_local above
    seg = np.repeat(np.arange(len(lengths)), lengths)
    n = sum(lengths) // cp
    for r in range(cp):
        for s in range(cp):
            j = (r - s) % cp
            a = src[r * n:(r + 1) * n][:, None]
            b = src[j * n:(j + 1) * n][None, :]
            want = (seg[a] == seg[b]) & (b <= a)
            assert np.array_equal(oracle.step_mask(cu, cp, r, s).astype(bool), want)


# ---------------------------------------------------------------- balance and tiles

@pytest.mark.parametrize("name", ["c1", "c2"])
def test_rank_pairs_closed_form(name):
    """Per-sequence zigzag gives every rank exactly sum_i L_i (L_i + 1) / (2 CP)
    visible pairs, the balance the split is for."""
    w = synthetic.WORKLOADS[name]
    L = np.array(synthetic.lengths_for(w), dtype=np.int64)
    got = oracle.rank_pairs(synthetic.cu_seqlens_for(w), w.cp)
    assert np.all(got == (L * (L + 1)).sum() // (2 * w.cp))


def closed_form_tiles(lengths, cp, rank, step, bm, bn):
    """Tiles from chunk geometry: within one sequence, query chunk a and key
    chunk b are fully visible when a > b, invisible when a < b, and lower
    triangular when a == b (offset o sees offsets <= o)."""
    j = (rank - step) % cp
    out = []
    qbase = 0
    for L in lengths:
        c = L // (2 * cp)
        qch = [(rank, qbase), (2 * cp - 1 - rank, qbase + c)]
        kch = [(j, qbase), (2 * cp - 1 - j, qbase + c)]
        for qa, qs in qch:
            for a0 in range(0, c, bm):
                a1 = min(a0 + bm, c)
                for kb, ks in kch:
                    for b0 in range(0, c, bn):
                        b1 = min(b0 + bn, c)
                        if qa > kb or (qa == kb and b1 - 1 <= a0):
                            kind = 1
                        elif qa < kb or b0 > a1 - 1:
                            continue
                        else:
                            kind = 2
                        out.append((qs + a0, qs + a1, ks + b0, ks + b1, kind))
        qbase += 2 * c
    return sorted(out)


@pytest.mark.parametrize("lengths,cp,bm,bn", [
    ((96, 64, 96), 2, 16, 16), ((96, 64, 96), 2, 128, 64), ((8, 24, 16), 4, 4, 2),
    ((48,), 3, 5, 3), ((6, 6, 12), 3, 1, 1), ((64, 32), 2, 8, 32),
])
def test_tiles_match_chunk_geometry(lengths, cp, bm, bn):
    cu = synthetic.make_cu_seqlens(lengths)
    for r in range(cp):
        for s in range(cp):
            got = [tuple(int(x) for x in t) for t in oracle.tiles(cu, cp, r, s, bm, bn)]
            assert got == closed_form_tiles(list(lengths), cp, r, s, bm, bn), (r, s)


def test_tiles_cover_visible_pairs_exactly():
    lengths = [8, 24, 16]
    cp, bm, bn = 4, 4, 3
    cu = synthetic.make_cu_seqlens(lengths)
    for r in range(cp):
        for s in range(cp):
            m = oracle.step_mask(cu, cp, r, s)
            cover = np.zeros_like(m, dtype=np.int32)
            for q0, q1, k0, k1, kind in oracle.tiles(cu, cp, r, s, bm, bn):
                blk = m[q0:q1, k0:k1]
                assert blk.any()
                assert (kind == 1) == bool(blk.all())
                cover[q0:q1, k0:k1] += 1
            assert np.all(cover[m.astype(bool)] == 1)


# ---------------------------------------------------------------- backward

def torch_reference_bwd(q, k, v, do, lengths, scale):
    q = torch.as_tensor(q, dtype=torch.float64).clone().requires_grad_(True)
    k = torch.as_tensor(k, dtype=torch.float64).clone().requires_grad_(True)
    v = torch.as_tensor(v, dtype=torch.float64).clone().requires_grad_(True)
    hq, hkv = q.shape[1], k.shape[1]
    G = hq // hkv
    outs = []
    start = 0
    for L in lengths:
        qs = q[start:start + L].transpose(0, 1)
        ks = k[start:start + L].repeat_interleave(G, dim=1).transpose(0, 1)
        vs = v[start:start + L].repeat_interleave(G, dim=1).transpose(0, 1)
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            qs, ks, vs, is_causal=True, scale=scale).transpose(0, 1))
        start += L
    o = torch.cat(outs)
    (o * torch.as_tensor(do, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("lengths,hq,hkv,d", [((16, 8, 24), 4, 2, 8), ((32,), 8, 1, 16), ((12, 4), 2, 2, 4)])
def test_bwd_matches_torch_autograd(lengths, hq, hkv, d):
    q, k, v, do = rand_inputs(13, lengths, hq, hkv, d, with_do=True)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, synthetic.make_cu_seqlens(lengths), scale)
    rq, rk, rv = torch_reference_bwd(q, k, v, do, lengths, scale)
    assert np.abs(dq - rq).max() < 1e-11
    assert np.abs(dk - rk).max() < 1e-11
    assert np.abs(dv - rv).max() < 1e-11


def test_bwd_finite_differences():
    lengths = [6, 4]
    hq, hkv, d = 2, 1, 3
    q, k, v, do = (x.double() for x in rand_inputs(17, lengths, hq, hkv, d, with_do=True))
    cu = synthetic.make_cu_seqlens(lengths)
    scale = 0.7
    dq, dk, dv = oracle.attn_bwd(q.float(), k.float(), v.float(), do.float(), cu, scale)
    # loss = <O, dO>; central differences in float64 through the oracle's forward
    # (inputs are float32, so perturb by exactly representable steps).
    eps = 2.0 ** -10

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq.float(), kk.float(), vv.float(), cu, scale)
        return float((o * do.numpy()).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0), (3, 1 if name == "q" else 0, 2), (7, 0, 1), (9, 0, 0)]:
            xp = x.clone(); xp[idx] += eps
            xm = x.clone(); xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 2e-5, (name, idx, fd, g[idx])


def test_bwd_zero_key_closed_form():
    """K = 0: uniform weights 1/n over the visible keys, so dQ = 0 and
    dV_k = sum over later rows q of the group of dO_q / n_q."""
    lengths = [10, 6]
    hq, hkv, d = 4, 2, 5
    q, _, v, do = rand_inputs(19, lengths, hq, hkv, d, with_do=True)
    k = torch.zeros((sum(lengths), hkv, d))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, synthetic.make_cu_seqlens(lengths), 0.6)
    assert np.abs(dq).max() < 1e-14
    dod = do.double().numpy()
    start = 0
    for L in lengths:
        n = np.arange(1, L + 1, dtype=np.float64)
        for g in range(hkv):
            contrib = dod[start:start + L, 2 * g:2 * g + 2].sum(axis=1) / n[:, None]   # [L,d]
            want = np.cumsum(contrib[::-1], axis=0)[::-1]
            assert np.abs(dv[start:start + L, g] - want).max() < 1e-12
        start += L


def test_bwd_dq_rows_equal_full():
    lengths = [16, 24]
    q, k, v, do = rand_inputs(23, lengths, 4, 2, 8, with_do=True)
    cu = synthetic.make_cu_seqlens(lengths)
    dq, _, _ = oracle.attn_bwd(q, k, v, do, cu, 0.35)
    rows = np.array([0, 15, 16, 39, 20])
    heads = np.array([1, 0, 3, 2, 1])
    got = oracle.attn_bwd_dq_rows(q, k, v, do, cu, 0.35, rows, heads)
    assert np.abs(got - dq[rows, heads]).max() < 1e-14


@pytest.mark.parametrize("lengths,hq,hkv,d", [((16, 8, 24), 4, 2, 8), ((32,), 8, 1, 16), ((12, 4), 2, 2, 4)])
def test_bwd_dkv_rows_match_torch_autograd(lengths, hq, hkv, d):
    """Every (key row, key/value head) of small packings against torch's
    autograd through SDPA in float64."""
    q, k, v, do = rand_inputs(29, lengths, hq, hkv, d, with_do=True)
    scale = 1.0 / math.sqrt(d)
    T = sum(lengths)
    rows = np.repeat(np.arange(T), hkv)
    kvh = np.tile(np.arange(hkv), T)
    dk, dv = oracle.attn_bwd_dkv_rows(q, k, v, do, synthetic.make_cu_seqlens(lengths), scale, rows, kvh)
    _, rk, rv = torch_reference_bwd(q, k, v, do, lengths, scale)
    assert np.abs(dk - rk[rows, kvh]).max() < 1e-11
    assert np.abs(dv - rv[rows, kvh]).max() < 1e-11


def test_bwd_dkv_rows_zero_key_closed_form():
    """K = 0: every visible key has weight 1/n_q (n_q = q - start + 1), O_q is
    the running mean of V and D_q = <dO_q, O_q>, so per sequence and group
      dV_k = sum_{q>=k} sum_h dO_q / n_q,
      dK_k = scale * [ (sum_{q>=k} sum_h Q_q dO_q^T / n_q) V_k - sum_{q>=k} sum_h D_q Q_q / n_q ],
    written here with reverse cumulative sums."""
    lengths = [10, 6, 14]
    hq, hkv, d = 4, 2, 5
    G = hq // hkv
    q, _, v, do = (x.double().numpy() for x in rand_inputs(31, lengths, hq, hkv, d, with_do=True))
    k = np.zeros((sum(lengths), hkv, d))
    scale = 0.45
    cu = synthetic.make_cu_seqlens(lengths)
    T = sum(lengths)
    rows = np.repeat(np.arange(T), hkv)
    kvh = np.tile(np.arange(hkv), T)
    dk, dv = oracle.attn_bwd_dkv_rows(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                                      do.astype(np.float32), cu, scale, rows, kvh)
    q, v, do = q.astype(np.float32).astype(np.float64), v.astype(np.float32).astype(np.float64), \
        do.astype(np.float32).astype(np.float64)
    start = 0
    for L in lengths:
        n = np.arange(1, L + 1, dtype=np.float64)
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            vs = v[start:start + L, g]                                         # [L,d]
            o = np.cumsum(vs, axis=0) / n[:, None]                             # running mean
            dos = do[start:start + L, hs]                                      # [L,G,d]
            qs = q[start:start + L, hs]
            D = (dos * o[:, None, :]).sum(-1)                                  # [L,G]
            rev = lambda x: np.cumsum(x[::-1], axis=0)[::-1]
            want_dv = rev(dos.sum(1) / n[:, None])
            A = rev(np.einsum("lgi,lgj->lij", qs, dos) / n[:, None, None])     # [L,d,d]
            B = rev((D[:, :, None] * qs).sum(1) / n[:, None])                  # [L,d]
            want_dk = scale * (np.einsum("lij,lj->li", A, vs) - B)
            sel = (rows >= start) & (rows < start + L) & (kvh == g)
            assert np.abs(dv[sel] - want_dv).max() < 1e-12
            assert np.abs(dk[sel] - want_dk).max() < 1e-12
        start += L


def test_bwd_dkv_rows_heads_with_zero_upstream_add_nothing():
    """The head subset a caller may pass is exact when dO vanishes on the
    other heads: full-group sums equal the subset's, and both equal the full
    backward's rows (sampled keys, first and last of each sequence included)."""
    lengths = [24, 40]
    hq, hkv, d = 8, 2, 8
    q, k, v, do = rand_inputs(37, lengths, hq, hkv, d, with_do=True)
    do = do.clone()
    keep = [1, 6]
    for h in range(hq):
        if h not in keep:
            do[:, h] = 0
    cu = synthetic.make_cu_seqlens(lengths)
    rows = np.array([0, 23, 24, 63, 5, 40, 12])
    kvh = np.array([0, 1, 1, 0, 1, 0, 0])
    full = oracle.attn_bwd_dkv_rows(q, k, v, do, cu, 0.3, rows, kvh)
    sub = oracle.attn_bwd_dkv_rows(q, k, v, do, cu, 0.3, rows, kvh, heads_on=keep)
    _, rk, rv = torch_reference_bwd(q, k, v, do, lengths, 0.3)
    for a, b, ref in ((full[0], sub[0], rk), (full[1], sub[1], rv)):
        assert np.array_equal(a, b)
        assert np.abs(a - ref[rows, kvh]).max() < 1e-11


def test_bwd_dkv_rows_with_forward_row_stats():
    """Row statistics taken from the oracle's forward (LSE, and D = <dO, O>)
    give the same dK, dV as the ones the function computes itself
    (D = sum_k P dP): the two definitions of D agree."""
    lengths = [20, 44]
    hq, hkv, d = 4, 2, 8
    q, k, v, do = rand_inputs(41, lengths, hq, hkv, d, with_do=True)
    cu = synthetic.make_cu_seqlens(lengths)
    o, lse = oracle.attn_fwd(q, k, v, cu, 0.3)
    dsum = (o * do.double().numpy()).sum(-1).T.copy()          # [hq, T]
    rows = np.array([0, 19, 20, 63, 7, 33, 50])
    kvh = np.array([1, 0, 1, 1, 0, 0, 1])
    own = oracle.attn_bwd_dkv_rows(q, k, v, do, cu, 0.3, rows, kvh)
    given = oracle.attn_bwd_dkv_rows(q, k, v, do, cu, 0.3, rows, kvh, row_stats=(lse, dsum))
    for a, b in zip(own, given):
        assert np.abs(a - b).max() < 1e-12
