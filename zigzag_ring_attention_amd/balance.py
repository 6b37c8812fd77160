"""Packing-aware balance study: per-rank useful and issued attention work of
ways to split a packed batch of documents over CP ranks.

    python -m zigzag_ring_attention_amd.balance [--bm 128 --bn 64]

The pages raise the question this answers.  Packing documents of very
different lengths into one micro-batch unbalances ring attention, and the
fix suggested there is on the data side: keep long and short sequences out
of the same micro-batch (MiniMax-01 issue #6, "Question about varlen ring
attention").  Zigzag balances the causal mask of one sequence by giving rank
r chunks r and 2CP-1-r (ring-attention-pytorch issue #20, "Zigzag attention
support?"), and it was noted to be troublesome with packing; a different
reordering is needed for packed data (MaxText PR #1133).  The layout the
kernels use applies the zigzag split to every document separately.

Strategies (each gives every rank a list of contiguous row ranges, "chunks",
of the packed stream):
  doc_zigzag     every document cut into 2CP chunks; rank r holds chunks r and
                 2CP-1-r of every document (the layout of the kernels);
  stream_zigzag  the packed stream cut into 2CP equal chunks, rank r holds
                 chunks r and 2CP-1-r, document boundaries ignored;
  contiguous     rank r holds stream rows [r T/CP, (r+1) T/CP) (plain ring).
and, on top of any of them, length-bucketed micro-batches: the documents,
sorted by length, are packed into micro-batches of about equal token count
and each micro-batch is split separately.

Work of rank r:
  useful  = sum over its query rows q of the keys q sees (same document, not
            later): position of q in its document + 1;
  issued  = area of the BM x BN tiles holding at least one visible pair, with
            the query rows of each of the rank's chunks and the key rows of
            each chunk of the stream cut into tiles that restart at every
            chunk start (in a ring, rank r meets every other rank's chunks).
Both are summed over all ring steps; the balance is max over ranks / mean.
"""
from __future__ import annotations

import argparse
import sys
from typing import Dict, List, Tuple

import numpy as np

Chunks = List[Tuple[int, int]]   # (first stream row, length)


def doc_zigzag(cu: np.ndarray, cp: int) -> List[Chunks]:
    out: List[Chunks] = [[] for _ in range(cp)]
    for i in range(len(cu) - 1):
        s, L = int(cu[i]), int(cu[i + 1] - cu[i])
        if L % (2 * cp):
            raise ValueError("document %d: length %d is not a multiple of 2*cp" % (i, L))
        c = L // (2 * cp)
        for r in range(cp):
            out[r] += [(s + r * c, c), (s + (2 * cp - 1 - r) * c, c)]
    return out


def stream_zigzag(cu: np.ndarray, cp: int) -> List[Chunks]:
    T = int(cu[-1])
    if T % (2 * cp):
        raise ValueError("total %d is not a multiple of 2*cp" % T)
    c = T // (2 * cp)
    return [[(r * c, c), ((2 * cp - 1 - r) * c, c)] for r in range(cp)]


def contiguous(cu: np.ndarray, cp: int) -> List[Chunks]:
    T = int(cu[-1])
    if T % cp:
        raise ValueError("total %d is not a multiple of cp" % T)
    n = T // cp
    return [[(r * n, n)] for r in range(cp)]


STRATEGIES = {"doc_zigzag": doc_zigzag, "stream_zigzag": stream_zigzag, "contiguous": contiguous}


def useful_per_rank(cu: np.ndarray, ranks: List[Chunks]) -> np.ndarray:
    """Visible (query, key) pairs of every rank's query rows."""
    T = int(cu[-1])
    doc = np.searchsorted(cu, np.arange(T), side="right") - 1
    seen = np.arange(T, dtype=np.int64) - cu[doc] + 1          # keys row q sees
    pref = np.concatenate([[0], np.cumsum(seen)])
    return np.array([sum(int(pref[s + n] - pref[s]) for s, n in ch) for ch in ranks], dtype=np.int64)


def _tiles(chunks: Chunks, step: int) -> np.ndarray:
    t = [(s + o, s + min(o + step, n)) for s, n in chunks for o in range(0, n, step)]
    return np.array(t, dtype=np.int64).reshape(-1, 2)


def issued_per_rank(cu: np.ndarray, ranks: List[Chunks], bm: int, bn: int) -> np.ndarray:
    """Area of the visited tiles of every rank (query tiles of its chunks x
    key tiles of every chunk of the stream)."""
    cu = np.asarray(cu, dtype=np.int64)
    keys = _tiles([c for ch in ranks for c in ch], bn)          # every chunk of the stream
    k0, k1 = keys[:, 0], keys[:, 1]
    out = []
    for ch in ranks:
        total = 0
        for q0, q1 in _tiles(ch, bm):
            # a key tile is visited when some document d inside the query tile
            # has a key row in [k0, k1) at or before its last query row in the
            # tile: max(k0, start_d) <= min(k1, min(q1, end_d)) - 1
            d0 = int(np.searchsorted(cu, q0, side="right") - 1)
            d1 = int(np.searchsorted(cu, q1 - 1, side="right") - 1)
            vis = np.zeros(len(k0), dtype=bool)
            for d in range(d0, d1 + 1):
                qmax = min(int(q1), int(cu[d + 1])) - 1
                vis |= np.maximum(k0, cu[d]) <= np.minimum(k1 - 1, qmax)
            total += int((q1 - q0) * (k1 - k0)[vis].sum())
        out.append(total)
    return np.array(out, dtype=np.int64)


def buckets(lengths: List[int], n_mb: int) -> List[List[int]]:
    """Documents sorted by length, cut into n_mb micro-batches of about equal
    token count (long documents together, short ones together)."""
    order = sorted(lengths, reverse=True)
    target = sum(lengths) / n_mb
    out: List[List[int]] = [[]]
    acc = 0
    for L in order:
        if acc >= target * len(out) and len(out) < n_mb:
            out.append([])
        out[-1].append(L)
        acc += L
    return out


def study(lengths: List[int], cp: int, bm: int, bn: int, strategy: str, n_mb: int = 1) -> Dict[str, float]:
    """Balance of `strategy` over `cp` ranks, optionally on length-bucketed
    micro-batches (n_mb > 1): work summed over the micro-batches per rank."""
    groups = buckets(lengths, n_mb) if n_mb > 1 else [list(lengths)]
    u = np.zeros(cp, dtype=np.int64)
    iss = np.zeros(cp, dtype=np.int64)
    worst_mb = 1.0
    for g in groups:
        cu = np.concatenate([[0], np.cumsum(np.asarray(g, dtype=np.int64))])
        ranks = STRATEGIES[strategy](cu, cp)
        ug = useful_per_rank(cu, ranks)
        ig = issued_per_rank(cu, ranks, bm, bn)
        u += ug
        iss += ig
        worst_mb = max(worst_mb, float(ig.max() / ig.mean()))
    return {
        "useful_max_over_mean": float(u.max() / u.mean()),
        "issued_max_over_mean": float(iss.max() / iss.mean()),
        "tile_efficiency": float(u.sum() / iss.sum()),
        "worst_microbatch_issued_max_over_mean": worst_mb,
        "useful_pairs": int(u.sum()),
    }


def main(argv=None) -> int:
    import synthetic
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--bm", type=int, default=128)
    ap.add_argument("--bn", type=int, default=64)
    args = ap.parse_args(argv)
    # two long documents packed with many short ones (the mix the pages warn
    # about): 2 x 16384 plus log-uniform [64, 1024] lengths up to 65536 tokens
    mixed = [16384, 16384] + synthetic.lengths_loguniform(9, 32768, 64, 1024, 16)
    mixes = [("c2 (8192 tokens, lengths ~U[128,4096])", synthetic.lengths_for(synthetic.WORKLOADS["c2"]), 4),
             ("c4 (65536 tokens, lengths log-U[64,16384])", synthetic.lengths_for(synthetic.WORKLOADS["c4"]), 8),
             ("2 x 16384 + short log-U[64,1024] (65536 tokens)", mixed, 8)]
    print("| length mix | CP | split | micro-batches | useful max/mean | issued max/mean | tile efficiency |")
    print("|---|---|---|---|---|---|---|")
    for label, lengths, cp in mixes:
        for strategy in STRATEGIES:
            for n_mb in (1, 4):
                r = study(lengths, cp, args.bm, args.bn, strategy, n_mb)
                print("| %s | %d | %s | %d | %.3f | %.3f | %.3f |" % (
                    label, cp, strategy, n_mb, r["useful_max_over_mean"], r["issued_max_over_mean"],
                    r["tile_efficiency"]))
    return 0


if __name__ == "__main__":
    sys.exit(main())
