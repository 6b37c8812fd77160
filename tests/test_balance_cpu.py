"""The packing-aware balance study, pinned: the document-level zigzag counts
equal the planner's own per-rank pair counts, 1x1 tiles issue exactly the
useful pairs, a contiguous split of one causal sequence has the closed-form
imbalance (2CP-1)/CP, and every split does the same total useful work."""
import numpy as np
import pytest

import synthetic
from zigzag_ring_attention_amd import balance as B

zz = pytest.importorskip("zigzag_ring_attention_amd")


@pytest.mark.parametrize("lengths,cp,bm,bn", [
    (tuple(synthetic.lengths_for(synthetic.WORKLOADS["c4"])), 8, 128, 64),
    ((96, 64, 96), 2, 16, 8),
    ((8, 24, 16), 4, 4, 3),
])
def test_doc_zigzag_matches_planner(lengths, cp, bm, bn):
    cu = synthetic.make_cu_seqlens(lengths)
    ranks = B.doc_zigzag(cu, cp)
    plan = zz.Plan(cu, cp, 2, 2, 32, "f32", bm, bn)
    want_u = [sum(plan.pair_counts(r, s)[0] for s in range(cp)) for r in range(cp)]
    want_i = [sum(plan.pair_counts(r, s)[1] for s in range(cp)) for r in range(cp)]
    assert list(B.useful_per_rank(cu, ranks)) == want_u
    assert list(B.issued_per_rank(cu, ranks, bm, bn)) == want_i


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_unit_tiles_issue_exactly_the_useful_pairs(seed):
    cp = 3
    lengths = synthetic.random_lengths(seed, 5, 7, cp)
    cu = synthetic.make_cu_seqlens(lengths)
    for name, split in B.STRATEGIES.items():
        if int(cu[-1]) % (2 * cp):
            continue
        ranks = split(cu, cp)
        assert list(B.issued_per_rank(cu, ranks, 1, 1)) == list(B.useful_per_rank(cu, ranks)), name


@pytest.mark.parametrize("cp", [2, 4, 8, 16])
def test_contiguous_split_of_one_sequence_closed_form(cp):
    L = 64 * cp
    cu = synthetic.make_cu_seqlens([L])
    u = B.useful_per_rank(cu, B.contiguous(cu, cp))
    n = L // cp
    want = np.array([n * r * n + n * (n + 1) // 2 for r in range(cp)])
    assert np.array_equal(u, want)
    assert abs(u.max() / u.mean() - (2 * cp - 1) / cp) < 2.0 / n


def test_stream_zigzag_of_one_document_is_doc_zigzag():
    cu = synthetic.make_cu_seqlens([512])
    assert B.stream_zigzag(cu, 4) == B.doc_zigzag(cu, 4)


def test_every_split_does_the_same_useful_work():
    lengths = synthetic.lengths_for(synthetic.WORKLOADS["c2"])
    cu = synthetic.make_cu_seqlens(lengths)
    total = sum(L * (L + 1) // 2 for L in lengths)
    for name, split in B.STRATEGIES.items():
        assert int(B.useful_per_rank(cu, split(cu, 4)).sum()) == total, name
    for n_mb in (1, 4):
        assert B.study(lengths, 4, 128, 64, "doc_zigzag", n_mb)["useful_pairs"] == total
