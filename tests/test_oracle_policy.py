"""Pins of the oracle's policy variants.  CPU only.

Shared scores across the KV heads of a sequence ([H2O] "Formulating
Cumulative Attention Scores": a token's score sums the attention of every
head of the layer, so all heads of a sequence evict the same tokens):

  * brute force on small inputs: the victims are the m smallest (shared sum,
    slot) pairs among the candidates, found by a full sort, the sum taken in
    fp32 with heads in ascending order;
  * with one KV head it is the ordinary selection; with every head holding
    the same integer-valued row (exact sums) it equals each head's own
    selection, ties included;
  * heads that do not hold the same tokens in the same slots are refused for
    their sequence only.
"""
import numpy as np
import pytest

import oracle

rng = np.random.default_rng


def _brute(scores, n, budget, recent):
    B, Hkv, ms = scores.shape
    out = []
    for b in range(B):
        acc = scores[b, 0, :n].astype(np.float32)
        for h in range(1, Hkv):
            acc = (acc + scores[b, h, :n]).astype(np.float32)
        m = max(0, n - budget)
        nc = max(0, n - recent)
        order = np.lexsort((np.arange(nc), acc[:nc]))
        out.append(np.sort(order[:m]))
    return out


@pytest.mark.parametrize("seed,integer", [(0, False), (1, True), (2, False)])
def test_shared_selection_brute_force(seed, integer):
    r = rng(seed)
    B, Hkv, ms, n, budget, recent = 3, 4, 64, 57, 20, 6
    if integer:   # many ties
        scores = r.integers(0, 4, (B, Hkv, ms)).astype(np.float32)
    else:
        scores = r.uniform(0, 1, (B, Hkv, ms)).astype(np.float32)
    seq = np.full((B, Hkv), n, np.int32)
    pos = np.broadcast_to(np.arange(ms, dtype=np.int32), (B, Hkv, ms)).copy()
    vic, nv = oracle.select_shared(scores, seq, pos, budget, recent)
    want = _brute(scores, n, budget, recent)
    for b in range(B):
        for h in range(Hkv):
            assert nv[b, h] == n - budget
            assert np.array_equal(vic[b, h, :nv[b, h]], want[b])


def test_one_head_and_identical_heads_reduce_to_the_per_head_selection():
    r = rng(5)
    B, ms, n, budget, recent = 2, 80, 70, 33, 8
    s1 = r.uniform(0, 2, (B, 1, ms)).astype(np.float32)
    seq1 = np.full((B, 1), n, np.int32)
    pos1 = np.broadcast_to(np.arange(ms, dtype=np.int32), (B, 1, ms)).copy()
    vs, ns = oracle.select_shared(s1, seq1, pos1, budget, recent)
    vp, np_ = oracle.select(s1.reshape(B, ms), seq1.reshape(B), budget, recent)
    assert np.array_equal(ns.reshape(-1), np_) and np.array_equal(vs.reshape(B, ms), vp)
    Hkv = 5
    si = r.integers(0, 6, (B, 1, ms)).astype(np.float32)
    s5 = np.repeat(si, Hkv, axis=1)
    vs5, ns5 = oracle.select_shared(s5, np.full((B, Hkv), n, np.int32),
                                    np.broadcast_to(np.arange(ms, dtype=np.int32),
                                                    (B, Hkv, ms)).copy(), budget, recent)
    vpi, npi = oracle.select(si.reshape(B, ms), np.full(B, n, np.int32), budget, recent)
    for h in range(Hkv):
        assert np.array_equal(ns5[:, h], npi)
        assert np.array_equal(vs5[:, h], vpi)


def test_misaligned_heads_are_refused_per_sequence():
    r = rng(7)
    B, Hkv, ms, n = 3, 2, 48, 40
    scores = r.uniform(0, 1, (B, Hkv, ms)).astype(np.float32)
    seq = np.full((B, Hkv), n, np.int32)
    pos = np.broadcast_to(np.arange(ms, dtype=np.int32), (B, Hkv, ms)).copy()
    seq[0, 1] = n - 1                  # unequal lengths
    pos[2, 1, 5] = 99                  # a slot holding another token
    vic, nv = oracle.select_shared(scores, seq, pos, 20, 4)
    assert nv[0].tolist() == [-1, -1] and nv[2].tolist() == [-1, -1]
    assert nv[1].tolist() == [20, 20]
    pos[2, 1, 5] = 5
    pos[2, 1, 45] = 99                 # past the length: not a token
    _, nv2 = oracle.select_shared(scores, seq, pos, 20, 4)
    assert nv2[2].tolist() == [20, 20]


def test_per_unit_budgets_brute_force():
    """Each unit's victims are the m = n - budget smallest (score, slot) pairs
    among its first n - recent slots (full sort), with its own pair; invalid
    pairs and lengths give -1."""
    r = rng(9)
    U, ms = 8, 96
    scores = r.integers(0, 6, (U, ms)).astype(np.float32)
    seq = r.integers(0, ms + 1, U).astype(np.int32)
    budget = r.integers(1, 60, U).astype(np.int32)
    recent = np.minimum(r.integers(0, 20, U), budget - 1).astype(np.int32)
    budget[5], recent[5] = 10, 10          # recent >= budget: refused
    seq[6] = ms + 1                        # past the capacity: refused
    vic, nv = oracle.select_budgets(scores, seq, budget, recent)
    for u in range(U):
        if u in (5, 6):
            assert nv[u] == -1
            continue
        n = int(seq[u])
        m = max(0, n - int(budget[u]))
        nc = max(0, n - int(recent[u]))
        order = np.lexsort((np.arange(nc), scores[u, :nc]))
        assert nv[u] == m
        assert np.array_equal(vic[u, :m], np.sort(order[:m]))
