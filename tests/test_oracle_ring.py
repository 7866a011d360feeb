"""Pins of the oracle's SnapKV ring-buffer decode step (oracle.ring_step) to
what the policy book's SnapKV entry fixes.  CPU only.

  * "How it works": every observed step writes each cached token's weight
    into its ring at the current index and advances the index modulo
    obsWindow; the new token enters with an all-zero ring.  The weight
    written for a cached token equals the already pinned SUM score of the
    step's single query (oracle.score with the input builder's LSE), so the
    ring holds exactly the window sum's terms, minus each token's weight on
    its own admission step.
  * A null attention vector writes nothing and leaves the index.
  * Eviction: sums of each ring (index 0 upward), max-pooled over the
    poolKernel tokens centred on each in position order (clamped), the
    smallest (pooled, position) outside the recent window is dropped; brute
    force with a sort by position and a sliding maximum; poolKernel 1 leaves
    the plain sums; equal scores drop the lower position; with recent 0 the
    new token itself can be the one dropped.
  * Ranks: each slot's index in position order, after in-place overwrites.
  * Refusals: recentWindow >= budget, obsWindow 0, an even poolKernel.
"""
import numpy as np
import pytest

import oracle
from tests.helpers import rounded_window_inputs
from tests.test_oracle_h2o_step import _enc, _state, _stream_inputs

rng = np.random.default_rng


def _ring(st, W):
    return oracle.ring_state(st, W)


def _step(st, keys, vals, qs, t, budget, recent, pool, observe=1):
    B = st["B"]
    return oracle.ring_step(st, _enc(qs[t], st), _enc(keys[:, :, t], st), _enc(vals[:, :, t], st),
                            np.full(B, t, np.int32), np.full(B, observe, np.int32), budget, recent,
                            pool)


def test_ring_weights_are_the_single_query_sum_scores():
    B, Hkv, G, D, n0, T, W = 2, 2, 2, 32, 5, 14, 4
    keys, vals, qs = _stream_inputs(3, B, Hkv, G, D, T)
    budget = 32
    st = _ring(_state(keys, vals, n0, budget, G), W)
    ch = _state(keys, vals, n0, budget, G)          # the appended cache, for the score oracle
    for t in range(n0, T):
        idx = int(st["ring"][0, 0])
        st, ev, _, _ = _step(st, keys, vals, qs, t, budget, 4, 1)
        assert (ev == -1).all() and (st["ring"] == (idx + 1) % W).all()
        for b in range(B):
            for h in range(Hkv):
                blk = ch["block_table"][b, h, t // 16]
                ch["k_pool"][blk, t % 16] = keys[b, h, t]
                ch["v_pool"][blk, t % 16] = vals[b, h, t]
        ch["pos"][:, :, t] = t
        ch["seq_len"][:] = t + 1
        ch["q"] = np.ascontiguousarray(qs[t][:, :, None, :], np.float32)
        ch["q_pos"] = np.full((B, 1), t, np.int32)
        lse64, _ = oracle.lse_a(ch)
        lse32, _ = rounded_window_inputs(ch, lse64)
        want = oracle.score(ch, lse32, oracle.SUM)["sum"]
        got = st["hist"][:, :, idx, :t]
        assert np.allclose(got, want[:, :, :t], rtol=2e-6, atol=1e-30), t
        assert (st["hist"][:, :, :, t] == 0).all()   # the new token: a zero ring
        assert (st["pos"][:, :, t] == t).all()


def test_ring_wraps_and_null_steps_are_inert():
    B, Hkv, G, D, T, W = 1, 2, 2, 16, 12, 3
    keys, vals, qs = _stream_inputs(4, B, Hkv, G, D, T)
    st = _ring(_state(keys, vals, 2, 32, G), W)
    written = {}
    for t in range(2, T):
        observe = 0 if t in (5, 6) else 1
        before = st
        idx = int(st["ring"][0, 0])
        st, ev, _, _ = _step(st, keys, vals, qs, t, 32, 2, 1, observe=observe)
        if observe:
            assert (st["ring"] == (idx + 1) % W).all()
            written[t] = idx
            # only the index written changed in the cached rows
            other = [w for w in range(W) if w != idx]
            assert np.array_equal(st["hist"][:, :, other, :t], before["hist"][:, :, other, :t])
        else:
            assert np.array_equal(st["ring"], before["ring"])
            assert np.array_equal(st["hist"][:, :, :, :t], before["hist"][:, :, :, :t])
    # the observed steps cycle through the indices, skipping the null steps
    obs = [t for t in range(2, T) if t not in (5, 6)]
    assert [written[t] for t in obs] == [i % W for i in range(len(obs))]


def _brute_victim(st, u, t, recent, pool):
    """(evicted position, pooled) by a sort by position and a sliding max."""
    B, Hkv = st["B"], st["Hkv"]
    b, h = divmod(u, Hkv)
    n = int(st["seq_len"][b, h])
    W = st["hist"].shape[2]
    S = []
    for j in range(n):
        acc = np.float32(0)
        for w in range(W):
            acc = np.float32(acc + st["hist"][b, h, w, j])
        S.append(acc)
    S.append(np.float32(0))
    P = list(st["pos"][b, h, :n]) + [t]
    order = np.argsort(P, kind="stable")
    r = (pool - 1) // 2
    pooled = np.zeros(n + 1, np.float32)
    for k in range(n + 1):
        win = order[max(0, k - r):min(n, k + r) + 1]
        pooled[order[k]] = max(S[i] for i in win)
    cand = [i for i in range(n + 1) if t - P[i] >= recent]
    best = min(cand, key=lambda i: (pooled[i], P[i]))
    return P[best]


@pytest.mark.parametrize("seed,pool,recent,W", [(0, 1, 3, 4), (1, 3, 2, 4), (2, 7, 5, 8),
                                                 (3, 5, 0, 2), (4, 3, 1, 6)])
def test_eviction_by_brute_force(seed, pool, recent, W):
    r = rng(seed)
    B, Hkv, G, D, n = 2, 3, 2, 16, 24
    keys, vals, qs = _stream_inputs(seed + 10, B, Hkv, G, D, 64)
    st = _ring(_state(keys, vals, n, n, G), W)
    # positions in shuffled slot order, rings with values on a coarse grid (ties)
    for b in range(B):
        for h in range(Hkv):
            st["pos"][b, h, :n] = r.permutation(np.arange(40))[:n]
    st = _ring(st, W)
    st["hist"][:, :, :, :n] = (r.integers(0, 5, (B, Hkv, W, n)) / 8).astype(np.float32)
    t = 50
    want = [_brute_victim(st, u, t, recent, pool) for u in range(B * Hkv)]
    new, ev, _, _ = oracle.ring_step(st, _enc(qs[0], st), _enc(keys[:, :, 0], st),
                                     _enc(vals[:, :, 0], st), np.full(B, t, np.int32),
                                     np.zeros(B, np.int32), n, recent, pool)
    assert ev.reshape(-1).tolist() == want
    for u in range(B * Hkv):
        b, h = divmod(u, Hkv)
        if want[u] == t:     # the new token dropped: nothing changes
            assert np.array_equal(new["pos"][b, h], st["pos"][b, h])
            continue
        slot = int(np.flatnonzero(st["pos"][b, h, :n] == want[u])[0])
        assert new["pos"][b, h, slot] == t and (new["hist"][b, h, :, slot] == 0).all()
        p = new["pos"][b, h, :n]
        assert np.array_equal(new["rank"][b, h, :n], np.argsort(np.argsort(p)))


def test_new_token_dropped_and_ties_drop_the_lower_position():
    B, Hkv, G, D, n, W = 1, 1, 1, 16, 8, 2
    keys, vals, qs = _stream_inputs(7, B, Hkv, G, D, 16)
    st = _ring(_state(keys, vals, n, n, G), W)
    st["hist"][:, :, :, :n] = 1.0
    new, ev, _, _ = oracle.ring_step(st, _enc(qs[0], st), _enc(keys[:, :, 0], st),
                                     _enc(vals[:, :, 0], st), np.full(B, 20, np.int32),
                                     np.zeros(B, np.int32), n, 0, 1)
    assert ev[0, 0] == 20 and np.array_equal(new["pos"], st["pos"])   # zero ring: lowest
    new, ev, _, _ = oracle.ring_step(st, _enc(qs[0], st), _enc(keys[:, :, 0], st),
                                     _enc(vals[:, :, 0], st), np.full(B, 20, np.int32),
                                     np.zeros(B, np.int32), n, 2, 1)
    assert ev[0, 0] == 0            # all sums tie: the lowest candidate position


def test_ranks_follow_positions_through_a_long_stream():
    B, Hkv, G, D, T, budget, W = 2, 2, 2, 16, 90, 20, 5
    keys, vals, qs = _stream_inputs(8, B, Hkv, G, D, T)
    st = _ring(_state(keys, vals, 0, budget, G), W)
    fl = np.arange(200, 240, dtype=np.int32)
    for t in range(T):
        st, ev, fl, fc = oracle.ring_step(st, _enc(qs[t], st), _enc(keys[:, :, t], st),
                                          _enc(vals[:, :, t], st), np.full(B, t, np.int32),
                                          np.full(B, t % 7 != 3, np.int32), budget, 4, 3)
        for b in range(B):
            for h in range(Hkv):
                n = int(st["seq_len"][b, h])
                p = st["pos"][b, h, :n]
                assert np.array_equal(st["rank"][b, h, :n], np.argsort(np.argsort(p)))
                assert sorted(p.tolist())[-4:] == list(range(max(0, t - 3), t + 1))[-min(4, n):]


def test_refusals():
    B, Hkv, G, D = 1, 1, 1, 16
    keys, vals, qs = _stream_inputs(9, B, Hkv, G, D, 4)
    st = _ring(_state(keys, vals, 2, 16, G), 2)
    for budget, recent, pool in ((8, 8, 1), (8, 2, 2), (8, 2, 0)):
        with pytest.raises(ValueError):
            oracle.ring_step(st, _enc(qs[2], st), _enc(keys[:, :, 2], st), _enc(vals[:, :, 2], st),
                             np.full(B, 2, np.int32), np.ones(B, np.int32), budget, recent, pool)
    st0 = dict(st)
    st0["hist"] = np.zeros(st["hist"].shape[:2] + (0,) + st["hist"].shape[3:], np.float32)
    with pytest.raises(ValueError):
        oracle.ring_step(st0, _enc(qs[2], st), _enc(keys[:, :, 2], st), _enc(vals[:, :, 2], st),
                         np.full(B, 2, np.int32), np.ones(B, np.int32), 8, 2, 1)
