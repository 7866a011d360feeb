"""Pins of the oracle's H2O decode step (oracle.h2o_step) to what the pages and
the mathematics fix.  CPU only.

  * [H2O] "Verification Unit Test": 16 steps, budget 8 (4 heavy + 4 recent):
    a token that draws the attention of every query stays; one that draws
    none is pruned; the recent window is always kept.
  * The step equals the already pinned chain append -> accumulate (score with
    ACCUMULATE) -> select -> compact ([H2O] "Step-by-Step Eviction
    Lifecycle"): the same positions are evicted at every step and the kept
    tokens carry the same running scores.  Only the slot a token lands in
    differs: the step overwrites the pruned slot in place ([H2O]
    "PagedAttention Memory Integration"), the chain packs the rows in order.
  * Closed forms: equal keys give every attended token 1/(n+1) per query row.
  * Conservation: the kept (pos, K, V) rows are the old ones minus the victim
    plus the new token.
  * Edge cases: recent = 0 (the new token itself can be pruned), appends that
    take a block from the free list in (b, h) order, and the refusals.
  * The step's attention output equals the input builder's (oracle.lse_a, an
    independent function) on the chain's appended cache; equal keys give the
    mean of the value rows; a dominant key gives its own value row.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import manual_case, rounded_window_inputs

rng = np.random.default_rng


def _stream_inputs(seed, B, Hkv, G, D, total, plant=None, plant_at=0, std=0.5):
    """Keys and values of positions 0..total-1 [B,Hkv,total,D] and one query
    per position [total,B,Hq,D]; optionally a key planted on (plant > 0) or
    against (plant < 0) the queries' shared direction."""
    r = rng(seed)
    u = r.normal(0, 1, D)
    u /= np.linalg.norm(u)
    keys = r.normal(0, std, (B, Hkv, total, D))
    vals = r.normal(0, 1, (B, Hkv, total, D))
    qs = r.normal(0, std, (total, B, Hkv * G, D))
    if plant is not None:
        qs = qs + np.sqrt(D) * u
        keys[:, :, plant_at] += plant * np.sqrt(D) * u
    return keys, vals, qs


def _state(keys, vals, n0, capacity, G, dtype="f32", scale=None, seq_len=None, **kw):
    B, Hkv, _, D = keys.shape
    k_rows = np.zeros((B, Hkv, capacity, D))
    v_rows = np.zeros((B, Hkv, capacity, D))
    k_rows[:, :, :n0] = keys[:, :, :n0]
    v_rows[:, :, :n0] = vals[:, :, :n0]
    seq = np.full((B, Hkv), n0, np.int32) if seq_len is None else seq_len
    st = manual_case(k_rows, v_rows, np.zeros((B, Hkv * G, 1, D)), np.zeros((B, 1)), seq_len=seq,
                     dtype=dtype, scale=(1 / np.sqrt(D)) if scale is None else scale, **kw)
    st["score"] = np.zeros((B, Hkv, st["max_blocks"] * 16), np.float32)
    return st


def _enc(x, st):
    return synth.encode(np.asarray(x, np.float64), st["dtype"])


def _step_attn(st, keys, vals, qs, t, budget, recent, **kw):
    B = st["B"]
    return oracle.h2o_step(st, _enc(qs[t], st), _enc(keys[:, :, t], st), _enc(vals[:, :, t], st),
                           np.full(B, t, np.int32), budget, recent, want_attn=True, **kw)


def _step(st, keys, vals, qs, t, budget, recent, **kw):
    B = st["B"]
    return oracle.h2o_step(st, _enc(qs[t], st), _enc(keys[:, :, t], st), _enc(vals[:, :, t], st),
                           np.full(B, t, np.int32), budget, recent, **kw)


def _kept(st, u=(0, 0)):
    n = int(st["seq_len"][u])
    ps = st["pos"][u][:n]
    return dict(zip(ps.tolist(), st["score"][u][:n].tolist()))


def _rows(st, which, u, slot):
    blk = st["block_table"][u][slot // 16]
    return st[which][blk, slot % 16]


def test_page_self_test_heavy_hitter_kept():
    """[H2O] "Verification Unit Test" rebuilt on q.k: 16 steps, budget 8,
    recent 4, 4 query heads, D 64."""
    def run(plant, token=0):
        keys, vals, qs = _stream_inputs(11, 1, 1, 4, 64, 16, plant=plant, plant_at=token)
        st = _state(keys, vals, 0, 8, 4)
        for t in range(16):
            st, ev, _, _ = _step(st, keys, vals, qs, t, 8, 4)
            assert (ev[0, 0] == -1) if t < 8 else (0 <= ev[0, 0] <= t - 4)
            assert int(st["seq_len"][0, 0]) == min(t + 1, 8)
        return sorted(_kept(st))
    kept = run(1.0)
    assert len(kept) == 8 and 0 in kept
    assert kept[-4:] == [12, 13, 14, 15]
    assert 6 in run(1.0, token=6)
    assert 0 not in run(-1.0)


@pytest.mark.parametrize("seed,budget,recent", [(1, 12, 4), (2, 9, 1), (3, 20, 7)])
def test_step_equals_append_accumulate_select_compact(seed, budget, recent):
    B, Hkv, G, D, T = 2, 2, 2, 32, 48
    keys, vals, qs = _stream_inputs(seed, B, Hkv, G, D, T)
    st = _state(keys, vals, 0, budget, G)
    ch = _state(keys, vals, 0, budget + 1, G)  # one slot past the budget for the append
    acc = np.zeros((B, Hkv, ch["max_blocks"] * 16), np.float32)
    for t in range(T):
        st, ev, _, _, attn, aabs = _step_attn(st, keys, vals, qs, t, budget, recent)
        # the chain: append at slot n, accumulate, then evict down to the budget
        n = int(ch["seq_len"][0, 0])
        for b in range(B):
            for h in range(Hkv):
                blk = ch["block_table"][b, h, n // 16]
                ch["k_pool"][blk, n % 16] = keys[b, h, t]
                ch["v_pool"][blk, n % 16] = vals[b, h, t]
        ch["pos"][:, :, n] = t
        ch["seq_len"][:] = n + 1
        acc[:, :, n] = 0.0
        ch["q"] = np.ascontiguousarray(qs[t][:, :, None, :], np.float32)
        ch["q_pos"] = np.full((B, 1), t, np.int32)
        lse64, a64 = oracle.lse_a(ch, want_a=True)
        # the step's attention output is the input builder's, over the same keys
        assert np.all(np.abs(attn - a64[:, :, 0, :]) <= 1e-12 * aabs + 1e-300), t
        lse32, _ = rounded_window_inputs(ch, lse64)
        acc = oracle.score(ch, lse32, oracle.SUM | oracle.ACCUMULATE, prev_sum=acc)["sum"]
        acc = np.nan_to_num(acc, nan=0.0).astype(np.float32)
        evicted = np.full((B, Hkv), -1)
        if n + 1 > budget:
            vic, nv = oracle.select(acc, ch["seq_len"], budget, recent)
            assert (nv == 1).all()
            for u in range(B * Hkv):
                evicted.reshape(-1)[u] = ch["pos"].reshape(B * Hkv, -1)[u, vic[u, 0]]
            ch, _, _, _ = oracle.compact(ch, vic, nv, score_row=acc)
            acc = ch.pop("score_row")
        assert np.array_equal(ev, evicted), t
        for b in range(B):
            for h in range(Hkv):
                a = _kept(st, (b, h))
                n2 = int(ch["seq_len"][b, h])
                c = dict(zip(ch["pos"][b, h, :n2].tolist(), acc[b, h, :n2].tolist()))
                assert sorted(a) == sorted(c), (t, b, h)
                for p in a:
                    assert abs(a[p] - c[p]) <= 1e-5 * abs(c[p]) + 1e-30, (t, b, h, p)


def test_equal_keys_closed_form():
    """Equal keys: every query row spreads 1/(n+1) over the n cached tokens and
    itself; from zero scores each token then holds G/(n+1), all tie, and the
    lowest position outside the recent window is pruned."""
    B, Hkv, G, D, n, budget, recent = 1, 2, 3, 16, 10, 10, 3
    keys = np.ones((B, Hkv, n + 1, D)) * 0.25
    vals = rng(5).normal(0, 1, (B, Hkv, n + 1, D))
    qs = rng(6).normal(0, 1, (n + 1, B, Hkv * G, D))
    st = _state(keys, vals, n, budget, G)
    st["pos"][:, :, :n] = np.arange(100, 100 + n)  # positions need not start at 0
    t = 100 + n
    new, ev, _, _ = oracle.h2o_step(st, _enc(qs[n], st), _enc(keys[:, :, n], st),
                                    _enc(vals[:, :, n], st), np.full(B, t, np.int32), budget,
                                    recent)
    assert (ev == 100).all()
    for h in range(Hkv):
        kept = _kept(new, (0, h))
        assert sorted(kept) == list(range(101, 100 + n)) + [t]
        for p, v in kept.items():
            assert v == pytest.approx(G / (n + 1), rel=1e-6)
        assert int(new["pos"][0, h, 0]) == t  # the pruned slot 0 holds the new token


def test_conservation_and_untouched_slots():
    B, Hkv, G, D, budget, recent = 2, 3, 2, 16, 24, 5
    keys, vals, qs = _stream_inputs(21, B, Hkv, G, D, budget + 1)
    st = _state(keys, vals, budget, budget, G)
    st["score"][:, :, :budget] = rng(22).uniform(0, 1, (B, Hkv, budget)).astype(np.float32)
    new, ev, _, _ = _step(st, keys, vals, qs, budget, budget, recent)
    for b in range(B):
        for h in range(Hkv):
            u = (b, h)
            victim_pos = int(ev[b, h])
            assert 0 <= victim_pos <= budget - recent  # outside the recent window
            slot = int(np.nonzero(st["pos"][u][:budget] == victim_pos)[0][0])
            for s in range(budget):
                if s == slot:
                    assert int(new["pos"][u][s]) == budget
                    assert np.array_equal(_rows(new, "k_pool", u, s), _enc(keys[b, h, budget], st))
                    assert np.array_equal(_rows(new, "v_pool", u, s), _enc(vals[b, h, budget], st))
                else:
                    assert new["pos"][u][s] == st["pos"][u][s]
                    assert np.array_equal(_rows(new, "k_pool", u, s), _rows(st, "k_pool", u, s))
                    assert np.array_equal(_rows(new, "v_pool", u, s), _rows(st, "v_pool", u, s))


def test_recent_zero_can_drop_the_new_token():
    """With no recent window the new token competes too: a key pointing away
    from every query draws almost no attention and is pruned at once."""
    B, Hkv, G, D, budget = 1, 1, 4, 32, 6
    keys, vals, qs = _stream_inputs(31, B, Hkv, G, D, budget + 1, plant=-1.0, plant_at=budget)
    st = _state(keys, vals, budget, budget, G)
    st["score"][:] = 1.0
    new, ev, _, _ = _step(st, keys, vals, qs, budget, budget, 0)
    assert ev[0, 0] == budget
    assert np.array_equal(new["pos"], st["pos"]) and np.array_equal(new["k_pool"], st["k_pool"])
    assert (new["score"][0, 0, :budget] > 1.0).all()  # the cached tokens still accumulate
    # with a recent window of 1 the new token is protected and a cached one goes
    new1, ev1, _, _ = _step(st, keys, vals, qs, budget, budget, 1)
    assert 0 <= ev1[0, 0] < budget


def test_append_takes_blocks_in_head_order():
    B, Hkv, G, D, budget = 2, 2, 2, 8, 40
    keys, vals, qs = _stream_inputs(41, B, Hkv, G, D, 40)
    seq = np.array([[16, 5], [32, 0]], np.int32)
    st = _state(keys, vals, 0, budget, G, seq_len=seq, spare_blocks=4)
    for b in range(B):
        for h in range(Hkv):
            n = seq[b, h]
            st["pos"][b, h, :n] = np.arange(n)
            if n % 16 == 0:
                st["block_table"][b, h, n // 16:] = -1  # the next block is not allocated yet
    used = set(st["block_table"][st["block_table"] >= 0].tolist())
    spare = [x for x in range(st["num_blocks"]) if x not in used][:3]
    free = np.array(spare + [-1] * 5, np.int32)
    t = np.array([40, 40], np.int32)
    new, ev, fl, fc = oracle.h2o_step(st, _enc(qs[0], st), _enc(keys[:, :, 0], st),
                                      _enc(vals[:, :, 0], st), t, budget, 4, free_list=free,
                                      free_count=3)
    assert (ev == -1).all()
    assert np.array_equal(new["seq_len"], seq + 1)
    # heads (0,0) n=16, (1,0) n=32, (1,1) n=0 need a block: top of the stack first, (b, h) order
    assert fc == 0
    assert new["block_table"][0, 0, 1] == free[2]
    assert new["block_table"][1, 0, 2] == free[1]
    assert new["block_table"][1, 1, 0] == free[0]
    assert new["block_table"][0, 1, 0] == st["block_table"][0, 1, 0]
    for b in range(B):
        for h in range(Hkv):
            n = seq[b, h]
            assert new["pos"][b, h, n] == 40
            assert np.array_equal(_rows(new, "k_pool", (b, h), n), _enc(keys[b, h, 0], st))


def test_refusals_leave_heads_unchanged():
    B, Hkv, G, D, budget = 1, 3, 2, 8, 16
    keys, vals, qs = _stream_inputs(51, B, Hkv, G, D, 20)
    seq = np.array([[17, 16, 8]], np.int32)  # over the budget; full; a bad block id
    st = _state(keys, vals, 0, budget + 16, G, seq_len=seq)
    st["pos"][0, :, :17] = np.arange(17)
    st["block_table"][0, 2, 0] = st["num_blocks"] + 5
    new, ev, _, _ = oracle.h2o_step(st, _enc(qs[0], st), _enc(keys[:, :, 0], st),
                                    _enc(vals[:, :, 0], st), np.array([30], np.int32), budget, 2)
    assert ev[0, 0] == -2 and ev[0, 2] == -4
    assert ev[0, 1] >= 0
    for h in (0, 2):
        assert np.array_equal(new["score"][0, h], st["score"][0, h])
        assert new["seq_len"][0, h] == st["seq_len"][0, h]
    # an empty free list refuses an append that needs a block
    st2 = _state(keys, vals, 0, budget, G, seq_len=np.array([[0, 0, 0]], np.int32))
    st2["block_table"][0, 1, 0] = -1
    new2, ev2, _, fc2 = oracle.h2o_step(st2, _enc(qs[0], st2), _enc(keys[:, :, 0], st2),
                                        _enc(vals[:, :, 0], st2), np.array([0], np.int32), budget,
                                        2, free_list=np.zeros(4, np.int32), free_count=0)
    assert ev2[0].tolist() == [-1, -3, -1] and fc2 == 0
    with pytest.raises(ValueError):
        oracle.h2o_step(st2, _enc(qs[0], st2), _enc(keys[:, :, 0], st2), _enc(vals[:, :, 0], st2),
                        np.array([0], np.int32), budget, budget)  # recent >= budget


def test_attention_output_closed_forms():
    """Equal keys: the output is the mean of the n cached value rows and the new
    one.  One key far above the others: the output is that key's value row."""
    B, Hkv, G, D, n, budget = 1, 2, 3, 16, 10, 12
    keys = np.ones((B, Hkv, n + 1, D)) * 0.25
    vals = rng(61).normal(0, 1, (B, Hkv, n + 1, D))
    qs = rng(62).normal(0, 1, (n + 1, B, Hkv * G, D))
    st = _state(keys, vals, n, budget, G)
    _, ev, _, _, attn, aabs = oracle.h2o_step(st, _enc(qs[n], st), _enc(keys[:, :, n], st),
                                              _enc(vals[:, :, n], st), np.full(B, n, np.int32),
                                              budget, 2, want_attn=True)
    assert (ev == -1).all()
    v32 = synth.decode(_enc(vals, st), "f32").astype(np.float64)
    mean = v32.mean(axis=2)                                   # [B, Hkv, D]
    want = np.repeat(mean, G, axis=1)                         # every row of the group
    assert np.allclose(attn, want, rtol=1e-12, atol=1e-12)
    assert np.all(aabs >= np.abs(attn) - 1e-12)
    # a dominant key: the planted token draws all the weight
    keys2, vals2, qs2 = _stream_inputs(63, 1, 1, 4, 32, 9, plant=4.0, plant_at=3)
    st2 = _state(keys2, vals2, 8, 12, 4, scale=1.0)
    _, _, _, _, attn2, _ = oracle.h2o_step(st2, _enc(qs2[8], st2), _enc(keys2[:, :, 8], st2),
                                           _enc(vals2[:, :, 8], st2), np.full(1, 8, np.int32),
                                           12, 2, want_attn=True)
    v3 = synth.decode(_enc(vals2[0, 0, 3], st2), "f32").astype(np.float64)
    assert np.allclose(attn2[0], np.repeat(v3[None], 4, axis=0), rtol=0, atol=1e-9)

