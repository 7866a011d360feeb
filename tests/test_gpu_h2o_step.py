"""GPU parity of kvev_h2o_step, the H2O decode step, against oracle.h2o_step.

Two ways of running a stream of decode steps:

* isolated steps: before every step the GPU receives the oracle's state, so
  each step is compared on its own (positions, K / V rows slot by slot
  bit-exact, running scores to the score tolerance);
* a free-running chain: the GPU's state evolves by its own steps.  The two
  sides prune the same token unless two candidates' scores lie within the
  tolerance of each other; then the GPU's choice must lie in that band of the
  oracle's cutoff (the oracle's own scores, from a run of the same step with
  room for one more token, which appends instead of pruning), and that head
  is followed by invariants only from then on.

Blocks taken from the free list by heads appending in the same step may come
out in any order on the GPU: the taken set and the remaining list are
compared, the rows through each side's own block table.  When the list runs
short within a step, which heads get the last blocks is that order too:
test_short_free_list checks that case by its counts.
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import FLT_MIN, TOL, dev, device_cache, host

pytestmark = pytest.mark.gpu
rng = np.random.default_rng


def _say(msg):
    print(f"[h2o] {msg}", flush=True)


# ------------------------------------------------------------------ states


def _scaled_state(seed, dtype, B, Hkv, G, D, budget, n0, spare=None, bad_head=None, fresh=True):
    """A stream state with per-head lengths n0 [B, Hkv] (positions 0..n-1),
    running scores drawn around what one step adds (G / budget), heads at a
    block boundary with no block allocated there, a free list of spare pool
    blocks, and optionally one head whose first block id is out of range."""
    r = rng(seed)
    cap_blocks = (budget + 1 + 15) // 16 + 1
    U = B * Hkv
    if spare is None:  # enough for every append: the order of pops is then immaterial
        spare = U * cap_blocks
    num_blocks = U * cap_blocks + spare
    perm = synth.shuffled(num_blocks, seed, 7)
    bt = perm[:U * cap_blocks].reshape(B, Hkv, cap_blocks).astype(np.int32).copy()
    edt = np.uint16 if dtype == "bf16" else np.float32
    k_pool = synth.encode(r.normal(0, 0.5, (num_blocks, 16, D)), dtype).astype(edt)
    v_pool = synth.encode(r.normal(0, 1.0, (num_blocks, 16, D)), dtype).astype(edt)
    pos = np.zeros((B, Hkv, cap_blocks * 16), np.int32)
    score = np.zeros((B, Hkv, cap_blocks * 16), np.float32)
    for b in range(B):
        for h in range(Hkv):
            n = int(n0[b, h])
            m = max(0, min(n, cap_blocks * 16))
            pos[b, h, :m] = np.arange(m)
            score[b, h, :m] = r.uniform(0.0, 2.0 * G / budget, m).astype(np.float32)
            if fresh and 0 <= n < budget and n % 16 == 0:
                bt[b, h, n // 16:] = -1   # the append opens a block from the free list
    if bad_head is not None:
        bt.reshape(U, cap_blocks)[bad_head, 0] = num_blocks + 3
    free = np.full(num_blocks, -1, np.int32)
    spare_ids = perm[U * cap_blocks:]
    free[:spare_ids.size] = spare_ids
    return dict(dtype=dtype, B=B, Hkv=Hkv, G=G, D=D, W=1, max_blocks=cap_blocks,
                num_blocks=num_blocks, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                seq_len=np.ascontiguousarray(n0, dtype=np.int32).copy(), pos=pos, score=score,
                scale=1.0 / np.sqrt(D)), free, int(spare_ids.size)


def _step_inputs(seed, step, dtype, B, Hkv, G, D, u_dirs):
    """Query rows (with the heads' planted direction), new key and value."""
    r = rng([seed, step])
    q = r.normal(0, 0.5, (B, Hkv * G, D))
    q += np.repeat(u_dirs, G, axis=1) * np.sqrt(D) * 0.5
    k = r.normal(0, 0.5, (B, Hkv, D))
    hot = r.uniform(0, 1, (B, Hkv)) < 0.1             # a tenth of the tokens: heavy hitters
    k += hot[..., None] * u_dirs * np.sqrt(D) * 0.5
    v = r.normal(0, 1.0, (B, Hkv, D))
    return synth.encode(q, dtype), synth.encode(k, dtype), synth.encode(v, dtype)


class Dev:
    """Device copy of a stream state and its free list."""

    def __init__(self, st, free, fc):
        self.c = device_cache(st)
        self.score = dev(st["score"])
        self.fl = dev(free)
        self.fc = dev(np.array([fc], np.int32))
        self.ws = {}

    def step(self, st, q, k, v, t, budget, recent, attn=None):
        key = (st["G"], budget)
        if key not in self.ws:  # zero-filled once, left zero by every call
            self.ws[key] = K.new_h2o_workspace(self.c, st["G"], budget)
        return K.h2o_step(self.c, dev(q), dev(k), dev(v), dev(t), st["G"], st["scale"],
                          self.score, budget, recent, self.fl, self.fc, self.ws[key],
                          attn_out=attn)

    def state(self, like):
        out = dict(like)
        out.update(k_pool=host(self.c.k_pool), v_pool=host(self.c.v_pool),
                   block_table=host(self.c.block_table), seq_len=host(self.c.seq_len),
                   pos=host(self.c.pos), score=host(self.score))
        return out, host(self.fl), int(host(self.fc)[0])


# ------------------------------------------------------------- comparisons


def _row(st, which, u, s):
    return st[which][st["block_table"].reshape(-1, st["max_blocks"])[u, s // 16], s % 16]


def _flat(st, key):
    return st[key].reshape(st["B"] * st["Hkv"], -1)


def _close(g, o, tol):
    return abs(float(g) - float(o)) <= tol * max(abs(float(o)), FLT_MIN)


def _slot_rows(st, which, u, n):
    """Rows of slots [0, n) of head u through the head's own block table."""
    bt = st["block_table"].reshape(-1, st["max_blocks"])[u]
    s = np.arange(n)
    return st[which][bt[s // 16], s % 16]


def _scores_close(g, o, tol):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return np.abs(g - o) <= tol * np.maximum(np.abs(o), FLT_MIN)


def _same_slots(g, o, u, n, tol, what):
    """Slots [0, n) of head u: positions and K / V rows equal, scores close."""
    gp, op = _flat(g, "pos")[u, :n], _flat(o, "pos")[u, :n]
    assert np.array_equal(gp, op), f"{what}: positions differ"
    for which in ("k_pool", "v_pool"):
        eq = (_slot_rows(g, which, u, n) == _slot_rows(o, which, u, n)).all(axis=-1)
        assert eq.all(), f"{what}: {which} row of slot {int(np.flatnonzero(~eq)[0])} differs"
    ok = _scores_close(_flat(g, "score")[u, :n], _flat(o, "score")[u, :n], tol)
    if not ok.all():
        s = int(np.flatnonzero(~ok)[0])
        raise AssertionError(f"{what}: score of slot {s}: gpu {_flat(g, 'score')[u, s]!r} "
                             f"oracle {_flat(o, 'score')[u, s]!r}")


def _all_scores(before, q, k, v, t, budget, recent):
    """The oracle's running scores after the step's attention for every cached
    slot: the same step with room for one more token appends, pruning none."""
    spare = np.arange(before["num_blocks"], dtype=np.int32)  # any ids: the copy is discarded
    st, _, _, _ = oracle.h2o_step(before, q, k, v, t, budget + 1, recent, free_list=spare,
                                  free_count=spare.size)
    return st["score"].reshape(before["B"] * before["Hkv"], -1)


def compare_step(before, g, o, ev_g, ev_o, allsc, t, budget, recent, tol, what, heads=None):
    """Verdict per head of one step taken from the same `before` state: 'same',
    or 'band' (the pruned tokens differ, inside the tolerance band).  allsc:
    a function returning the oracle's scores of every slot after the step's
    attention (called only when the pruned tokens differ)."""
    U = before["B"] * before["Hkv"]
    ev_g, ev_o = ev_g.reshape(-1), ev_o.reshape(-1)
    verdict = {}
    for u in (range(U) if heads is None else heads):
        b = u // before["Hkv"]
        n = int(_flat(before, "seq_len")[u, 0])
        tag = f"{what} head {u}"
        if ev_o[u] < -1:  # refused: the head is untouched on both sides
            assert ev_g[u] == ev_o[u], f"{tag}: code {ev_g[u]} vs {ev_o[u]}"
            verdict[u] = "same"
            if g is None:
                continue
            m = max(0, min(n, _flat(before, "pos").shape[1]))
            assert np.array_equal(_flat(g, "pos")[u, :m], _flat(before, "pos")[u, :m]), tag
            for j in range(m):
                assert _close(_flat(g, "score")[u, j], _flat(before, "score")[u, j], tol), tag
            assert _flat(g, "seq_len")[u, 0] == n, tag
            continue
        if ev_g[u] == ev_o[u]:
            verdict[u] = "same"
            if g is None:
                continue
            n_after = int(_flat(o, "seq_len")[u, 0])
            assert int(_flat(g, "seq_len")[u, 0]) == n_after, tag
            _same_slots(g, o, u, n_after, tol, tag)
            continue
        # different pruned tokens: both candidates, the GPU's inside the band
        # of the oracle's cutoff (scores after this step's attention)
        assert ev_o[u] >= 0 and ev_g[u] >= 0, f"{tag}: {ev_g[u]} vs {ev_o[u]}"
        tb = int(t[b])
        assert tb - ev_g[u] >= recent, f"{tag}: pruned {ev_g[u]} inside the recent window"
        pos_b = _flat(before, "pos")[u, :n]
        sc_all = allsc()

        def score_of(p):  # the new token sits at slot n of the appending run
            if p == tb:
                return float(sc_all[u, n])
            return float(sc_all[u, int(np.flatnonzero(pos_b == p)[0])])
        c, x = score_of(int(ev_o[u])), score_of(int(ev_g[u]))
        assert abs(x - c) <= tol * max(abs(c), FLT_MIN), \
            f"{tag}: pruned {ev_g[u]} (score {x!r}) against {ev_o[u]} (cutoff {c!r})"
        if g is not None:  # the GPU's own state: new token in the slot it pruned
            hit = pos_b == ev_g[u]
            gp = _flat(g, "pos")[u, :n]
            assert (gp[hit] == tb).all() and np.array_equal(gp[~hit], pos_b[~hit]), tag
            assert _scores_close(_flat(g, "score")[u, :n][~hit], sc_all[u, :n][~hit], tol).all(), tag
        verdict[u] = "band"
    return verdict


def _lazy(fn):
    box = []

    def get():
        if not box:
            box.append(fn())
        return box[0]
    return get


def check_attention(g_attn, o_attn, o_abs, ev_o, Hkv, G, tol, what):
    """The step's attention output of the heads that were not refused:
    |g - o| <= tol * sum_j p_j |v_j| per element (the error bound of a weighted
    sum whose weights carry relative error up to tol)."""
    B = g_attn.shape[0]
    for b in range(B):
        for h in range(Hkv):
            if ev_o[b, h] < -1:
                continue
            rows = slice(h * G, (h + 1) * G)
            err = np.abs(g_attn[b, rows].astype(np.float64) - o_attn[b, rows])
            bound = tol * o_abs[b, rows] + 1e-30
            assert (err <= bound).all(), (
                f"{what} head ({b},{h}): attention output off by {float((err / bound).max()):.2f}x "
                f"the bound")


def check_free_lists(before_bt, g, o, fl_g, fc_g, fl_o, fc_o):
    """Same number taken, the same remaining list, the same set of taken blocks."""
    assert fc_g == fc_o
    assert np.array_equal(fl_g[:fc_o], fl_o[:fc_o])
    new_g = g["block_table"][(before_bt < 0) & (g["block_table"] >= 0)]
    new_o = o["block_table"][(before_bt < 0) & (o["block_table"] >= 0)]
    assert sorted(new_g.tolist()) == sorted(new_o.tolist())


# ------------------------------------------------------------------- cases

CASES = [
    # dtype, D, G, budget, recent, head with a bad block id
    ("bf16", 128, 4, 100, 20, None),
    ("f32", 64, 2, 40, 0, None),
    ("bf16", 64, 8, 57, 1, 7),
    ("f32", 128, 4, 48, 6, None),
]


def _lengths(B, Hkv, budget):
    """Ragged starts: appends, a full head, an empty one, one on a block
    boundary, one above the budget (refused at every step)."""
    pick = [budget - 10, budget, 0, 32, budget + 3, budget - 1, 16, 5]
    return np.array([pick[i % len(pick)] for i in range(B * Hkv)], np.int32).reshape(B, Hkv)


@pytest.mark.parametrize("dtype,D,G,budget,recent,bad", CASES)
def test_isolated_steps(dtype, D, G, budget, recent, bad):
    B, Hkv, steps = 2, 4, 48
    seed = 100 + D + budget
    st, free, fc = _scaled_state(seed, dtype, B, Hkv, G, D, budget, _lengths(B, Hkv, budget),
                                 bad_head=bad)
    dirs = rng(seed).normal(0, 1, (B, Hkv, D))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    t0 = budget + 8
    counts = {"same": 0, "band": 0}
    _say(f"{dtype} D{D} G{G} budget {budget} recent {recent}: {steps} isolated steps")
    for i in range(steps):
        q, k, v = _step_inputs(seed, i, dtype, B, Hkv, G, D, dirs)
        t = np.full(B, t0 + i, np.int32)
        o, ev_o, fl_o, fc_o, o_attn, o_abs = oracle.h2o_step(st, q, k, v, t, budget, recent,
                                                             free_list=free, free_count=fc,
                                                             want_attn=True)
        d = Dev(st, free, fc)
        attn = torch.full((B, Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
        ev_g = host(d.step(st, q, k, v, t, budget, recent, attn=attn))
        torch.cuda.synchronize()
        g, fl_g, fc_g = d.state(st)
        check_attention(host(attn), o_attn, o_abs, ev_o, Hkv, G, TOL[dtype], f"step {i}")
        allsc = _lazy(lambda: _all_scores(st, q, k, v, t, budget, recent))
        for vv in compare_step(st, g, o, ev_g, ev_o, allsc, t, budget, recent, TOL[dtype],
                               f"step {i}").values():
            counts[vv] += 1
        check_free_lists(st["block_table"], g, o, fl_g, fc_g, fl_o, fc_o)
        st, free, fc = o, fl_o, fc_o
    _say(f"heads x steps: {counts}")
    assert counts["same"] >= 0.95 * (counts["same"] + counts["band"])


@pytest.mark.parametrize("dtype,D,G,budget,recent,bad", CASES[:2])
def test_free_running_chain(dtype, D, G, budget, recent, bad):
    B, Hkv, steps = 2, 4, 64
    seed = 200 + D + budget
    st, free, fc = _scaled_state(seed, dtype, B, Hkv, G, D, budget, _lengths(B, Hkv, budget))
    dirs = rng(seed).normal(0, 1, (B, Hkv, D))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    t0 = budget + 8
    d = Dev(st, free, fc)
    o, fl_o, fc_o = st, free, fc
    U = B * Hkv
    diverged = set()
    _say(f"{dtype} D{D} G{G} budget {budget} recent {recent}: {steps} free-running steps")
    for i in range(steps):
        q, k, v = _step_inputs(seed, i, dtype, B, Hkv, G, D, dirs)
        t = np.full(B, t0 + i, np.int32)
        before_o = o
        o, ev_o, fl_o, fc_o = oracle.h2o_step(o, q, k, v, t, budget, recent, free_list=fl_o,
                                              free_count=fc_o)
        ev_g = host(d.step(st, q, k, v, t, budget, recent))
        torch.cuda.synchronize()
        g, fl_g, fc_g = d.state(st)
        allsc = _lazy(lambda: _all_scores(before_o, q, k, v, t, budget, recent))
        live = [u for u in range(U) if u not in diverged]
        for u, vv in compare_step(before_o, g, o, ev_g, ev_o, allsc, t, budget, recent,
                                  TOL[dtype], f"step {i}", heads=live).items():
            if vv == "band":
                diverged.add(u)
        for u in diverged:  # followed by invariants only
            n = int(_flat(g, "seq_len")[u, 0])
            e = int(ev_g.reshape(-1)[u])
            tb = t0 + i
            assert n <= budget and e >= -1
            p = set(_flat(g, "pos")[u, :n].tolist())
            assert len(p) == n                       # positions unique
            assert tb in p or e == tb                # the new token placed or dropped
            assert e < 0 or tb - e >= recent         # nothing pruned inside the window
        check_free_lists(before_o["block_table"], g, o, fl_g, fc_g, fl_o, fc_o)
    _say(f"{dtype} D{D}: {len(diverged)} of {U} heads pruned a different token inside the "
         f"tolerance band")
    assert len(diverged) <= U // 2


def test_h2o_stream_870_full_size():
    """The decode workload at its real shape: B8, 8 KV heads x 4 query heads,
    D128, bf16, 806 -> 870 tokens in 64 appending steps, then 192 steps that
    prune one token each (budget 870, recent 435).  The GPU chain runs free
    beside the oracle's: pruned positions compared at every step, whole states
    every 16th step and at the end."""
    cfg = synth.CONFIGS["h2o_stream_870"]
    case = synth.make_case(cfg)
    B, Hkv, D = cfg.B, cfg.Hkv, cfg.D
    st = dict(case)
    st["score"] = np.zeros((B, Hkv, case["max_blocks"] * 16), np.float32)
    free = np.full(case["num_blocks"], -1, np.int32)
    d = Dev(st, free, 0)
    o, fl_o, fc_o = st, free, 0
    U = B * Hkv
    diverged = set()
    counts = {"append": 0, "prune": 0}
    _say(f"h2o_stream_870: {cfg.decode_steps} steps, oracle beside")
    for i in range(cfg.decode_steps):
        q, _ = synth.make_queries(cfg, 0, 1, case["dirs"], step=i)
        q = np.ascontiguousarray(q.reshape(B, cfg.Hq, D))
        k, v = synth.decode_token_kv(case, i)
        t = np.full(B, cfg.L + i, np.int32)
        before_o = o
        o, ev_o, fl_o, fc_o = oracle.h2o_step(o, q, k, v, t, cfg.budget, cfg.recent,
                                              free_list=fl_o, free_count=fc_o)
        ev_g = host(d.step(st, q, k, v, t, cfg.budget, cfg.recent))
        full = i % 16 == 15 or i == cfg.decode_steps - 1
        g = d.state(st)[0] if full else None
        allsc = _lazy(lambda: _all_scores(before_o, q, k, v, t, cfg.budget, cfg.recent))
        live = [u for u in range(U) if u not in diverged]
        for u, vv in compare_step(before_o, g, o, ev_g, ev_o, allsc, t, cfg.budget, cfg.recent,
                                  TOL[cfg.dtype], f"step {i}", heads=live).items():
            if vv == "band":
                diverged.add(u)
        counts["append" if i < cfg.budget - cfg.L else "prune"] += 1
        assert ((ev_g == -1) if i < cfg.budget - cfg.L else (ev_g >= 0)).all(), i
        if i % 64 == 63:
            _say(f"step {i + 1} done, {len(diverged)} heads diverged inside the band")
    assert fc_o == 0 and int(host(d.fc)[0]) == 0
    _say(f"{counts}; {len(diverged)} of {U} heads pruned a different token inside the band")
    assert len(diverged) <= U // 10


def test_short_free_list():
    """Heads that open a block in the same step, with fewer free blocks than
    heads: as many appends as blocks, the others refused with -3 and left
    unchanged; the taken blocks are the top of the list."""
    dtype, D, G, budget, recent = "bf16", 64, 2, 64, 8
    B, Hkv = 2, 4
    n0 = np.array([[16, 32, 48, 0], [16, 20, 64, 0]], np.int32)  # six heads open a block
    st, free, fc = _scaled_state(7, dtype, B, Hkv, G, D, budget, n0)
    free = free.copy()
    avail = 3
    d = Dev(st, free, avail)
    dirs = rng(7).normal(0, 1, (B, Hkv, D))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    q, k, v = _step_inputs(7, 0, dtype, B, Hkv, G, D, dirs)
    t = np.full(B, budget + 8, np.int32)
    ev = host(d.step(st, q, k, v, t, budget, recent)).reshape(-1)
    torch.cuda.synchronize()
    g, fl_g, fc_g = d.state(st)
    opens = [u for u in range(B * Hkv) if n0.reshape(-1)[u] < budget and n0.reshape(-1)[u] % 16 == 0]
    assert len(opens) == 6
    got = [u for u in opens if ev[u] == -1]
    assert len(got) == avail and all(ev[u] == -3 for u in opens if u not in got)
    assert fc_g == 0
    taken = sorted(int(_flat(g, "block_table")[u, n0.reshape(-1)[u] // 16]) for u in got)
    assert taken == sorted(free[:avail].tolist())
    # each head: the oracle's result for that head alone, with the block it got
    for u in range(B * Hkv):
        one = {key: (st[key].copy() if isinstance(st[key], np.ndarray) else st[key]) for key in st}
        seq = one["seq_len"].reshape(-1)
        for x in range(B * Hkv):
            if x != u:
                seq[x] = budget + 1  # refused with -2, untouched
        fl = np.full(4, -1, np.int32)
        cnt = 0
        if u in got:
            fl[0] = _flat(g, "block_table")[u, n0.reshape(-1)[u] // 16]
            cnt = 1
        o, ev_o, _, _ = oracle.h2o_step(one, q, k, v, t, budget, recent, free_list=fl,
                                        free_count=cnt)
        assert ev_o.reshape(-1)[u] == ev[u], u
        if ev[u] == -3:
            assert _flat(g, "seq_len")[u, 0] == n0.reshape(-1)[u]
            assert np.array_equal(_flat(g, "score")[u], _flat(st, "score")[u])
        else:
            _same_slots(g, o, u, int(_flat(o, "seq_len")[u, 0]), TOL[dtype], f"head {u}")


def test_graph_replay_matches_eager():
    """A run of decode steps captured as one HIP graph gives, on every replay
    from the same state, exactly the state the eager steps give (every head
    has its blocks, so no step depends on the order of free-list pops)."""
    dtype, D, G, budget, recent = "bf16", 128, 4, 100, 20
    B, Hkv, steps = 2, 4, 12
    seed = 301
    st, free, fc = _scaled_state(seed, dtype, B, Hkv, G, D, budget, _lengths(B, Hkv, budget),
                                 fresh=False)
    dirs = rng(seed).normal(0, 1, (B, Hkv, D))
    dirs /= np.linalg.norm(dirs, axis=-1, keepdims=True)
    d = Dev(st, free, fc)
    ins = []
    for i in range(steps):
        q, k, v = _step_inputs(seed, i, dtype, B, Hkv, G, D, dirs)
        ins.append((dev(q), dev(k), dev(v), dev(np.full(B, budget + 8 + i, np.int32))))
    ws = K.new_h2o_workspace(d.c, G, budget)
    ev = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    tensors = (d.c.k_pool, d.c.v_pool, d.c.block_table, d.c.seq_len, d.c.pos, d.score, d.fl, d.fc)
    snap = [t.clone() for t in tensors]

    def run():
        for q, k, v, t in ins:
            K.h2o_step(d.c, q, k, v, t, G, st["scale"], d.score, budget, recent, d.fl, d.fc, ws, ev)

    def restore():
        for t, s0 in zip(tensors, snap):
            t.copy_(s0)
        torch.cuda.synchronize()

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in tensors] + [ev.clone()]
    restore()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in tensors] + [ev.clone()]
        names = ("k_pool", "v_pool", "block_table", "seq_len", "pos", "score", "free_list",
                 "free_count", "evicted")
        for name, a, b in zip(names, got, eager):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
        U = B * Hkv  # arrival counters, then error flags at the next 256 bytes: left zero
        assert not host(ws[:4 * U]).any() and not host(ws[256:256 + 4 * U]).any()

