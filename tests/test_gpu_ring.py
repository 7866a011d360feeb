"""GPU parity of kvev_ring_step, SnapKV's decode-time ring buffer, against
oracle.ring_step.

Isolated steps: before every step the GPU receives the oracle's state (cache,
rings, ring indices, ranks), so each step is compared on its own.  The ring
weights are fp32 on the GPU and double rounded to fp32 in the oracle, so the
ring entry written by a step is compared to the tolerance (relative 1e-5:
both sides compute in fp32 or better whatever the cache dtype) and every
other ring entry bit for bit.  The dropped token must be the oracle's, or
its pooled score must lie within the tolerance of the oracle's choice (the
oracle's own pooled scores, from a run of the same step with room for one
more token, which appends instead of dropping); then that head is not
compared further in the step.  Positions, ranks, ring indices and K/V rows
are compared bit for bit.

A free-running chain at the full decode shape (B8, 8 KV heads x 4, D128,
budget 870, obsWindow 32, poolKernel 7, recent 32, 256 steps with null steps
among them) follows the same rule step by step, each side evolving by its own
steps (so every ring entry is compared to the tolerance); a head whose
dropped token differs inside the band is followed by invariants from then
on.
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import dev, device_cache, host
from tests.test_oracle_h2o_step import _enc, _state, _stream_inputs

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _say(msg):
    print(f"[ring] {msg}", flush=True)


def _pooled(st, u, t, pool):
    """Pooled scores of the n + 1 tokens (cached slots, then the new token)
    from a state whose rings already hold the step's weights."""
    B, Hkv = st["B"], st["Hkv"]
    b, h = divmod(u, Hkv)
    n = int(st["seq_len"][b, h])
    W = st["hist"].shape[2]
    S = np.zeros(n + 1, np.float32)
    for j in range(n):
        acc = np.float32(0)
        for w in range(W):
            acc = np.float32(acc + st["hist"][b, h, w, j])
        S[j] = acc
    P = np.array(list(st["pos"][b, h, :n]) + [t])
    order = np.argsort(P, kind="stable")
    r = (pool - 1) // 2
    pooled = np.zeros(n + 1, np.float32)
    for k in range(n + 1):
        pooled[order[k]] = S[order[max(0, k - r):min(n, k + r) + 1]].max()
    return pooled, P


class Dev:
    def __init__(self, st, free, fc):
        self.c = device_cache(st)
        self.fl = dev(free)
        self.fc = dev(np.array([fc], np.int32))
        self.load_ring(st)

    def load_ring(self, st):
        self.ring = K.RingState.__new__(K.RingState)
        self.ring.W = st["hist"].shape[2]
        self.ring.ws = {}
        self.ring.hist = dev(st["hist"])
        self.ring.ring = dev(st["ring"])
        self.ring.rank = dev(st["rank"])

    def step(self, st, q, k, v, t, observe, budget, recent, pool):
        return K.ring_step(self.c, self.ring, dev(q), dev(k), dev(v), dev(t), dev(observe),
                           st["G"], st["scale"], budget, recent, pool, self.fl, self.fc)

    def state(self, like):
        out = dict(like)
        out.update(k_pool=host(self.c.k_pool), v_pool=host(self.c.v_pool),
                   block_table=host(self.c.block_table), seq_len=host(self.c.seq_len),
                   pos=host(self.c.pos), hist=host(self.ring.hist), ring=host(self.ring.ring),
                   rank=host(self.ring.rank))
        return out


def _row(st, which, u, s):
    return st[which][st["block_table"].reshape(-1, st["max_blocks"])[u, s // 16], s % 16]


def _compare(pre, o, oev, g, gev, t, budget, recent, pool, wide, ring0, observe, skip=(),
             chain=False):
    """One step's outputs; returns the heads whose dropped token differs
    inside the band.  In a chain every ring entry was written by the side's
    own steps, so all of them are compared to the tolerance."""
    B, Hkv = pre["B"], pre["Hkv"]
    diverged = []
    for u in range(B * Hkv):
        if u in skip:
            continue
        b, h = divmod(u, Hkv)
        ge, oe = int(gev.reshape(-1)[u]), int(oev.reshape(-1)[u])
        if ge != oe:
            assert ge >= 0 and oe >= 0, (u, ge, oe)
            pooled, P = _pooled(wide, u, t, pool)
            pg = pooled[list(P).index(ge)]
            po = pooled[list(P).index(oe)]
            assert t - ge >= recent
            assert abs(float(pg) - float(po)) <= TOL * max(abs(float(po)), 1e-30), (u, pg, po)
            diverged.append(u)
            continue
        n = int(o["seq_len"][b, h])
        assert int(g["seq_len"][b, h]) == n
        assert np.array_equal(g["pos"][b, h, :n], o["pos"][b, h, :n]), u
        assert np.array_equal(g["rank"][b, h, :n], o["rank"][b, h, :n]), u
        assert g["ring"][b, h] == o["ring"][b, h], u
        for s in range(n):
            assert np.array_equal(_row(g, "k_pool", u, s), _row(o, "k_pool", u, s)), (u, s)
            assert np.array_equal(_row(g, "v_pool", u, s), _row(o, "v_pool", u, s)), (u, s)
        gh, oh = g["hist"][b, h, :, :n], o["hist"][b, h, :, :n]
        written = int(ring0[b, h]) if observe[b] else -1
        for w in range(gh.shape[0]):
            if w == written or chain:
                err = np.abs(gh[w].astype(np.float64) - oh[w])
                assert (err <= TOL * np.maximum(np.abs(oh[w]), 1e-30) + 1e-12).all(), (u, w)
            else:
                assert np.array_equal(gh[w], oh[w]), (u, w)
    return diverged


def _ring_case(seed, dtype, B, Hkv, G, D, budget, n0, W, steps=40):
    keys, vals, qs = _stream_inputs(seed, B, Hkv, G, D, max(512, n0 + steps))
    st = _state(keys, vals, n0, budget + 1, G, dtype=dtype)
    st = oracle.ring_state(st, W)
    return st, keys, vals, qs


CASES = [
    # dtype, D, G, budget, recent, W, pool, n0[, B, Hkv, steps]
    ("bf16", 128, 4, 100, 20, 8, 7, 96),
    ("f32", 64, 2, 40, 0, 3, 1, 38),
    ("bf16", 64, 8, 57, 1, 5, 5, 50),
    ("f32", 128, 4, 48, 6, 16, 3, 44),
    # budgets over 1024 (four slots per thread in the last workgroup), rings
    # of more than 32 entries, a pooling radius past 8
    ("bf16", 64, 2, 1300, 40, 40, 19, 1290),
    # 256 heads: one workgroup per head, whose 700 slots exceed one pass of
    # its thread pairs over the ring entries
    ("bf16", 64, 1, 700, 16, 6, 5, 694, 32, 8, 10),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_isolated_steps(case):
    dtype, D, G, budget, recent, W, pool, n0 = case[:8]
    B, Hkv, steps = case[8:] if len(case) > 8 else (2, 3, 40)
    st, keys, vals, qs = _ring_case(7 + D + G, dtype, B, Hkv, G, D, budget, n0, W, steps)
    d = Dev(st, np.full(st["num_blocks"], -1, np.int32), 0)
    drops = 0
    for i, t in enumerate(range(n0, n0 + steps)):
        observe = np.array([int((t + b) % 5 != 0) for b in range(B)], np.int32)
        q, k, v = _enc(qs[t], st), _enc(keys[:, :, t], st), _enc(vals[:, :, t], st)
        tp = np.full(B, t, np.int32)
        d = Dev(st, np.full(st["num_blocks"], -1, np.int32), 0)   # the oracle's state
        gev = host(d.step(st, q, k, v, tp, observe, budget, recent, pool))
        g = d.state(st)
        o, oev, _, _ = oracle.ring_step(st, q, k, v, tp, observe, budget, recent, pool)
        wide, _, _, _ = oracle.ring_step(st, q, k, v, tp, observe, budget + 1, recent, pool)
        _compare(st, o, oev, g, gev, t, budget, recent, pool, wide, st["ring"], observe)
        drops += int((oev >= 0).sum())
        st = o
    assert drops > 0
    _say(f"{case}: {drops} drops over {steps} steps")


def test_free_running_chain_full_decode_shape():
    """B8, 8 KV heads x 4, D128 bf16; 806 cached tokens grow to the budget
    870, then one token is dropped per step; obsWindow 32, poolKernel 7,
    recent 32; every seventh step of a sequence is a null step."""
    cfg = synth.CONFIGS["h2o_stream_870"]
    case = synth.make_case(cfg)
    B, Hkv, G = cfg.B, cfg.Hkv, cfg.G
    budget, recent, W, pool = cfg.budget, 32, 32, 7
    st = oracle.ring_state(dict(case), W)
    d = Dev(st, np.full(case["num_blocks"], -1, np.int32), 0)
    gone = set()
    total = 0
    for i in range(cfg.decode_steps):
        t = cfg.L + i
        q, _ = synth.make_queries(cfg, 0, 1, case["dirs"], step=i)
        q = q.reshape(B, cfg.Hq, cfg.D)
        k, v = synth.decode_token_kv(case, i)
        tp = np.full(B, t, np.int32)
        observe = np.array([int((i + b) % 7 != 3) for b in range(B)], np.int32)
        ring0 = st["ring"].copy()
        gev = host(d.step(st, q, k, v, tp, observe, budget, recent, pool))
        o, oev, _, _ = oracle.ring_step(st, q, k, v, tp, observe, budget, recent, pool)
        g = d.state(st)
        wide = None
        if not np.array_equal(gev, oev):
            wide, _, _, _ = oracle.ring_step(st, q, k, v, tp, observe, budget + 1, recent, pool)
        div = _compare(st, o, oev, g, gev, t, budget, recent, pool, wide, ring0, observe,
                       skip=gone, chain=True)
        gone.update(div)
        total += int((oev >= 0).sum())
        st = o
        if i % 32 == 0:
            _say(f"step {i}: {len(gone)} heads diverged inside the band")
    # every head, diverged or not: the budget, the recent window, ranks in position order
    g = d.state(st)
    for u in range(B * Hkv):
        b, h = divmod(u, Hkv)
        n = int(g["seq_len"][b, h])
        p = g["pos"][b, h, :n]
        assert n == budget and len(set(p.tolist())) == n
        assert set(range(t - recent + 1, t + 1)) <= set(p.tolist())
        assert np.array_equal(g["rank"][b, h, :n], np.argsort(np.argsort(p)))
    _say(f"chain: {total} drops, {len(gone)} of {B * Hkv} heads diverged inside the band")


def test_ring_init_and_appends_with_free_list_pops():
    """kvev_ring_init matches oracle.ring_state; an append that opens a block
    takes it from the top of the free list."""
    B, Hkv, G, D, W = 1, 2, 2, 64, 4
    keys, vals, qs = _stream_inputs(31, B, Hkv, G, D, 64)
    st = _state(keys, vals, 32, 64, G, dtype="bf16")
    st["pos"][0, 1, :32] = np.random.default_rng(3).permutation(100)[:32]   # shuffled order
    st = oracle.ring_state(st, W)
    dc = device_cache(st)
    rs = K.RingState(dc, W)
    torch.cuda.synchronize()
    assert (host(rs.hist) == 0).all() and (host(rs.ring) == 0).all()
    assert np.array_equal(host(rs.rank)[:, :, :32], st["rank"][:, :, :32])
    # slot 32 opens logical block 2: it comes from the free list
    st["block_table"][:, :, 2:] = -1
    free = np.full(st["num_blocks"], -1, np.int32)
    spare = [int(x) for x in range(st["num_blocks"]) if x not in set(st["block_table"].ravel())]
    free[:2] = spare[:2]
    d = Dev(st, free, 2)
    t = 200
    q, k, v = _enc(qs[0], st), _enc(keys[:, :, 40], st), _enc(vals[:, :, 40], st)
    gev = host(d.step(st, q, k, v, np.full(B, t, np.int32), np.ones(B, np.int32), 48, 4, 3))
    o, oev, ofl, ofc = oracle.ring_step(st, q, k, v, np.full(B, t, np.int32), np.ones(B, np.int32),
                                        48, 4, 3, free_list=free, free_count=2)
    assert (gev == -1).all() and (oev == -1).all()
    assert int(host(d.fc)[0]) == ofc == 0
    g = d.state(st)
    taken_g = sorted(g["block_table"][0, :, 2].tolist())
    assert taken_g == sorted(o["block_table"][0, :, 2].tolist()) == sorted(spare[:2])
    for h in range(Hkv):
        assert np.array_equal(g["rank"][0, h, :33], o["rank"][0, h, :33])
        assert np.array_equal(_row(g, "k_pool", h, 32), k[0, h])
