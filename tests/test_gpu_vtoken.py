"""GPU parity of vToken's liveness marks (kvev_vtok_evict) and lazy,
threshold-gated reclamation (kvev_vtok_reclaim) against oracle.vtok_evict and
oracle.vtok_reclaim.

Both sides are integer work and copies, and both take the same decisions in
the same order (first fit in (b, h) order, destinations from the top of the
free list, sources appended after every head has planned), so every output
is compared bit for bit: both pools whole, block tables, positions, liveness,
live counts, score rows, the free list and its count, and the statistics.

States are built here: shuffled block ids, ragged lengths (empty heads and
partial tail blocks among them), random liveness with some full and some
empty blocks, -1 entries left by earlier reclamations, and a few heads the
call must skip (a length past the capacity, a block id past the pool, a live
count out of range).
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import dev, device_cache, host

pytestmark = pytest.mark.gpu
rng = np.random.default_rng


def _say(msg):
    print(f"[vtok] {msg}", flush=True)


def _state(seed, dtype="bf16", D=128, B=2, Hkv=3, max_blocks=12, spare=40, holes=True,
           bad=()):
    """A vToken state with shuffled ids and a free list of the unused ids.
    bad: (kind, unit) pairs with kind "len", "id" or "count"."""
    r = rng(seed)
    U = B * Hkv
    num_blocks = U * max_blocks + spare
    perm = synth.shuffled(num_blocks, seed, 11)
    bt = perm[:U * max_blocks].reshape(B, Hkv, max_blocks).astype(np.int32).copy()
    edt = np.uint16 if dtype == "bf16" else np.float32
    k_pool = synth.encode(r.normal(0, 1, (num_blocks, 16, D)), dtype).astype(edt)
    v_pool = synth.encode(r.normal(0, 1, (num_blocks, 16, D)), dtype).astype(edt)
    ms = max_blocks * 16
    seq = r.integers(0, ms + 1, size=(B, Hkv)).astype(np.int32)
    seq.reshape(-1)[0] = ms                # a head at capacity
    if U > 2:
        seq.reshape(-1)[1] = 0             # an empty head
        seq.reshape(-1)[2] = ms - 5        # a partial tail block
    pos = np.zeros((B, Hkv, ms), np.int32)
    live = np.zeros((B, Hkv, ms), np.uint8)
    for u in range(U):
        b, h = divmod(u, Hkv)
        n = int(seq[b, h])
        pos[b, h] = r.permutation(1 << 20)[:ms].astype(np.int32)   # any unique positions
        nb = (n + 15) // 16
        for lb in range(nb):
            lo, hi = lb * 16, min(n, lb * 16 + 16)
            kind = r.integers(0, 5)
            if kind == 0:
                keep = np.ones(hi - lo, bool)                     # full
            elif kind == 1:
                keep = np.zeros(hi - lo, bool)                    # every token evicted
            else:
                keep = r.uniform(0, 1, hi - lo) < r.uniform(0.1, 0.9)
            live[b, h, lo:hi] = keep
        bt[b, h, nb:] = -1
        if holes and nb > 3:               # entries freed by an earlier reclamation
            for lb in r.choice(nb - 1, size=min(2, nb - 2), replace=False):
                bt[b, h, lb] = -1
                live[b, h, lb * 16:lb * 16 + 16] = 0
    block_live = live.reshape(B, Hkv, max_blocks, 16).sum(-1).astype(np.int32)
    for kind, u in bad:
        b, h = divmod(u, Hkv)
        if kind == "len":
            seq[b, h] = ms + 16
        elif kind == "id":
            bt[b, h, 0] = num_blocks + 5
        elif kind == "count":
            seq[b, h] = ms
            bt[b, h, 1] = perm[u * max_blocks + 1]
            block_live[b, h, 1] = 17
    used = set(bt[bt >= 0].tolist())
    free = np.array([x for x in perm.tolist() if x not in used and x < num_blocks], np.int32)
    fl = np.full(num_blocks + 8, -1, np.int32)
    fl[:free.size] = free
    score = r.uniform(0, 1, (B, Hkv, ms)).astype(np.float32)
    st = dict(dtype=dtype, B=B, Hkv=Hkv, D=D, max_blocks=max_blocks, num_blocks=num_blocks,
              k_pool=k_pool, v_pool=v_pool, block_table=bt, seq_len=seq, pos=pos, live=live,
              block_live=block_live, score=score)
    return st, fl, int(free.size)


class Dev:
    """Device copy of a vToken state."""

    def __init__(self, st, fl, fc):
        self.c = device_cache(st)
        self.live = dev(st["live"])
        self.block_live = dev(st["block_live"])
        self.score = dev(st["score"])
        self.fl = dev(fl)
        self.fc = dev(np.array([fc], np.int32))
        self.ws = None

    def reclaim(self, theta, max_sources, with_score=True, stream=None):
        if self.ws is None or self.ws_ms < max_sources:
            self.ws = K.new_vtok_workspace(self.c, max_sources)
            self.ws_ms = max_sources
        return K.vtok_reclaim(self.c, self.live, self.block_live, theta, max_sources, self.fl,
                              self.fc, self.ws, score=self.score if with_score else None,
                              stream=stream)

    def evict(self, vic, nv):
        if getattr(self, "ews", None) is None:
            self.ews = K.new_vtok_evict_workspace(self.c)
        return K.vtok_evict(self.c, self.live, self.block_live, dev(vic), dev(nv), self.ews)

    def state(self, like):
        out = dict(like)
        out.update(k_pool=host(self.c.k_pool), v_pool=host(self.c.v_pool),
                   block_table=host(self.c.block_table), pos=host(self.c.pos),
                   live=host(self.live), block_live=host(self.block_live),
                   score=host(self.score))
        return out, host(self.fl), int(host(self.fc)[0])


def _same(o, g, keys, what=""):
    for k in keys:
        if not np.array_equal(o[k], g[k]):
            bad = np.argwhere(o[k] != g[k])
            raise AssertionError(f"{what}: {k} differs at {len(bad)} places, first "
                                 f"{bad[0].tolist()}: oracle {o[k][tuple(bad[0])]!r} "
                                 f"gpu {g[k][tuple(bad[0])]!r}")


STATE_KEYS = ("k_pool", "v_pool", "block_table", "pos", "live", "block_live", "score")


def _compare_reclaim(st, fl, fc, d, theta, max_sources, stats_g, with_score=True, what=""):
    o, ofl, ofc, ost = oracle.vtok_reclaim(st, theta, max_sources, fl, fc, with_score=with_score)
    torch.cuda.synchronize()
    g, gfl, gfc = d.state(st)
    keys = STATE_KEYS if with_score else STATE_KEYS[:-1]
    _same(o, g, keys, what)
    assert gfc == ofc, (what, gfc, ofc)
    assert np.array_equal(gfl[:gfc], ofl[:ofc]), what
    assert host(stats_g).tolist() == ost.tolist(), (what, host(stats_g).tolist(), ost.tolist())
    return o, ofl, ofc, ost


# ------------------------------------------------------------------ marks


@pytest.mark.parametrize("seed", [0, 1])
def test_evict_marks_bit_exact(seed):
    st, fl, fc = _state(seed, B=2, Hkv=4, max_blocks=10)
    U, ms = 8, 160
    r = rng(100 + seed)
    vic = np.full((2, 4, ms), -1, np.int32)
    nv = np.zeros((2, 4), np.int32)
    for u in range(U):
        b, h = divmod(u, 4)
        cand = np.flatnonzero(st["live"][b, h])
        m = int(r.integers(0, max(1, cand.size - 8)))
        v = r.permutation(cand)[:m].tolist()
        if u == 3:   # invalid victims: negative, past the length, already dead, a repeat
            dead = np.flatnonzero(st["live"][b, h, :int(st["seq_len"][b, h])] == 0)
            v += [-4, int(st["seq_len"][b, h]) + 1, ms + 7] + dead[:2].tolist()
            if v[:1]:
                v.append(v[0])
        vic[b, h, :len(v)] = v
        nv[b, h] = len(v)
    _say(f"evict seed {seed}: {int(nv.sum())} victims")
    d = Dev(st, fl, fc)
    status = d.evict(vic, nv)
    o, ostatus = oracle.vtok_evict(st, vic, nv)
    torch.cuda.synchronize()
    assert int(host(status)[0]) == ostatus
    assert ostatus == 1
    assert np.array_equal(host(d.live), o["live"])
    assert np.array_equal(host(d.block_live), o["block_live"])
    # a clean batch leaves the status at 0
    nv2 = np.zeros_like(nv)
    assert int(host(d.evict(vic, nv2))[0]) == 0


# ------------------------------------------------------------ reclamation


CASES = [
    # dtype, D, B, Hkv, max_blocks, spare, free count cap, theta, max_sources, bad
    ("bf16", 128, 2, 3, 12, 200, None, 0.25, 8, ()),                  # every plan fits
    ("f32", 64, 2, 4, 20, 200, None, 0.10, 64, (("len", 5),)),
    ("bf16", 64, 1, 8, 16, 6, 5, 0.0, 16, (("id", 2), ("count", 6))),  # first fit, deferrals
    ("f32", 128, 3, 2, 9, 0, 0, 0.0, 4, ()),                          # no headroom at all
    ("bf16", 128, 4, 8, 40, 300, None, 0.25, 2, ()),                  # the smallest batch
    ("bf16", 128, 2, 2, 300, 5000, None, 0.25, 4096, ()),             # long heads, one batch
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[1]}-{c[2]}x{c[3]}-"
                         f"mb{c[4]}-fc{c[6]}-th{c[7]}-ms{c[8]}")
def test_reclaim_bit_exact(case):
    dtype, D, B, Hkv, mb, spare, cap, theta, ms, bad = case
    st, fl, fc = _state(7 + mb, dtype=dtype, D=D, B=B, Hkv=Hkv, max_blocks=mb, spare=spare,
                        bad=bad)
    if cap is not None:   # only the first `cap` entries of the list are free
        fc = min(fc, cap)
    _say(f"reclaim {case}: free {fc}")
    d = Dev(st, fl, fc)
    stats = d.reclaim(theta, ms)
    o, ofl, ofc, ost = _compare_reclaim(st, fl, fc, d, theta, ms, stats, what=str(case))
    _say(f"stats {ost.tolist()}")
    if bad:
        assert ost[9] != 0
    if cap == 0:
        assert ost[0] == 0 and ost[1] > 0
    elif cap is not None:
        assert ost[0] > 0 and ost[1] > 0
    else:
        assert ost[1] == 0 and ost[0] > 0


def test_reclaim_without_score_row():
    st, fl, fc = _state(3, B=2, Hkv=2, max_blocks=12, spare=100)
    d = Dev(st, fl, fc)
    stats = d.reclaim(0.1, 16, with_score=False)
    _compare_reclaim(st, fl, fc, d, 0.1, 16, stats, with_score=False, what="no score")
    assert np.array_equal(host(d.score), st["score"])


def test_free_count_out_of_range_admits_nothing():
    st, fl, fc = _state(4, B=1, Hkv=4, max_blocks=12, spare=100)
    d = Dev(st, fl, fc)
    d.fc.fill_(st["num_blocks"] + 1)     # more entries than blocks: refused on the device
    stats = d.reclaim(0.0, 16)
    torch.cuda.synchronize()
    s = host(stats)
    assert s[9] & 8 and s[0] == 0 and s[3] == 0
    assert int(host(d.fc)[0]) == st["num_blocks"] + 1
    assert np.array_equal(host(d.c.block_table), st["block_table"])


def test_chain_of_marks_and_reclamations():
    """Each side evolves by its own calls: marks, a reclamation, more marks,
    another, with the free list carried over; identical at every stage."""
    st, fl, fc = _state(21, B=2, Hkv=4, max_blocks=24, spare=60)
    d = Dev(st, fl, fc)
    r = rng(5)
    for it in range(4):
        U, ms = 8, 24 * 16
        vic = np.full((2, 4, ms), -1, np.int32)
        nv = np.zeros((2, 4), np.int32)
        for u in range(U):
            b, h = divmod(u, 4)
            cand = np.flatnonzero(st["live"][b, h, :int(st["seq_len"][b, h])])
            m = int(r.integers(0, cand.size // 3 + 1))
            vic[b, h, :m] = r.permutation(cand)[:m]
            nv[b, h] = m
        st, _ = oracle.vtok_evict(st, vic, nv)
        d.evict(vic, nv)
        stats = d.reclaim(0.25, 6)
        st, fl, fc, ost = _compare_reclaim(st, fl, fc, d, 0.25, 6, stats, what=f"iteration {it}")
        _say(f"iteration {it}: stats {ost.tolist()}")


def test_reclaim_on_a_relocation_stream():
    """The copies run on a stream of their own; the next reader waits on an
    event recorded after them (a GPU-side wait, no host synchronisation)."""
    st, fl, fc = _state(30, B=2, Hkv=4, max_blocks=30, spare=200)
    d = Dev(st, fl, fc)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    ready = torch.cuda.Event()
    ready.record(main)                          # the state is written on the main stream
    side.wait_event(ready)
    stats = d.reclaim(0.25, 32, stream=side)
    done = torch.cuda.Event()
    done.record(side)
    main.wait_event(done)
    # a reader on the main stream: the block table and both pools, copied there
    bt = d.c.block_table.clone()
    kp = d.c.k_pool.clone()
    vp = d.c.v_pool.clone()
    st_h = stats.clone()
    torch.cuda.synchronize()
    o, ofl, ofc, ost = oracle.vtok_reclaim(st, 0.25, 32, fl, fc, with_score=True)
    assert np.array_equal(host(bt), o["block_table"])
    assert np.array_equal(host(kp), o["k_pool"]) and np.array_equal(host(vp), o["v_pool"])
    assert host(st_h).tolist() == ost.tolist()
    assert ost[0] > 0


# ------------------------------------- sync_new_tokens and slot mapping


def test_sync_bit_exact():
    st, fl, fc = _state(71, B=2, Hkv=4, max_blocks=20, spare=200, holes=False)
    r = rng(72)
    U, ms = 8, 20 * 16
    new_len = st["seq_len"].copy()
    free = list(fl[:fc])
    for u in range(U):
        b, h = divmod(u, 4)
        n = int(st["seq_len"][b, h])
        m = min(ms, n + int(r.integers(0, 60)))
        for lb in range((n + 15) // 16, (m + 15) // 16):   # the caller's allocator
            st["block_table"][b, h, lb] = free.pop()
        new_len[b, h] = m
    new_len[0, 1] = int(st["seq_len"][0, 1]) - 1 if st["seq_len"][0, 1] > 0 else ms + 1  # -2
    n6 = int(st["seq_len"][1, 2])
    if n6 + 20 <= ms:                                   # a block without an id: -4
        new_len[1, 2] = n6 + 20
        st["block_table"][1, 2, (n6 + 19) // 16] = -1
    pos0 = np.array([1000, 5000], np.int32)
    d = Dev(st, fl, fc)
    status = K.vtok_sync(d.c, d.live, d.block_live, dev(new_len), dev(pos0))
    o, ostat = oracle.vtok_sync(st, new_len, pos0)
    torch.cuda.synchronize()
    assert host(status).tolist() == ostat.tolist()
    assert (ostat == 0).sum() >= 5 and (ostat == -2).sum() >= 1
    assert np.array_equal(host(d.c.seq_len), o["seq_len"])
    assert np.array_equal(host(d.c.pos), o["pos"])
    assert np.array_equal(host(d.live), o["live"])
    assert np.array_equal(host(d.block_live), o["block_live"])


@pytest.mark.parametrize("seed", [80, 81])
def test_slot_mapping_bit_exact_after_reclamation(seed):
    st, fl, fc = _state(seed, B=2, Hkv=4, max_blocks=30, spare=150, bad=(("len", 6),))
    d = Dev(st, fl, fc)
    d.reclaim(0.1, 16)
    g_slots, g_pos, g_cnt = K.vtok_slot_mapping(d.c, d.live)
    o, _, _, _ = oracle.vtok_reclaim(st, 0.1, 16, fl, fc, with_score=True)
    slots, positions, count = oracle.vtok_slot_mapping(o)
    torch.cuda.synchronize()
    gc = host(g_cnt)
    assert np.array_equal(gc, count) and count[1, 2] == -1
    gs, gp = host(g_slots), host(g_pos)
    for b in range(2):
        for h in range(4):
            k = max(0, int(count[b, h]))
            assert np.array_equal(gs[b, h, :k], slots[b, h, :k]), (b, h)
            assert np.array_equal(gp[b, h, :k], positions[b, h, :k]), (b, h)


# ---------------------------------------------- online checks of I1, I2


def _digest(d):
    return host(K.vtok_digest(d.c, d.live)).view(np.uint64)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("bf16", 64), ("f32", 128)])
def test_digest_and_check_match_the_oracle(dtype, D):
    st, fl, fc = _state(50 + D, dtype=dtype, D=D, B=2, Hkv=4, max_blocks=20, spare=80,
                        bad=(("len", 5),))
    d = Dev(st, fl, fc)
    g = _digest(d)
    o = oracle.vtok_digest(st)
    assert np.array_equal(g, o)
    cws = K.new_vtok_check_workspace(d.c)
    assert host(K.vtok_check(d.c, d.live, d.block_live, d.fl, d.fc, cws)).tolist() == \
        oracle.vtok_check(st, fl, fc).tolist()
    # planted faults, each against the oracle
    bt = st["block_table"].copy()
    bt[1, 2, 0] = bt[0, 0][bt[0, 0] >= 0][0]       # a second owner of a held block
    bt[1, 3, 1] = st["num_blocks"] + 2             # out of range
    bl = st["block_live"].copy()
    lb = int(np.flatnonzero(bt[0, 0] >= 0)[-1])
    bl[0, 0, lb] += 1                              # a count off by one
    m = dict(st, block_table=bt, block_live=bl)
    d2 = Dev(m, fl, fc)
    want = oracle.vtok_check(m, fl, fc)
    assert want[0] >= 1 and want[2] >= 1 and want[3] >= 1
    assert host(K.vtok_check(d2.c, d2.live, d2.block_live, d2.fl, d2.fc, cws)).tolist() == \
        want.tolist()
    assert np.array_equal(_digest(d2), oracle.vtok_digest(m))


def test_online_checks_around_reclamation():
    """I1: every head's digest is the same before and after the relocation;
    I2: every block held once, every live count right, after it."""
    st, fl, fc = _state(61, B=2, Hkv=4, max_blocks=40, spare=200)
    d = Dev(st, fl, fc)
    before = _digest(d)
    stats = d.reclaim(0.1, 64)
    after = _digest(d)
    cws = K.new_vtok_check_workspace(d.c)
    chk = host(K.vtok_check(d.c, d.live, d.block_live, d.fl, d.fc, cws))
    torch.cuda.synchronize()
    assert host(stats)[0] > 0
    assert np.array_equal(before, after) and np.array_equal(before, oracle.vtok_digest(st))
    assert chk.tolist() == [0, 0, 0, 0]


def test_full_size_random_eviction_layer():
    """One layer of the block-aware workload (B16, 8 KV heads, D128, 64000
    tokens: 4000 blocks a head, about 4.2 GB of K+V) with half of every head's
    tokens marked dead by a uniform random policy (16 recent protected), then
    one reclamation whose source batch covers the whole head (4096), in the
    launch configuration of the benchmark.  Every output against the oracle."""
    cfg = synth.CONFIGS["block_evict_64k"]
    U = cfg.B * cfg.Hkv
    case = synth.make_case(cfg, spare_blocks=U * 2048)
    _say("full size: state built")
    st = dict(case)
    st["live"], st["block_live"] = oracle.vtok_liveness(case)
    st["score"] = np.zeros((cfg.B, cfg.Hkv, case["max_blocks"] * 16), np.float32)
    vic, nv = synth.random_victims(case, cfg.budget, cfg.recent)
    used = set(case["block_table"][case["block_table"] >= 0].tolist())
    free = np.array([x for x in range(case["num_blocks"]) if x not in used], np.int32)
    fl = np.full(case["num_blocks"], -1, np.int32)
    fl[:free.size] = free
    d = Dev(st, fl, free.size)
    d.evict(vic, nv)
    before = _digest(d)
    stats = d.reclaim(0.25, 4096, with_score=False)
    after = _digest(d)
    cws = K.new_vtok_check_workspace(d.c)
    chk = host(K.vtok_check(d.c, d.live, d.block_live, d.fl, d.fc, cws))
    assert np.array_equal(before, after) and chk.tolist() == [0, 0, 0, 0]   # I1, I2 online
    _say("full size: GPU done; oracle")
    st2, _ = oracle.vtok_evict(st, vic, nv)
    o, ofl, ofc, ost = oracle.vtok_reclaim(st2, 0.25, 4096, fl, free.size)
    torch.cuda.synchronize()
    _say(f"full size: stats {ost.tolist()}")
    assert host(stats).tolist() == ost.tolist()
    assert ost[0] == U and ost[1] == 0
    for k, t in (("block_table", d.c.block_table), ("pos", d.c.pos), ("live", d.live),
                 ("block_live", d.block_live)):
        assert np.array_equal(host(t), o[k]), k
    gfc = int(host(d.fc)[0])
    assert gfc == ofc and np.array_equal(host(d.fl)[:gfc], ofl[:ofc])
    # the pools: every destination block whole (the rows the copies wrote)
    dest = np.setdiff1d(o["block_table"][o["block_table"] >= 0],
                        st2["block_table"][st2["block_table"] >= 0])
    kp, vp = host(d.c.k_pool), host(d.c.v_pool)
    assert np.array_equal(kp[dest], o["k_pool"][dest]) and np.array_equal(vp[dest], o["v_pool"][dest])
    assert np.array_equal(kp, o["k_pool"]) and np.array_equal(vp, o["v_pool"])
    assert np.array_equal(after, oracle.vtok_digest(o))


def test_algorithm1_runtime_loop():
    """The review's Algorithm 1 as a loop of decode steps, GPU beside the
    oracle: SyncNewTokens (one token a step), SelectVictims (a seeded random
    policy over the live tokens outside a recent window of 8), EvictToken,
    BuildSlotMapping, and every eighth step ReclaimAsync on a relocation stream
    that the next step waits for through an event.  Every table, pool and
    mapping is compared bit for bit at every step, and the online checks
    (digests equal across each reclamation, the block check clean) hold."""
    B, Hkv, D, mb = 2, 2, 64, 24
    st, fl, fc = _state(90, D=D, B=B, Hkv=Hkv, max_blocks=mb, spare=40, holes=False)
    # every block of the capacity allocated up front (the allocator's job);
    # the heads start at 100 live tokens
    used = set(st["block_table"][st["block_table"] >= 0].tolist())
    spare = [x for x in range(st["num_blocks"]) if x not in used]
    for b in range(B):
        for h in range(Hkv):
            for lb in range(mb):
                if st["block_table"][b, h, lb] < 0:
                    st["block_table"][b, h, lb] = spare.pop()
    st["seq_len"][:] = 0
    st["live"][:] = 0
    st["block_live"][:] = 0
    st, s0 = oracle.vtok_sync(st, np.full((B, Hkv), 100, np.int32), np.zeros(B, np.int32))
    assert (s0 == 0).all()
    fl = np.full(st["num_blocks"], -1, np.int32)
    fl[:len(spare)] = spare
    fc = len(spare)
    d = Dev(st, fl, fc)
    ws = K.new_vtok_workspace(d.c, 8)
    cws = K.new_vtok_check_workspace(d.c)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    r = rng(91)
    for step in range(40):
        t = 100 + step
        n = st["seq_len"].copy()
        # 1. SyncNewTokens
        K.vtok_sync(d.c, d.live, d.block_live, dev(n + 1), dev(np.full(B, t, np.int32)))
        st, ss = oracle.vtok_sync(st, n + 1, np.full(B, t, np.int32))
        assert (ss == 0).all()
        # 2-3. SelectVictims (random policy) and EvictToken
        vic = np.full((B, Hkv, mb * 16), -1, np.int32)
        nv = np.zeros((B, Hkv), np.int32)
        for b in range(B):
            for h in range(Hkv):
                m = int(st["seq_len"][b, h])
                ok = np.flatnonzero((st["live"][b, h, :m] != 0) & (st["pos"][b, h, :m] <= t - 8)
                                    & (st["block_table"][b, h, np.arange(m) // 16] >= 0))
                k = int(r.integers(0, 3))
                pick = r.choice(ok, size=min(k, ok.size), replace=False) if ok.size else []
                vic[b, h, :len(pick)] = pick
                nv[b, h] = len(pick)
        d.evict(vic, nv)
        st, es = oracle.vtok_evict(st, vic, nv)
        assert es == 0
        # 4. BuildSlotMapping
        gs, gp, gc = K.vtok_slot_mapping(d.c, d.live)
        os_, op, oc = oracle.vtok_slot_mapping(st)
        assert np.array_equal(host(gc), oc)
        for b in range(B):
            for h in range(Hkv):
                k = int(oc[b, h])
                assert np.array_equal(host(gs)[b, h, :k], os_[b, h, :k])
                assert np.array_equal(host(gp)[b, h, :k], op[b, h, :k])
        # 5. ReclaimAsync on the relocation stream, after this step's work
        if step % 8 == 7:
            before = _digest(d)
            ready = torch.cuda.Event()
            ready.record(main)
            side.wait_event(ready)
            K.vtok_reclaim(d.c, d.live, d.block_live, 0.25, 8, d.fl, d.fc, ws, stream=side)
            done = torch.cuda.Event()
            done.record(side)
            main.wait_event(done)   # the next step's reads wait on the GPU side only
            st, fl, fc, ost = oracle.vtok_reclaim(st, 0.25, 8, fl, fc)
            after = _digest(d)
            chk = host(K.vtok_check(d.c, d.live, d.block_live, d.fl, d.fc, cws))
            assert np.array_equal(before, after) and chk.tolist() == [0, 0, 0, 0]
            _say(f"step {step}: reclaimed {ost[0]} heads, {ost[3]} blocks freed")
        torch.cuda.synchronize()
        g, gfl, gfc = d.state(st)
        for key in ("block_table", "pos", "live", "block_live", "k_pool", "v_pool"):
            assert np.array_equal(g[key], st[key]), (step, key)
        assert np.array_equal(host(d.c.seq_len), st["seq_len"])
        assert gfc == fc and np.array_equal(gfl[:gfc], fl[:fc]), step


def test_vtoken_calls_leave_a_shared_workspace_state_alone():
    """The vToken calls write only past the workspace's state part: on one
    buffer shared with kvev_select, a selection after marks and a
    reclamation gives the victims a fresh buffer gives (claim words at the
    start of the buffer would have left its selection histograms non-zero)."""
    st, fl, fc = _state(5, B=2, Hkv=3, max_blocks=12)
    d = Dev(st, fl, fc)
    r = rng(55)
    U, ms = 6, 12 * 16
    vic = np.full((2, 3, ms), -1, np.int32)
    nv = np.zeros((2, 3), np.int32)
    for u in range(U):
        b, h = divmod(u, 3)
        cand = np.flatnonzero(st["live"][b, h])
        v = np.sort(r.permutation(cand)[:cand.size // 2])
        vic[b, h, :v.size] = v
        nv[b, h] = v.size
    n = max(K.new_vtok_evict_workspace(d.c).numel(), K.new_vtok_workspace(d.c, 8).numel(),
            K.new_workspace(d.c).numel())
    shared = torch.zeros(n, dtype=torch.uint8, device="cuda")
    K.vtok_evict(d.c, d.live, d.block_live, dev(vic), dev(nv), shared)
    K.vtok_reclaim(d.c, d.live, d.block_live, 0.0, 8, d.fl, d.fc, shared, score=d.score)
    scores = dev(r.uniform(0, 1, (2, 3, ms)).astype(np.float32))
    v1, n1 = K.select(d.c, scores, 40, 4, workspace=shared)
    v2, n2 = K.select(d.c, scores, 40, 4, workspace=K.new_workspace(d.c))
    torch.cuda.synchronize()
    n1, n2, v1, v2 = host(n1), host(n2), host(v1), host(v2)
    assert int(n1.sum()) > 0 and np.array_equal(n1, n2)
    for b in range(2):
        for h in range(3):
            m = int(n1[b, h])
            assert np.array_equal(v1[b, h, :m], v2[b, h, :m]), (b, h)
