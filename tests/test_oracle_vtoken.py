"""Pins of the oracle's vToken liveness and lazy reclamation to what the
review of the vToken paper fixes.  CPU only.

  * Section 3.2: evicting a token only clears its liveness bit (and the live
    count of its block); nothing moves.
  * Section 3.3, stage 3, and section 3.5, I4: a plan proceeds only when
    packing the sources' T live tokens into ceil(T/16) destinations frees
    strictly more blocks than it takes; destinations are filled completely
    one after the other, in logical order.
  * Section 3.3, stages 1 and 2: the waste threshold theta_F gates a head;
    destinations come from the free pool and a head that does not fit is
    deferred.
  * Section 3.5, I1 and I2: the live tokens (position, K, V) are conserved;
    every block is in exactly one of a table or the free list.  The moved
    tokens keep their relative order ("where possible": with a full block
    between two sources, a moved token passes over it).
  * Eq. 1: F before and after from the stats, by closed form.
  * Cross-check with the (separately pinned) eager compaction: with every
    non-full block a source, the live tokens come out in the same order.
"""
import collections

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import manual_case

rng = np.random.default_rng


def _state(fills, D=8, dtype="f32", seed=3, spare=8):
    """One head per entry of `fills`: a list of live counts per logical block
    (the last block is the growing tail); live slots are the first ones of each
    block; positions are the slot indices."""
    B, Hkv = 1, len(fills)
    nb = max(len(f) for f in fills)
    r = rng(seed)
    n_max = nb * 16
    k = r.normal(0, 1, (B, Hkv, n_max, D))
    v = r.normal(0, 1, (B, Hkv, n_max, D))
    seq = np.array([[len(f) * 16 for f in fills]], np.int32)
    st = manual_case(k, v, np.zeros((B, Hkv, 1, D)), np.zeros((B, 1)), seq_len=seq, dtype=dtype,
                     spare_blocks=spare)
    live = np.zeros((B, Hkv, nb * 16), np.uint8)
    for h, f in enumerate(fills):
        for lb, c in enumerate(f):
            live[0, h, lb * 16:lb * 16 + c] = 1
        st["block_table"][0, h, len(f):] = -1
    st["live"] = live
    st["block_live"] = live.reshape(B, Hkv, nb, 16).sum(-1).astype(np.int32)
    st["score"] = r.uniform(0, 1, (B, Hkv, nb * 16)).astype(np.float32)
    used = set(st["block_table"][st["block_table"] >= 0].tolist())
    free = np.array([b for b in range(st["num_blocks"]) if b not in used], np.int32)
    fl = np.full(st["num_blocks"] + 16, -1, np.int32)
    fl[:free.size] = free
    return st, fl, int(free.size)


def _live_tokens(st, h):
    """(pos, K row, V row) of the live tokens of head h, in logical order."""
    out = []
    bt = st["block_table"][0, h]
    for s in range(int(st["seq_len"][0, h])):
        if bt[s // 16] < 0 or not st["live"][0, h, s]:
            continue
        blk = bt[s // 16]
        out.append((int(st["pos"][0, h, s]), st["k_pool"][blk, s % 16].tobytes(),
                    st["v_pool"][blk, s % 16].tobytes()))
    return out


def test_evict_only_clears_bits():
    st, fl, fc = _state([[16, 16, 16]])
    vic = np.full((1, 1, 48), -1, np.int32)
    vic[0, 0, :4] = [3, 17, 18, 40]
    new, status = oracle.vtok_evict(st, vic, np.array([[4]], np.int32))
    assert status == 0
    assert new["block_live"][0, 0].tolist() == [15, 14, 15]
    assert new["live"][0, 0, [3, 17, 18, 40]].tolist() == [0, 0, 0, 0]
    assert np.array_equal(new["k_pool"], st["k_pool"]) and np.array_equal(new["pos"], st["pos"])
    # a slot already dead, out of range, or past the head's length is flagged
    vic[0, 0, :3] = [3, 48, 100]
    new2, status2 = oracle.vtok_evict(new, vic, np.array([[3]], np.int32))
    assert status2 == 1 and np.array_equal(new2["live"], new["live"])


def test_plan_needs_a_strict_decrease():
    # head 0: three sources with 5 live each -> 15 tokens, one destination: frees 2
    # head 1: two sources with 9 live each -> 18 tokens need 2 destinations: refused
    st, fl, fc = _state([[5, 5, 5, 16, 3], [9, 9, 7]])
    new, fl2, fc2, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc, with_score=True)
    assert stats[0] == 1 and stats[3] == 2 and stats[4] == 15
    bt0, bt1 = new["block_table"][0, 0], new["block_table"][0, 1]
    assert bt0[1] == -1 and bt0[2] == -1 and bt0[0] >= 0 and bt0[0] != st["block_table"][0, 0, 0]
    assert bt0[3] == st["block_table"][0, 0, 3] and bt0[4] == st["block_table"][0, 0, 4]
    assert np.array_equal(bt1[:3], st["block_table"][0, 1, :3])
    # the destination is filled completely with the tokens in logical order
    assert new["block_live"][0, 0].tolist()[:3] == [15, 0, 0]
    assert new["live"][0, 0, :16].tolist() == [1] * 15 + [0]
    assert new["pos"][0, 0, :15].tolist() == [0, 1, 2, 3, 4, 16, 17, 18, 19, 20, 32, 33, 34, 35, 36]
    want_sc = st["score"][0, 0, [0, 1, 2, 3, 4, 16, 17, 18, 19, 20, 32, 33, 34, 35, 36]]
    assert np.array_equal(new["score"][0, 0, :15], want_sc)
    # the three sources went to the free list, the destination came from it
    assert fc2 == fc - 1 + 3
    assert sorted(fl2[fc - 1:fc2].tolist()) == sorted(st["block_table"][0, 0, :3].tolist())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_conservation_unique_mapping_and_waste(seed):
    r = rng(seed)
    fills = [list(r.integers(0, 17, size=int(r.integers(3, 9)))) for _ in range(5)]
    st, fl, fc = _state(fills, seed=seed, spare=20)
    before = [_live_tokens(st, h) for h in range(5)]
    new, fl2, fc2, stats = oracle.vtok_reclaim(st, 0.1, 4, fl, fc)
    for h in range(5):
        after = _live_tokens(new, h)
        assert sorted(after) == sorted(before[h])         # I1: the same live tokens
        # the order among the moved tokens is kept ("where possible": a moved
        # token may pass over a full block that is not a source); every block
        # that is not a source keeps its tokens in place
        changed = [lb for lb in range(st["max_blocks"])
                   if st["block_table"][0, h, lb] != new["block_table"][0, h, lb]]
        moved = [t for t in before[h] if t[0] // 16 in changed]
        assert [t for t in after if t in moved] == moved
        for lb in range(st["max_blocks"]):
            if lb not in changed and new["block_table"][0, h, lb] >= 0:
                sl = slice(lb * 16, lb * 16 + 16)
                assert np.array_equal(new["live"][0, h, sl], st["live"][0, h, sl])
                assert np.array_equal(new["pos"][0, h, sl], st["pos"][0, h, sl])
    # I2: every block id exactly once across the tables and the free list
    ids = new["block_table"][new["block_table"] >= 0].tolist() + fl2[:fc2].tolist()
    assert sorted(ids) == list(range(new["num_blocks"]))
    # block_live agrees with the bits; Eq. 1 before and after from the stats
    assert np.array_equal(new["block_live"], new["live"].reshape(new["block_live"].shape + (16,)).sum(-1))
    live_tok = sum(len(b) for b in before)
    alloc0 = int((st["block_table"] >= 0).sum())
    alloc1 = int((new["block_table"] >= 0).sum())
    assert stats[6] == live_tok and stats[7] == alloc0 and stats[8] == alloc1
    assert stats[3] == alloc0 - alloc1 >= 0
    F0, F1 = 1 - live_tok / (16 * alloc0), 1 - live_tok / (16 * alloc1)
    assert F1 <= F0
    assert stats[5] == stats[4] * 2 * new["D"] * 4 * 2


def test_threshold_gates_a_head():
    # 2 blocks at 10 live + a full one + the tail: F = 1 - 48/64 = 0.25
    st, fl, fc = _state([[10, 10, 16, 12]])
    _, _, _, s_hi = oracle.vtok_reclaim(st, 0.25, 8, fl, fc)
    assert s_hi[0] == 0 and s_hi[2] == 1          # F is not above 0.25: left as it is
    _, _, _, s_lo = oracle.vtok_reclaim(st, 0.2, 8, fl, fc)
    assert s_lo[0] == 0 and s_lo[2] == 1          # above, but 20 tokens need 2 blocks: no gain
    st2, fl2, fc2 = _state([[6, 6, 16, 12]])
    _, _, _, s2 = oracle.vtok_reclaim(st2, 0.25, 8, fl2, fc2)
    assert s2[0] == 1 and s2[3] == 1              # 12 tokens into one block: frees one


def test_headroom_defers_heads_that_do_not_fit():
    # no free block at all: every plan is deferred and nothing changes
    st, fl, fc = _state([[3, 3, 3, 1], [4, 4, 4, 1], [2, 2, 2, 1]], spare=0)
    assert fc == 0
    new, _, fc0, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert stats[1] == 3 and stats[0] == 0 and fc0 == 0
    assert np.array_equal(new["block_table"], st["block_table"])
    # one free block: heads take destinations in (b, h) order from the top;
    # sources return to the list only after every head has planned, so the
    # first head fits and the two after it are deferred
    st1, fl1, fc1 = _state([[3, 3, 3, 1], [4, 4, 4, 1], [2, 2, 2, 1]], spare=1)
    assert fc1 == 1
    new1, fl_after, fc_after, s1 = oracle.vtok_reclaim(st1, 0.0, 8, fl1, fc1)
    assert s1[0] == 1 and s1[1] == 2 and fc_after == 3
    assert new1["block_table"][0, 0, 0] == fl1[0]


def test_max_sources_caps_the_plan():
    st, fl, fc = _state([[2, 2, 2, 2, 2, 2, 2, 2, 5]])
    _, _, _, s2 = oracle.vtok_reclaim(st, 0.0, 2, fl, fc)
    assert s2[4] == 4 and s2[3] == 1               # two sources, 4 tokens, one block freed
    _, _, _, s8 = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert s8[4] == 16 and s8[3] == 7              # eight sources, 16 tokens: one destination


def test_same_order_as_eager_compaction():
    """Every non-full block a source (and a full tail): the live tokens read in
    logical order equal what the eager, order-preserving compaction keeps."""
    r = rng(9)
    fills = [[int(x) for x in r.integers(0, 16, size=6)] + [16]]
    st, fl, fc = _state(fills, spare=10)
    new, _, _, _ = oracle.vtok_reclaim(st, 0.0, 64, fl, fc)
    lazy = _live_tokens(new, 0)
    # the same liveness as victims of the eager compaction
    n = int(st["seq_len"][0, 0])
    vic = np.flatnonzero(st["live"][0, 0, :n] == 0).astype(np.int32)
    v = np.full((1, 1, st["max_blocks"] * 16), -1, np.int32)
    v[0, 0, :vic.size] = vic
    eager, _, _, _ = oracle.compact(st, v, np.array([[vic.size]], np.int32),
                                    free_list=np.full(st["num_blocks"] + 16, -1, np.int32))
    m = int(eager["seq_len"][0, 0])
    ref = []
    for s in range(m):
        blk = eager["block_table"][0, 0, s // 16]
        ref.append((int(eager["pos"][0, 0, s]), eager["k_pool"][blk, s % 16].tobytes(),
                    eager["v_pool"][blk, s % 16].tobytes()))
    assert lazy == ref


def test_inconsistent_heads_are_skipped():
    """A head whose table holds a block id past the pool or a live count
    outside [0, 16] is skipped with a status bit and left as it is; a victim
    count above the list's capacity is flagged and clamped."""
    st, fl, fc = _state([[3, 3, 3, 1], [4, 4, 4, 1], [2, 2, 2, 1]], spare=10)
    st["block_live"][0, 1, 1] = 17
    new, _, _, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert stats[9] == 4 and stats[0] == 2
    assert np.array_equal(new["block_table"][0, 1], st["block_table"][0, 1])
    st["block_live"][0, 1, 1] = 4
    st["block_table"][0, 2, 0] = st["num_blocks"] + 1
    new, _, _, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert stats[9] == 4 and stats[0] == 2 and stats[7] == 8   # the skipped head is not counted
    st["seq_len"][0, 0] = st["max_blocks"] * 16 + 1
    _, _, _, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert stats[9] == 6 and stats[0] == 1
    st2, _, _ = _state([[16, 16]])
    vic = np.zeros((1, 1, 32), np.int32)
    vic[0, 0] = np.arange(32)
    new, status = oracle.vtok_evict(st2, vic, np.array([[40]], np.int32))
    assert status == 1 and new["live"][0, 0].sum() == 0 and new["block_live"][0, 0].tolist() == [0, 0]


# ------------------------------------------------ online checks of I1, I2

M64 = (1 << 64) - 1


def _unfmix64(h):
    """The inverse of MurmurHash3's finalizer, from its published steps: undo
    each xor-shift by 33 (two rounds suffice for 64 bits) and each multiply by
    the odd constant's inverse mod 2^64."""
    def unshift(x):
        return x ^ (x >> 33) ^ (x >> 66)
    h = unshift(h)
    h = (h * pow(0xc4ceb9fe1a85ec53, -1, 1 << 64)) & M64
    h = unshift(h)
    h = (h * pow(0xff51afd7ed558ccd, -1, 1 << 64)) & M64
    return unshift(h)


def test_fmix64_is_murmur3_finalizer():
    assert oracle.fmix64(0) == 0
    r = rng(4)
    for x in [1, 2, 3, M64, 1 << 63] + [int(v) for v in r.integers(0, 1 << 63, 50)]:
        y = oracle.fmix64(x)
        assert _unfmix64(y) == x, hex(x)
        assert y != x


def test_digest_follows_the_tokens_not_their_slots():
    st, fl, fc = _state([[5, 7, 16, 9, 3], [2, 2, 2, 2, 11]], spare=10)
    st["score"] = np.zeros_like(st["score"])
    d0 = oracle.vtok_digest(st)
    assert (d0 != 0).all()
    new, fl2, fc2, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert stats[0] == 2
    assert np.array_equal(oracle.vtok_digest(new), d0)          # I1 across a relocation
    # one token moved by hand to a free block: the same digest
    m = dict(new)
    m["k_pool"], m["v_pool"] = new["k_pool"].copy(), new["v_pool"].copy()
    m["block_table"], m["live"] = new["block_table"].copy(), new["live"].copy()
    m["pos"] = new["pos"].copy()
    lb = 2                                   # the full block: not a source, still in place
    old = m["block_table"][0, 0, lb]
    assert old == st["block_table"][0, 0, lb] and m["live"][0, 0, 32:48].all()
    dst = int(fl2[fc2 - 1])
    m["k_pool"][dst] = m["k_pool"][old]
    m["v_pool"][dst] = m["v_pool"][old]
    m["block_table"][0, 0, lb] = dst
    assert np.array_equal(oracle.vtok_digest(m), d0)


def test_digest_sees_every_live_byte_and_ignores_dead_ones():
    st, fl, fc = _state([[5, 7, 16, 9, 3], [2, 2, 2, 2, 11]], spare=4)
    d0 = oracle.vtok_digest(st)
    blk = st["block_table"][0, 0, 1]
    for pool, o, j in (("k_pool", 0, 0), ("v_pool", 6, 7), ("k_pool", 3, 5)):
        m = dict(st)
        m[pool] = st[pool].copy()
        m[pool].view(np.uint8).reshape(st["num_blocks"], 16, -1)[blk, o, j] ^= 1
        d = oracle.vtok_digest(m)
        assert d[0, 0] != d0[0, 0] and d[0, 1] == d0[0, 1], (pool, o, j)
    m = dict(st)
    m["pos"] = st["pos"].copy()
    m["pos"][0, 0, 17] += 1
    assert oracle.vtok_digest(m)[0, 0] != d0[0, 0]
    # a dead slot (block 1 keeps 7 of 16) changes nothing
    m = dict(st)
    m["k_pool"] = st["k_pool"].copy()
    m["k_pool"].view(np.uint8).reshape(st["num_blocks"], 16, -1)[blk, 12, :] ^= 0xff
    assert np.array_equal(oracle.vtok_digest(m), d0)
    # swapping the V rows of two live tokens (each keeps its own K and pos) changes it
    m = dict(st)
    m["v_pool"] = st["v_pool"].copy()
    b0 = st["block_table"][0, 0, 0]
    m["v_pool"][b0, [0, 1]] = st["v_pool"][b0, [1, 0]]
    assert oracle.vtok_digest(m)[0, 0] != d0[0, 0]
    # no live token: 0
    m = dict(st)
    m["live"] = np.zeros_like(st["live"])
    assert (oracle.vtok_digest(m) == 0).all()


def test_check_counts_every_kind_of_fault():
    st, fl, fc = _state([[5, 7, 16, 9, 3], [2, 2, 2, 2, 11]], spare=6)
    assert oracle.vtok_check(st, fl, fc).tolist() == [0, 0, 0, 0]
    new, fl2, fc2, _ = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert oracle.vtok_check(new, fl2, fc2).tolist() == [0, 0, 0, 0]   # I2 after a relocation
    m = dict(st)
    m["block_table"] = st["block_table"].copy()
    m["block_table"][0, 1, 0] = st["block_table"][0, 0, 0]           # two owners, one orphan
    assert oracle.vtok_check(m, fl, fc).tolist() == [1, 1, 0, 0]
    m["block_table"][0, 1, 0] = st["num_blocks"]                      # out of range
    assert oracle.vtok_check(m, fl, fc).tolist() == [0, 1, 1, 0]
    m = dict(st)
    m["block_live"] = st["block_live"].copy()
    m["block_live"][0, 0, 2] -= 1
    assert oracle.vtok_check(m, fl, fc).tolist() == [0, 0, 0, 1]
    fl_bad = fl.copy()
    fl_bad[0] = -7
    assert oracle.vtok_check(st, fl_bad, fc).tolist() == [0, 1, 1, 0]
    assert oracle.vtok_check(st, fl, fc - 1).tolist() == [0, 1, 0, 0]


# --------------------------------------- sync_new_tokens and slot mapping


def test_slot_mapping_is_eq2_on_a_dense_head_and_skips_dead_slots():
    st, fl, fc = _state([[16, 16, 9]])
    st["seq_len"][0, 0] = 41
    st["live"][0, 0, 32:41] = 1
    st["block_live"][0, 0, 2] = 9
    slots, positions, count = oracle.vtok_slot_mapping(st)
    bt = st["block_table"][0, 0]
    want = [int(bt[s // 16]) * 16 + s % 16 for s in range(41)]   # Eq. 2
    assert count[0, 0] == 41 and slots[0, 0, :41].tolist() == want
    assert positions[0, 0, :41].tolist() == st["pos"][0, 0, :41].tolist()
    vic = np.full((1, 1, 48), -1, np.int32)
    vic[0, 0, :3] = [0, 17, 40]
    new, _ = oracle.vtok_evict(st, vic, np.array([[3]], np.int32))
    s2, p2, c2 = oracle.vtok_slot_mapping(new)
    keep = [s for s in range(41) if s not in (0, 17, 40)]
    assert c2[0, 0] == 38 and s2[0, 0, :38].tolist() == [want[s] for s in keep]


def test_slot_mapping_reads_the_live_tokens_after_reclamation():
    r = rng(12)
    fills = [list(r.integers(0, 17, size=7)) for _ in range(3)]
    st, fl, fc = _state(fills, spare=30)
    new, _, _, stats = oracle.vtok_reclaim(st, 0.0, 8, fl, fc)
    assert stats[0] > 0
    slots, positions, count = oracle.vtok_slot_mapping(new)
    for h in range(3):
        got = [(int(positions[0, h, k]),
                new["k_pool"].reshape(-1, new["D"])[slots[0, h, k]].tobytes(),
                new["v_pool"].reshape(-1, new["D"])[slots[0, h, k]].tobytes())
               for k in range(count[0, h])]
        assert got == _live_tokens(new, h)                  # logical order, through Eq. 2
        assert sorted(got) == sorted(_live_tokens(st, h))   # and the same tokens as before


def test_sync_registers_new_tokens():
    st, fl, fc = _state([[16, 5], [16, 16, 16]])
    st["seq_len"][0] = [21, 48]
    new, status = oracle.vtok_sync(st, np.array([[30, 48]], np.int32), np.array([100], np.int32))
    assert status.tolist() == [[0, 0]]
    assert new["seq_len"][0].tolist() == [30, 48]
    assert new["live"][0, 0, 21:30].all() and new["block_live"][0, 0, 1] == 5 + 9
    assert new["pos"][0, 0, 21:30].tolist() == list(range(100, 109))
    assert np.array_equal(new["pos"][0, 1], st["pos"][0, 1])        # nothing new
    # then marked dead, the counts return: sync and evict are inverse on counts
    vic = np.full((1, 2, 48), -1, np.int32)
    vic[0, 0, :9] = np.arange(21, 30)
    back, s2 = oracle.vtok_evict(new, vic, np.array([[9, 0]], np.int32))
    assert s2 == 0 and np.array_equal(back["block_live"], st["block_live"])
    # a shrinking length, one past the capacity, a block without an id
    bad, status = oracle.vtok_sync(st, np.array([[20, 49]], np.int32), np.array([0], np.int32))
    assert status.tolist() == [[-2, -2]] and np.array_equal(bad["live"], st["live"])
    st["block_table"][0, 0, 1] = -1
    bad, status = oracle.vtok_sync(st, np.array([[25, 48]], np.int32), np.array([0], np.int32))
    assert status.tolist() == [[-4, 0]]
