"""GPU parity of the fused entry point kvev_evict (score + select + compact in
one call).

Against the three separate calls on the same inputs it must be bit-exact
everywhere: victims, n_victims, the compacted K/V rows, pos, seq_len, block
table, free list, stats and the compacted score row.  Against the oracle it
follows the end-to-end rule: victim sets may differ only where an oracle
score lies within the score tolerance of the oracle's cutoff, and the
compaction of the GPU's victims equals the oracle's compaction of them.
Workloads span several tiles, ragged heads (0, 1, 16, 17 and odd lengths),
heads that lose nothing, an inconsistent head and back-to-back calls on one
workspace.
"""
import numpy as np
import pytest

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import KIND, TOL, Run, check_eviction_vs_oracle_chain, dev
from tests.helpers import rounded_window_inputs

pytestmark = pytest.mark.gpu

def _ragged(B, H, L, seed=0):
    r = np.random.default_rng(seed)
    seq = np.full(B * H, L, np.int32)
    picks = [L - 1, L // 2 + 3, min(17, L), 1, 0, min(16, L)]
    for i in range(1, seq.size):
        seq[i] = picks[(i - 1) % len(picks)] if i % 2 else max(0, L - int(r.integers(0, min(40, L))))
    return seq.reshape(B, H)


def _inputs(case, kind):
    lse64, a64 = oracle.lse_a(case, want_a=(kind == "drop"))
    return rounded_window_inputs(case, lse64, a64)


def _assert_same(a, b, seq_before):
    """Bit-exact comparison of two eviction results (live data only)."""
    assert np.array_equal(a["nv"], b["nv"])
    assert np.array_equal(a["seq"], b["seq"])
    assert np.array_equal(a["bt"], b["bt"])
    assert a["fc"] == b["fc"]
    assert np.array_equal(a["fl"][:a["fc"]], b["fl"][:b["fc"]])
    assert np.array_equal(a["stats"], b["stats"])
    B, H = seq_before.shape
    for bb in range(B):
        for h in range(H):
            m = int(a["nv"][bb, h])
            if m > 0:
                assert np.array_equal(a["vic"][bb, h, :m], b["vic"][bb, h, :m]), (bb, h)
            n2 = int(a["seq"][bb, h])
            if not 0 <= n2 <= a["pos"].shape[-1]:
                continue
            assert np.array_equal(a["pos"][bb, h, :n2], b["pos"][bb, h, :n2]), (bb, h)
            sa, sb = a["score"][bb, h, :n2], b["score"][bb, h, :n2]
            assert np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), (bb, h)
            for s in range(0, n2, 16):
                blk = a["bt"][bb, h, s // 16]
                e = min(16, n2 - s)
                assert np.array_equal(a["k"][blk, :e], b["k"][blk, :e]), (bb, h, s)
                assert np.array_equal(a["v"][blk, :e], b["v"][blk, :e]), (bb, h, s)


FUSED_CASES = [
    # name, overrides, kind, pool, budget, recent, ragged
    ("tiny_f32", {}, "pool", 5, 128, 32, False),
    ("tiny_f32", {}, "sum", 1, 100, 8, False),
    ("tiny_f32", {}, "drop", 1, 64, 16, False),
    ("tiny_f32", dict(D=128, L=700, W=12, B=2), "pool", 3, 200, 16, True),
    ("snapkv_prefill_32k", dict(B=2, Hkv=3, L=3001), "pool", 7, 500, 32, True),
    ("snapkv_prefill_32k", dict(B=1, Hkv=2, L=2000, D=64), "pool", 33, 300, 8, False),
    ("dropkv_128k", dict(Hkv=2, L=4099), "drop", 1, 600, 32, True),
    ("block_evict_64k", dict(B=2, Hkv=2, L=2500), "sum", 1, 1200, 16, True),
    ("h2o_decode_4k", dict(B=2, Hkv=2, L=1000, decode_steps=0), "sum", 1, 200, 100, True),
]


@pytest.mark.parametrize("name,over,kind,pool,budget,recent,ragged", FUSED_CASES,
                         ids=[f"{c[0]}-{c[2]}-{i}" for i, c in enumerate(FUSED_CASES)])
def test_evict_equals_three_calls(name, over, kind, pool, budget, recent, ragged):
    cfg = synth.CONFIGS[name].scaled(**over)
    seq = _ragged(cfg.B, cfg.Hkv, cfg.L, 5) if ragged else None
    case = synth.make_case(cfg, seq_len=seq, spare_blocks=5)
    lse32, a32 = _inputs(case, kind)
    f = Run(case)
    f.fused(kind, lse32, a32, pool, budget, recent)
    t = Run(case)
    t.three_calls(kind, lse32, a32, pool, budget, recent)
    _assert_same(f.state(), t.state(), case["seq_len"])


def test_evict_accumulate_equals_three_calls():
    """H2O's running sums: ACCUMULATE adds this step's window sum to the row."""
    cfg = synth.CONFIGS["h2o_decode_4k"].scaled(B=2, Hkv=2, L=900, decode_steps=0)
    case = synth.make_case(cfg, seq_len=_ragged(2, 2, 900, 3))
    lse32, _ = _inputs(case, "sum")
    prev = np.random.default_rng(4).uniform(0, 2, (2, 2, case["max_blocks"] * 16)).astype(np.float32)
    f = Run(case, prev=prev)
    f.fused("sum", lse32, None, 1, 300, 30, accumulate=True)
    t = Run(case, prev=prev)
    t.three_calls("sum", lse32, None, 1, 300, 30, accumulate=True)
    _assert_same(f.state(), t.state(), case["seq_len"])


def test_evict_back_to_back_on_one_workspace():
    """Two eviction steps in a row (the second on the compacted cache with a
    smaller budget): the workspace state left by the first is clean."""
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=2, Hkv=2, L=2600)
    case = synth.make_case(cfg, seq_len=_ragged(2, 2, 2600, 9))
    lse32, _ = _inputs(case, "pool")
    f, t = Run(case), Run(case)
    for budget in (1000, 400):
        f.fused("pool", lse32, None, 7, budget, 32)
        t.three_calls("pool", lse32, None, 7, budget, 32)
        _assert_same(f.state(), t.state(), case["seq_len"])


def test_evict_inconsistent_head_is_flagged_and_left_alone():
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=1, Hkv=3, L=700)
    case = synth.make_case(cfg)
    lse32, _ = _inputs(case, "pool")
    case = dict(case)
    case["seq_len"] = np.array([[700, 10**6, 650]], np.int32)
    f = Run(case, free_prefix=0)
    f.fused("pool", lse32, None, 7, 300, 8)
    st = f.state()
    assert st["nv"].tolist() == [[400, -1, 350]]
    assert st["stats"][4] & 2
    assert st["seq"].tolist() == [[300, 10**6, 300]]
    t = Run(case, free_prefix=0)
    t.three_calls("pool", lse32, None, 7, 300, 8)
    _assert_same(st, t.state(), case["seq_len"])


ORACLE_CASES = [
    ("snapkv_prefill_32k", dict(B=2, Hkv=4, L=4000), "pool", 7, 500, 32),
    ("dropkv_128k", dict(Hkv=2, L=6000), "drop", 1, 300, 32),
    ("block_evict_64k", dict(B=2, Hkv=2, L=3000), "sum", 1, 1500, 16),
    ("tiny_f32", {}, "pool", 5, 128, 32),
]


@pytest.mark.parametrize("name,over,kind,pool,budget,recent", ORACLE_CASES,
                         ids=[c[0] for c in ORACLE_CASES])
def test_evict_matches_oracle(name, over, kind, pool, budget, recent):
    cfg = synth.CONFIGS[name].scaled(**over)
    case = synth.make_case(cfg)
    lse32, a32 = _inputs(case, kind)
    kg, ko, key = KIND[kind]
    orc = oracle.score(case, lse32, ko, pool, a32=a32)[key]
    o32 = orc.astype(np.float32)
    ov, on = oracle.select(np.nan_to_num(o32, nan=0.0), case["seq_len"], budget, recent)
    f = Run(case, free_prefix=0)
    f.fused(kind, lse32, a32, pool, budget, recent)
    st = f.state()
    # the oracle's own chain: its victims, then its compaction of them carrying its scores
    new, ofl, ofc, ostats = oracle.compact(case, ov, on, score_row=np.nan_to_num(o32, nan=0.0),
                                           free_list=np.full(case["num_blocks"] + 8, -1, np.int32),
                                           free_count=0)
    nd = check_eviction_vs_oracle_chain(case, st, ov, on, new, ofl, ofc, ostats, o32,
                                        TOL[cfg.dtype])
    print(f"{name}: {nd} heads with victims differing inside the tolerance band", flush=True)


def test_evict_on_two_streams_equals_sequential():
    """Independent caches (the layers of one model) evicted concurrently on
    two streams, each with its own workspace and outputs, end bit-exact equal
    to the same evictions run one after the other on one stream."""
    import torch

    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=2, Hkv=4, L=3001)
    cases = [synth.make_case(cfg.scaled(seed=cfg.seed + i), seq_len=_ragged(2, 4, 3001, 11 + i))
             for i in range(4)]
    inputs = [_inputs(c, "pool")[0] for c in cases]
    seq_runs = [Run(c) for c in cases]
    for r, lse32 in zip(seq_runs, inputs):
        r.fused("pool", lse32, None, 7, 700, 32)
    par_runs = [Run(c) for c in cases]
    lses = [dev(x) for x in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    for i, (r, lse) in enumerate(zip(par_runs, lses)):
        with torch.cuda.stream(streams[i % 2]):
            r.stats = K.evict(r.dc, r.q, lse, r.qp, r.case["scale"], r.case["G"], K.POOL, 700, 32,
                              r.score, r.vic, r.nv, r.fl, r.fc, r.ws, pool_kernel=7)
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    for a, b, c in zip(seq_runs, par_runs, cases):
        _assert_same(a.state(), b.state(), c["seq_len"])


@pytest.mark.parametrize("kind,pool", [("sum", 1), ("pool", 5)])
def test_evict_at_the_slot_limit_matches_oracle(kind, pool):
    """One head at the library's largest size: 1,048,576 slots (65536 blocks,
    1024 selection chunks), 8 short of full.  The fused pass (score, the
    selection shared by 512 workgroups, compaction) against the oracle's
    chain, as above."""
    cfg = synth.CONFIGS["tiny_f32"].scaled(B=1, Hkv=1, G=1, W=1, L=(1 << 20) - 8)
    case = synth.make_case(cfg)
    assert case["max_blocks"] * 16 == 1 << 20
    lse32, a32 = _inputs(case, kind)
    kg, ko, key = KIND[kind]
    orc = oracle.score(case, lse32, ko, pool, a32=a32)[key]
    o32 = orc.astype(np.float32)
    budget, recent = 300_000, 64
    ov, on = oracle.select(np.nan_to_num(o32, nan=0.0), case["seq_len"], budget, recent)
    f = Run(case, free_prefix=0)
    f.fused(kind, lse32, a32, pool, budget, recent)
    st = f.state()
    new, ofl, ofc, ostats = oracle.compact(case, ov, on, score_row=np.nan_to_num(o32, nan=0.0),
                                           free_list=np.full(case["num_blocks"] + 8, -1, np.int32),
                                           free_count=0)
    nd = check_eviction_vs_oracle_chain(case, st, ov, on, new, ofl, ofc, ostats, o32,
                                        TOL[cfg.dtype])
    assert int(st["stats"][0]) == (case["seq_len"][0, 0] + 15) // 16 - (budget + 15) // 16
    print(f"slot limit, {kind}: {nd} heads with victims differing inside the tolerance band",
          flush=True)
