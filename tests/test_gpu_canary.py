"""Canary fills: memory an eviction pass must not write keeps its bits.

Before the pass, every spare block of the pool (in no head's table) and
every row at or past a head's length (the tail of its last block and the
allocated blocks after it) hold a NaN pattern with a payload, and those
slots' positions and the free list's unused entries hold sentinels.  After
kvev_evict (or the three separate calls) the whole K and V pools, pos, the
block table, seq_len, the free list (sentinel tail included) and the stats
must equal, bit for bit, the oracle's compaction of the GPU's own victims,
which writes only the kept rows' destinations ([VTOK] section 3.5, I2:
every live token keeps one slot, and nothing else is touched).  The only
slots left out are those the boundary leaves unspecified: [n', 16 *
ceil(n'/16)) of each head.  The canaries also show that rows past a head's
length never reach its scores (a NaN there would rank above every finite
score and change the victims).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_helpers import Run, dev, host
from tests.test_gpu_evict import _inputs, _ragged

pytestmark = pytest.mark.gpu

CANARY = {"bf16": np.uint16(0x7FA5), "f32": np.uint32(0x7FA5A5A5)}
POS_SENTINEL = -7
FREE_SENTINEL = -99


def _canary_case(name, over, seed):
    cfg = synth.CONFIGS[name].scaled(**over)
    case = synth.make_case(cfg, seq_len=_ragged(cfg.B, cfg.Hkv, cfg.L, seed), spare_blocks=9)
    c = CANARY[case["dtype"]]
    k = case["k_pool"].view(c.dtype)
    v = case["v_pool"].view(c.dtype)
    bt = case["block_table"]
    used = np.zeros(case["num_blocks"], bool)
    used[bt[bt >= 0]] = True
    k[~used] = c
    v[~used] = c
    ms = case["max_blocks"] * 16
    for b in range(case["B"]):
        for h in range(case["Hkv"]):
            n = int(case["seq_len"][b, h])
            s = np.arange(n, ms)
            rows = bt[b, h, s // 16]
            k[rows, s % 16] = c
            v[rows, s % 16] = c
            case["pos"][b, h, n:] = POS_SENTINEL
    return case, int((~used).sum())


CASES = [
    # name, overrides, kind, pool, budget, recent, path
    ("snapkv_prefill_32k", dict(B=2, Hkv=3, L=1500), "pool", 7, 400, 32, "fused"),
    ("snapkv_prefill_32k", dict(B=2, Hkv=3, L=1500), "pool", 7, 400, 32, "separate"),
    ("dropkv_128k", dict(Hkv=2, L=1700), "drop", 1, 300, 32, "fused"),       # 256-row window
    ("tiny_f32", dict(B=2, L=700), "sum", 1, 200, 16, "fused"),
    ("block_evict_64k", dict(B=2, Hkv=2, L=2000), "sum", 1, 1000, 16, "separate"),
]


@pytest.mark.parametrize("name,over,kind,pool,budget,recent,path", CASES,
                         ids=[f"{c[0]}-{c[2]}-{c[6]}" for c in CASES])
def test_pass_writes_only_kept_destinations(name, over, kind, pool, budget, recent, path):
    case, spare = _canary_case(name, over, 4)
    assert spare == 9
    lse32, a32 = _inputs(case, kind)
    r = Run(case, free_prefix=3)
    fl0 = host(r.fl).copy()
    fl0[3:] = FREE_SENTINEL
    r.fl = dev(fl0)
    if path == "fused":
        r.fused(kind, lse32, a32, pool, budget, recent)
    else:
        r.three_calls(kind, lse32, a32, pool, budget, recent)
    st = r.state()
    assert int(st["nv"].sum()) > 0
    new, ofl, ofc, ostats = oracle.compact(case, st["vic"], st["nv"], free_list=fl0, free_count=3)
    assert np.array_equal(st["seq"], new["seq_len"])
    assert np.array_equal(st["bt"], new["block_table"])
    assert st["fc"] == ofc and np.array_equal(st["fl"], ofl)  # the sentinel tail included
    assert np.array_equal(st["stats"], ostats)
    # rows and positions: everything except each head's unspecified slots
    c = CANARY[case["dtype"]]
    keep_rows = np.ones(case["k_pool"].shape[:2], bool)
    keep_pos = np.ones(case["pos"].shape, bool)
    for b in range(case["B"]):
        for h in range(case["Hkv"]):
            n2 = int(new["seq_len"][b, h])
            s = np.arange(n2, -(-n2 // 16) * 16)
            keep_rows[new["block_table"][b, h, s // 16], s % 16] = False
            keep_pos[b, h, s] = False
    for key in ("k", "v"):
        g = st[key].view(c.dtype)
        o = new[f"{key}_pool"].view(c.dtype)
        bad = np.argwhere(keep_rows & np.any(g != o, axis=-1))
        assert bad.size == 0, (key, bad[:5].tolist())
    assert np.array_equal(st["pos"][keep_pos], new["pos"][keep_pos])
    # the canaries are still where the oracle kept them (spare blocks whole)
    assert np.all(st["k"].view(c.dtype)[~np.isin(np.arange(case["num_blocks"]),
                                                 case["block_table"])] == c)
