"""GPU parity of the policy variants against the oracle.

Shared scores across the KV heads of a sequence (kvev_select_shared against
oracle.select_shared): given identical fp32 per-head scores, both sides sum
the heads in fp32 in ascending order and select on the sum, so victims and
counts are compared bit for bit, on ragged sequences, many ties, refused
sequences (heads holding different tokens), and a full 64000-token layer of
the block-aware shape.  The chain SUM score -> shared selection -> compaction
is compared with the oracle's compaction of the same victims.
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
    print(f"[policy] {msg}", flush=True)


def _shared_case(seed, B, Hkv, ms, integer):
    r = rng(seed)
    if integer:
        scores = r.integers(0, 5, (B, Hkv, ms)).astype(np.float32)
    else:
        scores = r.uniform(0, 1, (B, Hkv, ms)).astype(np.float32)
    seq = np.repeat(r.integers(0, ms + 1, (B, 1)), Hkv, axis=1).astype(np.int32)
    seq[0, :] = ms
    pos = np.broadcast_to(np.arange(ms, dtype=np.int32), (B, Hkv, ms)).copy()
    return scores, seq, pos


class _Cache:
    """A device cache whose pools are never read by the selection."""

    def __init__(self, B, Hkv, ms, seq, pos):
        self.B, self.Hkv, self.ms = B, Hkv, ms
        mb = ms // 16
        k = torch.zeros((1, 16, 64), dtype=torch.bfloat16, device="cuda")
        bt = torch.zeros((B, Hkv, mb), dtype=torch.int32, device="cuda")
        self.c = K.Cache(k, k.clone(), bt, dev(seq), dev(pos))


@pytest.mark.parametrize("seed,B,Hkv,ms,budget,recent,integer", [
    (0, 3, 4, 1024, 300, 32, False),
    (1, 4, 8, 2048, 500, 16, True),      # many ties: the lower slot goes first
    (2, 2, 2, 16384, 4000, 64, False),   # several selection chunks
    (3, 5, 1, 512, 100, 10, False),      # one head: the ordinary selection
])
def test_shared_selection_bit_exact(seed, B, Hkv, ms, budget, recent, integer):
    scores, seq, pos = _shared_case(seed, B, Hkv, ms, integer)
    if B > 2:
        seq[2, -1] = max(0, seq[2, 0] - 1)        # unequal lengths: refused
        if Hkv > 1:
            pos[1, 1, 3] = 10 ** 6                # another token in one slot: refused
            seq[1, :] = np.maximum(seq[1, :], 8)
    c = _Cache(B, Hkv, ms, seq, pos)
    ws = K.new_select_shared_workspace(c.c)
    v, n = K.select_shared(c.c, dev(scores), budget, recent, ws)
    ov, on = oracle.select_shared(scores, seq, pos, budget, recent)
    gv, gn = host(v), host(n)
    assert np.array_equal(gn, on), (gn, on)
    for b in range(B):
        for h in range(Hkv):
            m = int(on[b, h])
            if m > 0:
                assert np.array_equal(gv[b, h, :m], ov[b, h, :m]), (b, h)
    _say(f"seed {seed}: counts {on[:, 0].tolist()}")
    # a second call on the same workspace gives the same result
    v2, n2 = K.select_shared(c.c, dev(scores), budget, recent, ws)
    assert np.array_equal(host(n2), gn)
    gv2 = host(v2)
    for b in range(B):
        for h in range(Hkv):
            m = max(0, int(on[b, h]))
            assert np.array_equal(gv2[b, h, :m], gv[b, h, :m]), (b, h)


def test_shared_chain_score_select_compact():
    """SUM scores on the GPU, one victim set per sequence, then every head
    compacted with it: the compaction equals the oracle's on the same victims,
    and every head of a sequence keeps the same positions."""
    cfg = synth.CONFIGS["block_evict_64k"].scaled(B=2, Hkv=4, L=3000)
    case = synth.make_case(cfg, spare_blocks=8)
    dc = device_cache(case)
    q = dev(case["q"])
    qp = dev(case["q_pos"])
    ws_wa = K.new_workspace(dc, case["G"], case["W"])
    lse, _ = K.window_attn(dc, q, qp, case["scale"], case["G"], ws_wa)
    score = dc.score_buffer()
    K.score(dc, q, lse, qp, case["scale"], case["G"], K.SUM, 1, sum=score)
    ws = K.new_select_shared_workspace(dc)
    budget, recent = 1500, 16
    v, n = K.select_shared(dc, score, budget, recent, ws)
    gscore = host(score)
    ov, on = oracle.select_shared(gscore, case["seq_len"], case["pos"], budget, recent)
    assert np.array_equal(host(n), on) and (on == 1500).all()
    assert np.array_equal(host(v)[:, :, :1500], ov[:, :, :1500])
    fl = dev(np.full(case["num_blocks"] + 8, -1, np.int32))
    fc = dev(np.zeros(1, np.int32))
    wsc = K.new_workspace(dc)
    stats = K.compact(dc, v, n, fl, fc, wsc)
    torch.cuda.synchronize()
    new, ofl, ofc, ost = oracle.compact(case, ov, on, free_list=np.full(case["num_blocks"] + 8, -1,
                                                                       np.int32))
    assert np.array_equal(host(dc.seq_len), new["seq_len"])
    assert np.array_equal(host(dc.block_table), new["block_table"])
    assert np.array_equal(host(dc.pos), new["pos"])
    assert np.array_equal(host(dc.k_pool), new["k_pool"])
    assert np.array_equal(host(dc.v_pool), new["v_pool"])
    assert host(stats).tolist()[:4] == ost.tolist()[:4]
    p = host(dc.pos)
    for h in range(1, cfg.Hkv):
        assert np.array_equal(p[:, h, :1500], p[:, 0, :1500])


def test_shared_selection_full_layer():
    """One 64000-token layer of the block-aware shape (B16, 8 KV heads):
    every sequence's victims bit-exact against the oracle."""
    B, Hkv, ms = 16, 8, 64000
    r = rng(11)
    scores = r.uniform(0, 1, (B, Hkv, ms)).astype(np.float32)
    seq = np.full((B, Hkv), ms, np.int32)
    pos = np.broadcast_to(np.arange(ms, dtype=np.int32), (B, Hkv, ms)).copy()
    c = _Cache(B, Hkv, ms, seq, pos)
    ws = K.new_select_shared_workspace(c.c)
    v, n = K.select_shared(c.c, dev(scores), 32000, 16, ws)
    ov, on = oracle.select_shared(scores, seq, pos, 32000, 16)
    assert np.array_equal(host(n), on) and (on == 32000).all()
    assert np.array_equal(host(v)[:, :, :32000], ov[:, :, :32000])


def test_per_head_budgets_bit_exact():
    """kvev_select_budgets against oracle.select_budgets: four layers stacked
    along the batch axis with an asymmetric schedule (early layers: long
    recent windows and few heavy hitters; deep layers: the reverse), plus
    invalid pairs and lengths that give -1."""
    r = rng(21)
    layers, B, Hkv, ms = 4, 3, 4, 4096
    U = layers * B * Hkv
    scores = r.integers(0, 50, (layers * B, Hkv, ms)).astype(np.float32)
    seq = r.integers(ms // 2, ms + 1, (layers * B, Hkv)).astype(np.int32)
    heavy = np.array([256, 512, 768, 1024], np.int32)      # per layer
    recent = np.array([768, 512, 256, 64], np.int32)
    bud = np.repeat(heavy + recent, B * Hkv).reshape(layers * B, Hkv).copy()
    rec = np.repeat(recent, B * Hkv).reshape(layers * B, Hkv).copy()
    bud[1, 2], rec[1, 2] = 100, 100        # recent >= budget: -1
    bud[5, 0] = 0                          # no budget: -1
    seq[7, 3] = ms + 5                     # past the capacity: -1
    c = _Cache(layers * B, Hkv, ms, seq, np.zeros((layers * B, Hkv, ms), np.int32))
    ws = K.new_workspace(c.c)
    v, n = K.select_budgets(c.c, dev(scores), dev(bud), dev(rec), ws)
    ov, on = oracle.select_budgets(scores.reshape(U, ms), seq.reshape(U), bud.reshape(U),
                                   rec.reshape(U))
    gv, gn = host(v).reshape(U, ms), host(n).reshape(U)
    assert np.array_equal(gn, on)
    assert (on == -1).sum() == 3
    for u in range(U):
        m = max(0, int(on[u]))
        assert np.array_equal(gv[u, :m], ov[u, :m]), u
    # the scalar entry point gives the same victims on a uniform schedule
    bu = np.full((layers * B, Hkv), 900, np.int32)
    ru = np.full((layers * B, Hkv), 50, np.int32)
    seq[7, 3] = ms
    c2 = _Cache(layers * B, Hkv, ms, seq, np.zeros((layers * B, Hkv, ms), np.int32))
    v1, n1 = K.select_budgets(c2.c, dev(scores), dev(bu), dev(ru), ws)
    vic = dev(np.full((layers * B, Hkv, ms), -1, np.int32))
    nv = dev(np.zeros((layers * B, Hkv), np.int32))
    K.select(c2.c, dev(scores), 900, 50, vic, nv, ws)
    assert np.array_equal(host(n1), host(nv))
    h1, h2, hn = host(v1), host(vic), host(nv)
    for b in range(layers * B):
        for h in range(Hkv):
            m = int(hn[b, h])
            assert np.array_equal(h1[b, h, :m], h2[b, h, :m])
