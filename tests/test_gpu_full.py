"""GPU parity at the five workloads' full sizes.

The scaled-down cases in the other files compare every output; here the
workloads run at their real shapes:

* SnapKV prefill, 32K context (B4, 8 KV heads x 4, D128): the fused entry
  point kvev_evict in the launch configuration the benchmark times, every
  head against the oracle's chain; plus the full pooled score array from
  kvev_score.
* DropKV residual scoring, 128K context (B1, 8 KV heads x 8): kvev_evict with
  the residual score, every head against the oracle's chain.
* Block-aware eviction of the 70B GQA shape: each of its eight 64000-token
  layers (B16, 8 KV heads x 8, about 4.2 GB of K+V each, its own seeded
  data) through kvev_evict, every head of every layer against the oracle's
  chain (scores, victims, compaction) and the closed-form block count.
* H2O decode accumulation (B8, 8 KV heads x 4, 4096 -> 4352 tokens): the 256
  decode steps of ACCUMULATE scoring, then select and compact, every head
  against the oracle run through the same schedule.

Tolerances and the end-to-end rule are those of the scaled tests: scores to
2e-3 relative (bf16 caches, fp32 accumulation); victim sets equal or
differing only inside that band around the oracle's cutoff; compaction
bit-exact.
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import (KIND, TOL, Run, assert_scores_close,
                               check_eviction_vs_oracle_chain, dev, device_cache, host)
from tests.helpers import rounded_window_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[full] {msg}", flush=True)


def _evict_full(name, layer=0):
    cfg = synth.CONFIGS[name]
    kind = cfg.flags[0]
    kg, ko, key = KIND[kind]
    case = synth.make_case(cfg, layer=layer)
    if layer:
        name = f"{name} layer {layer}"
    _say(f"{name}: oracle window inputs")
    lse64, a64 = oracle.lse_a(case, want_a=(kind == "drop"))
    lse32, a32 = rounded_window_inputs(case, lse64, a64)
    _say(f"{name}: oracle scores")
    o32 = oracle.score(case, lse32, ko, cfg.pool_kernel, a32=a32)[key].astype(np.float32)
    _say(f"{name}: kvev_score on the full cache")
    r = Run(case, free_prefix=0)
    a_dev = dev(a32) if a32 is not None else None
    out = K.score(r.dc, r.q, dev(lse32), r.qp, case["scale"], case["G"], kg, cfg.pool_kernel,
                  **{key: r.dc.score_buffer()}, a=a_dev)
    torch.cuda.synchronize()
    worst = assert_scores_close(host(out[key]), o32.astype(np.float64), case["seq_len"],
                                TOL[cfg.dtype], key)
    _say(f"{name}: scores within tolerance, worst relative error {worst:.2e}")
    del out
    _say(f"{name}: kvev_evict")
    r.fused(kind, lse32, a32, cfg.pool_kernel, cfg.budget, cfg.recent)
    st = r.state()
    ov, on = oracle.select(np.nan_to_num(o32, nan=0.0), case["seq_len"], cfg.budget, cfg.recent)
    new, ofl, ofc, ostats = oracle.compact(case, ov, on, score_row=np.nan_to_num(o32, nan=0.0),
                                           free_list=np.full(case["num_blocks"] + 8, -1, np.int32),
                                           free_count=0)
    nd = check_eviction_vs_oracle_chain(case, st, ov, on, new, ofl, ofc, ostats, o32,
                                        TOL[cfg.dtype])
    _say(f"{name}: stats {st['stats'].tolist()}, {nd} heads with victims differing inside the "
         f"tolerance band")
    return st


def test_snapkv_prefill_32k_full_size():
    st = _evict_full("snapkv_prefill_32k")
    assert st["stats"][0] == 4 * 8 * (2048 - 128)  # blocks freed: 32768 -> 2048 tokens per head


def test_dropkv_128k_full_size():
    st = _evict_full("dropkv_128k")
    assert st["stats"][0] == 8 * (8192 - (6553 + 15) // 16)


@pytest.mark.parametrize("layer", range(8))
def test_block_evict_64k_layer_full_size(layer):
    """Each of the eight layers (its own seeded keys, values, queries and
    planted heavy hitters), every one of its 128 heads against the oracle."""
    st = _evict_full("block_evict_64k", layer)
    assert st["stats"][0] == 16 * 8 * (4000 - 2000)  # 64000 -> 32000 tokens per head


def test_h2o_decode_4k_full_schedule():
    cfg = synth.CONFIGS["h2o_decode_4k"]
    case = synth.make_case(cfg)
    B, H, G, D = case["B"], case["Hkv"], case["G"], case["D"]
    ms = case["max_blocks"] * 16
    dc = device_cache(case)
    gsum = dev(np.zeros((B, H, ms), np.float32))
    osum = np.zeros((B, H, ms), np.float32)
    _say(f"{cfg.decode_steps} decode steps of ACCUMULATE scoring, oracle beside")
    for t in range(cfg.decode_steps):
        n = cfg.L + t + 1  # the step's token is appended, then scored
        q, q_pos = synth.make_queries(cfg, 0, 1, case["dirs"], step=t)
        step = dict(case, seq_len=np.full((B, H), n, np.int32), q=q, q_pos=q_pos, W=1)
        lse64, _ = oracle.lse_a(step)
        lse32, _ = rounded_window_inputs(step, lse64)
        o = oracle.score(step, lse32, oracle.SUM | oracle.ACCUMULATE, 1, prev_sum=osum)["sum"]
        osum = np.nan_to_num(o, nan=0.0).astype(np.float32)
        dc.seq_len.fill_(n)
        K.score(dc, dev(q), dev(lse32), dev(q_pos), case["scale"], G, K.SUM | K.ACCUMULATE, 1,
                sum=gsum)
        if t % 64 == 63:
            torch.cuda.synchronize()
            _say(f"step {t + 1} done")
    torch.cuda.synchronize()
    final = dict(case, seq_len=np.full((B, H), cfg.L_final, np.int32))
    worst = assert_scores_close(host(gsum), osum.astype(np.float64), final["seq_len"],
                                TOL[cfg.dtype], "accumulated sum")
    _say(f"accumulated sums within tolerance, worst relative error {worst:.2e}")
    budget, recent = cfg.budget, cfg.recent  # 20% and 10% of the final 4352 tokens
    assert (budget, recent) == (int(0.2 * cfg.L_final), int(0.1 * cfg.L_final))
    ws = K.new_workspace(dc)
    vic, nv = K.select(dc, gsum, budget, recent, workspace=ws)
    fl = dev(np.full(case["num_blocks"] + 8, -1, np.int32))
    fc = dev(np.zeros(1, np.int32))
    stats = K.compact(dc, vic, nv, fl, fc, ws, score_row=gsum)
    torch.cuda.synchronize()
    st = dict(k=host(dc.k_pool), v=host(dc.v_pool), bt=host(dc.block_table), seq=host(dc.seq_len),
              pos=host(dc.pos), fl=host(fl), fc=int(host(fc)[0]), stats=host(stats),
              vic=host(vic), nv=host(nv), score=host(gsum))
    ov, on = oracle.select(osum, final["seq_len"], budget, recent)
    new, ofl, ofc, ostats = oracle.compact(final, ov, on, score_row=osum,
                                           free_list=np.full(case["num_blocks"] + 8, -1, np.int32))
    nd = check_eviction_vs_oracle_chain(final, st, ov, on, new, ofl, ofc, ostats, osum,
                                        TOL[cfg.dtype])
    _say(f"stats {st['stats'].tolist()}, {nd} heads with victims differing inside the band")
    assert st["stats"][0] == B * H * (272 - (870 + 15) // 16)
