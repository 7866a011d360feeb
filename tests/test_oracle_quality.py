"""What each score is for, checked on the generator's planted structure.

None of the pages prints a recall figure for these synthetic inputs, so these
tests fix the direction and target of each score instead.  A selection that
evicted the highest scores, a score with a flipped sign, or a pooled or
residual term that missed its target would fail one of them:

- H2O guide (heavy-hitter oracle): tokens whose keys lie on the queries'
  shared direction draw the most attention.  The accumulated SUM score keeps
  every one of them.
- SnapKV policy entry (observation window, pooling): planted salient spans are
  kept whole at a budget a few times their size.
- DropKV explainer (the residual score): value rows near the attention output
  change it least when dropped.  At a budget that leaves exactly their number
  to evict, they are the victims.
"""
import math

import numpy as np

import oracle
import synth
from tests.helpers import rounded_window_inputs


def _scored(name, flag, key, **kw):
    cfg = synth.CONFIGS[name].scaled(**kw)
    case = synth.make_case(cfg)
    lse, a = oracle.lse_a(case, want_a=bool(flag & oracle.DROP))
    lse32, a32 = rounded_window_inputs(case, lse, a if flag & oracle.DROP else None)
    sc = oracle.score(case, lse32, flag, cfg.pool_kernel, a32=a32)[key]
    # the generator lays tokens out in slot order: slot s holds position s
    U = cfg.B * cfg.Hkv
    assert np.array_equal(case["pos"].reshape(U, -1)[:, :cfg.L], np.tile(np.arange(cfg.L), (U, 1)))
    return cfg, case, sc.astype(np.float32)


def test_h2o_sum_keeps_planted_heavy_hitters():
    cfg, case, sc = _scored("h2o_decode_4k", oracle.SUM, "sum", B=1, Hkv=2, L=2048, W=8,
                            decode_steps=0, budget=256, recent=32)
    vic, nv = oracle.select(sc, case["seq_len"], cfg.budget, cfg.recent)
    for u in range(cfg.B * cfg.Hkv):
        planted = np.flatnonzero(case["plant"][u, :cfg.L])
        assert planted.size == math.ceil(cfg.plant_frac * cfg.L)
        assert nv[u] == cfg.L - cfg.budget
        assert not np.isin(planted, vic[u, :nv[u]]).any(), u


def test_snapkv_pool_keeps_planted_spans():
    cfg, case, sc = _scored("snapkv_prefill_32k", oracle.POOL, "pooled", B=1, Hkv=2, L=4096,
                            budget=256)
    vic, nv = oracle.select(sc, case["seq_len"], cfg.budget, cfg.recent)
    for u in range(cfg.B * cfg.Hkv):
        spans = np.flatnonzero(case["plant"][u, :cfg.L])
        assert spans.size >= math.ceil(cfg.plant_frac * cfg.L)
        assert 4 * spans.size < cfg.budget
        assert not np.isin(spans, vic[u, :nv[u]]).any(), u


def test_dropkv_residual_evicts_near_mean_rows():
    cfg, case, sc = _scored("dropkv_128k", oracle.DROP, "drop", B=1, Hkv=2, L=4096)
    v = synth.decode(case["v_pool"], "bf16").astype(np.float64)
    for h in range(cfg.Hkv):
        rows = v[case["block_table"][0, h, np.arange(cfg.L) // 16], np.arange(cfg.L) % 16]
        near = np.linalg.norm(rows, axis=1) < 0.2 * math.sqrt(cfg.D)
        assert abs(near.mean() - cfg.nearmean_frac) < 0.03
        target = np.flatnonzero(near[:cfg.L - cfg.recent])
        vic, nv = oracle.select(sc[:, h:h + 1], case["seq_len"][:, h:h + 1],
                                cfg.L - target.size, cfg.recent)
        assert nv[0] == target.size
        assert np.array_equal(vic[0, :nv[0]], target), h
