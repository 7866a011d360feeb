"""The seeded input generator: determinism and the planted structure."""
import math

import numpy as np

import synth


def test_counter_generator_is_deterministic_and_offsettable():
    a = synth.normal(1000, 5, 7)
    b = synth.normal(1000, 5, 7)
    c = synth.normal(500, 5, 7, offset=500)
    assert np.array_equal(a, b) and np.array_equal(a[500:], c)
    assert not np.array_equal(a, synth.normal(1000, 5, 8))
    x = synth.normal(200000, 1, 1)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    u = synth.uniform(200000, 1, 2)
    assert u.min() > 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.005


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 65504.0, 1e-30], np.float32)
    bits = synth.to_bf16(vals)
    back = synth.bf16_to_f32(bits)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2**-6
    assert back[3] == -2.5
    assert np.all(np.abs(back - vals) <= np.abs(vals) * 2**-8)


def test_case_is_reproducible_and_paged():
    cfg = synth.CONFIGS["tiny_f32"]
    c1, c2 = synth.make_case(cfg), synth.make_case(cfg)
    for k in ("k_pool", "v_pool", "block_table", "q"):
        assert np.array_equal(c1[k], c2[k])
    bt = c1["block_table"].reshape(-1)
    assert sorted(bt.tolist()) == list(range(c1["num_blocks"]))      # a permutation of the pool
    assert not np.array_equal(bt, np.arange(bt.size))                  # and not the identity
    assert abs(synth.decode(c1["k_pool"], "f32").std() - 1 / 8) < 0.01


def test_planted_heavy_hitters_and_spans():
    cfg = synth.CONFIGS["h2o_decode_4k"].scaled(B=1, Hkv=2, L=1000, decode_steps=24)
    case = synth.make_case(cfg)
    count = math.ceil(0.02 * cfg.L_final)
    assert np.all(case["plant"].sum(axis=1) == count)
    # planted keys carry +3*sqrt(2) along the head direction u
    k = synth.decode(case["k_pool"], "bf16").astype(np.float64)
    u = case["dirs"][0]
    proj = np.array([k[case["block_table"][0, 0, s // 16], s % 16] @ u for s in range(cfg.L_final)])
    pl = case["plant"][0, :cfg.L_final].astype(bool)
    assert abs(proj[pl].mean() - 3 * math.sqrt(2)) < 0.5 and abs(proj[~pl].mean()) < 0.2

    cs = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=1, Hkv=2, L=4096)
    case = synth.make_case(cs)
    for u in range(2):
        m = case["plant"][u, :cs.L]
        assert m.sum() >= math.ceil(0.01 * cs.L) and m[cs.L - cs.W:].sum() == 0
        edges = np.flatnonzero(np.diff(np.concatenate([[0], m, [0]]).astype(int)))
        lens = edges[1::2] - edges[::2]
        assert lens.min() >= 8 and lens.max() <= 64 * 2   # adjacent spans may touch


def test_near_mean_value_rows():
    cfg = synth.CONFIGS["dropkv_128k"].scaled(Hkv=1, L=8192)
    case = synth.make_case(cfg)
    v = synth.decode(case["v_pool"], "bf16").astype(np.float64)
    norms = np.array([np.linalg.norm(v[case["block_table"][0, 0, s // 16], s % 16])
                      for s in range(cfg.L)])
    small = norms < 0.2 * math.sqrt(cfg.D)
    assert abs(small.mean() - 0.1) < 0.02
    assert abs(np.median(norms[small]) - 0.05 * math.sqrt(cfg.D)) < 0.05
