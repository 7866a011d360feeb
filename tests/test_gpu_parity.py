"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Scores: |gpu - oracle| <= tol * max(|oracle|, FLT_MIN), tol = 1e-5 for fp32
caches and 2e-3 for bf16 caches (fp32 accumulation).  Selection on identical
fp32 scores and compaction on identical victims: bit-exact.  End to end,
victim sets may differ only where an oracle score lies within the tolerance
of the oracle's cutoff.  Sizes span several tiles and a ragged tail.
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import (TOL, assert_scores_close, check_eviction_vs_oracle_chain, dev,
                               device_cache, device_window, host)
from tests.helpers import manual_case, rounded_window_inputs

pytestmark = pytest.mark.gpu

FLAG_MAP = {"sum": (oracle.SUM, K.SUM), "pool": (oracle.POOL, K.POOL), "drop": (oracle.DROP, K.DROP)}


def _flags(kinds):
    o = g = 0
    for k in kinds:
        o |= FLAG_MAP[k][0]
        g |= FLAG_MAP[k][1]
    return o, g


def _ragged(B, H, L, rng_seed=0):
    r = np.random.default_rng(rng_seed)
    seq = np.full((B, H), L, np.int32)
    flat = seq.reshape(-1)
    picks = [L - 1, L // 2 + 3, min(17, L), 1, 0, min(16, L)]
    for i in range(1, flat.size):
        flat[i] = picks[(i - 1) % len(picks)] if i % 2 else L - int(r.integers(0, min(40, L)))
    return seq


def _run_score(case, kinds, pool_kernel, want_a, prev=None):
    lse64, a64 = oracle.lse_a(case, want_a=want_a)
    lse32, a32 = rounded_window_inputs(case, lse64, a64)
    of, gf = _flags(kinds)
    if prev is not None:
        of |= oracle.ACCUMULATE
        gf |= K.ACCUMULATE
    orc = oracle.score(case, lse32, of, pool_kernel, a32=a32, prev_sum=prev)
    dc = device_cache(case)
    q, qp = device_window(case)
    s_buf = dev(prev.copy()) if prev is not None else None
    out = K.score(dc, q, dev(lse32), qp, case["scale"], case["G"], gf, pool_kernel, sum=s_buf,
                  a=dev(a32) if a32 is not None else None)
    torch.cuda.synchronize()
    return orc, {k: (host(v) if v is not None else None) for k, v in out.items()}, lse32, a32


SCORE_CASES = [
    # name, config overrides, kinds, pool kernel, ragged
    ("tiny_f32", {}, ("sum", "pool", "drop"), 5, False),
    ("tiny_f32", dict(D=128, L=700, W=12, B=2), ("sum", "pool", "drop"), 3, True),
    ("snapkv_prefill_32k", dict(B=2, Hkv=3, L=3001), ("sum", "pool"), 7, True),
    ("snapkv_prefill_32k", dict(B=1, Hkv=2, L=2000, D=64), ("pool",), 33, False),
    ("snapkv_prefill_32k", dict(B=1, Hkv=2, L=1500, W=8), ("pool",), 63, True),
    ("snapkv_prefill_32k", dict(B=1, Hkv=2, L=1200), ("pool",), 1, False),
    ("dropkv_128k", dict(Hkv=2, L=4099), ("drop",), 1, True),
    ("dropkv_128k", dict(Hkv=2, L=2000, D=64, G=4), ("drop", "sum"), 1, False),
    ("h2o_decode_4k", dict(B=2, Hkv=2, L=1000, decode_steps=0), ("sum",), 1, True),
    ("block_evict_64k", dict(B=2, Hkv=2, L=2500), ("sum",), 1, True),
]


@pytest.mark.parametrize("name,over,kinds,pool,ragged", SCORE_CASES,
                         ids=[f"{c[0]}-{i}" for i, c in enumerate(SCORE_CASES)])
def test_score_matches_oracle(name, over, kinds, pool, ragged):
    cfg = synth.CONFIGS[name].scaled(**over)
    seq = _ragged(cfg.B, cfg.Hkv, cfg.L) if ragged else None
    case = synth.make_case(cfg, seq_len=seq)
    orc, gpu, _, _ = _run_score(case, kinds, pool, want_a="drop" in kinds)
    key = {"sum": "sum", "pool": "pooled", "drop": "drop"}
    for k in kinds:
        worst = assert_scores_close(gpu[key[k]], orc[key[k]], case["seq_len"], TOL[cfg.dtype],
                                    f"{name}/{k}")
        print(f"{name} {k}: worst relative error {worst:.3g}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_score_accumulate(dtype):
    """[H2O] lifecycle: the new step's attention is added to the stored score."""
    cfg = synth.CONFIGS["h2o_decode_4k"].scaled(B=1, Hkv=3, L=1700, D=64, dtype=dtype)
    case = synth.make_case(cfg, seq_len=_ragged(1, 3, 1700))
    prev = np.random.default_rng(5).uniform(0, 3, (1, 3, case["max_blocks"] * 16)).astype(np.float32)
    orc, gpu, _, _ = _run_score(case, ("sum",), 1, False, prev=prev)
    assert_scores_close(gpu["sum"], orc["sum"], case["seq_len"], TOL[dtype], "accumulate")


def test_score_page_worked_example_on_gpu():
    """[DROP] "Worked example" through the GPU kernel (fp32 cache, D 64)."""
    p = np.array([0.5, 0.3, 0.15, 0.05]); vals = np.array([5.0, 5.0, 15.0, 5.0]); n, D = 4, 64
    k = np.zeros((1, 1, n, D)); k[0, 0, :, 0] = np.log(p)
    v = np.zeros((1, 1, n, D)); v[0, 0, :, 0] = vals
    q = np.zeros((1, 1, 1, D)); q[..., 0] = 1.0
    case = manual_case(k, v, q, np.array([[n - 1]]), dtype="f32", scale=1.0)
    a = np.zeros((1, 1, 1, D), np.float32); a[..., 0] = 6.5
    dc = device_cache(case)
    qd, qp = device_window(case)
    out = K.score(dc, qd, dev(np.zeros((1, 1, 1), np.float32)), qp, 1.0, 1, K.DROP | K.SUM, a=dev(a))
    d = host(out["drop"])[0, 0, :n]
    np.testing.assert_allclose(d, [1.5, 9 / 14, 1.5, 3 / 38], rtol=1e-5)
    vic, nv = K.select(dc, out["drop"], 2, 0)
    assert host(vic)[0, 0, :host(nv)[0, 0]].tolist() == [1, 3]


# ------------------------------------------------------------- selection


def _score_rows(kind, U, ms, seed):
    r = np.random.default_rng(seed)
    if kind == "uniform":
        return r.uniform(0, 1, (U, ms)).astype(np.float32)
    if kind == "ties":
        return np.round(r.uniform(0, 6, (U, ms))).astype(np.float32)
    if kind == "special":
        s = np.round(r.normal(0, 2, (U, ms)), 1).astype(np.float32)
        s[:, ::7] = -0.0
        s[:, 3::7] = 0.0
        s[:, 5::11] = np.inf
        s[:, 6::13] = -np.inf
        s[:, 9::17] = np.nan
        return s
    if kind == "equal":
        return np.full((U, ms), 0.125, np.float32)
    if kind == "lognormal":
        return np.exp(r.normal(-6, 2, (U, ms))).astype(np.float32)
    raise ValueError(kind)


SELECT_CASES = [("uniform", 3000, 500, 32), ("ties", 3000, 700, 0), ("special", 2100, 300, 16),
                ("equal", 1500, 100, 10), ("lognormal", 40000, 2048, 32),
                ("lognormal", 4099, 5000, 32), ("ties", 17, 4, 3)]


@pytest.mark.parametrize("kind,L,budget,recent", SELECT_CASES)
def test_select_bit_exact_on_oracle_scores(kind, L, budget, recent):
    """Identical fp32 scores -> identical victims, in ascending order."""
    B, H = 2, 3
    seq = _ragged(B, H, L, 3)
    mb = (L + 15) // 16
    # select reads only seq_len and the score rows; the pools are placeholders
    case = dict(dtype="f32", B=B, Hkv=H, G=1, D=64, W=1, max_blocks=mb, num_blocks=B * H * mb,
                k_pool=np.zeros((B * H * mb, 16, 64), np.float32),
                v_pool=np.zeros((B * H * mb, 16, 64), np.float32),
                block_table=np.arange(B * H * mb, dtype=np.int32).reshape(B, H, mb),
                seq_len=seq, pos=np.zeros((B, H, mb * 16), np.int32))
    ms = case["max_blocks"] * 16
    scores = _score_rows(kind, B * H, ms, 11).reshape(B, H, ms)
    ov, on = oracle.select(scores, case["seq_len"], budget, recent)
    dc = device_cache(case)
    gv, gn = K.select(dc, dev(scores), budget, recent)
    gv, gn = host(gv).reshape(B * H, ms), host(gn).reshape(-1)
    assert np.array_equal(gn, on)
    for u in range(B * H):
        assert np.array_equal(gv[u, :on[u]], ov[u, :on[u]]), u


# ------------------------------------------------------------ compaction


def _pattern_victims(seq, ms, pattern, seed=0):
    r = np.random.default_rng(seed)
    U = seq.size
    vic = np.full((U, ms), -1, np.int32); nv = np.zeros(U, np.int32)
    for u in range(U):
        n = int(seq.reshape(-1)[u])
        if pattern == "random":
            sel = np.sort(r.choice(n, size=n // 2, replace=False)) if n else np.zeros(0, int)
        elif pattern == "first_only":
            sel = np.arange(min(1, n))
        elif pattern == "every_other":
            sel = np.arange(0, n, 2)
        elif pattern == "none":
            sel = np.zeros(0, int)
        elif pattern == "keep_recent":
            sel = np.arange(0, max(0, n - 37))
        elif pattern == "tail":
            sel = np.arange(max(0, n - 300), n)
        else:  # sparse: 94% evicted, like a 32K -> 2K prefill compression
            sel = np.sort(r.choice(n, size=int(n * 0.94), replace=False)) if n else np.zeros(0, int)
        vic[u, :len(sel)] = sel
        nv[u] = len(sel)
    return vic, nv


def _compact_both(case, vic, nv, with_score=True, free_prefix=3):
    B, H, ms = case["B"], case["Hkv"], case["max_blocks"] * 16
    score_row = np.random.default_rng(1).uniform(0, 1, (B, H, ms)).astype(np.float32)
    free0 = np.full(case["num_blocks"] + 8, -1, np.int32)
    free0[:free_prefix] = np.arange(free_prefix) + 10**6
    new, ofl, ofc, ostats = oracle.compact(case, vic, nv, score_row=score_row if with_score else None,
                                           free_list=free0, free_count=free_prefix)
    dc = device_cache(case)
    ws = K.new_workspace(dc)
    fl = dev(free0.copy())
    fc = dev(np.array([free_prefix], np.int32))
    sr = dev(score_row.copy()) if with_score else None
    stats = K.compact(dc, dev(vic.reshape(B, H, ms)), dev(nv.reshape(B, H)), fl, fc, ws,
                      score_row=sr)
    torch.cuda.synchronize()
    g = dict(k_pool=host(dc.k_pool), v_pool=host(dc.v_pool), block_table=host(dc.block_table),
             seq_len=host(dc.seq_len), pos=host(dc.pos), free_list=host(fl),
             free_count=int(host(fc)[0]), stats=host(stats),
             score=host(sr) if with_score else None)
    return new, ofl, ofc, ostats, g


def _assert_compaction_equal(case, new, ofl, ofc, ostats, g):
    B, H = case["B"], case["Hkv"]
    assert np.array_equal(g["seq_len"], new["seq_len"])
    assert np.array_equal(g["block_table"], new["block_table"])
    assert g["free_count"] == ofc
    assert np.array_equal(g["free_list"][:ofc], ofl[:ofc])
    assert np.array_equal(g["stats"], ostats)
    for b in range(B):
        for h in range(H):
            n2 = int(new["seq_len"][b, h])
            assert np.array_equal(g["pos"][b, h, :n2], new["pos"][b, h, :n2])
            if g["score"] is not None:
                assert np.array_equal(g["score"][b, h, :n2], new["score_row"][b, h, :n2])
            for s in range(0, n2, 16):
                blk = new["block_table"][b, h, s // 16]
                e = min(16, n2 - s)
                assert np.array_equal(g["k_pool"][blk, :e], new["k_pool"][blk, :e]), (b, h, s)
                assert np.array_equal(g["v_pool"][blk, :e], new["v_pool"][blk, :e]), (b, h, s)


@pytest.mark.parametrize("pattern", ["random", "first_only", "every_other", "none", "keep_recent",
                                     "tail", "sparse"])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_compact_bit_exact_on_oracle_victims(pattern, dtype, D):
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=2, Hkv=3, L=2600, D=D, dtype=dtype)
    case = synth.make_case(cfg, seq_len=_ragged(2, 3, 2600, 7), spare_blocks=11)
    vic, nv = _pattern_victims(case["seq_len"], case["max_blocks"] * 16, pattern)
    new, ofl, ofc, ostats, g = _compact_both(case, vic, nv, with_score=(D == 128))
    _assert_compaction_equal(case, new, ofl, ofc, ostats, g)


@pytest.mark.parametrize("pattern,dtype,D", [("first_only", "bf16", 128), ("random", "bf16", 128),
                                             ("every_other", "bf16", 128), ("tail", "bf16", 128),
                                             ("first_only", "f32", 64)])
def test_compact_beyond_the_staging_cap(pattern, dtype, D):
    """Heads with more than 4096 at-risk rows (20000 tokens: evicting slot 0
    shifts 19999 rows, half evicted leaves about 5000) move in rank order
    without staging; in the same call shorter heads (8000 and 12000 tokens
    with half evicted: 2000-3000 at-risk rows; 17 and 0 tokens) stage theirs.
    Bit-exact against the oracle."""
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=2, Hkv=3, L=20000, D=D, dtype=dtype)
    seq = np.array([[20000, 19999, 8000], [17, 12000, 0]], np.int32)
    case = synth.make_case(cfg, seq_len=seq, spare_blocks=5)
    vic, nv = _pattern_victims(case["seq_len"], case["max_blocks"] * 16, pattern)
    new, ofl, ofc, ostats, g = _compact_both(case, vic, nv, with_score=(D == 128))
    _assert_compaction_equal(case, new, ofl, ofc, ostats, g)
    assert ostats[3] > 4096 or pattern == "tail"


def test_compact_rejects_unsorted_victims_and_leaves_cache():
    """Victims not strictly ascending: the head is left unchanged and a status
    bit is set; the other heads are compacted."""
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=1, Hkv=2, L=600)
    case = synth.make_case(cfg)
    vic, nv = _pattern_victims(case["seq_len"], case["max_blocks"] * 16, "random")
    bad = vic.copy()
    bad[0, [3, 4]] = bad[0, [4, 3]]
    dc = device_cache(case)
    ws = K.new_workspace(dc)
    fl = dev(np.full(case["num_blocks"], -1, np.int32))
    fc = dev(np.zeros(1, np.int32))
    ms = case["max_blocks"] * 16
    stats = host(K.compact(dc, dev(bad.reshape(1, 2, ms)), dev(nv.reshape(1, 2)), fl, fc, ws))
    assert stats[4] & 1
    assert host(dc.seq_len)[0, 0] == 600 and host(dc.seq_len)[0, 1] == 600 - nv[1]
    k0 = host(dc.k_pool)
    assert np.array_equal(k0[case["block_table"][0, 0]], case["k_pool"][case["block_table"][0, 0]])


# ------------------------------------------------------------ end to end


E2E = [("snapkv_prefill_32k", dict(B=2, Hkv=4, L=4000), ("pool",), 7, 500, 32),
       ("dropkv_128k", dict(Hkv=2, L=6000), ("drop",), 1, 300, 32),
       ("block_evict_64k", dict(B=2, Hkv=2, L=3000), ("sum",), 1, 1500, 16),
       ("tiny_f32", {}, ("pool",), 5, 128, 32)]


@pytest.mark.parametrize("name,over,kinds,pool,budget,recent", E2E, ids=[e[0] for e in E2E])
def test_end_to_end(name, over, kinds, pool, budget, recent):
    """GPU score -> select -> compact against the oracle chain."""
    cfg = synth.CONFIGS[name].scaled(**over)
    case = synth.make_case(cfg)
    orc, gpu, lse32, a32 = _run_score(case, kinds, pool, want_a="drop" in kinds)
    key = {"sum": "sum", "pool": "pooled", "drop": "drop"}[kinds[0]]
    o32 = orc[key].astype(np.float32)
    dc = device_cache(case)
    gv, gn = K.select(dc, dev(gpu[key]), budget, recent)
    gvh, gnh = host(gv), host(gn)
    # compaction of the GPU's own victims on the device
    fl = dev(np.full(case["num_blocks"] + 8, -1, np.int32))
    fc = dev(np.zeros(1, np.int32))
    stats = K.compact(dc, gv, gn, fl, fc, K.new_workspace(dc))
    torch.cuda.synchronize()
    st = dict(k=host(dc.k_pool), v=host(dc.v_pool), bt=host(dc.block_table), seq=host(dc.seq_len),
              pos=host(dc.pos), fl=host(fl), fc=int(host(fc)[0]), stats=host(stats), vic=gvh,
              nv=gnh)
    # the oracle's own chain: its scores -> its victims -> its compaction
    ov, on = oracle.select(np.nan_to_num(o32, nan=0.0), case["seq_len"], budget, recent)
    new, ofl, ofc, ostats = oracle.compact(case, ov, on,
                                           free_list=np.full(case["num_blocks"] + 8, -1, np.int32))
    nd = check_eviction_vs_oracle_chain(case, st, ov, on, new, ofl, ofc, ostats, o32,
                                        TOL[cfg.dtype])
    print(f"{name}: {nd} heads with victims differing inside the tolerance band", flush=True)
    m = oracle.measure(case["seq_len"], ov, on)
    assert m["blocks_freed"] == ostats[0]


# ------------------------------------------------------- helper and misc


def _weighted_abs_values(case, lse64):
    """sum_j p_j |v_j| of every window row and d (float64, from the case's own
    rows): the scale of the output's error bound, which also covers outputs
    that cancel to near 0."""
    B, Hkv, G, W, D = case["B"], case["Hkv"], case["G"], case["W"], case["D"]
    kp = synth.decode(case["k_pool"], case["dtype"]).astype(np.float64)
    vp = synth.decode(case["v_pool"], case["dtype"]).astype(np.float64)
    q = synth.decode(case["q"], case["dtype"]).astype(np.float64)
    out = np.zeros((B, Hkv * G, W, D))
    for b in range(B):
        for h in range(Hkv):
            n = int(case["seq_len"][b, h])
            if n <= 0:
                continue
            j = np.arange(n)
            blk = case["block_table"][b, h, j // 16]
            k = kp[blk, j % 16]
            v = vp[blk, j % 16]
            pos = case["pos"][b, h, :n]
            for g in range(G):
                hq = h * G + g
                s = case["scale"] * q[b, hq] @ k.T                    # [W, n]
                live = pos[None, :] <= case["q_pos"][b][:, None]
                lse = lse64[b, hq][:, None]
                p = np.where(live & np.isfinite(lse), np.exp(np.where(live, s, 0.0) - lse), 0.0)
                out[b, hq] = p @ np.abs(v)
    return out


WA_CASES = [("tiny_f32", {}),
            ("tiny_f32", dict(D=128, G=8, W=40, L=700)),      # 320 rows: two workgroups a chunk
            ("dropkv_128k", dict(Hkv=2, L=5000)),               # 256 rows, bf16
            ("snapkv_prefill_32k", dict(B=1, Hkv=2, L=3000)),   # 128 rows
            ("snapkv_prefill_32k", dict(B=1, Hkv=1, L=600, D=64, G=3, W=3)),
            ("h2o_decode_4k", dict(B=2, Hkv=2, L=1000, decode_steps=0))]  # one query row a head


@pytest.mark.parametrize("name,over", WA_CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(WA_CASES)])
def test_window_attn_matches_oracle(name, over):
    """LSE and output of the window forward against the oracle's input
    builder (double).  LSE to 1e-5 absolute plus 1e-6 relative; the output to
    1e-4 * sum_j p_j |v_j| (the MFMA takes the weights as a bf16 high and low
    part for bf16 caches, p to a relative 2^-16; fp32 sums over chunks)."""
    cfg = synth.CONFIGS[name].scaled(**over)
    case = synth.make_case(cfg, seq_len=_ragged(cfg.B, cfg.Hkv, cfg.L, 2))
    lse64, a64 = oracle.lse_a(case, want_a=True)
    dc = device_cache(case)
    q, qp = device_window(case)
    ws = K.new_workspace(dc, cfg.G, cfg.W)
    lse, a = K.window_attn(dc, q, qp, case["scale"], cfg.G, ws, want_a=True)
    lse_only, none = K.window_attn(dc, q, qp, case["scale"], cfg.G, ws, want_a=False)
    torch.cuda.synchronize()
    assert a.dtype == torch.float32 and none is None  # fp32 output for bf16 caches too
    assert torch.equal(lse, lse_only)                    # the LSE does not depend on the output
    lse, a = host(lse).astype(np.float64), host(a).astype(np.float64)
    live = np.isfinite(lse64)
    assert np.array_equal(np.isfinite(lse), live)
    err = np.abs(lse[live] - lse64[live])
    assert np.all(err <= 1e-5 + 1e-6 * np.abs(lse64[live])), err.max()
    assert np.all(a[~live] == 0.0)
    bound = 1e-4 * _weighted_abs_values(case, lse64)
    worst = (np.abs(a - a64) / np.maximum(bound, 1e-30)).max()
    assert np.all(np.abs(a - a64) <= bound), worst
    print(f"{name} {over}: LSE worst {err.max():.2e}; output worst {worst * 1e-4:.2e} of "
          f"sum p|v|", flush=True)


def test_runs_are_bitwise_reproducible():
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=1, Hkv=2, L=3000)
    case = synth.make_case(cfg)
    lse64, _ = oracle.lse_a(case)
    lse = dev(lse64.astype(np.float32))
    dc = device_cache(case)
    q, qp = device_window(case)
    r1 = K.score(dc, q, lse, qp, case["scale"], cfg.G, K.POOL | K.SUM, 7)
    r2 = K.score(dc, q, lse, qp, case["scale"], cfg.G, K.POOL | K.SUM, 7)
    assert torch.equal(r1["pooled"], r2["pooled"]) and torch.equal(r1["sum"], r2["sum"])
    v1 = K.select(dc, r1["pooled"], 300, 32)
    v2 = K.select(dc, r2["pooled"], 300, 32)
    assert torch.equal(v1[0], v2[0]) and torch.equal(v1[1], v2[1])


def test_inconsistent_seq_len_is_flagged_not_used():
    cfg = synth.CONFIGS["snapkv_prefill_32k"].scaled(B=1, Hkv=2, L=400)
    case = synth.make_case(cfg)
    case["seq_len"] = np.array([[400, 10**6]], np.int32)
    dc = device_cache(case)
    scores = dev(np.ones((1, 2, case["max_blocks"] * 16), np.float32))
    _, nv = K.select(dc, scores, 100, 8)
    assert host(nv).tolist() == [[300, -1]]


# ------------------------------------------------------------ measurement


@pytest.mark.parametrize("pattern", ["random", "first_only", "every_other", "none", "keep_recent",
                                     "tail", "sparse"])
def test_measure_matches_oracle(pattern):
    """kvev_measure against the oracle's Eq. 1 waste and half-use shares on
    test-made victim lists (ragged heads, heads of 0, 1, 16 and 17 tokens)."""
    seq = np.array([[3001, 0, 1, 16], [17, 2048, 777, 4099]], np.int32)
    ms = 4112
    vic, nv = _pattern_victims(seq, ms, pattern, seed=3)
    g = K.measure(dev(seq), dev(vic.reshape(2, 4, ms)), dev(nv.reshape(2, 4)))
    o = oracle.measure(seq, vic, nv)
    for k in ("blocks_naive", "blocks_after", "live_tokens", "blocks_freed"):
        assert g[k] == int(o[k]), k
    for k in ("F_naive", "F_after", "frac_le_half_naive", "frac_le_half_after"):
        assert g[k] == o[k], k


def test_measure_full_size_block_evict_layer():
    """One 64000-token layer of the 70B GQA shape (B16, 8 KV heads): half of
    every head evicted at random, as the block-evict workload does."""
    B, H, L = 16, 8, 64000
    ms = 4000 * 16
    seq = np.full((B, H), L, np.int32)
    vic, nv = _pattern_victims(seq, ms, "random", seed=5)
    g = K.measure(dev(seq), dev(vic.reshape(B, H, ms)), dev(nv.reshape(B, H)))
    o = oracle.measure(seq, vic, nv)
    assert g["blocks_freed"] == int(o["blocks_freed"]) == B * H * (4000 - 2000)
    for k in ("blocks_naive", "blocks_after", "live_tokens"):
        assert g[k] == int(o[k]), k
    for k in ("F_naive", "F_after", "frac_le_half_naive", "frac_le_half_after"):
        assert g[k] == o[k], k
