"""GPU parity of DropKV's residual score where the attention weight p of a key
approaches 1 ([DROP] "The news", Lemma 1: the output shift from removing
key j is p_j/(1 - p_j) * (a - v_j), so its length grows without bound as
p_j -> 1 and is undefined at p_j = 1).

Window rows get one dominant key each, at weights from about 0.2 to 0.9999,
and one window query attends a single key (p = 1 up to the rounding of its
LSE: the term is then +inf when x = scale*q.k - lse >= 0, and 0 otherwise,
since a equals that key's value row).  The attention output a and the LSE
come from the oracle's input builder, rounded to fp32, identical for both
sides; the GPU scores must meet the score tolerance (1e-5 fp32, 2e-3 bf16)
everywhere, infinities included.  A window of 256 rows (G 8 x W 32) is
also run on bf16, where the rows are split over two workgroups per tile.
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
from tests.gpu_helpers import TOL, assert_scores_close, dev, device_cache, device_window, host
from tests.helpers import manual_case, rounded_window_inputs

pytestmark = pytest.mark.gpu

TARGETS = (0.2, 0.3, 0.9, 0.99, 0.999, 0.9999)


def _dominant_case(dtype, G, W, D=64, n=300, seed=0, Hkv=1):
    """Keys are small random rows; window row (g, w) looks along coordinate
    d = (g * W + w) % D and its dominant key carries a large value there, so
    that its weight is about TARGETS[(g * W + w) % len(TARGETS)].  Window
    query 0 sits at position 0 and attends key 0 alone."""
    r = np.random.default_rng(seed)
    k = r.normal(0, 1, (1, Hkv, n, D)) * 0.05
    v = r.normal(0, 1, (1, Hkv, n, D))
    q = np.zeros((1, Hkv * G, W, D))
    q_pos = np.full((1, W), n - 1, np.int32)
    q_pos[0, 0] = 0
    for h in range(Hkv):
        for g in range(G):
            for w in range(1, W):
                row = g * W + w
                d = row % D
                p = TARGETS[row % len(TARGETS)]
                j = 1 + (row * 7 + h) % (n - 1)
                # logit gap for weight p against about n - 1 logits near 0
                gap = np.log(p / (1.0 - p) * (n - 1))
                q[0, h * G + g, w, d] = 1.0
                k[0, h, j, d] = gap
            q[0, h * G + g, 0, 0] = 1.0
    return manual_case(k, v, q, q_pos, dtype=dtype, scale=1.0)


def _gpu_drop(case, lse32, a32):
    dc = device_cache(case)
    q, qp = device_window(case)
    out = K.score(dc, q, dev(lse32), qp, case["scale"], case["G"], K.DROP | K.SUM, 1,
                  a=dev(a32))
    torch.cuda.synchronize()
    return host(out["drop"]), host(out["sum"])


@pytest.mark.parametrize("dtype,G,W,D", [("f32", 2, 4, 64), ("bf16", 2, 4, 64),
                                         ("f32", 4, 8, 128), ("bf16", 4, 8, 128),
                                         ("bf16", 8, 32, 128)])
def test_dropkv_near_one_weights(dtype, G, W, D):
    case = _dominant_case(dtype, G, W, D=D)
    lse64, a64 = oracle.lse_a(case, want_a=True)
    lse32, a32 = rounded_window_inputs(case, lse64, a64)
    orc = oracle.score(case, lse32, oracle.DROP | oracle.SUM, a32=a32)
    gd, gs = _gpu_drop(case, lse32, a32)
    # the weights really reach the regime (key 0 aside, attended alone)
    p_max = float(np.nanmax(orc["sum"][0, 0, 1:]))
    assert p_max > 0.99, p_max
    worst = assert_scores_close(gd, orc["drop"], case["seq_len"], TOL[dtype], "drop")
    assert_scores_close(gs, orc["sum"], case["seq_len"], TOL[dtype], "sum")
    # key 0, attended alone by window query 0, is +inf or finite on both sides alike
    print(f"{dtype} G{G} W{W} D{D}: worst relative error {worst:.2e}; key 0: gpu {gd[0, 0, 0]!r} "
          f"oracle {orc['drop'][0, 0, 0]!r}", flush=True)


def test_dropkv_near_one_eviction_matches_oracle():
    """kvev_evict with DROP on dominant keys: victims and compaction against
    the oracle's own chain (the +inf and near-+inf keys are kept)."""
    from tests.gpu_helpers import Run, check_eviction_vs_oracle_chain
    case = _dominant_case("bf16", 4, 8, D=128, Hkv=2)
    lse64, a64 = oracle.lse_a(case, want_a=True)
    lse32, a32 = rounded_window_inputs(case, lse64, a64)
    o32 = oracle.score(case, lse32, oracle.DROP, a32=a32)["drop"].astype(np.float32)
    budget, recent = 60, 4
    ov, on = oracle.select(o32, case["seq_len"], budget, recent)
    f = Run(case, free_prefix=0)
    f.fused("drop", lse32, a32, 1, budget, recent)
    st = f.state()
    new, ofl, ofc, ostats = oracle.compact(case, ov, on, score_row=o32,
                                           free_list=np.full(case["num_blocks"] + 8, -1, np.int32),
                                           free_count=0)
    nd = check_eviction_vs_oracle_chain(case, st, ov, on, new, ofl, ofc, ostats, o32, TOL["bf16"])
    # every dominant key outscores the rest: none is a victim
    for h in range(2):
        vic = set(st["vic"][0, h, :int(st["nv"][0, h])].tolist())
        dom = {1 + (row * 7 + h) % (case["seq_len"][0, h] - 1) for row in range(32) if row % 8}
        assert not (dom & vic), (h, sorted(dom & vic))
    print(f"{nd} heads with victims differing inside the tolerance band", flush=True)


def test_dropkv_low_lse_fills_exact_queue_deterministically():
    """An LSE far below the rows' own (each weight scaled by e^8) puts most
    keys at p >= 1/4, more than the four exact terms per row the score kernel
    queues.  Not a parity
    case (the method's weights no longer sum to 1): the scores are NaN-free
    and two runs agree bit for bit (the workgroups that overflow score every
    pair by the expansion)."""
    r = np.random.default_rng(3)
    k = r.normal(0, 1, (1, 2, 300, 128))
    v = r.normal(0, 1, (1, 2, 300, 128))
    q = r.normal(0, 1, (1, 8, 8, 128))
    case = manual_case(k, v, q, np.full((1, 8), 299, np.int32), dtype="bf16", scale=128 ** -0.5)
    lse64, a64 = oracle.lse_a(case, want_a=True)
    lse32, a32 = rounded_window_inputs(case, lse64 - 8.0, a64)
    d1, s1 = _gpu_drop(case, lse32, a32)
    d2, s2 = _gpu_drop(case, lse32, a32)
    for h, n in enumerate(case["seq_len"][0]):
        assert not np.isnan(d1[0, h, :n]).any()
        assert np.array_equal(d1[0, h, :n], d2[0, h, :n])
        assert np.array_equal(s1[0, h, :n], s2[0, h, :n])
