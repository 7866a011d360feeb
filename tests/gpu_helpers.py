"""Moving seeded host cases to the GPU and back, and the comparison rules.
Test-only code."""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_eviction_qk_amd as K
import synth

FLT_MIN = np.finfo(np.float32).tiny
TOL = {"f32": 1e-5, "bf16": 2e-3}


def dev(arr: np.ndarray, dtype: str = "") -> torch.Tensor:
    """Host array -> GPU tensor; uint16 arrays are bf16 bit patterns."""
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def device_cache(case: dict) -> K.Cache:
    return K.Cache(dev(case["k_pool"]), dev(case["v_pool"]), dev(case["block_table"]),
                   dev(case["seq_len"]), dev(case["pos"]))


def device_window(case: dict):
    return dev(case["q"]), dev(case["q_pos"])


def assert_scores_close(gpu: np.ndarray, orc: np.ndarray, seq_len: np.ndarray, tol: float,
                        what: str = ""):
    """|g - o| <= tol * max(|o|, FLT_MIN) on the live slots; infinities must match."""
    B, H = seq_len.shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            n = int(seq_len[b, h])
            g = gpu[b, h, :n].astype(np.float64)
            o = orc[b, h, :n]
            inf = np.isinf(o)
            assert np.array_equal(np.isinf(g), inf), f"{what} ({b},{h}): infinities differ"
            assert np.array_equal(g[inf], o[inf]), f"{what} ({b},{h}): infinity signs differ"
            fin = ~inf
            err = np.abs(g[fin] - o[fin])
            bound = tol * np.maximum(np.abs(o[fin]), FLT_MIN)
            bad = np.flatnonzero(err > bound)
            assert bad.size == 0, (f"{what} ({b},{h}): {bad.size} slots off, first slot "
                                   f"{np.flatnonzero(fin)[bad[0]]}: gpu {g[fin][bad[0]]!r} "
                                   f"oracle {o[fin][bad[0]]!r}")
            if fin.any():
                worst = max(worst, float((err / np.maximum(np.abs(o[fin]), FLT_MIN)).max()))
    return worst


def victims_agree_up_to_tolerance(gv, gn, ov, on, orc_scores32, seq_len, budget, recent, tol):
    """End-to-end rule: counts equal; a slot may be in one set and not the
    other only if its oracle score lies within tol of the oracle's cutoff."""
    U = seq_len.size
    gv = gv.reshape(U, -1); ov = ov.reshape(U, -1)
    sc = orc_scores32.reshape(U, -1)
    n_diff = 0
    for u in range(U):
        assert gn.reshape(-1)[u] == on.reshape(-1)[u]
        m = int(on.reshape(-1)[u])
        a = set(gv[u, :m].tolist()); b = set(ov[u, :m].tolist())
        if a == b:
            continue
        if m == 0:
            continue
        cut = float(np.max(sc[u, ov[u, :m]]))
        for s in a ^ b:
            assert abs(float(sc[u, s]) - cut) <= tol * abs(cut) + 1e-30, (u, s, sc[u, s], cut)
            n_diff += 1
    return n_diff
