"""Moving seeded host cases to the GPU and back, and the comparison rules.
Test-only code."""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth

FLT_MIN = np.finfo(np.float32).tiny
TOL = {"f32": 1e-5, "bf16": 2e-3}
# score kind -> (library flag, oracle flag, oracle result key)
KIND = {"sum": (K.SUM, oracle.SUM, "sum"), "pool": (K.POOL, oracle.POOL, "pooled"),
        "drop": (K.DROP, oracle.DROP, "drop")}


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


def order_key(scores32: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 key of fp32 values (-0 == +0, NaN above +inf),
    for the brute-force selection checks."""
    u = np.ascontiguousarray(scores32, dtype=np.float32).view(np.uint32).copy()
    u[u == 0x80000000] = 0
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
    key[nan] = 0xFFFFFFFF
    return key


def brute_force_victims(scores32: np.ndarray, n: int, budget: int, recent: int) -> np.ndarray:
    """The m = max(0, n - budget) smallest (score, slot) pairs among the
    candidate slots [0, n - recent), in ascending slot order: a full sort."""
    m = max(0, n - budget)
    nc = max(0, n - recent)
    key = order_key(scores32[:nc])
    order = np.lexsort((np.arange(nc), key))  # key first, then slot
    return np.sort(order[:m]).astype(np.int32)


def phys_rows(block_table_row: np.ndarray, slots: np.ndarray) -> np.ndarray:
    return block_table_row[slots // 16].astype(np.int64) * 16 + slots % 16


def _close(g: np.ndarray, o: np.ndarray, tol: float) -> bool:
    g = g.astype(np.float64)
    o = o.astype(np.float64)
    inf = np.isinf(o)
    if not np.array_equal(np.isinf(g), inf) or not np.array_equal(g[inf], o[inf]):
        return False
    return bool(np.all(np.abs(g[~inf] - o[~inf]) <= tol * np.maximum(np.abs(o[~inf]), FLT_MIN)))


def check_compaction_by_definition(case, st, u, victims, kept_scores=None, tol=0.0):
    """Head u after compaction, against the definition on the given victims:
    row r (K, V, pos, and the score row if kept_scores is given) holds the
    r-th kept token of the cache before the call.  Returns (moved, at_risk)."""
    B, H, D = case["B"], case["Hkv"], case["D"]
    b, h = divmod(u, H)
    n = int(case["seq_len"].reshape(-1)[u])
    keep = np.ones(n, bool)
    keep[victims] = False
    kept = np.flatnonzero(keep)
    n2 = kept.size
    assert int(st["seq"][b, h]) == n2, u
    r = np.arange(n2)
    src = phys_rows(case["block_table"][b, h], kept)
    dst = phys_rows(st["bt"][b, h], r)
    assert np.array_equal(st["pos"][b, h, :n2], case["pos"][b, h, kept]), u
    assert np.array_equal(st["k"].reshape(-1, D)[dst], case["k_pool"].reshape(-1, D)[src]), u
    assert np.array_equal(st["v"].reshape(-1, D)[dst], case["v_pool"].reshape(-1, D)[src]), u
    if kept_scores is not None:
        assert _close(st["score"][b, h, :n2], kept_scores[kept], tol), u
    return int(np.count_nonzero(kept != r)), int(np.count_nonzero((kept != r) & (kept < n2)))


def check_eviction_vs_oracle_chain(case, st, ov, on, o_new, ofl, ofc, ostats, orc32, tol,
                                   units=None):
    """A GPU eviction result `st` (after select + compact) against the
    oracle's own chain: oracle victims `ov`/`on` from the oracle's scores
    `orc32`, then the oracle's compaction of them (`o_new`, `ofl`, `ofc`,
    `ostats`).

    Per head (all heads, or `units`): the victim sets are equal, or differ only
    where the oracle score lies within `tol` of the oracle's cutoff.  Equal
    sets: the compacted rows, pos and score row equal the oracle's.  Sets that
    differ inside the band: the GPU's compaction is checked against the
    definition on its own victims.  The block table, free list, seq_len and
    blocks freed depend only on the victim counts and equal the oracle's
    everywhere.  Returns the number of heads whose victim sets differ."""
    B, H, D = case["B"], case["Hkv"], case["D"]
    U = B * H
    ms = case["max_blocks"] * 16
    all_units = units is None
    units = range(U) if units is None else units
    gv = st["vic"].reshape(U, ms)
    gn = st["nv"].reshape(-1)
    ov = ov.reshape(U, ms)
    on = on.reshape(-1)
    sc = orc32.reshape(U, ms)
    seq0 = case["seq_len"].reshape(-1)
    kg, vg = st["k"].reshape(-1, D), st["v"].reshape(-1, D)
    ko, vo = o_new["k_pool"].reshape(-1, D), o_new["v_pool"].reshape(-1, D)
    with_score = "score_row" in o_new and st.get("score") is not None
    assert np.array_equal(gn, on), "victim counts"
    assert np.array_equal(st["seq"], o_new["seq_len"])
    assert np.array_equal(st["bt"], o_new["block_table"])
    assert st["fc"] == ofc and np.array_equal(st["fl"][:ofc], ofl[:ofc])
    assert st["stats"][0] == ostats[0] and st["stats"][4] == ostats[4]
    differ = moved = at_risk = 0
    for u in units:
        b, h = divmod(u, H)
        n, m = int(seq0[u]), int(on[u])
        if not 0 <= n <= ms:
            continue
        n2 = n - m
        gset = gv[u, :m]
        if np.array_equal(gset, ov[u, :m]):
            r = np.arange(n2)
            dst = phys_rows(st["bt"][b, h], r)
            assert np.array_equal(st["pos"][b, h, :n2], o_new["pos"][b, h, :n2]), u
            assert np.array_equal(kg[dst], ko[dst]), u
            assert np.array_equal(vg[dst], vo[dst]), u
            if with_score:
                assert _close(st["score"][b, h, :n2], o_new["score_row"][b, h, :n2], tol), u
            keep = np.ones(n, bool)
            keep[gset] = False
            kept = np.flatnonzero(keep)
            moved += int(np.count_nonzero(kept != r))
            at_risk += int(np.count_nonzero((kept != r) & (kept < n2)))
            continue
        differ += 1
        cut = float(np.max(sc[u, ov[u, :m]]))
        for s in np.setxor1d(gset, ov[u, :m]):
            o = float(sc[u, s])
            assert abs(o - cut) <= tol * abs(cut) + 1e-30, (u, int(s), o, cut)
        mv, ar = check_compaction_by_definition(case, st, u, gset,
                                                sc[u] if with_score else None, tol)
        moved += mv
        at_risk += ar
    if all_units:
        row_bytes = D * (2 if case["dtype"] == "bf16" else 4)
        assert st["stats"][1] == moved and st["stats"][3] == at_risk
        assert st["stats"][2] == moved * 4 * row_bytes
        if differ == 0:
            assert np.array_equal(st["stats"], ostats)
    return differ


class Run:
    """One device copy of the case plus every buffer an eviction step touches."""

    def __init__(self, case, prev=None, free_prefix=3):
        self.case = case
        self.dc = device_cache(case)
        self.q, self.qp = device_window(case)
        B, H, ms = case["B"], case["Hkv"], case["max_blocks"] * 16
        self.ws = K.new_workspace(self.dc, case["G"], case["W"])
        free0 = np.full(case["num_blocks"] + 8, -1, np.int32)
        free0[:free_prefix] = np.arange(free_prefix) + 10**6
        self.fl = dev(free0)
        self.fc = dev(np.array([free_prefix], np.int32))
        self.score = dev(prev.copy()) if prev is not None else dev(np.zeros((B, H, ms), np.float32))
        self.vic = dev(np.full((B, H, ms), -1, np.int32))
        self.nv = dev(np.zeros((B, H), np.int32))
        self.stats = None

    def fused(self, kind, lse32, a32, pool, budget, recent, accumulate=False):
        flags = KIND[kind][0] | (K.ACCUMULATE if accumulate else 0)
        self.stats = K.evict(self.dc, self.q, dev(lse32), self.qp, self.case["scale"],
                             self.case["G"], flags, budget, recent, self.score, self.vic, self.nv,
                             self.fl, self.fc, self.ws, pool_kernel=pool,
                             a=dev(a32) if a32 is not None else None)
        torch.cuda.synchronize()

    def three_calls(self, kind, lse32, a32, pool, budget, recent, accumulate=False):
        flags = KIND[kind][0] | (K.ACCUMULATE if accumulate else 0)
        kw = {KIND[kind][2]: self.score}
        K.score(self.dc, self.q, dev(lse32), self.qp, self.case["scale"], self.case["G"], flags,
                pool, a=dev(a32) if a32 is not None else None, **kw)
        K.select(self.dc, self.score, budget, recent, self.vic, self.nv, self.ws)
        self.stats = K.compact(self.dc, self.vic, self.nv, self.fl, self.fc, self.ws,
                               score_row=self.score)
        torch.cuda.synchronize()

    def state(self):
        return dict(k=host(self.dc.k_pool), v=host(self.dc.v_pool), bt=host(self.dc.block_table),
                    seq=host(self.dc.seq_len), pos=host(self.dc.pos), fl=host(self.fl),
                    fc=int(host(self.fc)[0]), stats=host(self.stats), score=host(self.score),
                    vic=host(self.vic), nv=host(self.nv))
