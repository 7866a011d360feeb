"""Plain CPU reference of attention-score KV-cache eviction (ctypes wrapper).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``kv_cache_eviction_qk_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (scalar loops, double precision); this
file only marshals numpy arrays.  Build: ``gcc -O2 -shared`` into
``liboracle.so`` next to the source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")

SUM, POOL, DROP, ACCUMULATE = 1, 2, 4, 8


def build(force: bool = False) -> str:
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp"
        # -ffp-contract=off keeps every product and sum a separate double rounding
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class Cache(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32), ("is_bf16", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("seq_len", ctypes.c_void_p),
                ("pos", ctypes.c_void_p)]


class Window(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("obs_window", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("q_pos", ctypes.c_void_p), ("scale", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        L.orc_lse_a.argtypes = [P, P, P, P, P, ctypes.c_int]
        L.orc_score.argtypes = [P, P, ctypes.c_int, ctypes.c_int, P, P, P, P, P, ctypes.c_int]
        L.orc_select.argtypes = [P, P, i32, i32, i32, i32, P, P]
        L.orc_compact.argtypes = [P, P, i32, i32, P, P, P, P, i32, i32, P, P, P, P, i32, P]
        L.orc_measure.argtypes = [P, P, P, i32, i32, P]
        L.orc_h2o_step.argtypes = [P, P, i32, i32, P, P, P, P, i32, i32, i32, i32, i32, P, P, P,
                                   P, ctypes.c_double, i32, i32, P, P, P, P, P]
        L.orc_vtok_evict.argtypes = [P, P, P, P, i32, i32, P, P, P]
        L.orc_fmix64.argtypes = [ctypes.c_uint64]
        L.orc_select_shared.argtypes = [P, P, P, i32, i32, i32, i32, i32, P, P]
        L.orc_select_budgets.argtypes = [P, P, i32, i32, P, P, P, P]
        L.orc_vtok_sync.argtypes = [P, P, P, P, P, i32, i32, i32, i32, P, P, P]
        L.orc_vtok_slot_mapping.argtypes = [P, P, P, P, i32, i32, i32, P, P, P]
        L.orc_ring_step.argtypes = [P, P, i32, i32, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                    P, P, P, P, P, ctypes.c_double, i32, i32, i32, i32, P, P, P]
        L.orc_fmix64.restype = ctypes.c_uint64
        L.orc_vtok_digest.argtypes = [P, P, i32, P, P, P, P, i32, i32, i32, P]
        L.orc_vtok_check.argtypes = [P, P, P, i32, i32, i32, P, i32, P]
        L.orc_vtok_reclaim.argtypes = [P, P, i32, i32, P, P, P, P, P, P, i32, i32, i32,
                                       ctypes.c_double, i32, P, P, i32, P]
        for f in (L.orc_lse_a, L.orc_score, L.orc_select, L.orc_compact, L.orc_measure,
                  L.orc_h2o_step, L.orc_vtok_evict, L.orc_vtok_reclaim, L.orc_vtok_digest,
                  L.orc_vtok_check, L.orc_select_shared, L.orc_select_budgets,
                  L.orc_ring_step, L.orc_vtok_sync, L.orc_vtok_slot_mapping):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def default_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _cache(case: dict) -> Cache:
    return Cache(case["B"], case["Hkv"], case["D"], case["max_blocks"], case["num_blocks"],
                 1 if case["dtype"] == "bf16" else 0, _p(case["k_pool"]), _p(case["v_pool"]),
                 _p(case["block_table"]), _p(case["seq_len"]), _p(case["pos"]))


def _window(case: dict, lse=None, a=None) -> Window:
    # the softmax scale as the library receives it (fp32); `a` as fp32
    if a is not None:
        assert a.dtype == np.float32, "the window output a is fp32"
    return Window(case["G"], case["W"], _p(case["q"]), _p(lse), _p(a), _p(case["q_pos"]),
                  float(np.float32(case["scale"])))


def _mask(case: dict, units) -> Optional[np.ndarray]:
    if units is None:
        return None
    m = np.zeros(case["B"] * case["Hkv"], np.uint8)
    m[np.asarray(units, dtype=np.int64)] = 1
    return m


def lse_a(case: dict, want_a: bool = False, units=None, nthreads: int = 0):
    """LSE [B,Hq,W] and attention output [B,Hq,W,D] of the window queries, in double."""
    B, Hq, W, D = case["B"], case["Hkv"] * case["G"], case["W"], case["D"]
    lse = np.zeros((B, Hq, W), np.float64)
    a = np.zeros((B, Hq, W, D), np.float64) if want_a else None
    c, w = _cache(case), _window(case)
    rc = lib().orc_lse_a(ctypes.byref(c), ctypes.byref(w), _p(lse), _p(a), _p(_mask(case, units)),
                         nthreads or default_threads())
    assert rc == 0, rc
    return lse, a


def score(case: dict, lse32: np.ndarray, flags: int, pool_kernel: int = 1, a32=None,
          prev_sum: Optional[np.ndarray] = None, units=None, nthreads: int = 0):
    """Scores in double: dict with 'sum', 'pooled', 'drop' arrays [B,Hkv,max_slots]
    (slots >= seq_len are NaN).  Returns None for the kinds not requested."""
    B, Hkv, ms = case["B"], case["Hkv"], case["max_blocks"] * 16
    shape = (B, Hkv, ms)
    # the SUM buffer is needed internally for POOL too; only returned if asked
    s = np.full(shape, np.nan) if flags & SUM else None
    pl = np.full(shape, np.nan) if flags & POOL else None
    dr = np.full(shape, np.nan) if flags & DROP else None
    lse32 = np.ascontiguousarray(lse32, dtype=np.float32)
    prev = None if prev_sum is None else np.ascontiguousarray(prev_sum, dtype=np.float32)
    c, w = _cache(case), _window(case, lse32, a32)
    rc = lib().orc_score(ctypes.byref(c), ctypes.byref(w), flags, pool_kernel, _p(prev), _p(s),
                         _p(pl), _p(dr), _p(_mask(case, units)), nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle score refused the arguments (rc={rc})")
    return {"sum": s, "pooled": pl, "drop": dr}


def select(scores32: np.ndarray, seq_len: np.ndarray, budget: int, recent: int):
    """Victims [U, max_slots] (first n_victims valid) and n_victims [U] from fp32 scores."""
    scores32 = np.ascontiguousarray(scores32, dtype=np.float32)
    U = int(np.prod(seq_len.shape))
    ms = scores32.size // U
    seq = np.ascontiguousarray(seq_len, dtype=np.int32).reshape(-1)
    vic = np.full((U, ms), -1, np.int32)
    nv = np.zeros(U, np.int32)
    rc = lib().orc_select(_p(scores32), _p(seq), U, ms, budget, recent, _p(vic), _p(nv))
    if rc != 0:
        raise ValueError(f"oracle select refused the arguments (rc={rc})")
    return vic, nv


def compact(case: dict, victims: np.ndarray, n_victims: np.ndarray,
            score_row: Optional[np.ndarray] = None, free_list: Optional[np.ndarray] = None,
            free_count: int = 0):
    """Compacts a COPY of the case's cache.  Returns (new_case, free_list, free_count, stats)."""
    new = dict(case)
    for k in ("k_pool", "v_pool", "block_table", "seq_len", "pos"):
        new[k] = case[k].copy()
    U = case["B"] * case["Hkv"]
    if free_list is None:
        free_list = np.full(case["num_blocks"], -1, np.int32)
    free_list = free_list.copy()
    fc = np.array([free_count], np.int32)
    stats = np.zeros(5, np.int64)
    sc = None if score_row is None else np.ascontiguousarray(score_row, dtype=np.float32).copy()
    elem = 2 if case["dtype"] == "bf16" else 4
    rc = lib().orc_compact(_p(new["k_pool"]), _p(new["v_pool"]), elem, case["D"],
                           _p(new["block_table"]), _p(new["seq_len"]), _p(new["pos"]), _p(sc), U,
                           case["max_blocks"], _p(np.ascontiguousarray(victims, dtype=np.int32)),
                           _p(np.ascontiguousarray(n_victims, dtype=np.int32)), _p(free_list),
                           _p(fc), free_list.size, _p(stats))
    if rc != 0:
        raise ValueError(f"oracle compact refused the arguments (rc={rc})")
    if sc is not None:
        new["score_row"] = sc
    return new, free_list, int(fc[0]), stats


def measure(seq_len_before: np.ndarray, victims: np.ndarray, n_victims: np.ndarray) -> dict:
    U = int(np.prod(seq_len_before.shape))
    ms = victims.size // U
    out = np.zeros(8, np.float64)
    rc = lib().orc_measure(_p(np.ascontiguousarray(seq_len_before, dtype=np.int32).reshape(-1)),
                           _p(np.ascontiguousarray(victims, dtype=np.int32)),
                           _p(np.ascontiguousarray(n_victims, dtype=np.int32)), U, ms, _p(out))
    assert rc == 0
    keys = ("F_naive", "F_after", "frac_le_half_naive", "frac_le_half_after", "blocks_naive",
            "blocks_after", "live_tokens", "blocks_freed")
    return dict(zip(keys, out.tolist()))


def h2o_step(state: dict, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             t_pos: np.ndarray, budget: int, recent: int, free_list: Optional[np.ndarray] = None,
             free_count: int = 0, want_attn: bool = False):
    """One H2O decode step on a COPY of `state` (a case dict plus 'score', the
    running fp32 score [B,Hkv,max_slots]).  q [B,Hq,D], k_new / v_new
    [B,Hkv,D] in the cache dtype, t_pos [B].  Returns (new_state, evicted_pos
    [B,Hkv], free_list, free_count), plus, with want_attn, the attention
    output [B,Hq,D] and its sum_j p_j |v_j| [B,Hq,D] (double; NaN for heads
    that were refused)."""
    new = dict(state)
    for k in ("k_pool", "v_pool", "block_table", "seq_len", "pos"):
        new[k] = state[k].copy()
    new["score"] = np.ascontiguousarray(state["score"], dtype=np.float32).copy()
    B, Hkv = state["B"], state["Hkv"]
    if free_list is None:
        free_list = np.full(max(1, state["num_blocks"]), -1, np.int32)
    free_list = np.ascontiguousarray(free_list, dtype=np.int32).copy()
    fc = np.array([free_count], np.int32)
    ev = np.zeros((B, Hkv), np.int32)
    edt = np.uint16 if state["dtype"] == "bf16" else np.float32
    attn = np.full((B, Hkv * state["G"], state["D"]), np.nan) if want_attn else None
    aabs = np.full((B, Hkv * state["G"], state["D"]), np.nan) if want_attn else None
    rc = lib().orc_h2o_step(_p(new["k_pool"]), _p(new["v_pool"]),
                            1 if state["dtype"] == "bf16" else 0, state["D"],
                            _p(new["block_table"]), _p(new["seq_len"]), _p(new["pos"]),
                            _p(new["score"]), B, Hkv, state["max_blocks"], state["num_blocks"],
                            state["G"], _p(np.ascontiguousarray(q, dtype=edt)),
                            _p(np.ascontiguousarray(k_new, dtype=edt)),
                            _p(np.ascontiguousarray(v_new, dtype=edt)),
                            _p(np.ascontiguousarray(t_pos, dtype=np.int32)), float(np.float32(state["scale"])),
                            budget, recent, _p(free_list), _p(fc), _p(ev), _p(attn), _p(aabs))
    if rc != 0:
        raise ValueError(f"oracle h2o_step refused the arguments (rc={rc})")
    if want_attn:
        return new, ev, free_list, int(fc[0]), attn, aabs
    return new, ev, free_list, int(fc[0])


def vtok_liveness(state: dict):
    """The vToken liveness view of a dense state: every slot below seq_len is
    live.  Returns (live uint8 [B,Hkv,max_slots], block_live int32
    [B,Hkv,max_blocks])."""
    B, Hkv, mb = state["B"], state["Hkv"], state["max_blocks"]
    live = np.zeros((B, Hkv, mb * 16), np.uint8)
    for b in range(B):
        for h in range(Hkv):
            live[b, h, :int(state["seq_len"][b, h])] = 1
    block_live = live.reshape(B, Hkv, mb, 16).sum(axis=-1).astype(np.int32)
    return live, block_live


def vtok_evict(state: dict, victims: np.ndarray, n_victims: np.ndarray):
    """Marks victim slots dead on a COPY of state's 'live' / 'block_live'.
    Returns (new_state, status)."""
    new = dict(state)
    new["live"] = state["live"].copy()
    new["block_live"] = state["block_live"].copy()
    U = state["B"] * state["Hkv"]
    st = np.zeros(1, np.int32)
    rc = lib().orc_vtok_evict(_p(np.ascontiguousarray(state["block_table"], dtype=np.int32)),
                              _p(np.ascontiguousarray(state["seq_len"], dtype=np.int32)),
                              _p(new["live"]), _p(new["block_live"]), U, state["max_blocks"],
                              _p(np.ascontiguousarray(victims, dtype=np.int32)),
                              _p(np.ascontiguousarray(n_victims, dtype=np.int32)), _p(st))
    assert rc == 0
    return new, int(st[0])


def vtok_reclaim(state: dict, theta_f: float, max_sources: int, free_list: np.ndarray,
                 free_count: int, with_score: bool = False):
    """Lazy reclamation on a COPY of state (pools, block_table, pos, live,
    block_live and, with with_score, 'score').  Returns (new_state,
    free_list, free_count, stats[10])."""
    new = dict(state)
    for k in ("k_pool", "v_pool", "block_table", "pos", "live", "block_live"):
        new[k] = state[k].copy()
    sc = None
    if with_score:
        sc = new["score"] = np.ascontiguousarray(state["score"], dtype=np.float32).copy()
    fl = np.ascontiguousarray(free_list, dtype=np.int32).copy()
    fc = np.array([free_count], np.int32)
    stats = np.zeros(10, np.int64)
    U = state["B"] * state["Hkv"]
    elem = 2 if state["dtype"] == "bf16" else 4
    rc = lib().orc_vtok_reclaim(_p(new["k_pool"]), _p(new["v_pool"]), elem, state["D"],
                                _p(new["block_table"]),
                                _p(np.ascontiguousarray(state["seq_len"], dtype=np.int32)),
                                _p(new["pos"]), _p(sc), _p(new["live"]), _p(new["block_live"]), U,
                                state["max_blocks"], state["num_blocks"], float(theta_f),
                                max_sources, _p(fl), _p(fc), fl.size, _p(stats))
    if rc != 0:
        raise ValueError(f"oracle vtok_reclaim refused the arguments (rc={rc})")
    return new, fl, int(fc[0]), stats



def fmix64(k: int) -> int:
    """MurmurHash3's 64-bit finalizer, as the oracle's C code computes it."""
    return int(lib().orc_fmix64(k & 0xFFFFFFFFFFFFFFFF))


def vtok_digest(state: dict) -> np.ndarray:
    """Per-head order-independent digest of the live tokens (I1's online
    check): uint64 [B, Hkv]."""
    U = state["B"] * state["Hkv"]
    out = np.zeros((state["B"], state["Hkv"]), np.uint64)
    row_bytes = state["D"] * (2 if state["dtype"] == "bf16" else 4)
    rc = lib().orc_vtok_digest(_p(np.ascontiguousarray(state["k_pool"])),
                               _p(np.ascontiguousarray(state["v_pool"])), row_bytes,
                               _p(np.ascontiguousarray(state["block_table"], dtype=np.int32)),
                               _p(np.ascontiguousarray(state["seq_len"], dtype=np.int32)),
                               _p(np.ascontiguousarray(state["pos"], dtype=np.int32)),
                               _p(np.ascontiguousarray(state["live"], dtype=np.uint8)), U,
                               state["max_blocks"], state["num_blocks"], _p(out))
    assert rc == 0
    return out


def vtok_check(state: dict, free_list: np.ndarray, free_count: int) -> np.ndarray:
    """I2's online check: int64 [4] = {blocks held more than once, blocks held
    by nobody, references out of range, live-count mismatches}."""
    out = np.zeros(4, np.int64)
    rc = lib().orc_vtok_check(_p(np.ascontiguousarray(state["block_table"], dtype=np.int32)),
                              _p(np.ascontiguousarray(state["live"], dtype=np.uint8)),
                              _p(np.ascontiguousarray(state["block_live"], dtype=np.int32)),
                              state["B"] * state["Hkv"], state["max_blocks"], state["num_blocks"],
                              _p(np.ascontiguousarray(free_list, dtype=np.int32)), int(free_count),
                              _p(out))
    assert rc == 0
    return out


def select_shared(scores32: np.ndarray, seq_len: np.ndarray, pos: np.ndarray, budget: int,
                  recent: int):
    """Victims [B, Hkv, max_slots] and n_victims [B, Hkv] of the selection on
    each sequence's scores summed over its KV heads (fp32, heads ascending)."""
    scores32 = np.ascontiguousarray(scores32, dtype=np.float32)
    B, Hkv = seq_len.shape
    ms = scores32.size // (B * Hkv)
    vic = np.full((B, Hkv, ms), -1, np.int32)
    nv = np.zeros((B, Hkv), np.int32)
    rc = lib().orc_select_shared(_p(scores32), _p(np.ascontiguousarray(seq_len, dtype=np.int32)),
                                 _p(np.ascontiguousarray(pos, dtype=np.int32)), B, Hkv, ms,
                                 budget, recent, _p(vic), _p(nv))
    if rc != 0:
        raise ValueError(f"oracle select_shared refused the arguments (rc={rc})")
    return vic, nv


def select_budgets(scores32: np.ndarray, seq_len: np.ndarray, budget: np.ndarray,
                   recent: np.ndarray):
    """Victims [U, max_slots] and n_victims [U] with a (budget, recent) pair
    per unit."""
    scores32 = np.ascontiguousarray(scores32, dtype=np.float32)
    U = int(np.prod(seq_len.shape))
    ms = scores32.size // U
    vic = np.full((U, ms), -1, np.int32)
    nv = np.zeros(U, np.int32)
    rc = lib().orc_select_budgets(_p(scores32), _p(np.ascontiguousarray(seq_len, dtype=np.int32)),
                                  U, ms, _p(np.ascontiguousarray(budget, dtype=np.int32)),
                                  _p(np.ascontiguousarray(recent, dtype=np.int32)), _p(vic), _p(nv))
    assert rc == 0
    return vic, nv


def ring_state(state: dict, obs_window: int):
    """Adds the ring-buffer adaptation's state to a COPY of a stream state:
    hist fp32 [B,Hkv,obs_window,max_slots] (zeros), ring int32 [B,Hkv] (0)
    and rank int32 [B,Hkv,max_slots] (each slot's index in position order)."""
    new = dict(state)
    B, Hkv, mb = state["B"], state["Hkv"], state["max_blocks"]
    new["hist"] = np.zeros((B, Hkv, obs_window, mb * 16), np.float32)
    new["ring"] = np.zeros((B, Hkv), np.int32)
    rank = np.zeros((B, Hkv, mb * 16), np.int32)
    for b in range(B):
        for h in range(Hkv):
            n = int(state["seq_len"][b, h])
            p = state["pos"][b, h, :n]
            rank[b, h, :n] = np.argsort(np.argsort(p, kind="stable"), kind="stable")
    new["rank"] = rank
    return new


def ring_step(state: dict, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
              t_pos: np.ndarray, observe: np.ndarray, budget: int, recent: int,
              pool_kernel: int, free_list: Optional[np.ndarray] = None, free_count: int = 0):
    """One decode step of the SnapKV ring-buffer adaptation on a COPY of a
    ring state (see ring_state).  Returns (new_state, evicted_pos [B,Hkv],
    free_list, free_count)."""
    new = dict(state)
    for k in ("k_pool", "v_pool", "block_table", "seq_len", "pos", "hist", "ring", "rank"):
        new[k] = np.ascontiguousarray(state[k]).copy()
    B, Hkv = state["B"], state["Hkv"]
    W = state["hist"].shape[2]
    is_bf16 = 1 if state["dtype"] == "bf16" else 0
    if free_list is None:
        free_list = np.full(state["num_blocks"], -1, np.int32)
    fl = np.ascontiguousarray(free_list, dtype=np.int32).copy()
    fc = np.array([free_count], np.int32)
    ev = np.zeros((B, Hkv), np.int32)
    rc = lib().orc_ring_step(_p(new["k_pool"]), _p(new["v_pool"]), is_bf16, state["D"],
                             _p(new["block_table"]), _p(new["seq_len"]), _p(new["pos"]),
                             _p(new["hist"]), _p(new["ring"]), _p(new["rank"]), B, Hkv,
                             state["max_blocks"], state["num_blocks"], state["G"],
                             _p(np.ascontiguousarray(q)), _p(np.ascontiguousarray(k_new)),
                             _p(np.ascontiguousarray(v_new)),
                             _p(np.ascontiguousarray(t_pos, dtype=np.int32)),
                             _p(np.ascontiguousarray(observe, dtype=np.int32)),
                             float(np.float32(state["scale"])), budget, recent, W, pool_kernel, _p(fl),
                             _p(fc), _p(ev))
    if rc != 0:
        raise ValueError(f"oracle ring_step refused the arguments (rc={rc})")
    return new, ev, fl, int(fc[0])


def vtok_sync(state: dict, new_len: np.ndarray, pos0: np.ndarray):
    """sync_new_tokens on a COPY of a vToken state: slots [seq_len, new_len)
    become live at positions pos0[b] + k.  Returns (new_state, status [B,Hkv])."""
    new = dict(state)
    for k in ("seq_len", "pos", "live", "block_live"):
        new[k] = np.ascontiguousarray(state[k]).copy()
    B, Hkv = state["B"], state["Hkv"]
    stat = np.zeros((B, Hkv), np.int32)
    rc = lib().orc_vtok_sync(_p(np.ascontiguousarray(state["block_table"], dtype=np.int32)),
                             _p(new["seq_len"]), _p(new["pos"]), _p(new["live"]),
                             _p(new["block_live"]), B, Hkv, state["max_blocks"],
                             state["num_blocks"], _p(np.ascontiguousarray(new_len, dtype=np.int32)),
                             _p(np.ascontiguousarray(pos0, dtype=np.int32)), _p(stat))
    assert rc == 0
    return new, stat


def vtok_slot_mapping(state: dict):
    """Eq. 2 for every live token, in logical order: (slots [B,Hkv,max_slots],
    positions [B,Hkv,max_slots], count [B,Hkv])."""
    B, Hkv, mb = state["B"], state["Hkv"], state["max_blocks"]
    slots = np.full((B, Hkv, mb * 16), -1, np.int32)
    positions = np.full((B, Hkv, mb * 16), -1, np.int32)
    count = np.zeros((B, Hkv), np.int32)
    rc = lib().orc_vtok_slot_mapping(_p(np.ascontiguousarray(state["block_table"], dtype=np.int32)),
                                     _p(np.ascontiguousarray(state["seq_len"], dtype=np.int32)),
                                     _p(np.ascontiguousarray(state["pos"], dtype=np.int32)),
                                     _p(np.ascontiguousarray(state["live"], dtype=np.uint8)),
                                     B * Hkv, mb, state["num_blocks"], _p(slots), _p(positions),
                                     _p(count))
    assert rc == 0
    return slots, positions, count
