"""The C-ABI boundary on the CPU: the library loads, exports every function
include/kvev.h declares, and refuses bad arguments on the host before any
work is enqueued (no GPU is touched: every call here fails validation)."""
import ctypes
import os
import re

import pytest

import torch

import kv_cache_eviction_qk_amd as K

# These calls pass fake device pointers and rely on host validation refusing
# them; they are run only where no GPU can be reached.
pytestmark = pytest.mark.skipif(torch.cuda.device_count() > 0,
                                reason="fake-pointer validation tests run only without a GPU")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000   # never dereferenced: validation fails first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvev.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(kvev_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function():
    L = K.load_library()
    names = declared_functions()
    assert set(names) == set(K.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    header = open(HEADER).read() if "HEADER" in globals() else open(
        os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                     "kvev.h")).read()
    declared = int(re.search(r"#define KVEV_ABI_VERSION (\d+)", header).group(1))
    assert L.kvev_abi_version() == K.ABI_VERSION == declared
    for code in (0, -1, -2, -3, -4):
        assert K.strerror(code)


def cache(**kw):
    d = dict(batch=2, kv_heads=2, head_dim=128, block_size=16, max_blocks=8, num_blocks=32,
             dtype=K.BF16, k_pool=FAKE, v_pool=FAKE, block_table=FAKE, seq_len=FAKE, pos=FAKE)
    d.update(kw)
    return K.CacheStruct(**d)


def window(**kw):
    d = dict(group=2, obs_window=4, q=FAKE, lse=FAKE, a=FAKE, q_pos=FAKE, scale=0.1)
    d.update(kw)
    return K.WindowStruct(**d)


def score(c, w, flags=K.SUM, pool=1, s=FAKE, p=FAKE, d=FAKE):
    return K.load_library().kvev_score(ctypes.byref(c) if c else None,
                                       ctypes.byref(w) if w else None, flags, pool, s, p, d,
                                       None, 0, None)


def evict(c, w, flags=K.POOL, pool=3, budget=8, recent=2, ptrs=None, cap=1 << 20,
          ws=FAKE, ws_bytes=1 << 40):
    p = dict(score=FAKE, victims=FAKE, n_victims=FAKE, free_list=FAKE, free_count=FAKE,
             stats=FAKE)
    p.update(ptrs or {})
    return K.load_library().kvev_evict(
        ctypes.byref(c) if c else None, ctypes.byref(w) if w else None, flags, pool, budget,
        recent, p["score"], p["victims"], p["n_victims"], p["free_list"], p["free_count"], cap,
        p["stats"], ws, ws_bytes, None)


BAD_CACHES = [dict(head_dim=96), dict(head_dim=256), dict(block_size=32), dict(batch=0),
              dict(kv_heads=0), dict(max_blocks=0), dict(num_blocks=0), dict(dtype=7),
              dict(k_pool=None), dict(v_pool=None), dict(block_table=None), dict(seq_len=None),
              dict(pos=None)]


@pytest.mark.parametrize("kw", BAD_CACHES)
def test_bad_cache_refused_everywhere(kw):
    L = K.load_library()
    c = cache(**kw)
    assert score(c, window()) == K.EINVAL
    assert L.kvev_select(ctypes.byref(c), FAKE, 8, 2, FAKE, FAKE, None, 0, None) == K.EINVAL
    assert L.kvev_compact(ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, 1 << 20, FAKE, FAKE,
                          1 << 40, None) == K.EINVAL
    assert L.kvev_window_attn(ctypes.byref(c), ctypes.byref(window()), FAKE, None, FAKE,
                              1 << 40, None) == K.EINVAL
    assert evict(c, window()) == K.EINVAL
    assert L.kvev_workspace_bytes(ctypes.byref(c), 1, 1) == 0


@pytest.mark.parametrize("wkw,flags,pool,expect", [
    (dict(group=0), K.SUM, 1, K.EINVAL),
    (dict(obs_window=0), K.SUM, 1, K.EINVAL),         # SnapKV: a zero window is refused
    (dict(q=None), K.SUM, 1, K.EINVAL),
    (dict(lse=None), K.SUM, 1, K.EINVAL),
    (dict(q_pos=None), K.SUM, 1, K.EINVAL),
    (dict(scale=float("nan")), K.SUM, 1, K.EINVAL),
    (dict(), 0, 1, K.EINVAL),                          # no score kind
    (dict(), 16, 1, K.EINVAL),                         # unknown flag
    (dict(), K.ACCUMULATE, 1, K.EINVAL),               # accumulate without SUM
    (dict(), K.POOL, 0, K.EINVAL),
    (dict(), K.POOL, 4, K.EINVAL),                     # SnapKV: poolKernel must be odd
    (dict(), K.POOL, -3, K.EINVAL),
    (dict(), K.POOL, 2051, K.EUNSUPPORTED),
    (dict(), K.POOL | K.SUM | K.ACCUMULATE, 3, K.EINVAL),
    (dict(), K.DROP | K.SUM | K.ACCUMULATE, 1, K.EINVAL),
    (dict(a=None), K.DROP, 1, K.EINVAL),
    (dict(group=64, obs_window=65), K.SUM, 1, K.EUNSUPPORTED),
    # 512 DROP rows exceed one workgroup's LDS: split over workgroups, whose
    # raw sums need the workspace (none given here)
    (dict(group=8, obs_window=64), K.DROP, 1, K.ENOSPACE),
])
def test_score_refusals(wkw, flags, pool, expect):
    assert score(cache(), window(**wkw), flags, pool) == expect


def test_score_missing_outputs():
    assert score(cache(), window(), K.SUM, s=None) == K.EINVAL
    assert score(cache(), window(), K.POOL, 3, p=None) == K.EINVAL
    assert score(cache(), window(), K.DROP, d=None) == K.EINVAL
    assert score(None, window()) == K.EINVAL
    assert score(cache(), None) == K.EINVAL


@pytest.mark.parametrize("budget,recent", [(0, 0), (-1, 0), (8, 8), (8, 9), (8, -1)])
def test_select_refusals(budget, recent):
    """recentWindow >= budget is refused; the budget must be positive."""
    L = K.load_library()
    c = cache()
    assert L.kvev_select(ctypes.byref(c), FAKE, budget, recent, FAKE, FAKE, None, 0,
                         None) == K.EINVAL
    assert L.kvev_select(ctypes.byref(c), None, 8, 2, FAKE, FAKE, None, 0, None) == K.EINVAL


def test_select_needs_workspace():
    L = K.load_library()
    c = cache()
    ws = L.kvev_workspace_bytes(ctypes.byref(c), 1, 1)
    assert L.kvev_select(ctypes.byref(c), FAKE, 8, 2, FAKE, FAKE, None, ws, None) == K.ENOSPACE
    assert L.kvev_select(ctypes.byref(c), FAKE, 8, 2, FAKE, FAKE, FAKE, 64, None) == K.ENOSPACE


def test_compact_refusals():
    L = K.load_library()
    c = cache()
    ws = L.kvev_workspace_bytes(ctypes.byref(c), 1, 1)
    assert ws > 0
    args = [FAKE, FAKE, None, FAKE, FAKE, 64, FAKE, FAKE, ws, None]
    for i in (0, 1, 3, 4, 6):
        a = list(args); a[i] = None
        assert L.kvev_compact(ctypes.byref(c), *a) == K.EINVAL
    a = list(args); a[5] = 31              # free list smaller than the pool
    assert L.kvev_compact(ctypes.byref(c), *a) == K.ENOSPACE
    a = list(args); a[8] = ws - 1          # short workspace
    assert L.kvev_compact(ctypes.byref(c), *a) == K.ENOSPACE
    a = list(args); a[7] = None
    assert L.kvev_compact(ctypes.byref(c), *a) == K.ENOSPACE


def test_window_attn_refusals():
    L = K.load_library()
    c = cache()
    w = window()
    ws = L.kvev_workspace_bytes(ctypes.byref(c), 2, 4)
    # a 16-byte workspace is short for any shape (the partials alone need more)
    assert L.kvev_window_attn(ctypes.byref(c), ctypes.byref(w), FAKE, None, FAKE, 16,
                              None) == K.ENOSPACE
    assert L.kvev_window_attn(ctypes.byref(c), ctypes.byref(w), FAKE, None, None, ws,
                              None) == K.ENOSPACE
    assert L.kvev_window_attn(ctypes.byref(c), ctypes.byref(w), None, None, FAKE, ws,
                              None) == K.EINVAL
    w0 = window(obs_window=0)
    assert L.kvev_window_attn(ctypes.byref(c), ctypes.byref(w0), FAKE, None, FAKE, ws,
                              None) == K.EINVAL


def test_workspace_grows_with_the_cache():
    L = K.load_library()
    small = L.kvev_workspace_bytes(ctypes.byref(cache(max_blocks=8)), 1, 1)
    big = L.kvev_workspace_bytes(ctypes.byref(cache(max_blocks=64)), 1, 1)
    assert big > small
    # the staged at-risk rows may cover every slot of every head
    assert small >= 2 * 2 * 8 * 16 * 128 * 2 * 2
    assert big >= 2 * 2 * 64 * 16 * 128 * 2 * 2


def test_binding_has_no_cpu_path():
    """The binding only marshals: CPU tensors are refused, nothing is computed."""
    c = K.Cache(torch.zeros(4, 16, 64), torch.zeros(4, 16, 64),
                torch.zeros(1, 1, 4, dtype=torch.int32), torch.zeros(1, 1, dtype=torch.int32),
                torch.zeros(1, 1, 64, dtype=torch.int32))
    with pytest.raises(ValueError):
        c.struct()


@pytest.mark.parametrize("flags", [0, K.SUM | K.POOL, K.POOL | K.DROP, K.SUM | K.DROP,
                                   K.ACCUMULATE, K.POOL | K.ACCUMULATE, 16])
def test_evict_needs_one_score_kind(flags):
    assert evict(cache(), window(), flags=flags) == K.EINVAL


@pytest.mark.parametrize("budget,recent", [(0, 0), (-1, 0), (8, 8), (8, 9), (8, -1)])
def test_evict_budget_refusals(budget, recent):
    assert evict(cache(), window(), budget=budget, recent=recent) == K.EINVAL


@pytest.mark.parametrize("name", ["score", "victims", "n_victims", "free_list", "free_count",
                                  "stats"])
def test_evict_null_pointers(name):
    assert evict(cache(), window(), ptrs={name: None}) == K.EINVAL


def test_evict_refusals_of_the_parts():
    L = K.load_library()
    c = cache()
    ws = L.kvev_workspace_bytes(ctypes.byref(c), 1, 1)
    assert evict(None, window()) == K.EINVAL
    assert evict(c, None) == K.EINVAL
    assert evict(c, window(obs_window=0)) == K.EINVAL        # SnapKV: zero window refused
    assert evict(c, window(), pool=4) == K.EINVAL            # SnapKV: even pool kernel refused
    assert evict(c, window(a=None), flags=K.DROP) == K.EINVAL
    assert evict(c, window(), cap=31) == K.ENOSPACE          # free list smaller than the pool
    assert evict(c, window(), ws=None, ws_bytes=ws) == K.ENOSPACE
    assert evict(c, window(), ws_bytes=ws - 1) == K.ENOSPACE
    assert evict(c, window(group=64, obs_window=65), flags=K.DROP, pool=1) == K.EUNSUPPORTED
    # a split window needs room for its raw sums past the main workspace
    ws_big = L.kvev_workspace_bytes(ctypes.byref(c), 8, 64)
    assert ws_big > ws
    assert evict(c, window(group=8, obs_window=64), flags=K.DROP, pool=1,
                 ws_bytes=ws) == K.ENOSPACE


def test_misaligned_score_refused():
    """The score row feeds 16-byte vector loads: a pointer off 16 bytes is refused."""
    L = K.load_library()
    c = cache()
    ws = L.kvev_workspace_bytes(ctypes.byref(c), 1, 1)
    assert L.kvev_select(ctypes.byref(c), FAKE + 4, 8, 2, FAKE, FAKE, FAKE, ws, None) == K.EINVAL
    assert evict(c, window(), ptrs={"score": FAKE + 8}) == K.EINVAL


def test_measure_refusals():
    L = K.load_library()
    args = [FAKE, FAKE, FAKE, 4, 64, FAKE, None]
    for i in (0, 1, 2, 5):
        a = list(args); a[i] = None
        assert L.kvev_measure(*a) == K.EINVAL
    for units, ms in ((-1, 64), (4, 0), (4, 40)):  # max_slots: a positive multiple of 16
        a = list(args); a[3] = units; a[4] = ms
        assert L.kvev_measure(*a) == K.EINVAL


def test_h2o_step_refusals():
    """Every refusal of kvev_h2o_step is decided on the host, before a launch."""
    L = K.load_library()

    def call(c=None, group=4, budget=64, recent=8, ptrs=None, ws_bytes=1 << 30):
        c = cache(max_blocks=8) if c is None else c
        p = dict(q=FAKE, k=FAKE, v=FAKE, t=FAKE, s=FAKE, fl=FAKE, fc=FAKE, ev=FAKE, ws=FAKE)
        p.update(ptrs or {})
        return L.kvev_h2o_step(ctypes.byref(c), p["q"], p["k"], p["v"], p["t"], group, 0.1,
                               p["s"], budget, recent, p["fl"], p["fc"], p["ev"], None,
                               p["ws"], ws_bytes, None)

    for name in ("q", "k", "v", "t", "s", "fl", "fc", "ev"):
        assert call(ptrs={name: None}) == K.EINVAL, name
    assert call(c=cache(head_dim=96)) == K.EINVAL
    assert call(c=cache(k_pool=None)) == K.EINVAL
    assert call(group=0) == K.EINVAL
    assert call(budget=0) == K.EINVAL
    assert call(budget=129) == K.EINVAL          # above max_blocks * 16 = 128
    assert call(recent=-1) == K.EINVAL
    assert call(recent=64) == K.EINVAL           # recent window must leave room: < budget
    assert call(group=17) == K.EUNSUPPORTED
    big = cache(max_blocks=300)
    assert call(c=big, group=1, budget=4097) == K.EUNSUPPORTED
    assert call(c=big, group=8, budget=2050) == K.EUNSUPPORTED  # 8 * 2064 logits > 16384
    need = L.kvev_h2o_workspace_bytes(ctypes.byref(cache(max_blocks=8)), 4, 64)
    assert need > 0
    assert call(ptrs={"ws": None}) == K.ENOSPACE
    assert call(ws_bytes=need - 1) == K.ENOSPACE
    # the size query refuses what the step refuses
    assert L.kvev_h2o_workspace_bytes(ctypes.byref(cache(max_blocks=8)), 0, 64) == 0
    assert L.kvev_h2o_workspace_bytes(ctypes.byref(cache(max_blocks=8)), 4, 5000) == 0
    assert L.kvev_h2o_workspace_bytes(None, 4, 64) == 0


def test_vtok_refusals():
    """Every refusal of kvev_vtok_evict and kvev_vtok_reclaim is decided on the
    host, before a launch."""
    L = K.load_library()

    def evict(c=None, ptrs=None, ws_bytes=1 << 30):
        c = cache(max_blocks=8) if c is None else c
        p = dict(live=FAKE, bl=FAKE, vic=FAKE, nv=FAKE, st=FAKE, ws=FAKE)
        p.update(ptrs or {})
        return L.kvev_vtok_evict(ctypes.byref(c), p["live"], p["bl"], p["vic"], p["nv"], p["st"],
                                 p["ws"], ws_bytes, None)

    for name in ("live", "bl", "vic", "nv", "st"):
        assert evict(ptrs={name: None}) == K.EINVAL, name
    assert evict(ptrs={"live": FAKE + 4}) == K.EINVAL      # live must be 16-byte aligned
    assert evict(ptrs={"ws": FAKE + 8}) == K.EINVAL
    assert evict(c=cache(head_dim=96)) == K.EINVAL
    c8 = cache(max_blocks=8)
    need_e = L.kvev_vtok_evict_workspace_bytes(ctypes.byref(c8))
    assert need_e >= 2 * 2 * 128 * 4                       # a claim word per slot
    assert evict(ptrs={"ws": None}) == K.ENOSPACE
    assert evict(ws_bytes=need_e - 1) == K.ENOSPACE
    assert L.kvev_vtok_evict_workspace_bytes(None) == 0

    def reclaim(c=None, theta=0.25, max_sources=8, cap=None, ptrs=None, ws_bytes=1 << 30):
        c = cache(max_blocks=8) if c is None else c
        p = dict(live=FAKE, bl=FAKE, fl=FAKE, fc=FAKE, st=FAKE, ws=FAKE)
        p.update(ptrs or {})
        cap = c.num_blocks if cap is None else cap
        return L.kvev_vtok_reclaim(ctypes.byref(c), p["live"], p["bl"], None, theta, max_sources,
                                   p["fl"], p["fc"], cap, p["st"], p["ws"], ws_bytes, None)

    for name in ("live", "bl", "fl", "fc", "st"):
        assert reclaim(ptrs={name: None}) == K.EINVAL, name
    assert reclaim(ptrs={"live": FAKE + 4}) == K.EINVAL
    assert reclaim(ptrs={"ws": FAKE + 8}) == K.EINVAL
    assert reclaim(c=cache(pos=FAKE + 4)) == K.EINVAL
    for theta in (-0.1, 1.0, float("nan"), float("inf")):
        assert reclaim(theta=theta) == K.EINVAL, theta
    assert reclaim(max_sources=1) == K.EINVAL
    assert reclaim(max_sources=4097) == K.EINVAL
    assert reclaim(c=cache(batch=8193, kv_heads=1)) == K.EUNSUPPORTED
    c = cache(max_blocks=8)
    assert reclaim(c=c, cap=c.num_blocks - 1) == K.ENOSPACE
    need = L.kvev_vtok_workspace_bytes(ctypes.byref(c), 8)
    assert need > 0
    assert reclaim(ptrs={"ws": None}) == K.ENOSPACE
    assert reclaim(ws_bytes=need - 1) == K.ENOSPACE
    # the size query refuses what the call refuses
    assert L.kvev_vtok_workspace_bytes(ctypes.byref(c), 1) == 0
    assert L.kvev_vtok_workspace_bytes(ctypes.byref(c), 4097) == 0
    assert L.kvev_vtok_workspace_bytes(None, 8) == 0
    # it grows with max_sources (staged rows of every source)
    assert L.kvev_vtok_workspace_bytes(ctypes.byref(c), 64) > need


def test_vtok_check_refusals():
    L = K.load_library()
    c = cache(max_blocks=8)
    assert L.kvev_vtok_digest(ctypes.byref(c), None, FAKE, None) == K.EINVAL
    assert L.kvev_vtok_digest(ctypes.byref(c), FAKE, None, None) == K.EINVAL
    assert L.kvev_vtok_digest(ctypes.byref(c), FAKE + 4, FAKE, None) == K.EINVAL
    assert L.kvev_vtok_digest(ctypes.byref(c), FAKE, FAKE + 4, None) == K.EINVAL
    assert L.kvev_vtok_digest(ctypes.byref(cache(head_dim=96)), FAKE, FAKE, None) == K.EINVAL
    need = L.kvev_vtok_check_workspace_bytes(ctypes.byref(c))
    assert need >= c.num_blocks * 4
    assert L.kvev_vtok_check_workspace_bytes(None) == 0

    def check(ptrs=None, cap=64, ws_bytes=1 << 20):
        p = dict(live=FAKE, bl=FAKE, fl=FAKE, fc=FAKE, out=FAKE, ws=FAKE)
        p.update(ptrs or {})
        return L.kvev_vtok_check(ctypes.byref(c), p["live"], p["bl"], p["fl"], p["fc"], cap,
                                 p["out"], p["ws"], ws_bytes, None)

    for name in ("live", "bl", "fl", "fc", "out"):
        assert check(ptrs={name: None}) == K.EINVAL, name
    assert check(ptrs={"live": FAKE + 4}) == K.EINVAL
    assert check(ptrs={"out": FAKE + 4}) == K.EINVAL
    assert check(cap=-1) == K.EINVAL
    assert check(ptrs={"ws": None}) == K.ENOSPACE
    assert check(ws_bytes=need - 1) == K.ENOSPACE


def test_select_shared_refusals():
    L = K.load_library()
    c = cache(max_blocks=8)
    need = L.kvev_select_shared_workspace_bytes(ctypes.byref(c))
    assert need > 0 and L.kvev_select_shared_workspace_bytes(None) == 0

    def call(budget=64, recent=8, ptrs=None, ws_bytes=1 << 30):
        p = dict(s=FAKE, v=FAKE, n=FAKE, ws=FAKE)
        p.update(ptrs or {})
        return L.kvev_select_shared(ctypes.byref(c), p["s"], budget, recent, p["v"], p["n"],
                                    p["ws"], ws_bytes, None)

    for name in ("s", "v", "n"):
        assert call(ptrs={name: None}) == K.EINVAL, name
    assert call(ptrs={"s": FAKE + 4}) == K.EINVAL
    assert call(budget=0) == K.EINVAL
    assert call(recent=64) == K.EINVAL
    assert call(recent=-1) == K.EINVAL
    assert call(ptrs={"ws": None}) == K.ENOSPACE
    assert call(ws_bytes=need - 1) == K.ENOSPACE


def test_select_budgets_refusals():
    L = K.load_library()
    c = cache(max_blocks=8)
    need = L.kvev_workspace_bytes(ctypes.byref(c), 0, 0)

    def call(ptrs=None, ws_bytes=1 << 30):
        p = dict(s=FAKE, b=FAKE, r=FAKE, v=FAKE, n=FAKE, ws=FAKE)
        p.update(ptrs or {})
        return L.kvev_select_budgets(ctypes.byref(c), p["s"], p["b"], p["r"], p["v"], p["n"],
                                     p["ws"], ws_bytes, None)

    for name in ("s", "b", "r", "v", "n"):
        assert call(ptrs={name: None}) == K.EINVAL, name
    assert call(ptrs={"s": FAKE + 8}) == K.EINVAL
    assert call(ptrs={"ws": None}) == K.ENOSPACE
    assert call(ws_bytes=64) == K.ENOSPACE        # far below the selection's regions
    assert need > 64


def test_ring_step_refusals():
    L = K.load_library()
    c = cache(max_blocks=8)

    def call(group=4, budget=64, recent=8, W=4, pool=3, ptrs=None, cc=None, ws_bytes=1 << 30):
        p = dict(h=FAKE, r=FAKE, k=FAKE, q=FAKE, kn=FAKE, vn=FAKE, t=FAKE, o=FAKE, fl=FAKE,
                 fc=FAKE, ev=FAKE, ws=FAKE)
        p.update(ptrs or {})
        return L.kvev_ring_step(ctypes.byref(cc or c), p["h"], p["r"], p["k"], p["q"], p["kn"],
                                p["vn"], p["t"], p["o"], group, 0.1, budget, recent, W, pool,
                                p["fl"], p["fc"], p["ev"], p["ws"], ws_bytes, None)

    for name in ("h", "r", "k", "q", "kn", "vn", "t", "o", "fl", "fc", "ev"):
        assert call(ptrs={name: None}) == K.EINVAL, name
    assert call(group=0) == K.EINVAL
    assert call(recent=64) == K.EINVAL               # recentWindow >= budget
    assert call(W=0) == K.EINVAL                     # obsWindow of zero
    assert call(pool=2) == K.EINVAL                  # an even poolKernel
    assert call(pool=0) == K.EINVAL
    assert call(budget=129) == K.EINVAL              # above the capacity
    assert call(cc=cache(head_dim=96)) == K.EINVAL
    assert call(group=9) == K.EUNSUPPORTED
    big = cache(max_blocks=300)
    assert call(cc=big, group=1, budget=4097) == K.EUNSUPPORTED
    assert call(cc=big, group=8, budget=2048) == K.EUNSUPPORTED   # 8 * 2049 > 16384
    assert call(pool=131) == K.EUNSUPPORTED
    need = L.kvev_ring_workspace_bytes(ctypes.byref(c), 4, 64)
    assert need > 0
    assert call(ptrs={"ws": None}) == K.ENOSPACE
    assert call(ws_bytes=need - 1) == K.ENOSPACE
    # the size query refuses what the step refuses
    assert L.kvev_ring_workspace_bytes(ctypes.byref(c), 0, 64) == 0
    assert L.kvev_ring_workspace_bytes(ctypes.byref(c), 9, 64) == 0
    assert L.kvev_ring_workspace_bytes(ctypes.byref(c), 4, 4097) == 0
    assert L.kvev_ring_workspace_bytes(None, 4, 64) == 0
    assert L.kvev_ring_init(ctypes.byref(c), None, FAKE, FAKE, 4, None) == K.EINVAL
    assert L.kvev_ring_init(ctypes.byref(c), FAKE, FAKE, FAKE, 0, None) == K.EINVAL


def test_vtok_sync_and_mapping_refusals():
    L = K.load_library()
    c = cache(max_blocks=8)
    for i in range(5):
        p = [FAKE] * 5
        p[i] = None
        assert L.kvev_vtok_sync(ctypes.byref(c), *p, None) == K.EINVAL, i
    for i in range(4):
        p = [FAKE] * 4
        p[i] = None
        assert L.kvev_vtok_slot_mapping(ctypes.byref(c), *p, FAKE, 1 << 20, None) == K.EINVAL, i
    need = L.kvev_vtok_map_workspace_bytes(ctypes.byref(c))
    assert need >= 2 * 2 * 4
    assert L.kvev_vtok_slot_mapping(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, None, 1 << 20,
                                    None) == K.ENOSPACE
    assert L.kvev_vtok_slot_mapping(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
                                    None) == K.ENOSPACE
    bad = cache(head_dim=96)
    assert L.kvev_vtok_sync(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None) == K.EINVAL
    assert L.kvev_vtok_slot_mapping(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20,
                                    None) == K.EINVAL


def test_read_probe_library_refuses_bad_arguments():
    """The HBM read-rate probe (libkvev_probe.so, the benchmark's --hbm-probe
    mode) is built beside the eviction library and checks its arguments on
    the host before any launch."""
    from kv_cache_eviction_qk_amd import build as kbuild
    if not os.path.exists(kbuild.PROBE_OUT):
        pytest.skip("libkvev_probe.so not built")
    L = ctypes.CDLL(kbuild.PROBE_OUT)
    f = L.kvev_probe_read
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    ok = dict(pattern=1, depth=8, buf=FAKE, nbytes=1 << 20, lst=FAKE, grid=64, sink=FAKE)
    for bad in (dict(pattern=2), dict(pattern=-1), dict(depth=6), dict(buf=None),
                dict(nbytes=0), dict(nbytes=4097), dict(nbytes=1 << 43), dict(lst=None),
                dict(grid=0), dict(grid=65537), dict(sink=None)):
        a = dict(ok, **bad)
        assert f(a["pattern"], a["depth"], a["buf"], a["nbytes"], a["lst"], a["grid"], a["sink"],
                 None) == -1, bad
    g = L.kvev_probe_overlap
    g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    g.restype = ctypes.c_int
    ok = dict(mode=0, grid=256, iters=100, out=FAKE)
    for bad in (dict(mode=-1), dict(mode=6), dict(grid=0), dict(grid=65537), dict(iters=0),
                dict(iters=(1 << 24) + 1), dict(out=None)):
        a = dict(ok, **bad)
        assert g(a["mode"], a["grid"], a["iters"], a["out"], None) == -1, bad
    h = L.kvev_probe_barrier
    h.argtypes = g.argtypes
    h.restype = ctypes.c_int
    for bad in (dict(mode=-1), dict(mode=3), dict(grid=0), dict(grid=65537), dict(iters=0),
                dict(out=None)):
        a = dict(ok, **bad)
        assert h(a["mode"], a["grid"], a["iters"], a["out"], None) == -1, bad
