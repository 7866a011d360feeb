"""Attention-score KV-cache eviction on MI355X: Python binding of libkvev.

Thin ctypes layer over the C ABI in ``include/kvev.h``: it checks that the
torch tensors handed over have the expected device, dtype, shape and
layout, builds the argument structs and calls the library on the current
torch stream.  Every step of score, select and compact runs in the HIP
kernels of ``csrc/``; nothing here computes.  There is no fallback: if
``libkvev.so`` is missing or cannot be loaded, importing the library raises.

Names follow the C ABI: ``score``, ``select``, ``compact``, ``evict``
(score + select + compact in one fused call), ``window_attn``,
``workspace_bytes``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvev.so")

OK, EINVAL, ENOSPACE, EUNSUPPORTED, EDEVICE = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
SUM, POOL, DROP, ACCUMULATE = 1, 2, 4, 8
BLOCK_SIZE = 16

# the functions include/kvev.h declares
EXPORTS = ("kvev_score", "kvev_select", "kvev_compact", "kvev_evict", "kvev_evict_noalloc",
           "kvev_measure",
           "kvev_h2o_step", "kvev_h2o_workspace_bytes", "kvev_vtok_evict",
           "kvev_vtok_evict_workspace_bytes", "kvev_vtok_reclaim", "kvev_vtok_workspace_bytes",
           "kvev_vtok_digest", "kvev_vtok_check", "kvev_vtok_check_workspace_bytes",
           "kvev_select_shared", "kvev_select_shared_workspace_bytes", "kvev_select_budgets",
           "kvev_ring_step", "kvev_ring_workspace_bytes", "kvev_ring_init", "kvev_vtok_sync", "kvev_vtok_slot_mapping",
           "kvev_vtok_map_workspace_bytes",
           "kvev_window_attn",
           "kvev_workspace_bytes", "kvev_strerror", "kvev_abi_version")
ABI_VERSION = 17


class KvevError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {strerror(status)} ({status})")
        self.status = status


class CacheStruct(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k_pool", ctypes.c_void_p),
                ("v_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("pos", ctypes.c_void_p)]


class WindowStruct(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("obs_window", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("lse", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("q_pos", ctypes.c_void_p), ("scale", ctypes.c_float)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvev.so; raises if it is missing or lacks a declared symbol."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libkvev.so not built at {path}: run python -m "
                          "kv_cache_eviction_qk_amd.build")
    L = ctypes.CDLL(path)
    for name in EXPORTS:
        if not hasattr(L, name):
            raise ImportError(f"{path} does not export {name}")
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.kvev_score.argtypes = [P, P, i32, i32, P, P, P, P, sz, P]
    L.kvev_select.argtypes = [P, P, i32, i32, P, P, P, sz, P]
    L.kvev_compact.argtypes = [P, P, P, P, P, P, i32, P, P, sz, P]
    L.kvev_evict.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P, i32, P, P, sz, P]
    L.kvev_evict_noalloc.argtypes = [P, P, i32, i32, i32, i32, P, P, P, P, P, i32, P, P]
    L.kvev_window_attn.argtypes = [P, P, P, P, P, sz, P]
    L.kvev_measure.argtypes = [P, P, P, i32, i32, P, P]
    L.kvev_h2o_step.argtypes = [P, P, P, P, P, i32, ctypes.c_float, P, i32, i32, P, P, P, P, P,
                                sz, P]
    L.kvev_h2o_workspace_bytes.argtypes = [P, i32, i32]
    L.kvev_h2o_workspace_bytes.restype = sz
    L.kvev_vtok_evict.argtypes = [P, P, P, P, P, P, P, sz, P]
    L.kvev_vtok_evict_workspace_bytes.argtypes = [P]
    L.kvev_vtok_evict_workspace_bytes.restype = sz
    L.kvev_vtok_reclaim.argtypes = [P, P, P, P, ctypes.c_double, i32, P, P, i32, P, P, sz, P]
    L.kvev_vtok_workspace_bytes.argtypes = [P, i32]
    L.kvev_vtok_digest.argtypes = [P, P, P, P]
    L.kvev_select_shared.argtypes = [P, P, i32, i32, P, P, P, sz, P]
    L.kvev_select_budgets.argtypes = [P, P, P, P, P, P, P, sz, P]
    L.kvev_ring_step.argtypes = [P, P, P, P, P, P, P, P, P, i32, ctypes.c_float, i32, i32, i32,
                                 i32, P, P, P, P, sz, P]
    L.kvev_ring_workspace_bytes.argtypes = [P, i32, i32]
    L.kvev_ring_workspace_bytes.restype = sz
    L.kvev_ring_init.argtypes = [P, P, P, P, i32, P]
    L.kvev_vtok_sync.argtypes = [P, P, P, P, P, P, P]
    L.kvev_vtok_slot_mapping.argtypes = [P, P, P, P, P, P, sz, P]
    L.kvev_vtok_map_workspace_bytes.argtypes = [P]
    L.kvev_vtok_map_workspace_bytes.restype = sz
    L.kvev_select_shared_workspace_bytes.argtypes = [P]
    L.kvev_select_shared_workspace_bytes.restype = sz
    L.kvev_vtok_check.argtypes = [P, P, P, P, P, i32, P, P, sz, P]
    L.kvev_vtok_check_workspace_bytes.argtypes = [P]
    L.kvev_vtok_check_workspace_bytes.restype = sz
    L.kvev_vtok_workspace_bytes.restype = sz
    L.kvev_workspace_bytes.argtypes = [P, i32, i32]
    L.kvev_workspace_bytes.restype = sz
    L.kvev_strerror.argtypes = [ctypes.c_int]
    L.kvev_strerror.restype = ctypes.c_char_p
    L.kvev_abi_version.argtypes = []
    for f in (L.kvev_score, L.kvev_select, L.kvev_compact, L.kvev_evict, L.kvev_evict_noalloc,
              L.kvev_window_attn,
              L.kvev_measure, L.kvev_h2o_step, L.kvev_vtok_evict, L.kvev_vtok_reclaim,
              L.kvev_vtok_digest, L.kvev_vtok_check, L.kvev_select_shared,
              L.kvev_select_budgets, L.kvev_ring_step, L.kvev_ring_init, L.kvev_vtok_sync,
              L.kvev_vtok_slot_mapping, L.kvev_abi_version):
        f.restype = ctypes.c_int
    if L.kvev_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {L.kvev_abi_version()}, expected "
                          f"{ABI_VERSION}: rebuild it")
    _lib = L
    return L


def strerror(status: int) -> str:
    return load_library().kvev_strerror(status).decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise KvevError(rc, what)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype=None, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


@dataclasses.dataclass
class Cache:
    """One layer's paged KV cache on the GPU (layout of include/kvev.h)."""
    k_pool: torch.Tensor        # [num_blocks, 16, D], float32 or bfloat16
    v_pool: torch.Tensor
    block_table: torch.Tensor   # int32 [B, Hkv, max_blocks]
    seq_len: torch.Tensor       # int32 [B, Hkv]
    pos: torch.Tensor           # int32 [B, Hkv, max_blocks*16]

    @property
    def batch(self) -> int:
        return self.block_table.shape[0]

    @property
    def kv_heads(self) -> int:
        return self.block_table.shape[1]

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[2]

    @property
    def max_slots(self) -> int:
        return self.max_blocks * BLOCK_SIZE

    @property
    def head_dim(self) -> int:
        return self.k_pool.shape[-1]

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]

    @property
    def units(self) -> int:
        return self.batch * self.kv_heads

    @property
    def dtype_code(self) -> int:
        return BF16 if self.k_pool.dtype == torch.bfloat16 else F32

    def struct(self) -> CacheStruct:
        if self.k_pool.dtype not in (torch.float32, torch.bfloat16):
            raise ValueError("k_pool must be float32 or bfloat16")
        _need(self.k_pool, "k_pool")
        _need(self.v_pool, "v_pool", self.k_pool.dtype, self.k_pool.numel())
        if self.k_pool.dim() != 3 or self.k_pool.shape[1] != BLOCK_SIZE:
            raise ValueError("k_pool must be [num_blocks, 16, head_dim]")
        _need(self.block_table, "block_table", torch.int32)
        if self.block_table.dim() != 3:
            raise ValueError("block_table must be [B, Hkv, max_blocks]")
        _need(self.seq_len, "seq_len", torch.int32, self.units)
        _need(self.pos, "pos", torch.int32, self.units * self.max_slots)
        return CacheStruct(self.batch, self.kv_heads, self.head_dim, BLOCK_SIZE,
                           self.max_blocks, self.k_pool.shape[0], self.dtype_code,
                           _ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.block_table),
                           _ptr(self.seq_len), _ptr(self.pos))

    def score_buffer(self, fill: float = 0.0) -> torch.Tensor:
        return torch.full((self.batch, self.kv_heads, self.max_slots), fill, dtype=torch.float32,
                          device=self.k_pool.device)


def _window(cache: Cache, q, lse, q_pos, scale, group, a=None) -> WindowStruct:
    B, Hkv, D = cache.batch, cache.kv_heads, cache.head_dim
    if q.dim() != 4 or q.shape[0] != B or q.shape[1] != Hkv * group or q.shape[3] != D:
        raise ValueError(f"q must be [B, Hkv*G, W, D] = [{B}, {Hkv * group}, W, {D}]")
    W = q.shape[2]
    _need(q, "q", cache.k_pool.dtype)
    if lse is not None:
        _need(lse, "lse", torch.float32, B * Hkv * group * W)
    if a is not None:
        _need(a, "a", torch.float32, q.numel())  # the forward pass's output, fp32
    _need(q_pos, "q_pos", torch.int32, B * W)
    return WindowStruct(group, W, _ptr(q), _ptr(lse), _ptr(a), _ptr(q_pos), float(scale))


def workspace_bytes(cache: Cache, group: int = 1, obs_window: int = 1) -> int:
    c = cache.struct()
    return int(load_library().kvev_workspace_bytes(ctypes.byref(c), group, obs_window))


def new_workspace(cache: Cache, group: int = 1, obs_window: int = 1) -> torch.Tensor:
    """A zero-filled workspace for every entry point (the library keeps its
    persistent part zeroed from call to call)."""
    return torch.zeros(workspace_bytes(cache, group, obs_window), dtype=torch.uint8,
                       device=cache.k_pool.device)


def score(cache: Cache, q: torch.Tensor, lse: torch.Tensor, q_pos: torch.Tensor, scale: float,
          group: int, flags: int, pool_kernel: int = 1, sum: Optional[torch.Tensor] = None,
          pooled: Optional[torch.Tensor] = None, drop: Optional[torch.Tensor] = None,
          a: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
          stream=None) -> dict:
    """kvev_score.  Output buffers are allocated (filled with 0) when not given;
    so is the workspace, which only windows too large for one workgroup use."""
    L = load_library()
    c = cache.struct()
    w = _window(cache, q, lse, q_pos, scale, group, a)
    if workspace is None:
        workspace = new_workspace(cache, group, q.shape[2])
    _need(workspace, "workspace", torch.uint8)
    if flags & SUM and sum is None:
        sum = cache.score_buffer()
    if flags & POOL and pooled is None:
        pooled = cache.score_buffer()
    if flags & DROP and drop is None:
        drop = cache.score_buffer()
    for t, nm in ((sum, "sum"), (pooled, "pooled"), (drop, "drop")):
        if t is not None:
            _need(t, nm, torch.float32, cache.units * cache.max_slots)
    rc = L.kvev_score(ctypes.byref(c), ctypes.byref(w), flags, pool_kernel, _ptr(sum),
                      _ptr(pooled), _ptr(drop), _ptr(workspace), workspace.numel(),
                      _stream(stream))
    _check(rc, "kvev_score")
    return {"sum": sum, "pooled": pooled, "drop": drop}


def select(cache: Cache, score_row: torch.Tensor, budget: int, recent_window: int,
           victims: Optional[torch.Tensor] = None, n_victims: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None):
    """kvev_select -> (victims [B, Hkv, max_slots] int32, n_victims [B, Hkv] int32).
    `workspace`: a zero-filled uint8 buffer from new_workspace() (allocated here when None)."""
    L = load_library()
    c = cache.struct()
    if workspace is None:
        workspace = new_workspace(cache)
    _need(workspace, "workspace", torch.uint8)
    _need(score_row, "score", torch.float32, cache.units * cache.max_slots)
    dev = cache.k_pool.device
    if victims is None:
        victims = torch.full((cache.batch, cache.kv_heads, cache.max_slots), -1,
                             dtype=torch.int32, device=dev)
    if n_victims is None:
        n_victims = torch.zeros((cache.batch, cache.kv_heads), dtype=torch.int32, device=dev)
    _need(victims, "victims", torch.int32, cache.units * cache.max_slots)
    _need(n_victims, "n_victims", torch.int32, cache.units)
    rc = L.kvev_select(ctypes.byref(c), _ptr(score_row), budget, recent_window, _ptr(victims),
                       _ptr(n_victims), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "kvev_select")
    return victims, n_victims


def select_budgets(cache: Cache, score_row: torch.Tensor, budget: torch.Tensor,
                   recent_window: torch.Tensor, workspace: torch.Tensor,
                   victims: Optional[torch.Tensor] = None, n_victims: Optional[torch.Tensor] = None,
                   stream=None):
    """kvev_select_budgets: kvev_select with int32 [B, Hkv] budgets and recent
    windows on the GPU -> (victims, n_victims)."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(score_row, "score_row", torch.float32, B * Hkv * cache.max_slots)
    _need(budget, "budget", torch.int32, B * Hkv)
    _need(recent_window, "recent_window", torch.int32, B * Hkv)
    _need(workspace, "workspace", torch.uint8)
    if victims is None:
        victims = torch.empty((B, Hkv, cache.max_slots), dtype=torch.int32, device=score_row.device)
    if n_victims is None:
        n_victims = torch.empty((B, Hkv), dtype=torch.int32, device=score_row.device)
    _need(victims, "victims", torch.int32, B * Hkv * cache.max_slots)
    _need(n_victims, "n_victims", torch.int32, B * Hkv)
    _check(L.kvev_select_budgets(ctypes.byref(c), _ptr(score_row), _ptr(budget),
                                 _ptr(recent_window), _ptr(victims), _ptr(n_victims),
                                 _ptr(workspace), workspace.numel(), _stream(stream)),
           "kvev_select_budgets")
    return victims, n_victims


def new_select_shared_workspace(cache: Cache) -> torch.Tensor:
    n = load_library().kvev_select_shared_workspace_bytes(ctypes.byref(cache.struct()))
    if n == 0:
        raise KvevError(EINVAL, "kvev_select_shared_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=cache.k_pool.device)


def select_shared(cache: Cache, score_row: torch.Tensor, budget: int, recent_window: int,
                  workspace: torch.Tensor, victims: Optional[torch.Tensor] = None,
                  n_victims: Optional[torch.Tensor] = None, stream=None):
    """kvev_select_shared: one victim set per sequence from the per-head scores
    summed over its KV heads, given to every head -> (victims, n_victims)."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(score_row, "score_row", torch.float32, B * Hkv * cache.max_slots)
    _need(workspace, "workspace", torch.uint8)
    if victims is None:
        victims = torch.empty((B, Hkv, cache.max_slots), dtype=torch.int32, device=score_row.device)
    if n_victims is None:
        n_victims = torch.empty((B, Hkv), dtype=torch.int32, device=score_row.device)
    _need(victims, "victims", torch.int32, B * Hkv * cache.max_slots)
    _need(n_victims, "n_victims", torch.int32, B * Hkv)
    _check(L.kvev_select_shared(ctypes.byref(c), _ptr(score_row), budget, recent_window,
                                _ptr(victims), _ptr(n_victims), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "kvev_select_shared")
    return victims, n_victims


def compact(cache: Cache, victims: torch.Tensor, n_victims: torch.Tensor,
            free_list: torch.Tensor, free_count: torch.Tensor, workspace: torch.Tensor,
            stats: Optional[torch.Tensor] = None, score_row: Optional[torch.Tensor] = None,
            stream=None) -> torch.Tensor:
    """kvev_compact (mutates the cache in place) -> stats int64[5] on the GPU."""
    L = load_library()
    c = cache.struct()
    _need(victims, "victims", torch.int32, cache.units * cache.max_slots)
    _need(n_victims, "n_victims", torch.int32, cache.units)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    _need(workspace, "workspace", torch.uint8)
    if stats is None:
        stats = torch.zeros(5, dtype=torch.int64, device=cache.k_pool.device)
    _need(stats, "stats", torch.int64, 5)
    if score_row is not None:
        _need(score_row, "score_row", torch.float32, cache.units * cache.max_slots)
    rc = L.kvev_compact(ctypes.byref(c), _ptr(victims), _ptr(n_victims), _ptr(score_row),
                        _ptr(free_list), _ptr(free_count), free_list.numel(), _ptr(stats),
                        _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "kvev_compact")
    return stats


def evict(cache: Cache, q: torch.Tensor, lse: torch.Tensor, q_pos: torch.Tensor, scale: float,
          group: int, flags: int, budget: int, recent_window: int, score_row: torch.Tensor,
          victims: torch.Tensor, n_victims: torch.Tensor, free_list: torch.Tensor,
          free_count: torch.Tensor, workspace: torch.Tensor, pool_kernel: int = 1,
          a: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None,
          stream=None) -> torch.Tensor:
    """kvev_evict: score + select + compact of one layer in one call (mutates the
    cache, score_row, the free list) -> stats int64[5] on the GPU."""
    L = load_library()
    c = cache.struct()
    w = _window(cache, q, lse, q_pos, scale, group, a)
    n = cache.units * cache.max_slots
    _need(score_row, "score_row", torch.float32, n)
    _need(victims, "victims", torch.int32, n)
    _need(n_victims, "n_victims", torch.int32, cache.units)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    _need(workspace, "workspace", torch.uint8)
    if stats is None:
        stats = torch.zeros(5, dtype=torch.int64, device=cache.k_pool.device)
    _need(stats, "stats", torch.int64, 5)
    rc = L.kvev_evict(ctypes.byref(c), ctypes.byref(w), flags, pool_kernel, budget,
                      recent_window, _ptr(score_row), _ptr(victims), _ptr(n_victims),
                      _ptr(free_list), _ptr(free_count), free_list.numel(), _ptr(stats),
                      _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "kvev_evict")
    return stats


def evict_noalloc(cache: Cache, q: torch.Tensor, lse: torch.Tensor, q_pos: torch.Tensor,
                  scale: float, group: int, flags: int, budget: int, recent_window: int,
                  score_row: torch.Tensor, victims: torch.Tensor, n_victims: torch.Tensor,
                  free_list: torch.Tensor, free_count: torch.Tensor, stats: torch.Tensor,
                  pool_kernel: int = 1, a: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """kvev_evict_noalloc: kvev_evict in the library's static per-GPU scratch
    array (no workspace; the C call allocates nothing).  Every argument,
    stats included, is the caller's."""
    L = load_library()
    c = cache.struct()
    w = _window(cache, q, lse, q_pos, scale, group, a)
    n = cache.units * cache.max_slots
    _need(score_row, "score_row", torch.float32, n)
    _need(victims, "victims", torch.int32, n)
    _need(n_victims, "n_victims", torch.int32, cache.units)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    _need(stats, "stats", torch.int64, 5)
    rc = L.kvev_evict_noalloc(ctypes.byref(c), ctypes.byref(w), flags, pool_kernel, budget,
                              recent_window, _ptr(score_row), _ptr(victims), _ptr(n_victims),
                              _ptr(free_list), _ptr(free_count), free_list.numel(), _ptr(stats),
                              _stream(stream))
    _check(rc, "kvev_evict_noalloc")
    return stats


def measure(seq_len_before: torch.Tensor, victims: torch.Tensor, n_victims: torch.Tensor,
            out: Optional[torch.Tensor] = None, stream=None) -> dict:
    """kvev_measure: block-level waste of an eviction.  seq_len_before and
    n_victims: int32 [B, Hkv]; victims: int32 [B, Hkv, max_slots].  Returns the
    six integer sums (synchronising to read them) and the ratios derived from
    them: F_naive, F_after, frac_le_half_naive, frac_le_half_after."""
    L = load_library()
    units = seq_len_before.numel()
    _need(seq_len_before, "seq_len_before", torch.int32, units)
    _need(n_victims, "n_victims", torch.int32, units)
    _need(victims, "victims", torch.int32)
    if units == 0 or victims.numel() % units:
        raise ValueError("victims must hold max_slots entries per head")
    max_slots = victims.numel() // units
    if out is None:
        out = torch.empty(6, dtype=torch.int64, device=victims.device)
    _need(out, "out", torch.int64, 6)
    rc = L.kvev_measure(_ptr(seq_len_before), _ptr(victims), _ptr(n_victims), units, max_slots,
                        _ptr(out), _stream(stream))
    _check(rc, "kvev_measure")
    live, bn, ba, hn, ha, freed = (int(x) for x in out.cpu().tolist())
    return dict(live_tokens=live, blocks_naive=bn, blocks_after=ba, le_half_naive=hn,
                le_half_after=ha, blocks_freed=freed,
                F_naive=1.0 - live / (bn * 16.0) if bn else 0.0,
                F_after=1.0 - live / (ba * 16.0) if ba else 0.0,
                frac_le_half_naive=hn / bn if bn else 0.0,
                frac_le_half_after=ha / ba if ba else 0.0)


def new_h2o_workspace(cache: Cache, group: int, budget: int) -> torch.Tensor:
    """A zero-filled workspace for kvev_h2o_step on this cache shape."""
    n = load_library().kvev_h2o_workspace_bytes(ctypes.byref(cache.struct()), group, budget)
    if n == 0:
        raise KvevError(EUNSUPPORTED, "kvev_h2o_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=cache.k_pool.device)


def h2o_step(cache: Cache, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             t_pos: torch.Tensor, group: int, scale: float, score: torch.Tensor, budget: int,
             recent: int, free_list: torch.Tensor, free_count: torch.Tensor,
             workspace: torch.Tensor, evicted: Optional[torch.Tensor] = None,
             attn_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvev_h2o_step: one decode step of every KV head.  q [B, Hq, D], k_new and
    v_new [B, Hkv, D] in the cache dtype; t_pos int32 [B]; score fp32 [B, Hkv,
    max_slots] (running scores, updated); free_list int32, free_count int32
    [1]; workspace from new_h2o_workspace; attn_out (optional) fp32 [B, Hq,
    D] receives the step's attention output.  Returns evicted int32 [B, Hkv]
    (-1 appended, else the pruned position; -2, -3, -4 for a head left
    unchanged)."""
    L = load_library()
    c = cache.struct()
    B, Hkv, D = cache.batch, cache.kv_heads, cache.head_dim
    _need(q, "q", cache.k_pool.dtype, B * Hkv * group * D)
    _need(k_new, "k_new", cache.k_pool.dtype, B * Hkv * D)
    _need(v_new, "v_new", cache.k_pool.dtype, B * Hkv * D)
    _need(t_pos, "t_pos", torch.int32, B)
    _need(score, "score", torch.float32, B * Hkv * cache.max_slots)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    _need(workspace, "workspace", torch.uint8)
    if evicted is None:
        evicted = torch.empty((B, Hkv), dtype=torch.int32, device=q.device)
    _need(evicted, "evicted", torch.int32, B * Hkv)
    if attn_out is not None:
        _need(attn_out, "attn_out", torch.float32, B * Hkv * group * D)
    rc = L.kvev_h2o_step(ctypes.byref(c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(t_pos), group,
                         scale, _ptr(score), budget, recent, _ptr(free_list), _ptr(free_count),
                         _ptr(evicted), _ptr(attn_out), _ptr(workspace), workspace.numel(),
                         _stream(stream))
    _check(rc, "kvev_h2o_step")
    return evicted


def new_vtok_evict_workspace(cache: Cache) -> torch.Tensor:
    """A workspace for kvev_vtok_evict on this cache shape (4 bytes a slot)."""
    n = load_library().kvev_vtok_evict_workspace_bytes(ctypes.byref(cache.struct()))
    if n == 0:
        raise KvevError(EINVAL, "kvev_vtok_evict_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=cache.k_pool.device)


def vtok_evict(cache: Cache, live: torch.Tensor, block_live: torch.Tensor,
               victims: torch.Tensor, n_victims: torch.Tensor, workspace: torch.Tensor,
               status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvev_vtok_evict: mark the victim slots dead.  live uint8 [B, Hkv,
    max_slots], block_live int32 [B, Hkv, max_blocks] (both updated); victims
    int32 [B, Hkv, max_slots], n_victims int32 [B, Hkv]; workspace from
    new_vtok_evict_workspace.  Returns status int32 [1] (1 when a victim was
    out of range, already dead or repeated)."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(live, "live", torch.uint8, B * Hkv * cache.max_slots)
    _need(block_live, "block_live", torch.int32, B * Hkv * cache.max_blocks)
    _need(victims, "victims", torch.int32, B * Hkv * cache.max_slots)
    _need(n_victims, "n_victims", torch.int32, B * Hkv)
    _need(workspace, "workspace", torch.uint8)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=live.device)
    _need(status, "status", torch.int32, 1)
    rc = L.kvev_vtok_evict(ctypes.byref(c), _ptr(live), _ptr(block_live), _ptr(victims),
                           _ptr(n_victims), _ptr(status), _ptr(workspace), workspace.numel(),
                           _stream(stream))
    _check(rc, "kvev_vtok_evict")
    return status


def new_vtok_workspace(cache: Cache, max_sources: int) -> torch.Tensor:
    """A workspace for kvev_vtok_reclaim on this cache shape."""
    n = load_library().kvev_vtok_workspace_bytes(ctypes.byref(cache.struct()), max_sources)
    if n == 0:
        raise KvevError(EINVAL, "kvev_vtok_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=cache.k_pool.device)


def vtok_reclaim(cache: Cache, live: torch.Tensor, block_live: torch.Tensor, theta_f: float,
                 max_sources: int, free_list: torch.Tensor, free_count: torch.Tensor,
                 workspace: torch.Tensor, score: Optional[torch.Tensor] = None,
                 stats: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvev_vtok_reclaim: lazy, threshold-gated reclamation of every head.  live,
    block_live as in vtok_evict; score (optional) fp32 [B, Hkv, max_slots]
    moves with the tokens; free_list int32 (capacity >= num_blocks),
    free_count int32 [1]; workspace from new_vtok_workspace.  Returns stats
    int64 [10]."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(live, "live", torch.uint8, B * Hkv * cache.max_slots)
    _need(block_live, "block_live", torch.int32, B * Hkv * cache.max_blocks)
    if score is not None:
        _need(score, "score", torch.float32, B * Hkv * cache.max_slots)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    _need(workspace, "workspace", torch.uint8)
    if stats is None:
        stats = torch.empty(10, dtype=torch.int64, device=live.device)
    _need(stats, "stats", torch.int64, 10)
    rc = L.kvev_vtok_reclaim(ctypes.byref(c), _ptr(live), _ptr(block_live), _ptr(score),
                             float(theta_f), max_sources, _ptr(free_list), _ptr(free_count),
                             free_list.numel(), _ptr(stats), _ptr(workspace), workspace.numel(),
                             _stream(stream))
    _check(rc, "kvev_vtok_reclaim")
    return stats


def vtok_digest(cache: Cache, live: torch.Tensor, digest: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """kvev_vtok_digest: per-head digest of the live tokens (I1's online
    check).  Returns int64 [B, Hkv] holding the uint64 digests' bits."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(live, "live", torch.uint8, B * Hkv * cache.max_slots)
    if digest is None:
        digest = torch.empty((B, Hkv), dtype=torch.int64, device=live.device)
    _need(digest, "digest", torch.int64, B * Hkv)
    _check(L.kvev_vtok_digest(ctypes.byref(c), _ptr(live), _ptr(digest), _stream(stream)),
           "kvev_vtok_digest")
    return digest


def vtok_sync(cache: Cache, live: torch.Tensor, block_live: torch.Tensor, new_len: torch.Tensor,
              pos0: torch.Tensor, status: Optional[torch.Tensor] = None, stream=None):
    """kvev_vtok_sync: register the slots [seq_len, new_len) as live tokens at
    positions pos0[b] + k.  Returns status int32 [B, Hkv]."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(live, "live", torch.uint8, B * Hkv * cache.max_slots)
    _need(block_live, "block_live", torch.int32, B * Hkv * cache.max_blocks)
    _need(new_len, "new_len", torch.int32, B * Hkv)
    _need(pos0, "pos0", torch.int32, B)
    if status is None:
        status = torch.empty((B, Hkv), dtype=torch.int32, device=live.device)
    _need(status, "status", torch.int32, B * Hkv)
    _check(L.kvev_vtok_sync(ctypes.byref(c), _ptr(live), _ptr(block_live), _ptr(new_len),
                            _ptr(pos0), _ptr(status), _stream(stream)), "kvev_vtok_sync")
    return status


def vtok_slot_mapping(cache: Cache, live: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                      stream=None):
    """kvev_vtok_slot_mapping -> (slots, positions int32 [B, Hkv, max_slots],
    count int32 [B, Hkv]): every live token's physical row by Eq. 2."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(live, "live", torch.uint8, B * Hkv * cache.max_slots)
    if workspace is None:
        workspace = torch.empty(L.kvev_vtok_map_workspace_bytes(ctypes.byref(c)),
                                dtype=torch.uint8, device=live.device)
    _need(workspace, "workspace", torch.uint8)
    slots = torch.empty((B, Hkv, cache.max_slots), dtype=torch.int32, device=live.device)
    positions = torch.empty_like(slots)
    count = torch.empty((B, Hkv), dtype=torch.int32, device=live.device)
    _check(L.kvev_vtok_slot_mapping(ctypes.byref(c), _ptr(live), _ptr(slots), _ptr(positions),
                                    _ptr(count), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "kvev_vtok_slot_mapping")
    return slots, positions, count


def new_vtok_check_workspace(cache: Cache) -> torch.Tensor:
    n = load_library().kvev_vtok_check_workspace_bytes(ctypes.byref(cache.struct()))
    if n == 0:
        raise KvevError(EINVAL, "kvev_vtok_check_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=cache.k_pool.device)


def vtok_check(cache: Cache, live: torch.Tensor, block_live: torch.Tensor,
               free_list: torch.Tensor, free_count: torch.Tensor, workspace: torch.Tensor,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvev_vtok_check: I2 and the live counts.  Returns int64 [4] = {blocks
    held more than once, held by nobody, references out of range, live-count
    mismatches}."""
    L = load_library()
    c = cache.struct()
    B, Hkv = cache.batch, cache.kv_heads
    _need(live, "live", torch.uint8, B * Hkv * cache.max_slots)
    _need(block_live, "block_live", torch.int32, B * Hkv * cache.max_blocks)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty(4, dtype=torch.int64, device=live.device)
    _need(out, "out", torch.int64, 4)
    _check(L.kvev_vtok_check(ctypes.byref(c), _ptr(live), _ptr(block_live), _ptr(free_list),
                             _ptr(free_count), free_list.numel(), _ptr(out), _ptr(workspace),
                             workspace.numel(), _stream(stream)), "kvev_vtok_check")
    return out


class RingState:
    """The SnapKV ring-buffer state of a cache: hist fp32 [B, Hkv, W,
    max_slots], ring int32 [B, Hkv], rank int32 [B, Hkv, max_slots], and
    the step's zero-filled workspace per (group, budget), allocated by the
    first step that needs it (take that step before capturing a graph)."""

    def __init__(self, cache: Cache, obs_window: int, stream=None):
        B, Hkv, dev_ = cache.batch, cache.kv_heads, cache.k_pool.device
        self.W = obs_window
        self.ws = {}
        self.hist = torch.empty((B, Hkv, obs_window, cache.max_slots), dtype=torch.float32,
                                device=dev_)
        self.ring = torch.empty((B, Hkv), dtype=torch.int32, device=dev_)
        self.rank = torch.zeros((B, Hkv, cache.max_slots), dtype=torch.int32, device=dev_)
        _check(load_library().kvev_ring_init(ctypes.byref(cache.struct()), _ptr(self.hist),
                                             _ptr(self.ring), _ptr(self.rank), obs_window,
                                             _stream(stream)), "kvev_ring_init")


def ring_step(cache: Cache, state: RingState, q: torch.Tensor, k_new: torch.Tensor,
              v_new: torch.Tensor, t_pos: torch.Tensor, observe: torch.Tensor, group: int,
              scale: float, budget: int, recent: int, pool_kernel: int, free_list: torch.Tensor,
              free_count: torch.Tensor, evicted: Optional[torch.Tensor] = None,
              stream=None) -> torch.Tensor:
    """kvev_ring_step: one SnapKV ring-buffer decode step of every KV head.
    observe int32 [B] (0: a null step).  Returns evicted int32 [B, Hkv]."""
    L = load_library()
    c = cache.struct()
    B, Hkv, D = cache.batch, cache.kv_heads, cache.head_dim
    _need(q, "q", cache.k_pool.dtype, B * Hkv * group * D)
    _need(k_new, "k_new", cache.k_pool.dtype, B * Hkv * D)
    _need(v_new, "v_new", cache.k_pool.dtype, B * Hkv * D)
    _need(t_pos, "t_pos", torch.int32, B)
    _need(observe, "observe", torch.int32, B)
    _need(state.hist, "hist", torch.float32, B * Hkv * state.W * cache.max_slots)
    _need(free_list, "free_list", torch.int32)
    _need(free_count, "free_count", torch.int32, 1)
    if evicted is None:
        evicted = torch.empty((B, Hkv), dtype=torch.int32, device=q.device)
    _need(evicted, "evicted", torch.int32, B * Hkv)
    ws = state.ws.get((group, budget))
    if ws is None:
        n = L.kvev_ring_workspace_bytes(ctypes.byref(c), group, budget)
        if n == 0:
            raise KvevError(EUNSUPPORTED, "kvev_ring_workspace_bytes")
        ws = state.ws[(group, budget)] = torch.zeros(n, dtype=torch.uint8, device=q.device)
    _check(L.kvev_ring_step(ctypes.byref(c), _ptr(state.hist), _ptr(state.ring), _ptr(state.rank),
                            _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(t_pos), _ptr(observe), group,
                            scale, budget, recent, state.W, pool_kernel, _ptr(free_list),
                            _ptr(free_count), _ptr(evicted), _ptr(ws), ws.numel(),
                            _stream(stream)), "kvev_ring_step")
    return evicted


def window_attn(cache: Cache, q: torch.Tensor, q_pos: torch.Tensor, scale: float, group: int,
                workspace: torch.Tensor, want_a: bool = False, lse_out=None, a_out=None,
                stream=None):
    """kvev_window_attn -> (lse fp32 [B, Hq, W], a fp32 [B, Hq, W, D] or None)."""
    L = load_library()
    c = cache.struct()
    w = _window(cache, q, None, q_pos, scale, group)
    if lse_out is None:
        lse_out = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _need(lse_out, "lse_out", torch.float32, q.shape[0] * q.shape[1] * q.shape[2])
    if want_a and a_out is None:
        a_out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if a_out is not None:
        _need(a_out, "a_out", torch.float32, q.numel())
    _need(workspace, "workspace", torch.uint8)
    rc = L.kvev_window_attn(ctypes.byref(c), ctypes.byref(w), _ptr(lse_out), _ptr(a_out),
                            _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "kvev_window_attn")
    return lse_out, a_out
