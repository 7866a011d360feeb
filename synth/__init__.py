"""Seeded synthetic inputs for the KV-cache eviction path.

This module only builds inputs.  It holds none of the eviction method's
arithmetic; the CPU oracle and the GPU path both read the arrays it returns.
Random numbers come from a counter-based SplitMix64 generator with Box-Muller
normals, implemented in ``synth.c`` (built to ``libsynth.so`` next to it).

The workload recipes follow the shapes and structure of the pages' workloads
(H2O heavy hitters, SnapKV salient spans, DropKV near-mean value rows); the
public datasets the pages evaluate on are not reproduced, these seeded tensors
stand in for them.

Layout of a case (all numpy, host memory):
  k_pool, v_pool : [num_blocks, 16, D]   float32 or uint16 (bf16 bits)
  block_table    : int32 [B, Hkv, max_blocks], -1 = no block
  seq_len        : int32 [B, Hkv]           live tokens per KV head
  pos            : int32 [B, Hkv, max_blocks*16]  original position of a slot
  q              : [B, Hkv*G, W, D]          cache dtype
  q_pos          : int32 [B, W]             positions of the window queries
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
BLOCK = 16

# tensor ids for the counter streams
T_Q, T_K, T_V, T_DIR, T_PLANT, T_NEARMEAN, T_PERM, T_SPAN, T_DECODE_Q, T_MISC, T_VICTIM = range(1, 12)


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, u64 = ctypes.c_int64, ctypes.c_uint64
        L.synth_u64.argtypes = [u64, u64, u64]
        L.synth_u64.restype = u64
        L.synth_uniform.argtypes = [P, i64, u64, u64, i64]
        L.synth_normal.argtypes = [P, i64, u64, u64, i64]
        L.synth_f32_to_bf16.argtypes = [P, P, i64]
        L.synth_f64_to_bf16.argtypes = [P, P, i64]
        L.synth_bf16_to_f32.argtypes = [P, P, i64]
        L.synth_shuffle_i32.argtypes = [P, i64, u64, u64]
        L.synth_fill_paged.argtypes = [P, ctypes.c_int, P, i64, i64, i64, i64, P, u64, u64,
                                       P, P, P, ctypes.c_float, ctypes.c_int]
        L.synth_fill_paged.restype = ctypes.c_int
        L.synth_fill_rows.argtypes = [P, ctypes.c_int, i64, i64, u64, u64, P, P, P,
                                      ctypes.c_float]
        L.synth_fill_rows.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def stream_id(tensor: int, unit: int = 0, layer: int = 0) -> int:
    return (layer << 48) | (tensor << 32) | unit


def uniform(n: int, seed: int, stream: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform(_ptr(out), n, seed, stream, offset)
    return out


def normal(n: int, seed: int, stream: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normal(_ptr(out), n, seed, stream, offset)
    return out


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (round to nearest even, through float32); returns uint16 bits."""
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, np.uint16)
    if x.dtype == np.float64:
        lib().synth_f64_to_bf16(_ptr(x), _ptr(out), x.size)
    else:
        x32 = np.ascontiguousarray(x, dtype=np.float32)
        lib().synth_f32_to_bf16(_ptr(x32), _ptr(out), x32.size)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().synth_bf16_to_f32(_ptr(bits), _ptr(out), bits.size)
    return out


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Encode float data in the cache dtype ('f32' -> float32, 'bf16' -> uint16 bits)."""
    if dtype == "bf16":
        return to_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of cache-dtype data."""
    if dtype == "bf16":
        return bf16_to_f32(x)
    return np.asarray(x, dtype=np.float32)


def shuffled(n: int, seed: int, stream: int) -> np.ndarray:
    perm = np.arange(n, dtype=np.int32)
    lib().synth_shuffle_i32(_ptr(perm), n, seed, stream)
    return perm


@dataclasses.dataclass
class Config:
    """One workload.  Sizes are per layer; `recipe` picks the value structure."""
    name: str
    B: int
    Hkv: int
    G: int
    D: int
    L: int                 # live tokens per KV head when scoring starts
    W: int                 # observation window (queries per call)
    dtype: str             # "f32" or "bf16"
    recipe: str            # "iid", "heavy_hitters", "spans", "near_mean"
    flags: tuple           # score kinds used: subset of ("sum", "pool", "drop")
    pool_kernel: int = 1
    budget: int = 0
    recent: int = 0
    scale: Optional[float] = None   # softmax scale; None -> 1/sqrt(D)
    value_std: float = 1.0          # std of the iid draws
    decode_steps: int = 0           # H2O decode schedule: tokens appended one by one
    layers: int = 1
    seed: int = 1000
    plant_frac: float = 0.0
    plant_sigmas: float = 3.0
    nearmean_frac: float = 0.0
    nearmean_std: float = 0.05
    span_min: int = 8
    span_max: int = 64

    @property
    def Hq(self) -> int:
        return self.Hkv * self.G

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.D) if self.scale is None else self.scale

    @property
    def L_final(self) -> int:
        return self.L + self.decode_steps

    def scaled(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads.  Percent budgets are floored; where no recent window is
# given it equals the observation window.
CONFIGS = {
    "tiny_f32": Config("tiny_f32", B=1, Hkv=2, G=2, D=64, L=512, W=8, dtype="f32", recipe="iid",
                       flags=("sum", "pool", "drop"), pool_kernel=5, budget=128, recent=32,
                       scale=1.0, value_std=1.0 / 8.0, seed=1001),
    "h2o_decode_4k": Config("h2o_decode_4k", B=8, Hkv=8, G=4, D=128, L=4096, W=1, dtype="bf16",
                            recipe="heavy_hitters", flags=("sum",), decode_steps=256,
                            budget=870, recent=435, plant_frac=0.02, seed=1002),
    "snapkv_prefill_32k": Config("snapkv_prefill_32k", B=4, Hkv=8, G=4, D=128, L=32768, W=32,
                                 dtype="bf16", recipe="spans", flags=("pool",), pool_kernel=7,
                                 budget=2048, recent=32, plant_frac=0.01, seed=1003),
    "dropkv_128k": Config("dropkv_128k", B=1, Hkv=8, G=8, D=128, L=131072, W=32, dtype="bf16",
                          recipe="near_mean", flags=("drop",), budget=6553, recent=32,
                          nearmean_frac=0.1, seed=1004),
    "block_evict_64k": Config("block_evict_64k", B=16, Hkv=8, G=8, D=128, L=64000, W=16,
                              dtype="bf16", recipe="heavy_hitters", flags=("sum",), budget=32000,
                              recent=16, layers=8, plant_frac=0.02, seed=1005),
    # Decode-time H2O lifecycle at the decode workload's final budget (870 of
    # 4352 tokens, 435 recent): the cache enters with 806 tokens, so the first
    # 64 steps append and every later step prunes one token.
    "h2o_stream_870": Config("h2o_stream_870", B=8, Hkv=8, G=4, D=128, L=806, W=1, dtype="bf16",
                             recipe="heavy_hitters", flags=("sum",), decode_steps=256,
                             budget=870, recent=435, plant_frac=0.02, seed=1006),
    # SnapKV's decode-time ring buffer on the H2O decode lifecycle's shape:
    # obsWindow 32 (the field W), poolKernel 7, recent window 32, budget 870.
    "snap_ring_870": Config("snap_ring_870", B=8, Hkv=8, G=4, D=128, L=806, W=32, dtype="bf16",
                            recipe="heavy_hitters", flags=("pool",), pool_kernel=7,
                            decode_steps=256, budget=870, recent=32, plant_frac=0.02, seed=1008),
    # vToken lazy reclamation on one layer of the block-aware shape: half of
    # every head's 64000 tokens marked dead by a uniform random policy (the 16
    # most recent protected), then one reclamation over each head's blocks.
    "vtok_reclaim_64k": Config("vtok_reclaim_64k", B=16, Hkv=8, G=8, D=128, L=64000, W=16,
                               dtype="bf16", recipe="iid", flags=("sum",), budget=32000,
                               recent=16, seed=1007),
}


def _unit_dirs(cfg: Config, layer: int) -> np.ndarray:
    """One random unit direction per (b, kv head): [B*Hkv, D] float32."""
    U = cfg.B * cfg.Hkv
    z = normal(U * cfg.D, cfg.seed, stream_id(T_DIR, 0, layer)).reshape(U, cfg.D)
    z /= np.linalg.norm(z, axis=1, keepdims=True)
    return np.ascontiguousarray(z, dtype=np.float32)


def _heavy_hitter_mask(cfg: Config, layer: int, rows: int) -> np.ndarray:
    """plant_frac of all positions (uniform, without replacement) per unit."""
    U = cfg.B * cfg.Hkv
    mask = np.zeros((U, rows), np.uint8)
    count = int(math.ceil(cfg.plant_frac * cfg.L_final))
    for u in range(U):
        perm = shuffled(cfg.L_final, cfg.seed, stream_id(T_PLANT, u, layer))
        mask[u, perm[:count]] = 1
    return mask


def _span_mask(cfg: Config, layer: int, rows: int) -> np.ndarray:
    """Non-overlapping spans of span_min..span_max tokens, starts in [0, L-W),
    drawn until they cover at least ceil(plant_frac*L) positions."""
    U = cfg.B * cfg.Hkv
    mask = np.zeros((U, rows), np.uint8)
    need = int(math.ceil(cfg.plant_frac * cfg.L))
    hi = cfg.L - cfg.W
    for u in range(U):
        draws = uniform(4096, cfg.seed, stream_id(T_SPAN, u, layer))
        k = covered = 0
        while covered < need and k + 1 < draws.size:
            length = cfg.span_min + int(draws[k] * (cfg.span_max - cfg.span_min + 1))
            start = int(draws[k + 1] * hi)
            k += 2
            if start + length > hi or mask[u, start:start + length].any():
                continue
            mask[u, start:start + length] = 1
            covered += length
    return mask


def make_case(cfg: Config, layer: int = 0, seq_len: Optional[np.ndarray] = None,
              spare_blocks: int = 0, nthreads: int = 0) -> dict:
    """Build one layer's paged cache and observation window for `cfg`.

    seq_len overrides the live length per KV head (ragged tests); the
    capacity of every head is ceil(L_final/16) blocks.
    """
    B, Hkv, G, D, W = cfg.B, cfg.Hkv, cfg.G, cfg.D, cfg.W
    U = B * Hkv
    max_blocks = (cfg.L_final + BLOCK - 1) // BLOCK
    max_slots = max_blocks * BLOCK
    num_blocks = U * max_blocks + spare_blocks
    if nthreads <= 0:
        nthreads = max(1, min(16, len(os.sched_getaffinity(0))))
    is_bf16 = 1 if cfg.dtype == "bf16" else 0
    edt = np.uint16 if is_bf16 else np.float32

    perm = shuffled(num_blocks, cfg.seed, stream_id(T_PERM, 0, layer))
    block_table = np.full((B, Hkv, max_blocks), -1, np.int32)
    block_table.reshape(U, max_blocks)[:] = perm[:U * max_blocks].reshape(U, max_blocks)
    if seq_len is None:
        seq_len = np.full((B, Hkv), cfg.L, np.int32)
    seq_len = np.ascontiguousarray(seq_len, dtype=np.int32).reshape(B, Hkv)
    assert seq_len.min() >= 0 and seq_len.max() <= max_slots
    pos = np.broadcast_to(np.arange(max_slots, dtype=np.int32), (B, Hkv, max_slots)).copy()

    dirs = None
    plant = None
    row_scale_v = None
    if cfg.recipe in ("heavy_hitters", "spans"):
        dirs = _unit_dirs(cfg, layer)
        plant = (_heavy_hitter_mask(cfg, layer, max_slots) if cfg.recipe == "heavy_hitters"
                 else _span_mask(cfg, layer, max_slots))
    if cfg.recipe == "near_mean":
        r = uniform(U * max_slots, cfg.seed, stream_id(T_NEARMEAN, 0, layer)).reshape(U, max_slots)
        row_scale_v = np.where(r < cfg.nearmean_frac, cfg.nearmean_std, 1.0).astype(np.float32)
    row_scale_k = None
    if cfg.value_std != 1.0:
        row_scale_k = np.full((U, max_slots), cfg.value_std, np.float32)
        if row_scale_v is None:
            row_scale_v = row_scale_k
    # fill every slot up to capacity so decode appends find their rows in place
    fill_rows = np.full(U, cfg.L_final, np.int32)

    k_pool = np.zeros((num_blocks, BLOCK, D), edt)
    v_pool = np.zeros((num_blocks, BLOCK, D), edt)
    amp = cfg.plant_sigmas * math.sqrt(2.0)
    lib().synth_fill_paged(_ptr(k_pool), is_bf16, _ptr(block_table), U, max_blocks, max_slots, D,
                           _ptr(fill_rows), cfg.seed, stream_id(T_K, 0, layer), _ptr(row_scale_k),
                           _ptr(plant), _ptr(dirs), amp, nthreads)
    lib().synth_fill_paged(_ptr(v_pool), is_bf16, _ptr(block_table), U, max_blocks, max_slots, D,
                           _ptr(fill_rows), cfg.seed, stream_id(T_V, 0, layer), _ptr(row_scale_v),
                           None, None, 0.0, nthreads)

    q, q_pos = make_queries(cfg, layer, W, dirs, step=None)
    return dict(cfg=cfg, layer=layer, dtype=cfg.dtype, B=B, Hkv=Hkv, G=G, D=D, W=W,
                max_blocks=max_blocks, num_blocks=num_blocks, k_pool=k_pool, v_pool=v_pool,
                block_table=block_table, seq_len=seq_len, pos=pos, q=q, q_pos=q_pos,
                scale=cfg.softmax_scale, dirs=dirs, plant=plant)


def make_queries(cfg: Config, layer: int, W: int, dirs: Optional[np.ndarray],
                 step: Optional[int]) -> tuple:
    """Window queries [B, Hq, W, D] and their positions [B, W].

    Prefill windows sit at the last W positions of L.  A decode step t has one
    query, the token appended at position L + t, drawn from its own stream.
    Planted recipes add sqrt(D)*u of the query's KV head.
    """
    B, Hkv, G, D = cfg.B, cfg.Hkv, cfg.G, cfg.D
    Hq = Hkv * G
    n_rows = B * Hq * W
    dir_of_row = None
    if dirs is not None:
        unit = (np.arange(B)[:, None] * Hkv + np.arange(Hq)[None, :] // G)  # [B, Hq]
        dir_of_row = np.ascontiguousarray(np.repeat(unit[:, :, None], W, axis=2).reshape(-1),
                                          dtype=np.int32)
    row_scale = None
    if cfg.value_std != 1.0:
        row_scale = np.full(n_rows, cfg.value_std, np.float32)
    is_bf16 = 1 if cfg.dtype == "bf16" else 0
    q = np.zeros((B, Hq, W, D), np.uint16 if is_bf16 else np.float32)
    stream = stream_id(T_Q, 0, layer) if step is None else stream_id(T_DECODE_Q, step, layer)
    lib().synth_fill_rows(_ptr(q), is_bf16, n_rows, D, cfg.seed, stream, _ptr(row_scale),
                          _ptr(dir_of_row), _ptr(dirs), math.sqrt(D))
    if step is None:
        q_pos = np.broadcast_to(np.arange(cfg.L - W, cfg.L, dtype=np.int32), (B, W)).copy()
    else:
        q_pos = np.full((B, W), cfg.L + step, np.int32)
    return q, q_pos


def decode_token_kv(case: dict, step: int) -> tuple:
    """Key and value rows [B, Hkv, D] (cache dtype) of the token a decode step
    appends: position L + step, generated in place at that slot by make_case."""
    cfg = case["cfg"]
    s = cfg.L + step
    B, Hkv = case["B"], case["Hkv"]
    blk = case["block_table"][:, :, s // BLOCK]          # [B, Hkv]
    k = case["k_pool"][blk.reshape(-1), s % BLOCK].reshape(B, Hkv, -1)
    v = case["v_pool"][blk.reshape(-1), s % BLOCK].reshape(B, Hkv, -1)
    return np.ascontiguousarray(k), np.ascontiguousarray(v)



def random_victims(case: dict, budget: int, recent: int) -> tuple:
    """Victims of a uniform random eviction policy: for every KV head of
    length n, n - budget positions drawn without replacement from the first
    n - recent (none when n <= budget), ascending.  Returns (victims int32
    [B, Hkv, max_slots], -1 past the count; n_victims int32 [B, Hkv])."""
    cfg = case["cfg"]
    B, Hkv = case["B"], case["Hkv"]
    ms = case["max_blocks"] * BLOCK
    vic = np.full((B, Hkv, ms), -1, np.int32)
    nv = np.zeros((B, Hkv), np.int32)
    for b in range(B):
        for h in range(Hkv):
            n = int(case["seq_len"][b, h])
            m = n - budget
            if m <= 0:
                continue
            pool = n - recent
            perm = shuffled(pool, cfg.seed, stream_id(T_VICTIM, b * Hkv + h, case["layer"]))
            vic[b, h, :m] = np.sort(perm[:m])
            nv[b, h] = m
    return vic, nv
