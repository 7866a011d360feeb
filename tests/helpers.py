"""Small hand-built cases in the paged layout that both the oracle and the
GPU path read.  Test-only code: it lays out given logical rows, it computes
nothing of the method."""
from __future__ import annotations

import numpy as np

import synth

BLOCK = 16


def manual_case(k_rows, v_rows, q, q_pos, seq_len=None, dtype="f32", scale=1.0,
                perm_seed=7, extra_blocks=0, spare_blocks=0):
    """k_rows, v_rows: [B, Hkv, n_max, D] logical rows; q: [B, Hkv*G, W, D];
    q_pos: [B, W].  Rows are encoded in `dtype` and scattered to a shuffled
    block pool."""
    k_rows = np.asarray(k_rows, np.float64)
    v_rows = np.asarray(v_rows, np.float64)
    B, Hkv, n_max, D = k_rows.shape
    Hq, W = q.shape[1], q.shape[2]
    G = Hq // Hkv
    U = B * Hkv
    max_blocks = (n_max + BLOCK - 1) // BLOCK + extra_blocks
    max_slots = max_blocks * BLOCK
    num_blocks = U * max_blocks + spare_blocks
    perm = synth.shuffled(num_blocks, perm_seed, 99)
    bt = perm[:U * max_blocks].reshape(B, Hkv, max_blocks).astype(np.int32).copy()
    if seq_len is None:
        seq_len = np.full((B, Hkv), n_max, np.int32)
    seq_len = np.asarray(seq_len, np.int32).reshape(B, Hkv).copy()
    edt = np.uint16 if dtype == "bf16" else np.float32
    k_pool = np.zeros((num_blocks, BLOCK, D), edt)
    v_pool = np.zeros((num_blocks, BLOCK, D), edt)
    kf = synth.encode(k_rows.reshape(-1, D), dtype).reshape(B, Hkv, n_max, D)
    vf = synth.encode(v_rows.reshape(-1, D), dtype).reshape(B, Hkv, n_max, D)
    for b in range(B):
        for h in range(Hkv):
            for s in range(n_max):
                blk = bt[b, h, s // BLOCK]
                k_pool[blk, s % BLOCK] = kf[b, h, s]
                v_pool[blk, s % BLOCK] = vf[b, h, s]
    pos = np.broadcast_to(np.arange(max_slots, dtype=np.int32), (B, Hkv, max_slots)).copy()
    return dict(dtype=dtype, B=B, Hkv=Hkv, G=G, D=D, W=W, max_blocks=max_blocks,
                num_blocks=num_blocks, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                seq_len=seq_len, pos=pos, q=synth.encode(np.asarray(q, np.float64), dtype),
                q_pos=np.ascontiguousarray(q_pos, dtype=np.int32), scale=float(scale))


def logical_rows(case, which="k_pool"):
    """Decode the live rows back to [B, Hkv, max_slots, D] float64 (NaN past seq_len)."""
    B, Hkv, D, mb = case["B"], case["Hkv"], case["D"], case["max_blocks"]
    pool = synth.decode(case[which], case["dtype"]).astype(np.float64)
    out = np.full((B, Hkv, mb * BLOCK, D), np.nan)
    for b in range(B):
        for h in range(Hkv):
            n = case["seq_len"][b, h]
            for s in range(n):
                blk = case["block_table"][b, h, s // BLOCK]
                out[b, h, s] = pool[blk, s % BLOCK]
    return out


def rounded_window_inputs(case, lse64, a64=None):
    """LSE and the attention output as fp32: the precision in which both sides
    receive these forward-pass values, whatever the cache dtype."""
    lse32 = np.ascontiguousarray(lse64, dtype=np.float32)
    a32 = None if a64 is None else np.ascontiguousarray(a64, dtype=np.float32)
    return lse32, a32
