"""kvev_evict_noalloc, the eviction pass for callers that cannot allocate
(its workspace is the library's static per-GPU scratch array), against
kvev_evict on a workspace of its own.

Both run the same kernels, so every live output must be bit-exact: victims,
n_victims, the compacted K/V rows, pos, seq_len, block table, free list,
stats and the compacted score row.  Two calls in a row, the second on a
smaller cache with a split DropKV window (256 rows): the array keeps the
first call's contents, and the second call must clear what starts at zero
and read nothing else of them.  A cache shape whose pass needs more than
the array is refused before any work is enqueued.
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import synth
from tests.gpu_helpers import KIND, Run, dev
from tests.test_gpu_evict import _assert_same, _inputs, _ragged

pytestmark = pytest.mark.gpu

CALLS = [
    # name, overrides, kind, pool, budget, recent
    ("snapkv_prefill_32k", dict(B=2, Hkv=3, L=3001), "pool", 7, 500, 32),
    ("dropkv_128k", dict(Hkv=2, L=1500), "drop", 1, 300, 32),
]


def _noalloc(r: Run, kind, lse32, a32, pool, budget, recent):
    stats = torch.zeros(5, dtype=torch.int64, device=r.dc.k_pool.device)
    r.stats = K.evict_noalloc(r.dc, r.q, dev(lse32), r.qp, r.case["scale"], r.case["G"],
                              KIND[kind][0], budget, recent, r.score, r.vic, r.nv, r.fl, r.fc,
                              stats, pool_kernel=pool,
                              a=dev(a32) if a32 is not None else None)
    torch.cuda.synchronize()


def test_noalloc_equals_evict_two_calls():
    sizes = []
    for name, over, kind, pool, budget, recent in CALLS:
        cfg = synth.CONFIGS[name].scaled(**over)
        case = synth.make_case(cfg, seq_len=_ragged(cfg.B, cfg.Hkv, cfg.L, 5), spare_blocks=5)
        sizes.append(case["B"] * case["Hkv"] * case["max_blocks"])
        print(f"[no-alloc] {name} {over} {kind}: {sizes[-1]} blocks of slots", flush=True)
        lse32, a32 = _inputs(case, kind)
        n = Run(case)
        _noalloc(n, kind, lse32, a32, pool, budget, recent)
        f = Run(case)
        f.fused(kind, lse32, a32, pool, budget, recent)
        st = n.state()
        assert int(st["nv"].sum()) > 0
        _assert_same(st, f.state(), case["seq_len"])
    assert sizes[1] < sizes[0]  # the second call is the smaller one


def test_noalloc_refuses_a_shape_beyond_the_array():
    """256 heads of 65536 slots need 12 B x 16.8 M = 201 MB > 128 MiB: the
    call returns ENOSPACE and leaves every buffer as it was (nothing is
    enqueued).  The cache is a real one: every head empty."""
    d = "cuda"
    B, H, mb, nb = 16, 16, 4096, 16
    cache = K.Cache(torch.zeros(nb, 16, 128, dtype=torch.bfloat16, device=d),
                    torch.zeros(nb, 16, 128, dtype=torch.bfloat16, device=d),
                    torch.full((B, H, mb), -1, dtype=torch.int32, device=d),
                    torch.zeros(B, H, dtype=torch.int32, device=d),
                    torch.zeros(B, H, mb * 16, dtype=torch.int32, device=d))
    G, W = 4, 8
    q = torch.zeros(B, H * G, W, 128, dtype=torch.bfloat16, device=d)
    lse = torch.zeros(B, H * G, W, dtype=torch.float32, device=d)
    qp = torch.zeros(B, W, dtype=torch.int32, device=d)
    n = B * H * mb * 16
    score = torch.full((n,), 7.0, dtype=torch.float32, device=d)
    vic = torch.full((n,), -5, dtype=torch.int32, device=d)
    nv = torch.full((B * H,), -5, dtype=torch.int32, device=d)
    fl = torch.full((nb + 8,), -5, dtype=torch.int32, device=d)
    fc = torch.zeros(1, dtype=torch.int32, device=d)
    stats = torch.full((5,), -5, dtype=torch.int64, device=d)
    with pytest.raises(K.KvevError) as e:
        K.evict_noalloc(cache, q, lse, qp, 0.088, G, K.SUM, 100, 8, score, vic, nv, fl, fc, stats)
    assert e.value.status == K.ENOSPACE
    torch.cuda.synchronize()
    assert bool((score == 7.0).all()) and bool((vic == -5).all()) and bool((nv == -5).all())
    assert bool((stats == -5).all()) and int(fc.item()) == 0
