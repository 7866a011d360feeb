"""Resume: a decode schedule split in two, its state saved to a file and
loaded into fresh device buffers in between, ends bit for bit where the
uninterrupted schedule ends ([VTOK] section 3.5, I1: the cache's content
is checked by comparison; every piece of state the path carries between
calls lives in the caller's tensors, none in the library).

* H2O decode-time accumulation (the 4096-token workload's schedule at a
  reduced batch): ACCUMULATE scoring steps 0..127, save, load, steps
  128..255, then selection and compaction to the budget.
* The H2O decode step (kvev_h2o_step, attend + accumulate + prune per step):
  40 steps, save, load, 40 more.
Saved with torch.save and read back with torch.load(weights_only=True).
"""
import numpy as np
import pytest
import torch

import kv_cache_eviction_qk_amd as K
import oracle
import synth
from tests.gpu_helpers import dev, device_cache, host
from tests.helpers import rounded_window_inputs

pytestmark = pytest.mark.gpu


def _roundtrip(path, tensors):
    torch.save({k: t.cpu() for k, t in tensors.items()}, path)
    loaded = torch.load(path, weights_only=True)
    return {k: t.cuda() for k, t in loaded.items()}


def _cache_tensors(c):
    return dict(k_pool=c.k_pool, v_pool=c.v_pool, block_table=c.block_table, seq_len=c.seq_len,
                pos=c.pos)


def test_decode_accumulation_resumes_bitwise(tmp_path):
    cfg = synth.CONFIGS["h2o_decode_4k"].scaled(B=2, Hkv=2, L=1024)
    steps, split = cfg.decode_steps, cfg.decode_steps // 2
    assert steps == 256
    case = synth.make_case(cfg)
    B, H, G = case["B"], case["Hkv"], case["G"]
    ms = case["max_blocks"] * 16
    # every step's window query and LSE, shared by both runs
    inputs = []
    for t in range(steps):
        n = cfg.L + t + 1
        q, q_pos = synth.make_queries(cfg, 0, 1, case["dirs"], step=t)
        st = dict(case, seq_len=np.full((B, H), n, np.int32), q=q, q_pos=q_pos, W=1)
        lse64, _ = oracle.lse_a(st)
        lse32, _ = rounded_window_inputs(st, lse64)
        inputs.append((n, dev(q), dev(lse32), dev(q_pos)))

    def steps_on(c, ssum, t0, t1):
        for t in range(t0, t1):
            n, q, lse, qp = inputs[t]
            c.seq_len.fill_(n)
            K.score(c, q, lse, qp, case["scale"], G, K.SUM | K.ACCUMULATE, 1, sum=ssum)

    def finish(c, ssum):
        vic, nv = K.select(c, ssum, cfg.budget, cfg.recent)
        fl = torch.full((case["num_blocks"] + 8,), -1, dtype=torch.int32, device="cuda")
        fc = torch.zeros(1, dtype=torch.int32, device="cuda")
        stats = K.compact(c, vic, nv, fl, fc, K.new_workspace(c), score_row=ssum)
        torch.cuda.synchronize()
        out = {k: host(t) for k, t in _cache_tensors(c).items()}
        out.update(sum=host(ssum), vic=host(vic), nv=host(nv), fl=host(fl), fc=host(fc),
                   stats=host(stats))
        return out

    a = device_cache(case)
    asum = dev(np.zeros((B, H, ms), np.float32))
    steps_on(a, asum, 0, steps)
    whole = finish(a, asum)

    b = device_cache(case)
    bsum = dev(np.zeros((B, H, ms), np.float32))
    steps_on(b, bsum, 0, split)
    torch.cuda.synchronize()
    saved = _roundtrip(tmp_path / "decode.pt", dict(_cache_tensors(b), sum=bsum))
    del b, bsum
    c = K.Cache(saved["k_pool"], saved["v_pool"], saved["block_table"], saved["seq_len"],
                saved["pos"])
    steps_on(c, saved["sum"], split, steps)
    resumed = finish(c, saved["sum"])

    assert int(whole["nv"].sum()) > 0
    for k in whole:
        if k == "vic":
            for u in range(B * H):
                m = int(whole["nv"].reshape(-1)[u])
                assert np.array_equal(whole[k].reshape(B * H, ms)[u, :m],
                                      resumed[k].reshape(B * H, ms)[u, :m]), (k, u)
        elif k == "sum":  # slots past the new length are unspecified after compaction
            for u in range(B * H):
                n2 = int(whole["seq_len"].reshape(-1)[u])
                x = whole[k].reshape(B * H, ms)[u, :n2].view(np.uint32)
                y = resumed[k].reshape(B * H, ms)[u, :n2].view(np.uint32)
                assert np.array_equal(x, y), (k, u)
        else:
            assert np.array_equal(whole[k], resumed[k]), k


def test_h2o_decode_step_resumes_bitwise(tmp_path):
    cfg = synth.CONFIGS["h2o_stream_870"].scaled(B=2, Hkv=2)
    case = synth.make_case(cfg)
    B, H, G, D = case["B"], case["Hkv"], case["G"], case["D"]
    n0 = cfg.L
    steps, split = 80, 40
    budget, recent = n0 + 16, 8
    ms = case["max_blocks"] * 16
    seq = np.full((B, H), n0, np.int32)
    toks = [synth.decode_token_kv(case, t) for t in range(steps)]
    qs = [synth.make_queries(cfg, 0, 1, case["dirs"], step=t)[0][:, :, 0] for t in range(steps)]

    def fresh():
        c = device_cache(dict(case, seq_len=seq))
        state = dict(score=dev(np.zeros((B, H, ms), np.float32)),
                     fl=dev(np.full(case["num_blocks"] + 8, -1, np.int32)),
                     fc=dev(np.zeros(1, np.int32)))
        return c, state

    def run(c, state, t0, t1):
        ws = K.new_h2o_workspace(c, G, budget)
        ev = torch.empty((B, H), dtype=torch.int32, device="cuda")
        for t in range(t0, t1):
            kn, vn = toks[t]
            tpos = dev(np.full(B, n0 + t, np.int32))
            K.h2o_step(c, dev(qs[t]), dev(kn), dev(vn), tpos, G, case["scale"], state["score"],
                       budget, recent, state["fl"], state["fc"], ws, evicted=ev)
        torch.cuda.synchronize()

    a, sa = fresh()
    run(a, sa, 0, steps)
    b, sb = fresh()
    run(b, sb, 0, split)
    saved = _roundtrip(tmp_path / "step.pt", dict(_cache_tensors(b), **sb))
    del b, sb
    c = K.Cache(saved["k_pool"], saved["v_pool"], saved["block_table"], saved["seq_len"],
                saved["pos"])
    sc = {k: saved[k] for k in ("score", "fl", "fc")}
    run(c, sc, split, steps)
    for k, t in _cache_tensors(a).items():
        assert torch.equal(t, _cache_tensors(c)[k]), k
    assert host(a.seq_len).min() == budget  # the stream reached the budget and pruned
    for k in ("score", "fl", "fc"):
        x, y = host(sa[k]), host(sc[k])
        if k == "score":
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        else:
            assert np.array_equal(x, y), k
