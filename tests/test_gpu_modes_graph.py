"""The other output modes captured in a HIP graph: the sglang-compatible
records, the FP8 mode, the fake quant and the FP4 MQA-logits scorer, each
captured once and replayed three times with new inputs copied in (eager work)
between replays; every replay must equal the oracle on that replay's inputs,
byte for byte (the scorer: within its fp32 bound)."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import SENTINEL
from harness import assert_same, say

pytestmark = pytest.mark.gpu


def _capture(step):
    import torch
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _inputs(rep, T, H):
    wl = workloads.sweep_case(900 + rep, T, H, True, 64)
    return wl


def test_sglang_graph_replay():
    import torch
    from pack_token_amd import fp4idx
    dev = "cuda:0"
    T, H, n = 40, 32, 64
    base = _inputs(0, T, H)
    q = torch.from_numpy(base.q.view(np.int16)).to(dev)
    k = torch.from_numpy(base.k.view(np.int16)).to(dev)
    pos = torch.from_numpy(base.positions).to(dev)
    cs = torch.from_numpy(base.cos_sin).to(dev)
    slots = torch.arange(1, T + 1, dtype=torch.int64, device=dev)
    qp = torch.empty((T, H, 68), dtype=torch.uint8, device=dev)
    cache = torch.empty((n, 68), dtype=torch.uint8, device=dev)

    def step():
        fp4idx.q_rope_pack_sglang(q, pos, cs, q_packed=qp, pack_floor=1e-3)
        fp4idx.k_rope_pack_store_sglang(k, pos, cs, slots, cache, compress_ratio=2, pack_floor=1e-3)

    g = _capture(step)
    for rep in range(1, 4):
        wl = _inputs(rep, T, H)
        q.copy_(torch.from_numpy(wl.q.view(np.int16)).to(dev))
        k.copy_(torch.from_numpy(wl.k.view(np.int16)).to(dev))
        cache.fill_(SENTINEL)
        torch.cuda.synchronize()
        say(f"case sglang graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert_same("q_packed", qp.cpu().numpy(),
                    oracle.q_rope_pack_sglang(wl.q, base.positions, base.cos_sin, pack_floor=1e-3))
        ref = np.full((n, 68), SENTINEL, np.uint8)
        oracle.k_rope_pack_store_sglang(wl.k, base.positions, base.cos_sin,
                                        np.arange(1, T + 1, dtype=np.int64), ref,
                                        compress_ratio=2, pack_floor=1e-3)
        assert_same("index_k_cache", cache.cpu().numpy(), ref)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
def test_fp8_graph_replay(fmt):
    import torch
    from pack_token_amd import fp4idx
    dev = "cuda:0"
    T, H = 600, 32                       # above the small-batch size on purpose
    base = _inputs(10, T, H)
    q = torch.from_numpy(base.q.view(np.int16)).to(dev)
    k = torch.from_numpy(base.k.view(np.int16)).to(dev)
    pos = torch.from_numpy(base.positions).to(dev)
    cs = torch.from_numpy(base.cos_sin).to(dev)
    w = torch.from_numpy(base.weights).to(dev)
    slots = torch.from_numpy(base.slot_mapping).to(dev)
    q_out = torch.empty((T, H, 128), dtype=torch.uint8, device=dev)
    w_out = torch.empty((T, H), dtype=torch.int16, device=dev)
    kv = torch.empty((base.NB, 64, 128), dtype=torch.uint8, device=dev)
    ks = torch.empty((base.NB, 64), dtype=torch.float32, device=dev)
    ofmt = {"ue8m0": 0, "fp32": 1}[fmt]

    def step():
        fp4idx.q_rope_pack_fp8(q, pos, cs, w, q_out=q_out, weights_out=w_out, scale_fmt=fmt,
                               weights_scale=0.25)
        fp4idx.k_rope_pack_store_fp8(k, pos, cs, slots, kv, ks, scale_fmt=fmt)

    g = _capture(step)
    for rep in range(11, 14):
        wl = _inputs(rep, T, H)
        q.copy_(torch.from_numpy(wl.q.view(np.int16)).to(dev))
        k.copy_(torch.from_numpy(wl.k.view(np.int16)).to(dev))
        w.copy_(torch.from_numpy(wl.weights).to(dev))
        kv.fill_(SENTINEL)
        ks.fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"case fp8 graph replay {fmt} {rep}")
        g.replay()
        torch.cuda.synchronize()
        rq, rw = oracle.q_rope_pack_fp8(wl.q, base.positions, base.cos_sin, wl.weights,
                                        weights_scale=0.25, scale_fmt=ofmt)
        assert_same("q_out", q_out.cpu().numpy(), rq)
        assert_same("weights_out", w_out.cpu().numpy().view(np.uint16), rw)
        rkv = np.full((base.NB, 64, 128), SENTINEL, np.uint8)
        rks = np.full((base.NB, 64), np.nan, np.float32)
        oracle.k_rope_pack_store_fp8(wl.k, base.positions, base.cos_sin, base.slot_mapping, rkv,
                                     rks, scale_fmt=ofmt)
        assert_same("kv_cache", kv.cpu().numpy(), rkv)
        assert_same("kv_cache_scale", ks.cpu().numpy(), rks)


@pytest.mark.parametrize("mode", ["ue8m0_32", "e4m3_16"])
def test_fake_quant_graph_replay(mode):
    import torch
    from pack_token_amd import fp4idx
    dev = "cuda:0"
    T, H = 50, 32
    base = _inputs(20, T, H)
    x = torch.from_numpy(base.q.view(np.int16)).to(dev)
    pos = torch.from_numpy(base.positions).to(dev)
    cs = torch.from_numpy(base.cos_sin).to(dev)
    y = torch.empty((T, H, 128), dtype=torch.int16, device=dev)
    m = {"ue8m0_32": 0, "e4m3_16": 1}[mode]

    def step():
        fp4idx.rope_fake_quant(x, pos, cs, y=y, rows_per_position=H, mode=mode, compress_ratio=4)

    g = _capture(step)
    for rep in range(21, 24):
        wl = _inputs(rep, T, H)
        x.copy_(torch.from_numpy(wl.q.view(np.int16)).to(dev))
        torch.cuda.synchronize()
        say(f"case fake quant graph replay {mode} {rep}")
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.rope_fake_quant(wl.q, base.positions, base.cos_sin, rows_per_position=H,
                                     mode=m, compress_ratio=4)
        assert_same("y", y.cpu().numpy().view(np.uint16), ref)


@pytest.mark.parametrize("next_n,H", [(4, 32), (67, 64)])
def test_scorer_graph_replay(next_n, H):
    """The FP4 MQA-logits scorer (decode, and chunked prefill with its LDS
    fetch-ahead) captured once and replayed three times with new query and key
    bytes copied in between; every replay within the scorer's fp32 bound of the
    oracle, -inf and untouched entries identical."""
    import torch
    from pack_token_amd import fp4idx
    from test_gpu_scorer import SENT, check_scorer
    dev = "cuda:0"
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    base = workloads.scorer_case(5000 + next_n, 3, next_n, H, 1, 900)
    q, qs, w = up(base.q_out), up(base.q_scale_out), up(base.weights)
    kv, ks = up(base.kv_cache), up(base.kv_cache_scale)
    table, ctx = up(base.block_table), up(base.context_lens)
    stride = base.max_blocks * 64
    logits = torch.full((base.B * next_n, stride), float(SENT), dtype=torch.float32, device=dev)

    def step():
        fp4idx.paged_mqa_logits(q, qs, w, kv, ks, table, ctx, next_n, weights_scale=0.5,
                                logits=logits)

    g = _capture(step)
    import copy
    for rep in range(1, 4):
        rng = np.random.default_rng(rep)
        sc = copy.copy(base)   # same shapes, tables and scales; new codes and weights
        sc.q_out = rng.integers(0, 256, base.q_out.shape, dtype=np.uint8)
        sc.kv_cache = rng.integers(0, 256, base.kv_cache.shape, dtype=np.uint8)
        sc.weights = rng.random(base.weights.shape, dtype=np.float32)
        q.copy_(up(sc.q_out))
        qs.copy_(up(sc.q_scale_out))
        w.copy_(up(sc.weights))
        kv.copy_(up(sc.kv_cache))
        ks.copy_(up(sc.kv_cache_scale))
        logits.fill_(float(SENT))
        torch.cuda.synchronize()
        say(f"case scorer graph replay next_n={next_n} H={H} rep {rep}")
        g.replay()
        torch.cuda.synchronize()
        ref, bound = oracle.paged_mqa_logits(sc.q_out, sc.q_scale_out, sc.weights, sc.kv_cache,
                                             sc.kv_cache_scale, sc.block_table, sc.context_lens,
                                             next_n, weights_scale=0.5, with_bound=True)
        check_scorer(logits.cpu().numpy(), ref, bound, H)
