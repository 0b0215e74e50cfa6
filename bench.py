"""Benchmark of the fused q+k RoPE / FP4 pack + paged store on one MI355X.

One step = fp4idx_qk_rope_pack_store (query and key sides in one launch) over
the large-prefill workload (T = 131072 tokens, H = 64 heads, D = 128, neox
RoPE on dims 64..127, contiguous slots into 2048 cache blocks), inputs
resident in HBM before timing starts.  The same step as two launches
(fp4idx_q_rope_pack + fp4idx_k_rope_pack_store) is timed too and reported
under "two_call_step".  Prints one JSON line.

Algorithmic bytes (each input read once, each output written once):
  query launch, per token: 256H (q) + 4H (weights) + 8 (position) + 256 (cos/sin
      row) + 64H (q_out) + 64J (q scales) + 4H (weights_out)
  key launch, per token:   256 (k) + 8 (slot) + 64 + 4 (cache); its own reads of
      the position and the cos/sin row repeat the query launch's and are not credited
  step total, per token:   query + key = 21,844 B at H = 64.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "pack_token_amd", "csrc")
# the sources each profiled kernel is built from (a traffic record is used only
# while their hash matches the one it was taken on)
MAIN_SOURCES = ("fp4idx_device.h", "fp4idx_kernels.hip")
MODE_SOURCES = ("fp4idx_device.h", "fp4idx_modes.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qk_kernel_large_prefill_traffic.json")
PNR_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "qk_kernel_prefill_norm_rotate_traffic.json")
SGLANG_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q_sglang_kernel_sglang_prefill_traffic.json")
FP8_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "q_fp8_kernel_fp8_prefill_traffic.json")
FQ_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                               "fake_quant_token_kernel_fake_quant_prefill_traffic.json")
SCORER_SOURCES = ("fp4idx_internal.h", "fp4idx_scorer.hip")
SCORER_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                                   "mqa_logits_kernel_decode_scoring_traffic.json")


def q_bytes_per_token(H: int) -> int:
    J = ((H // 16) + 3) // 4 * 4
    return 256 * H + 4 * H + 8 + 256 + 64 * H + 64 * J + 4 * H


def k_bytes_per_token() -> int:
    return 256 + 8 + 64 + 4


def step_bytes_per_token(H: int) -> int:
    return q_bytes_per_token(H) + k_bytes_per_token()


def code_text(src: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string
    and character literals kept), so that a comment edit does not change the
    hash of the code a traffic record was taken on."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(sources=MAIN_SOURCES) -> str:
    """SHA-256 of the code of the sources a profiled kernel is built from."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def measured_traffic(path=TRAFFIC_FILE, sources=MAIN_SOURCES):
    """HBM bytes of one launch of the profiled kernel from committed rocprofv3
    FETCH_SIZE / WRITE_SIZE counts (scaled by a plain copy's counts), if they
    were taken on the current kernel sources; otherwise None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash(sources):
        return None
    return int(rec["bytes_per_launch"])


def host_cpu() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs, CPUs usable here."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_cpu_count": os.cpu_count(),
            "usable_cpus": len(os.sched_getaffinity(0))}


def median_wall(fn, reps: int = 3) -> float:
    """Median wall time (s) of reps calls of fn."""
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return sorted(ts)[len(ts) // 2]


def time_legs(legs: dict, K: int, W: int, rounds: int, stream, settle_ms: float = 0.0):
    """Times each leg (a list of calls launched back to back as one step) over
    exactly K steps per round, with only two events around the K steps.  W
    untimed steps of every leg come first, then untimed steps of the first leg
    until settle_ms of GPU time has passed (clock ramp-up).  The legs run in
    alternating order from round to round, so no leg always runs on the
    coldest or the warmest GPU.  Returns {leg: [ms per step of each round]}."""
    import torch

    names = list(legs)
    for name in names:
        for _ in range(W):
            for c in legs[name]:
                c()
    torch.cuda.synchronize()
    if settle_ms > 0:
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for c in legs[names[0]]:
            c()
        s1.record(stream)
        torch.cuda.synchronize()
        n = int(settle_ms / max(s0.elapsed_time(s1), 1e-3)) + 1
        for _ in range(n):
            for c in legs[names[0]]:
                c()
        torch.cuda.synchronize()
    out = {name: [] for name in names}
    for r in range(rounds):
        for name in (names if r % 2 == 0 else names[::-1]):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record(stream)
            for _ in range(K):
                for c in legs[name]:
                    c()
            t1.record(stream)
            torch.cuda.synchronize()
            out[name].append(t0.elapsed_time(t1) / K)
    return out


def launch_pass(calls, K: int, stream):
    """Per-launch durations (ms) of each call over K steps, each launch between
    its own pair of events on `stream` (a pass of its own, after the timed
    steps).  Returns ([mean per call], [median per call])."""
    import numpy as np
    import torch

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        for j, c in enumerate(calls):
            c()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    d = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(len(calls))]
    return [float(np.mean(x)) for x in d], [float(np.median(x)) for x in d]


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def oracle_baseline(run, n: int, what: str, T: int, threads: int = 1,
                    noun: str = "tokens") -> dict:
    """cpu_baseline record for run() processing n units (median of 3 walls)."""
    dt = median_wall(run)
    return {"value": n / dt, "unit": f"{noun}/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {T} {noun} ({what}), {threads} thread(s), median of 3 "
                      f"runs, {dt:.2f} s wall", **host_cpu()}


def cpu_baseline(wl, n_tokens: int, threads: int):
    """The CPU oracle (test infrastructure) on the first n_tokens tokens of the
    same workload, query + key path, timed on the host cores (median of 3 runs),
    and single-threaded on a smaller slice."""
    import oracle

    def run(n, th):
        kv, ks = wl.empty_cache()
        oracle.q_rope_pack(wl.q[:n], wl.positions[:n], wl.cos_sin, wl.weights[:n],
                           is_neox=wl.is_neox, rope_offset=wl.rope_offset,
                           apply_hadamard=wl.apply_hadamard, threads=th)
        oracle.k_rope_pack_store(wl.k[:n], wl.positions[:n], wl.cos_sin, wl.slot_mapping[:n], kv,
                                 ks, k_norm_gamma=wl.k_norm_gamma, k_norm_eps=wl.k_norm_eps,
                                 is_neox=wl.is_neox, rope_offset=wl.rope_offset,
                                 apply_hadamard=wl.apply_hadamard, threads=th)

    rec = oracle_baseline(lambda: run(n_tokens, threads), n_tokens,
                          "query + key path of the same workload", wl.T, threads)
    n1 = min(n_tokens, 8192)
    dt1 = median_wall(lambda: run(n1, 1))
    rec["single_thread_value"] = n1 / dt1
    rec["single_thread_sample"] = f"first {n1} tokens, 1 thread, median of 3 runs, {dt1:.2f} s wall"
    return rec


def oracle_parity(wl, outputs: dict, threads: int) -> dict:
    """The oracle (test infrastructure) on every token of the workload, its five
    outputs compared byte for byte with the GPU's: {path: mismatched bytes}."""
    import numpy as np

    import oracle

    q_out, qs, w_out = oracle.q_rope_pack(wl.q, wl.positions, wl.cos_sin, wl.weights,
                                          is_neox=wl.is_neox, rope_offset=wl.rope_offset,
                                          apply_hadamard=wl.apply_hadamard,
                                          scale_floor=wl.scale_floor, threads=threads)
    kv, ks = wl.empty_cache()
    kw = dict(k_norm_gamma=wl.k_norm_gamma, k_norm_eps=wl.k_norm_eps, is_neox=wl.is_neox,
              rope_offset=wl.rope_offset, apply_hadamard=wl.apply_hadamard,
              scale_floor=wl.scale_floor, threads=threads)
    if wl.background is not None:
        oracle.k_rope_pack_store(wl.background["k"], wl.background["positions"], wl.cos_sin,
                                 wl.background["slots"], kv, ks, **kw)
    oracle.k_rope_pack_store(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, kv, ks, **kw)
    ref = (q_out, qs, w_out.view(np.uint8), kv, ks)
    out = {}
    for path, got in outputs.items():
        bad = 0
        for g, r in zip(got, ref):
            g = g.view(np.uint8).reshape(-1)
            r = r.view(np.uint8).reshape(-1)
            if g.size != r.size:
                bad += max(g.size, r.size)
            else:
                bad += int(np.count_nonzero(g != r))
        out[path] = bad
    return out


FP4_MFMA_PEAK_TFLOPS = 10100.0
# fp32 vector lane operations per second: MI355X's published fp32 vector rate,
# 157.3 TFLOP/s with a fused multiply-add counted as two flops, is 78.6 T lane
# operations (an add, a multiply or a fused multiply-add each) per second.
# Plain (not packed) fp32 adds and fused multiply-adds issue at most of that
# rate (fp4idx_ceiling_valu, measured beside the ALU-bound kernels).
VALU_PEAK_GOPS = 157.3e3 / 2
VALU_CEILING_KINDS = ("fp32_add", "fp32_fma", "fp32_max", "bf16_pack", "fp4_convert")


def valu_ceiling(args, dev, kernel_gops: float) -> dict:
    """Issue rate of single VALU instruction kinds (fp4idx_ceiling_valu): 8
    workgroups of 256 threads per compute unit (8 wavefronts per SIMD), 8
    independent chains per lane; lane operations per second from the mean
    launch time, the fp32 adds again at 2 wavefronts per SIMD, and the
    ALU-bound kernel's rate as a fraction of the fp32-add rate."""
    import torch

    from pack_token_amd import fp4idx

    stream = torch.cuda.current_stream(dev)
    wg = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4096
    out = torch.empty(wg * 256, dtype=torch.int32, device=dev)
    rec = {"kernel": "valu_kernel (fp4idx_ceiling_valu)",
           "what": "lane operations per second of one instruction kind, 8 independent chains "
                   "per lane, 8 wavefronts per SIMD",
           "workgroups": wg, "iterations": iters}
    for kind in VALU_CEILING_KINDS:
        def call(kind=kind):
            fp4idx.ceiling_valu(kind, wg, iters, out)

        for _ in range(max(args.warmup, 2)):
            call()
        (ms,), _ = launch_pass([call], max(args.steps, 5), stream)
        rec[kind + "_Gops"] = wg * 256 * iters * 8 / (ms * 1e-3) / 1e9
    # the same adds at two wavefronts per SIMD (issue rate at low occupancy)
    wg2 = wg // 4

    def call2():
        fp4idx.ceiling_valu("fp32_add", wg2, iters, out)

    for _ in range(max(args.warmup, 2)):
        call2()
    (ms,), _ = launch_pass([call2], max(args.steps, 5), stream)
    rec["fp32_add_2_waves_per_simd_Gops"] = wg2 * 256 * iters * 8 / (ms * 1e-3) / 1e9
    rec["kernel_frac_of_fp32_add"] = kernel_gops / rec["fp32_add_Gops"]
    return rec


def alu_ops_per_token(H: int, hadamard: bool, norm: bool) -> int:
    """Algorithmic fp32 operations of one token on the Hadamard path: per
    128-row, RoPE 3 per rotated element (2 multiplies, 1 add), the FWHT 7 adds
    per element, its scale 1 multiply per element and the quantizer's scaling
    1 per element; the key RMSNorm 3 per element (square, sum, scale by the
    reciprocal root and gamma counted as one) -- comparisons, conversions and
    data movement not counted."""
    row = 64 * 3 + 128 * (1 + (8 if hadamard else 0))
    return (H + 1) * row + (128 * 3 if norm else 0)


def stream_ceiling(args, dev, read_b: int, write_b: int, kernel_gbs: float) -> dict:
    """The launch's read and written bytes as plain 1 KB streams (measured live),
    and the kernel's rate as a fraction of that stream's."""
    cg, cl, _, _ = measure_ceiling(args, dev, "stream_rw", rw=(read_b, write_b))
    return {"kernel": "stream_kernel (fp4idx_ceiling_stream)",
            "what": "the launch's read and written bytes as plain 1 KB streams, writes spread "
                    "over the reads",
            "read_bytes": read_b, "write_bytes": write_b, "GBps": cg, "launch_us": cl,
            "frac_of_peak": cg / HBM_PEAK_GBS, "kernel_frac_of_ceiling": kernel_gbs / cg}


def fp8_q_bytes_per_token(H: int) -> int:
    return 256 * H + 4 * H + 8 + 256 + 128 * H + 2 * H


def fp8_k_bytes_per_token() -> int:
    return 256 + 8 + 128 + 4


def bench_fp8(args, dev):
    """FP8 output mode over the large-prefill input (T = 131072, H = 64, neox,
    dims 64..127 rotated, contiguous slots): one step = fp4idx_q_rope_pack_fp8 +
    fp4idx_k_rope_pack_store_fp8 with ue8m0 scales; the same step with fp32
    scales is timed beside it.  Algorithmic bytes per token: query launch
    256H + 4H + 8 + 256 + 128H + 2H, key launch 256 + 8 + 128 + 4 (its position
    and cos/sin reads repeat the query launch's)."""
    import numpy as np
    import torch

    import oracle
    from pack_token_amd import fp4idx, workloads

    wl = workloads.large_prefill(T=args.tokens, H=args.heads)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k = up(wl.q.view(np.int16)), up(wl.k.view(np.int16))
    pos, cs, w = up(wl.positions), up(wl.cos_sin), up(wl.weights)
    slots = up(wl.slot_mapping)
    T, H = wl.T, wl.H
    q_out = torch.empty((T, H, 128), dtype=torch.uint8, device=dev)
    w_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((wl.NB, 64, 128), dtype=torch.uint8, device=dev)
    ks = torch.zeros((wl.NB, 64), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(fmt):
        def q_call():
            fp4idx.q_rope_pack_fp8(q, pos, cs, w, q_out=q_out, weights_out=w_out, scale_fmt=fmt,
                                   stream=stream)

        def k_call():
            fp4idx.k_rope_pack_store_fp8(k, pos, cs, slots, kv, ks, scale_fmt=fmt, stream=stream)

        legs = time_legs({"step": [q_call, k_call]}, args.steps, args.warmup, args.rounds, stream,
                         settle_ms=args.settle_ms)
        (q_l, k_l), _ = launch_pass([q_call, k_call], args.steps, stream)
        return median(legs["step"]), q_l, k_l

    ms, q_ms, k_ms = run("ue8m0")
    ms32, q_ms32, k_ms32 = run("fp32")
    qb = fp8_q_bytes_per_token(H) * T
    kb = fp8_k_bytes_per_token() * T
    q_gbs = qb / (q_ms * 1e-3) / 1e9
    rec = {
        "metric": "tokens/s and achieved HBM GB/s, FP8 (e4m3fn) q+k RoPE/quant + paged store",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16->e4m3fn", "data": "synthetic",
        "config": {"workload": "fp8_prefill", "tokens": T, "heads": H, "head_dim": 128,
                   "rope_dim": 64, "rope": "neox", "rope_offset": 64, "scale_fmt": "ue8m0",
                   "kv_blocks": wl.NB, "kv_block_size": 64, "slot_mapping": "contiguous",
                   "step": "fp4idx_q_rope_pack_fp8 + fp4idx_k_rope_pack_store_fp8"},
        "step_GBps": (qb + kb) / (ms * 1e-3) / 1e9,
        "q_kernel_us": q_ms * 1e3, "k_kernel_us": k_ms * 1e3,
        "fp32_scales": {"ms_per_step": ms32, "tokens_per_s": T / (ms32 * 1e-3),
                        "q_kernel_us": q_ms32 * 1e3, "k_kernel_us": k_ms32 * 1e3,
                        "q_kernel_GBps": qb / (q_ms32 * 1e-3) / 1e9},
        "roofline": {"kernel": "q_fp8_kernel<neox,ue8m0>", "bound": "hbm", "achieved": q_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": q_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(FP8_TRAFFIC_FILE, MODE_SOURCES) if (T, H) == (131072, 64)
                     else None,
                     "algorithmic_bytes_per_launch": qb, "launch_us": q_ms * 1e3},
    }
    if not args.no_ceilings:
        rec["ceiling"] = stream_ceiling(args, dev, (256 * H + 4 * H + 8 + 256) * T,
                                        (128 * H + 2 * H) * T, q_gbs)
    if not args.no_cpu_baseline:
        n = min(args.cpu_sample_tokens, T, 16384)

        def run():
            oracle.q_rope_pack_fp8(wl.q[:n], wl.positions[:n], wl.cos_sin, wl.weights[:n])
            rkv = np.zeros((wl.NB, 64, 128), np.uint8)
            rks = np.zeros((wl.NB, 64), np.float32)
            oracle.k_rope_pack_store_fp8(wl.k[:n], wl.positions[:n], wl.cos_sin,
                                         wl.slot_mapping[:n], rkv, rks)

        rec["cpu_baseline"] = oracle_baseline(run, n, "query + key, ue8m0", T)
    print(json.dumps(rec), flush=True)


def bench_fake_quant(args, dev):
    """RoPE tail + FP4 fake quant over the large-prefill query input (T = 131072
    tokens x H = 64 heads = 8.4 M rows of 128, neox, dims 64..127 rotated),
    per-16 E4M3 scales (the compressed-KV variant); per-32 UE8M0 timed beside it.
    Algorithmic bytes per token: 256H in + 256H out + 8 (position) + 256 (cos/sin)."""
    import numpy as np
    import torch

    import oracle
    from pack_token_amd import fp4idx, workloads

    wl = workloads.large_prefill(T=args.tokens, H=args.heads)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, pos, cs = up(wl.q.view(np.int16)), up(wl.positions), up(wl.cos_sin)
    T, H = wl.T, wl.H
    y = torch.empty((T, H, 128), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(mode):
        def call():
            fp4idx.rope_fake_quant(q, pos, cs, y=y, rows_per_position=H, mode=mode, stream=stream)
        legs = time_legs({"step": [call]}, args.steps, args.warmup, args.rounds, stream,
                         settle_ms=args.settle_ms)
        (l_ms,), _ = launch_pass([call], args.steps, stream)
        return median(legs["step"]), l_ms

    ms, l_ms = run("e4m3_16")
    ms8, l_ms8 = run("ue8m0_32")
    b = (512 * H + 8 + 256) * T
    gbs = b / (l_ms * 1e-3) / 1e9
    rec = {
        "metric": "tokens/s and achieved HBM GB/s, RoPE tail + FP4 fake quant (bf16 in, bf16 out)",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 (values on the e2m1 x e4m3 grid)",
        "data": "synthetic",
        "config": {"workload": "fake_quant_prefill", "tokens": T, "heads": H, "rows": T * H,
                   "head_dim": 128, "rope": "neox", "rope_offset": 64, "mode": "e4m3_16",
                   "step": "fp4idx_rope_fake_quant"},
        "ue8m0_32": {"ms_per_step": ms8, "launch_us": l_ms8 * 1e3,
                     "GBps": b / (l_ms8 * 1e-3) / 1e9},
        "roofline": {"kernel": "fake_quant_token_kernel<neox,e4m3_16>", "bound": "hbm",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(FQ_TRAFFIC_FILE, MODE_SOURCES) if (T, H) == (131072, 64)
                     else None,
                     "algorithmic_bytes_per_launch": b, "launch_us": l_ms * 1e3},
    }
    if not args.no_ceilings:
        rec["ceiling"] = stream_ceiling(args, dev, (256 * H + 8 + 256) * T, 256 * H * T, gbs)
    if not args.no_cpu_baseline:
        n = min(args.cpu_sample_tokens, T, 4096)
        rec["cpu_baseline"] = oracle_baseline(
            lambda: oracle.rope_fake_quant(wl.q[:n], wl.positions[:n], wl.cos_sin,
                                           rows_per_position=H, mode=oracle.FQ_E4M3_16),
            n, f"{n * H} rows, e4m3_16", T)
    print(json.dumps(rec), flush=True)


def sglang_q_bytes_per_token(H: int) -> int:
    return 256 * H + 8 + 256 + 68 * H


def sglang_k_bytes_per_token() -> int:
    return 256 + 8 + 68


def bench_sglang(args, dev):
    """sglang-compatible mode over the large-prefill input (T = 131072, H = 64,
    neox, dims 64..127 rotated): one step = fp4idx_q_rope_pack_sglang +
    fp4idx_k_rope_pack_store_sglang (two launches), keys to slots 1..T.
    Algorithmic bytes per token: query launch 256H + 8 + 256 + 68H, key launch
    256 + 8 + 68 (its position and cos/sin reads repeat the query launch's)."""
    import numpy as np
    import torch

    import oracle
    from pack_token_amd import fp4idx, workloads

    wl = workloads.large_prefill(T=args.tokens, H=args.heads)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, k = up(wl.q.view(np.int16)), up(wl.k.view(np.int16))
    pos, cs = up(wl.positions), up(wl.cos_sin)
    slots_np = wl.slot_mapping + 1
    slots = up(slots_np)
    T, H = wl.T, wl.H
    q_packed = torch.empty((T, H, 68), dtype=torch.uint8, device=dev)
    cache = torch.zeros((T + 1, 68), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def q_call():
        fp4idx.q_rope_pack_sglang(q, pos, cs, q_packed=q_packed, stream=stream)

    def k_call():
        fp4idx.k_rope_pack_store_sglang(k, pos, cs, slots, cache, stream=stream)

    K = args.steps
    legs = time_legs({"step": [q_call, k_call]}, K, args.warmup, args.rounds, stream,
                     settle_ms=args.settle_ms)
    ms_per_step = median(legs["step"])
    (q_ms, k_ms), _ = launch_pass([q_call, k_call], K, stream)
    qb = sglang_q_bytes_per_token(H) * T
    kb = sglang_k_bytes_per_token() * T
    q_gbs = qb / (q_ms * 1e-3) / 1e9
    rec = {
        "metric": "tokens/s and achieved HBM GB/s, sglang-compatible q+k RoPE/FP4 68-byte records",
        "value": T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16->e2m1 (two stages)",
        "data": "synthetic",
        "config": {"workload": "sglang_prefill", "tokens": T, "heads": H, "head_dim": 128,
                   "rope_dim": 64, "rope": "neox", "rope_offset": 64, "record_bytes": 68,
                   "slots": "1..T (slot 0 unpublished)",
                   "step": "fp4idx_q_rope_pack_sglang + fp4idx_k_rope_pack_store_sglang"},
        "step_GBps": (qb + kb) / (ms_per_step * 1e-3) / 1e9,
        "q_kernel_us": q_ms * 1e3, "k_kernel_us": k_ms * 1e3,
        "k_kernel_GBps": kb / (k_ms * 1e-3) / 1e9,
        "roofline": {"kernel": "q_sglang_kernel<neox>", "bound": "hbm", "achieved": q_gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": q_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(SGLANG_TRAFFIC_FILE, MODE_SOURCES) if (T, H) == (131072, 64)
                     else None,
                     "algorithmic_bytes_per_launch": qb,
                     "launch_us": q_ms * 1e3},
    }
    if not args.no_ceilings:
        rec["ceiling"] = stream_ceiling(args, dev, (256 * H + 8 + 256) * T, 68 * H * T, q_gbs)
    if not args.no_cpu_baseline:
        n = min(args.cpu_sample_tokens, T, 16384)

        def run():
            oracle.q_rope_pack_sglang(wl.q[:n], wl.positions[:n], wl.cos_sin)
            ref = np.zeros((n + 1, 68), np.uint8)
            oracle.k_rope_pack_store_sglang(wl.k[:n], wl.positions[:n], wl.cos_sin,
                                            np.arange(1, n + 1, dtype=np.int64), ref)

        rec["cpu_baseline"] = oracle_baseline(run, n, "query + key records", T)
    print(json.dumps(rec), flush=True)


def bench_scorer(args, dev):
    """fp4idx_paged_mqa_logits over a decode batch: 64 sequences x next_n 4 query
    tokens, H = 32, contexts U[4096, 131072] keys, every sequence on its own cache
    blocks (random FP4 bytes, e8m0 exponents U[118, 130])."""
    import numpy as np
    import torch

    from pack_token_amd import fp4idx, workloads

    B, next_n, H = 64, 4, 32
    sc = workloads.scorer_case(7, B, next_n, H, 4096, 131072)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, qs, w = up(sc.q_out), up(sc.q_scale_out), up(sc.weights)
    kv, ks = up(sc.kv_cache), up(sc.kv_cache_scale)
    table, ctx = up(sc.block_table), up(sc.context_lens)
    stride = sc.max_blocks * 64
    logits = torch.empty((B * next_n, stride), dtype=torch.float32, device=dev)

    def call():
        fp4idx.paged_mqa_logits(q, qs, w, kv, ks, table, ctx, next_n, logits=logits)

    K = args.steps
    stream = torch.cuda.current_stream(dev)
    legs = time_legs({"step": [call]}, K, args.warmup, args.rounds, stream,
                     settle_ms=args.settle_ms)
    ms_per_step = median(legs["step"])
    (launch_ms,), _ = launch_pass([call], K, stream)
    keys = int(sc.context_lens.astype(np.int64).sum())
    blocks = int(sum(-(-int(c) // 64) for c in sc.context_lens))
    J = workloads.q_scale_cols(H)
    T = B * next_n
    bytes_ = (keys * (64 + 4) + T * (64 * H + 64 * J + 4 * H) + blocks * 4 + B * 4
              + keys * next_n * 4)
    flops = 2.0 * 128 * H * next_n * keys
    gbs = bytes_ / (launch_ms * 1e-3) / 1e9
    tfs = flops / (launch_ms * 1e-3) / 1e12
    rec = {
        "metric": "FP4 paged MQA logits: keys scored per second and achieved HBM GB/s",
        "value": keys / (ms_per_step * 1e-3), "unit": "keys/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e2m1 x e2m1 -> fp32 (scaled MFMA)",
        "data": "synthetic",
        "config": {"workload": "decode_scoring", "sequences": B, "next_n": next_n, "heads": H,
                   "head_dim": 128, "kv_block_size": 64, "keys": keys, "context": "U[4096,131072]",
                   "relu": True},
        "roofline": {"kernel": "mqa_logits_flat_kernel<4,2,relu>", "bound": "hbm", "achieved": gbs,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic(SCORER_TRAFFIC_FILE, SCORER_SOURCES),
                     "algorithmic_bytes_per_launch": bytes_,
                     "launch_us": launch_ms * 1e3,
                     "mfma": {"achieved_TFLOPs": tfs, "peak_TFLOPs": FP4_MFMA_PEAK_TFLOPS,
                              "frac": tfs / FP4_MFMA_PEAK_TFLOPS,
                              "algorithmic_flops_per_launch": flops}},
    }
    if not args.no_ceilings:
        cg, cl, _, _ = measure_ceiling(args, dev, "paged_gather", sc)
        rec["ceiling"] = {"kernel": "gather_kernel (fp4idx_ceiling_paged_gather)",
                          "what": "the same block reads and logit writes, no arithmetic",
                          "GBps": cg, "launch_us": cl, "frac_of_peak": cg / HBM_PEAK_GBS,
                          "scorer_frac_of_ceiling": gbs / cg}
    if not args.no_cpu_baseline:
        import oracle

        # the first sequences of the batch, about 100 k keys
        nseq = int(np.searchsorted(np.cumsum(sc.context_lens.astype(np.int64)), 100_000)) + 1
        nseq = min(nseq, B)
        nq = nseq * next_n
        nkeys = int(sc.context_lens[:nseq].astype(np.int64).sum())
        rec["cpu_baseline"] = oracle_baseline(
            lambda: oracle.paged_mqa_logits(sc.q_out[:nq], sc.q_scale_out[:nq], sc.weights[:nq],
                                            sc.kv_cache, sc.kv_cache_scale,
                                            sc.block_table[:nseq], sc.context_lens[:nseq],
                                            next_n),
            nkeys, f"{nseq} sequence(s) x {next_n} query tokens x {H} heads", keys, noun="keys")
    print(json.dumps(rec), flush=True)


def bench_prefill_scoring(args, dev):
    """fp4idx_paged_mqa_logits on a chunked-prefill shape: one sequence of
    65,536 keys whose last 4,096 tokens are the queries (next_n = 4096, query
    tiles of 2), H = 64, random FP4 bytes and e8m0 exponents U[118, 130].
    Algorithmic work counts the causal pairs (key s at or before the query's
    position): 2 * 128 * H flops per pair on the matrix cores and 2 VALU
    operations per pair and head (ReLU, weighted accumulate); bytes are the
    inputs read once plus every logit of the [4096, 65536] rows written."""
    import numpy as np
    import torch

    from pack_token_amd import fp4idx, workloads

    B, next_n, H, ctx_len = 1, 4096, 64, 65536
    sc = workloads.scorer_case(11, B, next_n, H, ctx_len, ctx_len)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    q, qs, w = up(sc.q_out), up(sc.q_scale_out), up(sc.weights)
    kv, ks = up(sc.kv_cache), up(sc.kv_cache_scale)
    table, ctx = up(sc.block_table), up(sc.context_lens)
    stride = sc.max_blocks * 64
    logits = torch.empty((B * next_n, stride), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        fp4idx.paged_mqa_logits(q, qs, w, kv, ks, table, ctx, next_n, logits=logits)

    K = args.steps
    legs = time_legs({"step": [call]}, K, args.warmup, args.rounds, stream,
                     settle_ms=args.settle_ms)
    ms_per_step = median(legs["step"])
    (launch_ms,), _ = launch_pass([call], K, stream)
    pos = np.arange(ctx_len - next_n, ctx_len, dtype=np.int64)
    pairs = int((pos + 1).sum())
    flops = 2.0 * 128 * H * pairs
    valu_ops = 2.0 * H * pairs
    J = workloads.q_scale_cols(H)
    bytes_ = (ctx_len * (64 + 4) + next_n * (64 * H + 64 * J + 4 * H) + next_n * ctx_len * 4
              + (ctx_len // 64) * 4 + 4)
    tfs = flops / (launch_ms * 1e-3) / 1e12
    gops = valu_ops / (launch_ms * 1e-3) / 1e9
    gbs = bytes_ / (launch_ms * 1e-3) / 1e9
    rec = {
        "metric": "FP4 paged MQA logits, chunked prefill: causal query-key pairs scored per second",
        "value": pairs / (ms_per_step * 1e-3), "unit": "pairs/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "e2m1 x e2m1 -> fp32 (scaled MFMA)",
        "data": "synthetic",
        "config": {"workload": "prefill_scoring", "sequences": B, "next_n": next_n, "heads": H,
                   "head_dim": 128, "kv_block_size": 64, "context": ctx_len, "relu": True,
                   "causal_pairs": pairs},
        "roofline": {"kernel": "mqa_logits_kernel<2,4,relu,tiled>", "bound": "alu", "achieved": gops,
                     "peak": VALU_PEAK_GOPS, "unit": "Gop/s", "frac": gops / VALU_PEAK_GOPS,
                     "traffic": None, "algorithmic_ops_per_launch": valu_ops,
                     "launch_us": launch_ms * 1e3},
        "mfma_view": {"achieved_TFLOPs": tfs, "peak_TFLOPs": FP4_MFMA_PEAK_TFLOPS,
                      "frac": tfs / FP4_MFMA_PEAK_TFLOPS, "algorithmic_flops_per_launch": flops},
        "hbm_view": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": bytes_},
    }
    if not args.no_ceilings:
        rec["valu_ceiling"] = valu_ceiling(args, dev, gops)
    if not args.no_cpu_baseline:
        import oracle

        # the last 4 queries against the whole context (their causal pairs)
        nq = 4
        sub_pairs = int((pos[-nq:] + 1).sum())
        rec["cpu_baseline"] = oracle_baseline(
            lambda: oracle.paged_mqa_logits(sc.q_out[-nq:], sc.q_scale_out[-nq:],
                                            sc.weights[-nq:], sc.kv_cache, sc.kv_cache_scale,
                                            sc.block_table, np.array([ctx_len], np.int32), nq),
            sub_pairs, f"the last {nq} queries' causal pairs x {H} heads", pairs, noun="pairs")
    print(json.dumps(rec), flush=True)


def measure_ceiling(args, dev, kind: str, sc=None, rw=None):
    """One ceiling measurement (fp4idx_ceiling_stream / fp4idx_ceiling_paged_gather):
    plain HBM traffic of the shapes the kernels move, none of their arithmetic.
      stream_read   reads the bytes the headline step reads (17,168 per token
                    x 131,072 tokens at H = 64), writes nothing;
      stream_mix    the headline step's reads and writes (17,168 + 4,676 bytes
                    per token: 78.6% reads), writes spread over the reads;
      stream_copy   a 1:1 copy of the fake-quant input (256 bytes x 64 heads x
                    131,072 tokens read, as many written);
      paged_gather  the decode-scoring batch's key blocks (4,096 + 256 bytes per
                    block of every sequence) and its logit writes, with the
                    scorer's flat split over wavefronts (sc: that batch, if the
                    caller has it);
      stream_rw     rw = (read bytes, written bytes) of a caller's launch, writes
                    spread over the reads.
    Returns (GB/s from the mean launch time, mean launch us, median ms per step
    of the timed rounds, config)."""
    import numpy as np
    import torch

    from pack_token_amd import fp4idx, workloads

    stream = torch.cuda.current_stream(dev)
    T, H = args.tokens, args.heads
    if kind == "paged_gather":
        B, next_n = 64, 4
        if sc is None:
            sc = workloads.scorer_case(7, B, next_n, 32, 4096, 131072)
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        kv, ks = up(sc.kv_cache), up(sc.kv_cache_scale)
        table, ctx = up(sc.block_table), up(sc.context_lens)
        logits = torch.empty((B * next_n, sc.max_blocks * 64), dtype=torch.float32, device=dev)

        def call():
            fp4idx.ceiling_paged_gather(kv, ks, table, ctx, next_n, logits)

        keys = int(sc.context_lens.astype(np.int64).sum())
        blocks = int(sum(-(-int(c) // 64) for c in sc.context_lens))
        read_b = blocks * (4096 + 256) + blocks * 4 + B * 4
        write_b = keys * next_n * 4
        shape = {"sequences": B, "next_n": next_n, "keys": keys, "blocks": blocks,
                 "context": "U[4096,131072]"}
    else:
        J = ((H // 16) + 3) // 4 * 4
        if kind == "stream_rw":
            read_b, write_b = rw
        elif kind == "stream_copy":
            read_b = write_b = 256 * H * T
        else:
            read_b = (256 * H + 4 * H + 8 + 256 + 256 + 8) * T
            write_b = 0 if kind == "stream_read" else (64 * H + 64 * J + 4 * H + 68) * T
        read_b, write_b = -(-read_b // 1024) * 1024, -(-write_b // 1024) * 1024
        src = torch.zeros(read_b, dtype=torch.uint8, device=dev)
        dst = torch.zeros(max(write_b, 1024), dtype=torch.uint8, device=dev)

        def call():
            fp4idx.ceiling_stream(src, read_b, dst, write_b)

        shape = {"tokens": T, "heads": H, "read_bytes": read_b, "write_bytes": write_b,
                 "read_fraction": read_b / (read_b + write_b)}
    K = args.steps
    legs = time_legs({"step": [call]}, K, args.warmup, args.rounds, stream,
                     settle_ms=args.settle_ms)
    (launch_ms,), (launch_med,) = launch_pass([call], K, stream)
    total = read_b + write_b
    shape = dict(shape, bytes_per_launch=total, launch_us_median=launch_med * 1e3)
    return total / (launch_ms * 1e-3) / 1e9, launch_ms * 1e3, median(legs["step"]), shape


def bench_ceiling(args, dev, kind: str):
    """A ceiling measurement as its own bench line (see measure_ceiling)."""
    gbs, launch_us, ms, shape = measure_ceiling(args, dev, kind)
    rec = {
        "metric": "HBM GB/s of plain traffic (ceiling measurement, no arithmetic)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u8", "data": "synthetic",
        "config": dict({"workload": kind}, **{k: v for k, v in shape.items()
                                               if k not in ("bytes_per_launch",
                                                            "launch_us_median")}),
        "roofline": {"kernel": "gather_kernel" if kind == "paged_gather" else "stream_kernel",
                     "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": shape["bytes_per_launch"],
                     "launch_us": launch_us, "launch_us_median": shape["launch_us_median"]},
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_prefill",
                    choices=["large_prefill", "prefill_norm_rotate", "decode", "decode_scoring",
                             "prefill_scoring", "sglang_prefill", "fp8_prefill",
                             "fake_quant_prefill", "stream_read", "stream_mix", "stream_copy",
                             "paged_gather"],
                    help="large_prefill is the headline configuration; the other two are timed "
                         "for reference")
    ap.add_argument("--tokens", type=int, default=131072,
                    help="the prefill workloads")
    ap.add_argument("--heads", type=int, default=64, help="the prefill workloads")
    ap.add_argument("--cpu-sample-tokens", type=int, default=131072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the ceiling measurements reported beside the headline and the "
                         "decode scorer")
    ap.add_argument("--graph", choices=["auto", "on", "off"], default="auto",
                    help="time steps replayed from captured HIP graphs (auto: on for decode, where "
                         "host launch overhead exceeds the kernel time)")
    ap.add_argument("--graph-steps", type=int, default=10, help="steps captured per graph")
    ap.add_argument("--rounds", type=int, default=5,
                    help="timed rounds of K steps per leg (legs alternate; median reported)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed GPU time spent on steps after the warm-up steps, so clocks "
                         "have ramped up before timing")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="instead of the benchmark, time one plain device copy of this many MiB "
                         "(reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this path runs on one GPU only (every token is independent and no "
              "collective is on the hot path); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from pack_token_amd import fp4idx, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        reps = 3
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0.record()
        for _ in range(reps):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / reps
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n, "copies": reps + 1,
                          "us_per_copy": ms * 1e3, "GBps": 2 * n / (ms * 1e-3) / 1e9}), flush=True)
        return

    t_gen = time.perf_counter()
    if args.workload == "decode_scoring":
        bench_scorer(args, dev)
        return
    if args.workload == "prefill_scoring":
        bench_prefill_scoring(args, dev)
        return
    if args.workload == "sglang_prefill":
        bench_sglang(args, dev)
        return
    if args.workload == "fp8_prefill":
        bench_fp8(args, dev)
        return
    if args.workload == "fake_quant_prefill":
        bench_fake_quant(args, dev)
        return
    if args.workload in ("stream_read", "stream_mix", "stream_copy", "paged_gather"):
        bench_ceiling(args, dev, args.workload)
        return
    if args.workload == "large_prefill":
        wl = workloads.large_prefill(T=args.tokens, H=args.heads)
    else:
        wl = workloads.RECIPES[args.workload]()
    print(f"bench: generated {wl.name} T={wl.T} H={wl.H} in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q = up(wl.q.view(np.int16))
    k = up(wl.k.view(np.int16))
    pos = up(wl.positions)
    cs = up(wl.cos_sin)
    w = up(wl.weights)
    slots = up(wl.slot_mapping)
    T, H = wl.T, wl.H
    J = wl.J
    q_out = torch.empty((T, H, 64), dtype=torch.uint8, device=dev)
    qs = torch.empty((T, 1, 4, 16, J), dtype=torch.uint8, device=dev)
    w_out = torch.empty_like(w)
    kv = torch.full((wl.NB, 1, 4, 64, 16), workloads.SENTINEL, dtype=torch.uint8, device=dev)
    ks = torch.full((wl.NB, 1, 4, 64), workloads.SENTINEL, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    gamma = None if wl.k_norm_gamma is None else up(wl.k_norm_gamma.view(np.int16))

    # stream=None: each call goes to torch's current stream (the capture stream
    # while a graph is being recorded)
    common = dict(is_neox=wl.is_neox, rope_offset=wl.rope_offset,
                  apply_hadamard=wl.apply_hadamard, stream=None)
    kcommon = dict(common, k_norm_gamma=gamma, k_norm_eps=wl.k_norm_eps)
    def fill_background():
        # the cache's background keys, written before the step (not timed)
        fp4idx.k_rope_pack_store(up(wl.background["k"].view(np.int16)),
                                 up(wl.background["positions"]), cs, up(wl.background["slots"]),
                                 kv, ks, **kcommon)
        torch.cuda.synchronize()

    if wl.background is not None:
        fill_background()

    def q_call():
        fp4idx.q_rope_pack(q, pos, cs, w, q_out=q_out, q_scale_out=qs, weights_out=w_out, **common)

    def k_call():
        fp4idx.k_rope_pack_store(k, pos, cs, slots, kv, ks, **kcommon)

    def qk_call():
        fp4idx.qk_rope_pack_store(q, k, pos, cs, slots, kv, ks, w, q_out=q_out, q_scale_out=qs,
                                  weights_out=w_out, **kcommon)

    use_graph = args.graph == "on" or (args.graph == "auto" and wl.name == "decode")

    G = max(1, args.graph_steps)

    def graphed(fns):
        """A HIP graph holding G steps of fns (warmed up on a side stream first)."""
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for f in fns:
                f()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(G):
                for f in fns:
                    f()
        torch.cuda.synchronize()
        return g.replay

    K = args.steps
    R = max(1, args.rounds)
    # headline and two-call step: K steps per round between two events, legs
    # alternating in order from round to round, the median round reported
    legs = time_legs({"fused": [qk_call], "two_call": [q_call, k_call]}, K, args.warmup, R,
                     stream, settle_ms=args.settle_ms)
    ms_per_step, two_ms = median(legs["fused"]), median(legs["two_call"])
    # per-launch durations in a pass of their own (events around every launch)
    (fused_ms,), (fused_med_ms,) = launch_pass([qk_call], K, stream)
    (q_ms, k_ms), _ = launch_pass([q_call, k_call], K, stream)
    if use_graph:
        # step time from graph replays: K steps = ceil(K / G) replays of G steps
        reps = -(-K // G)
        K = reps * G
        glegs = time_legs({"fused": [graphed([qk_call])],
                           "two_call": [graphed([q_call, k_call])]}, reps,
                          max(1, args.warmup // G), R, stream)
        eager_ms_per_step, eager_two_ms = ms_per_step, two_ms
        ms_per_step, two_ms = median(glegs["fused"]) / G, median(glegs["two_call"]) / G

    step_bytes = step_bytes_per_token(H) * T
    achieved = step_bytes / (fused_ms * 1e-3) / 1e9
    traffic = None
    if wl.name == "large_prefill" and (T, H) == (131072, 64):
        traffic = measured_traffic()
    elif wl.name == "prefill_norm_rotate" and (T, H) == (16384, 64):
        traffic = measured_traffic(PNR_TRAFFIC_FILE)
    rec = {
        "metric": "tokens/s and achieved HBM GB/s (% of peak), fused q+k RoPE/FP4 pack+store",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->e2m1",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "heads": H, "head_dim": 128, "rope_dim": 64,
                   "rope": "neox" if wl.is_neox else "interleaved", "rope_offset": wl.rope_offset,
                   "key_rmsnorm": wl.k_norm_gamma is not None, "hadamard": wl.apply_hadamard,
                   "kv_blocks": wl.NB, "kv_block_size": 64,
                   "slot_mapping": "random distinct" if wl.background is not None else "contiguous",
                   "step": "fp4idx_qk_rope_pack_store (one launch)",
                   "graph_replay": use_graph, "graph_steps": G if use_graph else None},
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_hbm_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "timing": {"rounds": R, "fused_ms_per_step_rounds": legs["fused"],
                   "two_call_ms_per_step_rounds": legs["two_call"],
                   "settle_ms": args.settle_ms,
                   "note": "each round times K steps of each leg between two events, legs in "
                           "alternating order; ms_per_step is the median round; per-launch "
                           "durations come from a separate pass with events around every launch"},
        "two_call_step": {"calls": "fp4idx_q_rope_pack + fp4idx_k_rope_pack_store",
                          "ms_per_step": two_ms, "tokens_per_s": T / (two_ms * 1e-3),
                          "GBps": step_bytes / (two_ms * 1e-3) / 1e9,
                          "q_kernel_us": q_ms * 1e3, "k_kernel_us": k_ms * 1e3,
                          "q_kernel_GBps": q_bytes_per_token(H) * T / (q_ms * 1e-3) / 1e9},
        "roofline": {"kernel": "qk_kernel<neox=%d,hadamard=%d,norm=%d>" % (
                         wl.is_neox, wl.apply_hadamard, wl.k_norm_gamma is not None),
                     "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": step_bytes,
                     "launch_us": fused_ms * 1e3, "launch_us_median": fused_med_ms * 1e3},
    }
    if wl.name == "prefill_norm_rotate":
        rec["cache_note"] = ("%.1f MB per step against a 256 MB Infinity Cache: part of the "
                             "step's bytes can stay cache-resident between back-to-back steps, "
                             "so the HBM fraction is an upper estimate" % (step_bytes / 1e6))
        # with the Hadamard the kernel is bound by VALU issue, not by HBM
        ops = alu_ops_per_token(H, True, wl.k_norm_gamma is not None) * T
        gops = ops / (fused_ms * 1e-3) / 1e9
        hbm = rec["roofline"]
        rec["roofline"] = {"kernel": hbm["kernel"], "bound": "alu", "achieved": gops,
                           "peak": VALU_PEAK_GOPS, "unit": "Gop/s", "frac": gops / VALU_PEAK_GOPS,
                           "traffic": hbm["traffic"], "algorithmic_ops_per_launch": ops,
                           "launch_us": hbm["launch_us"],
                           "launch_us_median": hbm["launch_us_median"]}
        rec["hbm_view"] = {k: hbm[k] for k in ("achieved", "peak", "unit", "frac", "traffic",
                                               "algorithmic_bytes_per_launch")}
        if not args.no_ceilings:
            rec["valu_ceiling"] = valu_ceiling(args, dev, gops)
    if use_graph:
        rec["eager_ms_per_step"] = eager_ms_per_step
        rec["two_call_step"]["eager_ms_per_step"] = eager_two_ms
    if not args.no_ceilings and wl.name == "large_prefill":
        ceil = {}
        for kind in ("stream_read", "stream_mix"):
            cg, cl, _, shape = measure_ceiling(args, dev, kind)
            ceil[kind] = {"GBps": cg, "launch_us": cl, "frac_of_peak": cg / HBM_PEAK_GBS,
                          "read_bytes": shape["read_bytes"], "write_bytes": shape["write_bytes"]}
        ceil["kernel"] = "stream_kernel (fp4idx_ceiling_stream)"
        ceil["what"] = ("the step's read bytes alone, and its reads and writes in the same mix, as "
                        "plain 1 KB streams")
        ceil["fused_frac_of_stream_read"] = achieved / ceil["stream_read"]["GBps"]
        rec["ceilings"] = ceil
    if not args.no_cpu_baseline:
        # outputs of one fused launch and of one two-call step, each from
        # sentinel-filled buffers (untimed), for the parity check
        def outputs_of(calls):
            for o in (q_out, qs, kv, ks):
                o.fill_(workloads.SENTINEL)
            w_out.fill_(float("nan"))
            if wl.background is not None:
                fill_background()
            for c in calls:
                c()
            torch.cuda.synchronize()
            return tuple(x.cpu().numpy() for x in (q_out, qs, w_out, kv, ks))

        got = {"fused": outputs_of([qk_call]), "two_call": outputs_of([q_call, k_call])}
        threads = max(1, min(16, len(os.sched_getaffinity(0))))
        rec["cpu_baseline"] = cpu_baseline(wl, min(args.cpu_sample_tokens, T), threads)
        rec["parity"] = {"tokens": T, "outputs": ["q_out", "q_scale_out", "weights_out",
                                                  "kv_cache", "kv_cache_scale"],
                         "mismatched_bytes": oracle_parity(wl, got, threads),
                         "against": "the CPU oracle on every token, byte for byte"}
        del got
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
