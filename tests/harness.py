"""Shared helpers for the GPU parity tests: run a workload through the HIP
library (via its C-ABI binding) and through the CPU oracle, and compare
outputs byte for byte."""
from __future__ import annotations

import os

import numpy as np

import oracle
from pack_token_amd.workloads import SENTINEL, Workload

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg: str):
    print(msg, flush=True)


def dev_tensors(wl: Workload, device):
    import torch

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    d = {
        "q": t(wl.q.view(np.int16)),
        "k": t(wl.k.view(np.int16)),
        "positions": t(wl.positions),
        "cos_sin": t(wl.cos_sin),
        "weights": t(wl.weights),
        "slot_mapping": t(wl.slot_mapping),
        "gamma": None if wl.k_norm_gamma is None else t(wl.k_norm_gamma.view(np.int16)),
    }
    if wl.background is not None:
        d["bg_k"] = t(wl.background["k"].view(np.int16))
        d["bg_positions"] = t(wl.background["positions"])
        d["bg_slots"] = t(wl.background["slots"])
    return d


def gpu_run(wl: Workload, device="cuda:0", with_weights=True, positions_dtype=None, stream=None,
            fused=False):
    """Returns numpy (q_out, q_scale_out, weights_out, kv_cache, kv_cache_scale).
    fused=False: fp4idx_q_rope_pack then fp4idx_k_rope_pack_store; True: the single
    fp4idx_qk_rope_pack_store launch."""
    import torch

    from pack_token_amd import fp4idx

    d = dev_tensors(wl, device)
    pos = d["positions"] if positions_dtype is None else d["positions"].to(positions_dtype)
    T, H = wl.T, wl.H
    # outputs start as a sentinel so a byte the kernels never write shows up
    q_out = torch.full((T, H, 64), SENTINEL, dtype=torch.uint8, device=device)
    qs = torch.full((T, 1, 4, 16, wl.J), SENTINEL, dtype=torch.uint8, device=device)
    w_out = torch.full((T, H), float("nan"), dtype=torch.float32, device=device) if with_weights else None
    kv_np, ks_np = wl.empty_cache()
    kv = torch.from_numpy(kv_np).to(device)
    ks = torch.from_numpy(ks_np).to(device)
    common = dict(is_neox=wl.is_neox, rope_offset=wl.rope_offset, apply_hadamard=wl.apply_hadamard,
                  scale_floor=wl.scale_floor, stream=stream)
    if wl.background is not None:
        fp4idx.k_rope_pack_store(d["bg_k"], d["bg_positions"], d["cos_sin"], d["bg_slots"], kv, ks,
                                 k_norm_gamma=d["gamma"], k_norm_eps=wl.k_norm_eps, **common)
    if fused:
        fp4idx.qk_rope_pack_store(d["q"], d["k"], pos, d["cos_sin"], d["slot_mapping"], kv, ks,
                                  d["weights"] if with_weights else None, q_out=q_out,
                                  q_scale_out=qs, weights_out=w_out, k_norm_gamma=d["gamma"],
                                  k_norm_eps=wl.k_norm_eps, **common)
    else:
        fp4idx.q_rope_pack(d["q"], pos, d["cos_sin"], d["weights"] if with_weights else None,
                           q_out=q_out, q_scale_out=qs, weights_out=w_out, **common)
        fp4idx.k_rope_pack_store(d["k"], pos, d["cos_sin"], d["slot_mapping"], kv, ks,
                                 k_norm_gamma=d["gamma"], k_norm_eps=wl.k_norm_eps, **common)
    torch.cuda.synchronize()
    return (q_out.cpu().numpy(), qs.cpu().numpy(), None if w_out is None else w_out.cpu().numpy(),
            kv.cpu().numpy(), ks.cpu().numpy())


def oracle_run(wl: Workload, with_weights=True, threads=ORACLE_THREADS):
    q_out, qs, w_out = oracle.q_rope_pack(wl.q, wl.positions, wl.cos_sin,
                                          wl.weights if with_weights else None,
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
    return q_out, qs, w_out, kv, ks


NAMES = ("q_out", "q_scale_out", "weights_out", "kv_cache", "kv_cache_scale")


def assert_same(name, got, ref):
    if got is None and ref is None:
        return
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if got.dtype == np.float32:
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    bad = np.argwhere(got != ref)
    if bad.size:
        idx = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} of {got.size} elements differ; first at {idx}: "
                             f"gpu={got[idx]:#x} oracle={ref[idx]:#x}")


def assert_all_same(got, ref):
    for name, g, r in zip(NAMES, got, ref):
        assert_same(name, g, r)
