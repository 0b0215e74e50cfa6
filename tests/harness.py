"""Shared helpers for the GPU parity tests: run a workload through the HIP
library (via its C-ABI binding) and through the CPU oracle, and compare
outputs byte for byte."""
from __future__ import annotations

import os

import numpy as np

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import SENTINEL, Workload

ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def say(msg: str):
    print(msg, flush=True)


_LARGE_PREFILL = []


def large_prefill() -> Workload:
    """The large-prefill workload (131,072 tokens x 64 heads), generated once per
    test session and shared by the tests that use it (inputs are read-only)."""
    if not _LARGE_PREFILL:
        _LARGE_PREFILL.append(workloads.large_prefill())
    return _LARGE_PREFILL[0]


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


_RANDOM_T = [1, 2, 3, 5, 63, 64, 65, 127, 300, 511, 512, 513, 1000, 1023, 1024, 1025, 2047, 2049]


def random_case(seed):
    """A seeded random point of the whole input space: token counts around the
    block and small-batch boundaries, 16..256 heads, every RoPE mode, Hadamard
    and key RMSNorm on or off, value scales from 1e-3 to 1e3 with planted
    zero / subnormal / half-way groups, int32 or int64 positions (a few past
    max_pos or negative: clamped), slots with skips (-1) and a few past the end
    of the cache, three floors, weights present or not."""
    rng = np.random.Generator(np.random.PCG64(7000 + seed))
    T = int(rng.choice(_RANDOM_T))
    H = 16 * int(rng.integers(1, 17))
    scale = float(rng.choice([1.0, 40.0, 1e-3, 1e3]))
    q = workloads.to_bf16_bits(rng.standard_normal((T, H, 128), dtype=np.float32) * scale)
    k = workloads.to_bf16_bits(rng.standard_normal((T, 128), dtype=np.float32) * scale)
    workloads._plant_special_groups(rng, q.reshape(T * H, 128))
    workloads._plant_special_groups(rng, k)
    max_pos = int(rng.integers(1, 70000))
    positions = rng.integers(0, max_pos, T, dtype=np.int64)
    odd = rng.random(T) < 0.02
    positions[odd] = np.where(rng.random(int(odd.sum())) < 0.5, -1 - rng.integers(0, 5, int(odd.sum())),
                              max_pos + rng.integers(0, 1000, int(odd.sum())))
    if rng.integers(2):
        positions = positions.astype(np.int32)
    NB = -(-T // 64) + int(rng.integers(0, 3))
    slots = rng.permutation(NB * 64)[:T].astype(np.int64)
    u = rng.random(T)
    slots[u < 0.05] = -1
    slots[(u >= 0.05) & (u < 0.07)] = NB * 64 + rng.integers(0, 100)
    wl = workloads.Workload(f"random_{seed}_T{T}_H{H}", T, H, q, k, positions,
                            workloads.cos_sin_table(max_pos),
                            rng.random((T, H), dtype=np.float32), slots, NB,
                            is_neox=bool(rng.integers(2)), rope_offset=int(rng.choice([0, 64])),
                            apply_hadamard=bool(rng.integers(2)),
                            scale_floor=float(np.float32(rng.choice([2.0 ** -126, 1e-10, 1e-3]))))
    if rng.integers(2):
        wl.k_norm_gamma = workloads.to_bf16_bits(
            (1 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    return wl, bool(rng.integers(0, 4))
