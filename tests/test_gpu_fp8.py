"""GPU parity of the FP8 output mode (ROCm/aiter PR 5484 "API": the FP8
contract with its per-(token, head) q scale folded into weights_out, scale_fmt
ue8m0 or fp32; ROCm/aiter PR 4029 review: e4m3fn, largest value 448, on
gfx950): the HIP path through the C ABI against the CPU oracle, byte for byte
on codes, scales and folded weights, over both scale formats, every RoPE mode,
Hadamard and key RMSNorm, the edge-mix rows, every finite bf16 value under
every power-of-two scale, and the full-size prefill shape."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import SENTINEL
from harness import ORACLE_THREADS, assert_same, large_prefill, random_case, say

pytestmark = pytest.mark.gpu


def _t(a, dev="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_q(q, positions, cos_sin, weights, **kw):
    import torch
    from pack_token_amd import fp4idx
    T, H, _ = q.shape
    q_out = torch.full((T, H, 128), SENTINEL, dtype=torch.uint8, device="cuda:0")
    w_out = torch.full((T, H), -1, dtype=torch.int16, device="cuda:0")
    fp4idx.q_rope_pack_fp8(_t(q.view(np.int16)), _t(positions), _t(cos_sin), _t(weights),
                           q_out=q_out, weights_out=w_out, **kw)
    torch.cuda.synchronize()
    return q_out.cpu().numpy(), w_out.cpu().numpy().view(np.uint16)


def gpu_k(k, positions, cos_sin, slots, NB, gamma=None, **kw):
    import torch
    from pack_token_amd import fp4idx
    kv = torch.full((NB, 64, 128), SENTINEL, dtype=torch.uint8, device="cuda:0")
    ks = torch.full((NB, 64), float("nan"), dtype=torch.float32, device="cuda:0")
    fp4idx.k_rope_pack_store_fp8(_t(k.view(np.int16)), _t(positions), _t(cos_sin), _t(slots), kv,
                                 ks, k_norm_gamma=None if gamma is None else
                                 _t(gamma.view(np.int16)), **kw)
    torch.cuda.synchronize()
    return kv.cpu().numpy(), ks.cpu().numpy()


def check(wl, fmt, weights_scale=1.0, gamma=None, had=False, floor=None):
    kw = dict(is_neox=wl.is_neox, rope_offset=wl.rope_offset, apply_hadamard=had,
              scale_fmt=fmt)
    if floor is not None:
        kw["scale_floor"] = floor
    say(f"case fp8 {wl.name}: T={wl.T} H={wl.H} neox={wl.is_neox} ro={wl.rope_offset} "
        f"fmt={fmt} had={had} norm={gamma is not None} ws={weights_scale} floor={floor}")
    got_q, got_w = gpu_q(wl.q, wl.positions, wl.cos_sin, wl.weights,
                         weights_scale=weights_scale, **kw)
    ofmt = {"ue8m0": 0, "fp32": 1}[fmt]
    okw = dict(kw, scale_fmt=ofmt)
    ref_q, ref_w = oracle.q_rope_pack_fp8(wl.q, wl.positions, wl.cos_sin, wl.weights,
                                          weights_scale=weights_scale, **okw)
    assert_same("q_out", got_q, ref_q)
    assert_same("weights_out", got_w, ref_w)
    kv, ks = gpu_k(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, wl.NB, gamma,
                   k_norm_eps=1e-6, **kw)
    rkv = np.full((wl.NB, 64, 128), SENTINEL, np.uint8)
    rks = np.full((wl.NB, 64), np.nan, np.float32)
    oracle.k_rope_pack_store_fp8(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, rkv, rks,
                                 k_norm_gamma=gamma, k_norm_eps=1e-6, **okw)
    assert_same("kv_cache", kv, rkv)
    assert_same("kv_cache_scale", ks, rks)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
@pytest.mark.parametrize("pos32", [False, True])
def test_edge_mix(fmt, pos32):
    check(workloads.edge_mix(seed=500, T=300, positions_int32=pos32), fmt, weights_scale=0.3)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
@pytest.mark.parametrize("neox,ro", [(True, 64), (True, 0), (False, 64), (False, 0)])
@pytest.mark.parametrize("had", [False, True])
def test_modes(fmt, neox, ro, had):
    wl = workloads.sweep_case(510 + 2 * ro + neox, 37, 48, neox, ro)
    rng = np.random.default_rng(11)
    gamma = workloads.to_bf16_bits((1.0 + 0.1 * rng.standard_normal(128)).astype(np.float32))
    check(wl, fmt, weights_scale=1.0 / 8, gamma=gamma, had=had)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
@pytest.mark.parametrize("neox,ro", [(True, 64), (False, 0)])
@pytest.mark.parametrize("had", [False, True])
def test_overflow_rows(fmt, neox, ro, had):
    """Rows whose rotation leaves the fp32 range (one RoPE pair of
    largest-magnitude bf16 values in about half of the rows): the row amax
    is infinite."""
    check(workloads.overflow_case(71 + ro + neox, 300, 16, neox, ro, had), fmt, had=had)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
def test_floors_and_tiny_rows(fmt):
    wl = workloads.edge_mix(seed=520, T=64, H=16)
    q = wl.q.copy()
    q[::3] &= np.uint16(0x807F)               # every third token: subnormal or zero magnitudes
    wl.q = q
    for floor in (float(np.float32(2.0 ** -126)), 1e-3, 5.0):
        check(wl, fmt, floor=floor)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
def test_maximum_heads(fmt):
    check(workloads.sweep_case(779, 5, 2048, True, 64), fmt, weights_scale=2.0, had=True)


def test_empty():
    wl = workloads.tiny(T=0, H=16)
    q_out, w_out = gpu_q(wl.q, wl.positions, wl.cos_sin, wl.weights)
    assert q_out.shape == (0, 16, 128) and w_out.shape == (0, 16)


def _anchor_rows(anchors, per_row=63):
    """Rows whose dims 0..63 (left unrotated by the RoPE tail) carry one anchor
    -- the row's largest magnitude -- and 63 finite bf16 values below it."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb.astype(np.uint32) >> 7) & 0xFF) != 0xFF]
    mag = finite & 0x7FFF
    rows = []
    for anchor in anchors:
        vals = finite[mag <= anchor]
        n = -(-vals.size // per_row) * per_row
        vals = np.concatenate([vals, np.zeros(n - vals.size, np.uint16)]).reshape(-1, per_row)
        r = np.zeros((vals.shape[0], 128), np.uint16)
        r[:, 0] = anchor
        r[:, 1:64] = vals
        rows.append(r)
    rows = np.concatenate(rows)
    H = 64
    T = -(-rows.shape[0] // H)
    q = np.zeros((T * H, 128), np.uint16)
    q[: rows.shape[0]] = rows
    return q.reshape(T, H, 128), rows.shape[0]


def test_converter_exhaustive_ue8m0():
    """Every finite bf16 value under every power-of-two scale 2^(E-127) an
    amax can reach, E in [1, 247] (anchor 448 * 2^(E-127), or the largest
    bf16 at the top)."""
    anchors = []
    for E in range(1, 248):
        v = 448.0 * 2.0 ** (E - 127)
        anchors.append(0x7F7F if v > 3.3e38 else
                       int(workloads.to_bf16_bits(np.array([v], np.float32))[0]))
    q, n = _anchor_rows(sorted(set(anchors)))
    pos = np.zeros(q.shape[0], np.int64)
    cs = workloads.cos_sin_table(1)
    w = np.ones(q.shape[:2], np.float32)
    say(f"case fp8 converter_exhaustive_ue8m0: {n} rows, T={q.shape[0]}")
    got_q, got_w = gpu_q(q, pos, cs, w, scale_fmt="ue8m0")
    ref_q, ref_w = oracle.q_rope_pack_fp8(q, pos, cs, w, scale_fmt=0)
    assert_same("q_out", got_q, ref_q)
    assert_same("weights_out", got_w, ref_w)


def test_converter_fp32_scales():
    """Every finite bf16 value under 40 non-power-of-two anchors (fp32 scales
    with full significands), through the division and the e4m3 rounding."""
    rng = np.random.default_rng(12)
    anchors = workloads.to_bf16_bits((rng.uniform(1, 2, 40) * 2.0 ** rng.integers(-120, 120, 40))
                                     .astype(np.float32))
    q, n = _anchor_rows(sorted(set(int(a) for a in anchors)))
    pos = np.zeros(q.shape[0], np.int64)
    cs = workloads.cos_sin_table(1)
    w = rng.random(q.shape[:2], dtype=np.float32)
    say(f"case fp8 converter_fp32: {n} rows, T={q.shape[0]}")
    got_q, got_w = gpu_q(q, pos, cs, w, scale_fmt="fp32", weights_scale=0.7)
    ref_q, ref_w = oracle.q_rope_pack_fp8(q, pos, cs, w, scale_fmt=1, weights_scale=0.7)
    assert_same("q_out", got_q, ref_q)
    assert_same("weights_out", got_w, ref_w)


@pytest.mark.parametrize("fmt", ["ue8m0", "fp32"])
def test_large_prefill_full_size(fmt):
    """T = 131072, H = 64: the query codes and folded weights of every token and
    every key (codes and scales), byte for byte."""
    wl = large_prefill()
    say(f"case fp8 large_prefill fmt={fmt}")
    got_q, got_w = gpu_q(wl.q, wl.positions, wl.cos_sin, wl.weights, scale_fmt=fmt)
    ofmt = {"ue8m0": 0, "fp32": 1}[fmt]
    ref_q, ref_w = oracle.q_rope_pack_fp8(wl.q, wl.positions, wl.cos_sin, wl.weights,
                                          scale_fmt=ofmt, threads=ORACLE_THREADS)
    assert_same("q_out", got_q, ref_q)
    assert_same("weights_out", got_w, ref_w)
    assert not ((got_q & 0x7F) == 0x7F).any()       # no NaN codes anywhere
    del got_q, ref_q
    kv, ks = gpu_k(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, wl.NB, scale_fmt=fmt)
    rkv = np.full((wl.NB, 64, 128), SENTINEL, np.uint8)
    rks = np.full((wl.NB, 64), np.nan, np.float32)
    oracle.k_rope_pack_store_fp8(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, rkv, rks,
                                 scale_fmt=ofmt)
    assert_same("kv_cache", kv, rkv)
    assert_same("kv_cache_scale", ks, rks)


@pytest.mark.parametrize("seed", range(12))
def test_random_cases(seed):
    """Seeded random shapes and modes (the producer's random cases) in the FP8
    mode: either scale format, any weights scale, Hadamard and key RMSNorm as
    drawn, clamped positions and skipped / past-the-end slots."""
    wl, _ = random_case(100 + seed)
    rng = np.random.default_rng(seed)
    fmt = ["ue8m0", "fp32"][seed % 2]
    check(wl, fmt, weights_scale=float(rng.choice([1.0, 0.3, 1.0 / 8, 7.5])),
          gamma=wl.k_norm_gamma, had=wl.apply_hadamard, floor=wl.scale_floor)
