"""Pins for the oracle's compressed-KV pieces (sgl-project/sglang PR 39656
"Summary": the key store rotates a compressed row at its group's first
position; the torch-shaped RoPE + FP4 fake quant uses per-32 UE8M0 scales by
default and per-16 E4M3 scales for compressed KV, with the bf16 round trip
after RoPE and round-half-to-even; "Verification": compress ratios 1, 2, 4).
The fake-quant values are checked against an independent numpy/torch
evaluation: torch's float8_e4m3fn cast for the E4M3 scale, a nearest-value
search for the codes."""
import numpy as np
import pytest
import torch

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import bf16_bits_to_f32, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nearest_grid(m):
    """E2M1 magnitude code of m >= 0: nearest grid value, ties to the even
    code, above 6 saturating to code 7."""
    d = np.abs(m[..., None] - GRID)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, np.arange(8), 99)
    even = np.where(cand % 2 == 0, cand, 99).min(axis=-1)
    return np.where(even < 99, even, cand.min(axis=-1))


@pytest.mark.parametrize("r", [2, 4])
def test_compress_ratio_rotates_at_group_first_position(r):
    wl = workloads.sweep_case(20, 40, 16, True, 64)
    wl.positions[:] = np.arange(100, 140)
    slots = np.arange(1, 41, dtype=np.int64)
    got = np.zeros((41, 68), np.uint8)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, got, compress_ratio=r)
    first = wl.positions - wl.positions % r
    x = oracle.rope_rows(bf16_bits_to_f32(wl.k), wl.cos_sin[first])
    assert np.array_equal(got[1:], oracle.quantize_rows_two_stage(x))
    # every token of a group is rotated alike: identical rows give identical records
    k = np.repeat(wl.k[:1], 40, axis=0)
    same = np.zeros((41, 68), np.uint8)
    oracle.k_rope_pack_store_sglang(k, wl.positions, wl.cos_sin, slots, same, compress_ratio=r)
    for g in range(0, 40, r):
        assert (same[1 + g: 1 + g + r] == same[1 + g]).all()
    assert not np.array_equal(same[1], same[1 + r])


def test_ratio_one_is_the_plain_key_store():
    wl = workloads.sweep_case(21, 30, 16, False, 0)
    slots = np.arange(1, 31, dtype=np.int64)
    a = np.zeros((31, 68), np.uint8)
    b = np.zeros((31, 68), np.uint8)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, a, is_neox=False,
                                    rope_offset=0)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, b, is_neox=False,
                                    rope_offset=0, compress_ratio=1)
    assert np.array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, b, compress_ratio=3)


def test_ue8m0_fake_quant_is_the_decoded_quantizer():
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((300, 128)) * 2.0 ** rng.integers(-30, 30, (300, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :32] = -0.0
    x[2, 0] = np.float32(3.3e38)                 # codes 6/7 at e = 253: the value is infinite
    x = bf16_bits_to_f32(to_bf16_bits(x))
    y = oracle.fake_quant_rows(x, oracle.FQ_UE8M0_32)
    b, e = oracle.quantize_rows(x)
    nib = np.stack([b & 15, b >> 4], axis=-1).reshape(300, 128)
    mag = GRID[nib & 7] * np.ldexp(1.0, np.repeat(e.astype(np.int64), 32, axis=1) - 127)
    val = np.where(nib & 8, -mag, mag)
    want = torch.from_numpy(val).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, want)
    assert bf16_bits_to_f32(y[2, :1])[0] == np.inf


def test_e4m3_fake_quant_against_torch():
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((400, 128)) * 2.0 ** rng.integers(-12, 8, (400, 1))).astype(np.float32)
    x[0] = 0.0
    x[1, :16] = -0.0
    x[2, 16:32] = np.float32(1e-6) * np.sign(rng.standard_normal(16))   # scale rounds to 0
    x = bf16_bits_to_f32(to_bf16_bits(x))
    floor = float(np.float32(2.0 ** -126))
    y = oracle.fake_quant_rows(x, oracle.FQ_E4M3_16, floor)
    g = x.reshape(400, 8, 16).astype(np.float64)
    amax = np.abs(g).max(axis=-1)
    q = np.maximum((amax.astype(np.float32) / np.float32(6.0)), np.float32(floor))
    s = torch.from_numpy(q).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g.astype(np.float32) / s[..., None].astype(np.float32)).astype(np.float64)
    code = nearest_grid(np.abs(np.nan_to_num(ratio)))
    val = np.where(s[..., None] == 0, 0.0, GRID[code] * s[..., None])
    val = np.copysign(val, g)
    want = torch.from_numpy(val.reshape(400, 128)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(y, want.view(np.uint16))
    assert (y[2, 16:32] & 0x7FFF == 0).all()
    assert (y[1, :16] == 0x8000).all()


def test_e4m3_grid_groups_are_fixed_points():
    """x = code value * s with amax = 6 s for an e4m3 value s: the fake quant
    returns x unchanged."""
    rng = np.random.default_rng(24)
    s = np.array([0.5, 0.75, 1.125, 3.25, 2.0 ** -7, 96.0])
    x = np.copysign(GRID[rng.integers(0, 8, (6, 16))], rng.standard_normal((6, 16))) * s[:, None]
    x[:, 0] = 6.0 * s
    x = np.tile(x.reshape(-1), 2)[:128].reshape(1, 128)[:, :96]
    row = np.zeros((1, 128))
    row[0, :96] = x
    row = row.astype(np.float32)
    y = bf16_bits_to_f32(oracle.fake_quant_rows(row, oracle.FQ_E4M3_16))
    assert np.array_equal(y, row)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("r", [1, 2, 4])
def test_rope_fake_quant_composition(mode, r):
    wl = workloads.sweep_case(25 + r, 24, 32, True, 64, positions_int32=True)
    y = oracle.rope_fake_quant(wl.q, wl.positions, wl.cos_sin, rows_per_position=32,
                               compress_ratio=r, mode=mode)
    assert y.shape == wl.q.shape
    p = wl.positions.astype(np.int64)
    first = p - p % r
    cs = np.repeat(wl.cos_sin[first], 32, axis=0)
    x = oracle.rope_rows(bf16_bits_to_f32(wl.q).reshape(-1, 128), cs)
    assert np.array_equal(y.reshape(-1, 128), oracle.fake_quant_rows(x, mode))
