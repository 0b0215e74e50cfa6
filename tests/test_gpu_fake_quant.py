"""GPU parity of the RoPE tail + FP4 fake quant (sgl-project/sglang PR 39656
"Summary": per-32 UE8M0 scales by default, per-16 E4M3 scales for compressed
KV, bf16 round trip after RoPE, round half to even; "Verification": compress
ratios 1, 2, 4): the HIP path through the C ABI against the CPU oracle, bit
for bit on the bf16 outputs."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads
from harness import assert_same, random_case, say

pytestmark = pytest.mark.gpu

MODES = {"ue8m0_32": 0, "e4m3_16": 1}


def _t(a, dev="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_fq(x, positions, cos_sin, **kw):
    import torch
    from pack_token_amd import fp4idx
    y = torch.full(x.shape, -1, dtype=torch.int16, device="cuda:0")
    fp4idx.rope_fake_quant(_t(x.view(np.int16)), _t(positions), _t(cos_sin), y=y, **kw)
    torch.cuda.synchronize()
    return y.cpu().numpy().view(np.uint16)


def check(x, positions, cos_sin, mode, **kw):
    say(f"case fake_quant {x.shape} mode={mode} {kw}")
    got = gpu_fq(x, positions, cos_sin, mode=mode, **kw)
    ref = oracle.rope_fake_quant(x, positions, cos_sin, mode=MODES[mode], **kw)
    assert_same("y", got, ref)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("ratio", [1, 2, 4])
@pytest.mark.parametrize("pos32", [False, True])
def test_edge_mix_queries_and_keys(mode, ratio, pos32):
    wl = workloads.edge_mix(seed=600 + ratio, T=120, H=32, positions_int32=pos32)
    check(wl.q, wl.positions, wl.cos_sin, mode, rows_per_position=32, compress_ratio=ratio,
          is_neox=wl.is_neox, rope_offset=wl.rope_offset)
    check(wl.k, wl.positions, wl.cos_sin, mode, compress_ratio=ratio, is_neox=wl.is_neox,
          rope_offset=wl.rope_offset)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("neox,ro", [(True, 64), (True, 0), (False, 64), (False, 0)])
def test_modes_ragged(mode, neox, ro):
    wl = workloads.sweep_case(610 + ro + neox, 37, 48, neox, ro)
    check(wl.q, wl.positions, wl.cos_sin, mode, rows_per_position=48, is_neox=neox,
          rope_offset=ro)


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("neox,ro", [(True, 64), (False, 0)])
def test_overflow_rows(mode, neox, ro):
    """Rows whose rotation leaves the fp32 range (one RoPE pair of
    largest-magnitude bf16 values in about half of the rows)."""
    wl = workloads.overflow_case(81 + ro + neox, 37, 48, neox, ro, False)
    check(wl.q, wl.positions, wl.cos_sin, mode, rows_per_position=48, is_neox=neox,
          rope_offset=ro)
    check(wl.k, wl.positions, wl.cos_sin, mode, is_neox=neox, rope_offset=ro)


@pytest.mark.parametrize("mode", sorted(MODES))
def test_floors(mode):
    wl = workloads.edge_mix(seed=620, T=40, H=16)
    for floor in (0.0, 1e-3, 3.0):
        check(wl.k, wl.positions, wl.cos_sin, mode, scale_floor=floor, is_neox=False)


def _anchor_rows(anchors, group):
    """Rows whose dims 0..63 (left unrotated) hold groups of `group` values:
    one anchor (the group's largest magnitude) and group-1 finite bf16 values
    below it, every such value once per anchor."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb.astype(np.uint32) >> 7) & 0xFF) != 0xFF]
    mag = finite & 0x7FFF
    gs = []
    for anchor in anchors:
        vals = finite[mag <= anchor]
        k = group - 1
        n = -(-vals.size // k) * k
        vals = np.concatenate([vals, np.zeros(n - vals.size, np.uint16)]).reshape(-1, k)
        g = np.empty((vals.shape[0], group), np.uint16)
        g[:, 0] = anchor
        g[:, 1:] = vals
        gs.append(g)
    gs = np.concatenate(gs)
    per_row = 64 // group
    rows = -(-gs.shape[0] // per_row)
    flat = np.zeros((rows * per_row, group), np.uint16)
    flat[: gs.shape[0]] = gs
    x = np.zeros((rows, 128), np.uint16)
    x[:, :64] = flat.reshape(rows, 64)
    return x, gs.shape[0]


def test_e4m3_exhaustive():
    """Every finite bf16 value under anchors 6 s for every positive e4m3fn
    value s, plus anchors between them and above 6 * 448 (saturated scale)."""
    E = np.arange(127)
    s = np.where(E >> 3 == 0, (E & 7) * 2.0 ** -9, (8 + (E & 7)) * 2.0 ** ((E >> 3) - 10.0))
    a = np.concatenate([6 * s[1:], 6 * s[1:] * 1.03, [2688.0, 5000.0, 3.0e38]])
    anchors = sorted(set(int(b) for b in workloads.to_bf16_bits(a.astype(np.float32))))
    x, n = _anchor_rows(anchors, 16)
    pos = np.zeros(x.shape[0], np.int64)
    say(f"case fake_quant e4m3_exhaustive: {n} groups, rows={x.shape[0]}")
    check(x, pos, workloads.cos_sin_table(1), "e4m3_16")


def test_ue8m0_exhaustive():
    """Every finite bf16 value under every block exponent e in [1, 253]
    (anchor 6 * 2^(e-127), or the largest bf16 for 253, whose large codes
    have infinite values)."""
    anchors = [0x7F7F if e == 253 else int(workloads.to_bf16_bits(
        np.array([6.0 * 2.0 ** (e - 127)], np.float32))[0]) for e in range(1, 254)]
    x, n = _anchor_rows(anchors, 32)
    pos = np.zeros(x.shape[0], np.int64)
    say(f"case fake_quant ue8m0_exhaustive: {n} groups, rows={x.shape[0]}")
    check(x, pos, workloads.cos_sin_table(1), "ue8m0_32")


def test_empty():
    x = np.zeros((0, 128), np.uint16)
    assert gpu_fq(x, np.zeros(0, np.int64), workloads.cos_sin_table(4)).shape == (0, 128)


@pytest.mark.parametrize("seed", range(12))
def test_random_cases(seed):
    """Seeded random shapes and modes (the producer's random cases) through the
    RoPE tail + fake quant, queries (H rows per position) and keys, both
    scale modes, compress ratio 1, 2 or 4, the drawn floor."""
    wl, _ = random_case(300 + seed)
    mode = sorted(MODES)[seed % 2]
    kw = dict(compress_ratio=[1, 2, 4][seed % 3], is_neox=wl.is_neox, rope_offset=wl.rope_offset,
              scale_floor=wl.scale_floor)
    check(wl.q, wl.positions, wl.cos_sin, mode, rows_per_position=wl.H, **kw)
    check(wl.k, wl.positions, wl.cos_sin, mode, **kw)
