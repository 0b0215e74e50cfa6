"""GPU parity of the sglang-compatible mode (sgl-project/sglang PR 39656:
"Summary" -- RoPE, two quantization stages and the 68-byte index-K record;
review -- +0 codes and the separate floors of the two stages): the HIP path
through the C ABI against the CPU oracle, byte for byte, on the row matrix of
that page's "Verification" (rows {1, 5, 64, 300}, scales {1, 40, 1e-3} plus
zero, subnormal and half-way groups, int32/int64 positions), with the floors
equal and apart, every finite bf16 value under every stage-1 exponent, and
the full-size prefill shape."""
import numpy as np
import pytest

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import SENTINEL
from harness import ORACLE_THREADS, assert_same, large_prefill, random_case, say

pytestmark = pytest.mark.gpu

FMIN = float(np.float32(2.0 ** -126))
FLOORS = {"equal": (FMIN, FMIN), "fq_high": (1e-4, 1e-10), "pack_high": (FMIN, 1e-3),
          "fq_dominant": (1e-3, FMIN)}


def _t(a, dev="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_q(q, positions, cos_sin, **kw):
    import torch
    from pack_token_amd import fp4idx
    T, H, _ = q.shape
    out = torch.full((T, H, 68), SENTINEL, dtype=torch.uint8, device="cuda:0")
    fp4idx.q_rope_pack_sglang(_t(q.view(np.int16)), _t(positions), _t(cos_sin), q_packed=out, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_k(k, positions, cos_sin, slots, num_slots, gamma=None, **kw):
    import torch
    from pack_token_amd import fp4idx
    cache = torch.full((num_slots, 68), SENTINEL, dtype=torch.uint8, device="cuda:0")
    fp4idx.k_rope_pack_store_sglang(_t(k.view(np.int16)), _t(positions), _t(cos_sin), _t(slots),
                                    cache, k_norm_gamma=None if gamma is None else
                                    _t(gamma.view(np.int16)), **kw)
    torch.cuda.synchronize()
    return cache.cpu().numpy()


def check_both(wl, slots, num_slots, gamma=None, floors=(FMIN, FMIN), ratio=1):
    kw = dict(is_neox=wl.is_neox, rope_offset=wl.rope_offset, fake_quant_floor=floors[0],
              pack_floor=floors[1])
    say(f"case sglang {wl.name}: T={wl.T} H={wl.H} neox={wl.is_neox} ro={wl.rope_offset} "
        f"norm={gamma is not None} floors={floors} slots={num_slots}")
    got_q = gpu_q(wl.q, wl.positions, wl.cos_sin, **kw)
    ref_q = oracle.q_rope_pack_sglang(wl.q, wl.positions, wl.cos_sin, **kw)
    assert_same("q_packed", got_q, ref_q)
    got_k = gpu_k(wl.k, wl.positions, wl.cos_sin, slots, num_slots, gamma, k_norm_eps=1e-6,
                  compress_ratio=ratio, **kw)
    ref_k = np.full((num_slots, 68), SENTINEL, np.uint8)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, ref_k,
                                    k_norm_gamma=gamma, k_norm_eps=1e-6, compress_ratio=ratio,
                                    **kw)
    assert_same("index_k_cache", got_k, ref_k)


def with_slot_zero(wl):
    """The workload's slots with slot 0, -1 and one past the end planted."""
    slots = wl.slot_mapping.copy()
    num_slots = wl.NB * 64
    if wl.T >= 1:
        slots[0] = 0
    if wl.T >= 5:
        slots[2] = -1
        slots[4] = num_slots
    return slots, num_slots


@pytest.mark.parametrize("T", [1, 5, 64, 300])
@pytest.mark.parametrize("pos32", [False, True])
def test_row_matrix(T, pos32):
    wl = workloads.edge_mix(seed=300 + T, T=T, positions_int32=pos32)
    slots, n = with_slot_zero(wl)
    check_both(wl, slots, n)


@pytest.mark.parametrize("ratio", [2, 4])
@pytest.mark.parametrize("pos32", [False, True])
def test_compress_ratio(ratio, pos32):
    """Compressed key rows rotated at their group's first position (sglang PR
    39656 "Verification": compress ratios 1, 2, 4; ratio 1 is every other test)."""
    wl = workloads.edge_mix(seed=330 + ratio, T=300, positions_int32=pos32)
    slots, n = with_slot_zero(wl)
    check_both(wl, slots, n, ratio=ratio)


@pytest.mark.parametrize("floors", sorted(FLOORS))
def test_floors(floors):
    wl = workloads.edge_mix(seed=41, T=120, H=32)
    slots, n = with_slot_zero(wl)
    check_both(wl, slots, n, floors=FLOORS[floors])


@pytest.mark.parametrize("neox,ro", [(True, 64), (True, 0), (False, 64), (False, 0)])
def test_modes_with_rmsnorm(neox, ro):
    wl = workloads.sweep_case(51, 77, 48, neox, ro, positions_int32=not neox)
    rng = np.random.default_rng(52)
    gamma = workloads.to_bf16_bits((1.0 + 0.2 * rng.standard_normal(128)).astype(np.float32))
    slots, n = with_slot_zero(wl)
    check_both(wl, slots, n, gamma=gamma)


@pytest.mark.parametrize("neox,ro", [(True, 64), (True, 0), (False, 64), (False, 0)])
def test_overflow_rows(neox, ro):
    """Rows whose rotation leaves the fp32 range (one RoPE pair of
    largest-magnitude bf16 values in about half of the rows): the stage-1
    amax is infinite, so e1 = 254, and the infinite values take code 7."""
    wl = workloads.overflow_case(61 + ro + neox, 300, 16, neox, ro, False)
    ref = oracle.q_rope_pack_sglang(wl.q, wl.positions, wl.cos_sin, is_neox=neox, rope_offset=ro)
    assert (ref[:, :, 64:] == 254).any()  # the case reaches e = 254
    slots, n = with_slot_zero(wl)
    check_both(wl, slots, n)


def test_maximum_heads():
    """H = 2048 query records (139 KB per token) and ragged T."""
    wl = workloads.sweep_case(778, 5, 2048, False, 0)
    slots, n = with_slot_zero(wl)
    check_both(wl, slots, n)


def test_empty():
    wl = workloads.tiny(T=0, H=16)
    got = gpu_q(wl.q, wl.positions, wl.cos_sin)
    assert got.shape == (0, 16, 68)
    cache = gpu_k(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, 64)
    assert (cache == SENTINEL).all()


def _exhaustive_rows(anchor_for):
    """Groups that carry every finite bf16 value under each anchor (the group's
    largest magnitude), 31 values and the anchor per group, laid out as the
    unrotated groups 0-1 of query heads."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[((allb.astype(np.uint32) >> 7) & 0xFF) != 0xFF]
    mag = finite & 0x7FFF
    groups = []
    for anchor in anchor_for:
        vals = finite[mag <= anchor]
        n = -(-vals.size // 31) * 31
        vals = np.concatenate([vals, np.zeros(n - vals.size, np.uint16)]).reshape(-1, 31)
        g = np.empty((vals.shape[0], 32), np.uint16)
        g[:, 0] = anchor
        g[:, 1:] = vals
        groups.append(g)
    groups = np.concatenate(groups)
    H = 64
    rows = -(-groups.shape[0] // 2)
    T = -(-rows // H)
    q = np.zeros((T * H, 128), np.uint16)
    flat = np.zeros((T * H * 2, 32), np.uint16)
    flat[: groups.shape[0]] = groups
    q[:, :64] = flat.reshape(T * H, 64)
    return q.reshape(T, H, 128), groups.shape[0]


def test_two_stage_exhaustive():
    """Every finite bf16 value under every stage-1 exponent e1 in [1, 253]
    (anchor 6 * 2^(e1-127), or the largest bf16 for 253, whose fake-quant
    values overflow to infinity)."""
    anchors = [0x7F7F if e == 253 else int(workloads.to_bf16_bits(
        np.array([6.0 * 2.0 ** (e - 127)], np.float32))[0]) for e in range(1, 254)]
    q, ng = _exhaustive_rows(anchors)
    pos = np.zeros(q.shape[0], np.int64)
    cs = workloads.cos_sin_table(1)
    say(f"case sglang two_stage_exhaustive: {ng} groups, T={q.shape[0]}")
    assert_same("q_packed", gpu_q(q, pos, cs), oracle.q_rope_pack_sglang(q, pos, cs))


@pytest.mark.parametrize("floors", [(float(np.float32(1.5 * 2.0 ** 126)), FMIN),
                                    (FMIN, float(np.float32(1.5 * 2.0 ** 126))),
                                    (float(np.float32(2.0 ** 125)), float(np.float32(2.0 ** 120)))])
def test_extreme_floors(floors):
    """Floors that force e1 = 254 (the fake-quant values of codes >= 4 are
    infinite), e2 = 254, and e1 = 252 over every finite bf16 value."""
    q, ng = _exhaustive_rows([0x7F7F, 0x3F80, 0x0001])
    pos = np.zeros(q.shape[0], np.int64)
    cs = workloads.cos_sin_table(1)
    kw = dict(fake_quant_floor=floors[0], pack_floor=floors[1])
    say(f"case sglang extreme_floors {floors}: {ng} groups")
    assert_same("q_packed", gpu_q(q, pos, cs, **kw), oracle.q_rope_pack_sglang(q, pos, cs, **kw))


def test_large_prefill_full_size():
    """T = 131072, H = 64: every query record of every token and every key
    record, byte for byte."""
    wl = large_prefill()
    say(f"case sglang large_prefill: T={wl.T} H={wl.H}")
    got_q = gpu_q(wl.q, wl.positions, wl.cos_sin)
    ref_q = oracle.q_rope_pack_sglang(wl.q, wl.positions, wl.cos_sin, threads=ORACLE_THREADS)
    assert_same("q_packed", got_q, ref_q)
    del ref_q
    assert (got_q[..., 64:] >= 1).all() and (got_q[..., 64:] <= 254).all()
    del got_q
    slots = wl.slot_mapping + 1                 # slot 0 stays unpublished
    n = wl.NB * 64 + 1
    got_k = gpu_k(wl.k, wl.positions, wl.cos_sin, slots, n)
    ref_k = np.full((n, 68), SENTINEL, np.uint8)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, ref_k)
    assert_same("index_k_cache", got_k, ref_k)


@pytest.mark.parametrize("seed", range(12))
def test_random_cases(seed):
    """Seeded random shapes and modes (the producer's random cases) through the
    sglang-compatible records: any floor pair, compress ratio 1, 2 or 4, key
    RMSNorm as drawn, slot 0 and past-the-end slots among the draws."""
    wl, _ = random_case(200 + seed)
    rng = np.random.default_rng(seed)
    slots = wl.slot_mapping.copy()
    slots[rng.random(wl.T) < 0.03] = 0
    floors = FLOORS[sorted(FLOORS)[seed % len(FLOORS)]]
    check_both(wl, slots, wl.NB * 64, wl.k_norm_gamma, floors, ratio=[1, 2, 4][seed % 3])
