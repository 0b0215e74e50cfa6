"""Pins for the oracle's sglang-compatible mode (sgl-project/sglang PR 39656:
"Summary" -- two quantization stages and the 68-byte index-K record of 64
e2m1 bytes plus four block exponents; review -- the clear_negative_zero mask
and the packer's sign = (x < 0) & (idx != 0); the packer's floor differs
from the fake quant's, so packing the first stage directly gives other
bytes)."""
import numpy as np

import oracle
from pack_token_amd import workloads
from pack_token_amd.workloads import bf16_bits_to_f32, to_bf16_bits

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float32)


def clear_negative_zero(p):
    """The review's mask: bit 4k of (p | p>>1 | p>>2) & 0x11111111 is set iff a
    magnitude bit of nibble k is set; keep a sign bit only there."""
    p = np.asarray(p, np.uint32)
    nz = (p | (p >> 1) | (p >> 2)) & np.uint32(0x11111111)
    return p & (np.uint32(0x77777777) | (nz << np.uint32(3)))


def test_mask_identity_exhaustive_on_16_bits():
    p = np.arange(1 << 16, dtype=np.uint32)
    nib = np.stack([(p >> (4 * k)) & 15 for k in range(4)])
    got = clear_negative_zero(p)
    want = np.zeros_like(p)
    for k in range(4):
        n = nib[k]
        keep = np.where((n & 7) == 0, n & 7, n)        # sign survives iff magnitude != 0
        want |= keep << np.uint32(4 * k)
    assert np.array_equal(got, want)


def rows_with_max_code_7(rng, n):
    """Rows whose every group holds 6*2^k exactly, so stage 2 keeps stage 1's exponent."""
    x = rng.standard_normal((n, 128)).astype(np.float32)
    x = bf16_bits_to_f32(to_bf16_bits(x))
    g = np.abs(x.reshape(n, 4, 32)).max(axis=2)
    k = np.ceil(np.log2(g / 6.0))
    x = x.reshape(n, 4, 32)
    x[:, :, 0] = np.float32(6.0) * np.ldexp(np.float32(1.0), k.astype(np.int32))
    return bf16_bits_to_f32(to_bf16_bits(x.reshape(n, 128)))


def test_two_stage_equals_masked_one_stage_when_the_max_code_is_6():
    rng = np.random.default_rng(1)
    x = rows_with_max_code_7(rng, 300)
    one, e = oracle.quantize_rows(x)
    rec = oracle.quantize_rows_two_stage(x)
    assert np.array_equal(rec[:, 64:], e)
    masked = clear_negative_zero(one.view(np.uint32)).view(np.uint8)
    assert np.array_equal(rec[:, :64], masked.reshape(300, 64))


def test_two_stage_lowers_the_exponent_when_the_max_rounds_to_3():
    """amax = 3.25*2^k: stage 1 picks e = 127+k and rounds 3.25 to 3 (code 5);
    stage 2 sees amax 3*2^k, picks e = 126+k and re-encodes 3*2^k as 6 (code 7):
    packing the first stage directly would not give these bytes."""
    for k in (-10, 0, 7):
        x = np.zeros((1, 128), np.float32)
        x[0, :32] = np.float32(1.0 * 2.0 ** k)
        x[0, 0] = np.float32(3.25 * 2.0 ** k)
        x[0, 1] = np.float32(-0.1 * 2.0 ** k)            # rounds to zero: +0 code in stage 2
        one, e = oracle.quantize_rows(x)
        rec = oracle.quantize_rows_two_stage(x)
        assert e[0, 0] == 127 + k and rec[0, 64] == 126 + k
        assert one[0, 0] == (0x8 << 4) | 5                # stage-1 codes: 5 and -0
        assert rec[0, 0] == 7                              # stage 2: 6 (code 7), then +0
        assert rec[0, 1] == 0x44                           # 1*2^k at e = 126+k is 2: code 4
        assert not np.array_equal(rec[0, :64], clear_negative_zero(one.view(np.uint32)).view(np.uint8))


def test_separate_floors():
    x = np.zeros((2, 128), np.float32)
    x[1] = np.float32(1e-6)                               # tiny against a 1e-4 stage-1 floor
    f1, f2 = float(np.float32(1e-4)), float(np.float32(1e-10))
    rec = oracle.quantize_rows_two_stage(x, f1, f2)
    # all-zero rows and rows that stage 1 flushes to zero take the packer's floor exponent
    assert (rec[:, 64:] == 94).all()
    assert not rec[:, :64].any()
    # with the floors the other way round stage 1 keeps the values
    rec2 = oracle.quantize_rows_two_stage(x, f2, f1)
    assert (rec2[1, 64:] == 114).all() and (rec2[0, 64:] == 114).all()


def test_key_records_slot_zero_and_layout():
    wl = workloads.sweep_case(3, 12, 16, True, 64)
    wl.slot_mapping[:] = [0, 1, 2, 3, -1, 5, 6, 7, 8, 9, 10, 100]   # 0, -1 and 100 publish nothing
    cache = np.full((12, 68), 0xA5, np.uint8)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, wl.slot_mapping, cache)
    assert (cache[0] == 0xA5).all() and (cache[4] == 0xA5).all() and (cache[11] == 0xA5).all()
    # the record of a token is the two-stage quantization of its rotated row
    x = oracle.rope_rows(bf16_bits_to_f32(wl.k), wl.cos_sin[wl.positions])
    rec = oracle.quantize_rows_two_stage(x)
    for t, s in enumerate(wl.slot_mapping):
        if 0 < s < 12:
            assert np.array_equal(cache[s], rec[t])


def test_key_records_with_rmsnorm_and_interleaved_rope():
    rng = np.random.default_rng(5)
    wl = workloads.sweep_case(4, 40, 16, False, 0)
    gamma = to_bf16_bits(rng.uniform(0.5, 1.5, 128).astype(np.float32))
    cache = np.full((64, 68), 0xA5, np.uint8)
    slots = np.arange(1, 41, dtype=np.int64)
    oracle.k_rope_pack_store_sglang(wl.k, wl.positions, wl.cos_sin, slots, cache,
                                    k_norm_gamma=gamma, k_norm_eps=1e-6, is_neox=False,
                                    rope_offset=0)
    x = oracle.rmsnorm_rows(bf16_bits_to_f32(wl.k), gamma, 1e-6)
    x = oracle.rope_rows(x, wl.cos_sin[wl.positions], rope_offset=0, is_neox=False)
    assert np.array_equal(cache[1:41], oracle.quantize_rows_two_stage(x))
    assert (cache[0] == 0xA5).all() and (cache[41:] == 0xA5).all()


def test_query_records_per_head():
    wl = workloads.sweep_case(6, 9, 32, True, 64)
    qrec = oracle.q_rope_pack_sglang(wl.q, wl.positions, wl.cos_sin)
    assert qrec.shape == (9, 32, 68)
    cs = np.repeat(wl.cos_sin[wl.positions], 32, axis=0)
    x = oracle.rope_rows(bf16_bits_to_f32(wl.q).reshape(9 * 32, 128), cs)
    assert np.array_equal(qrec.reshape(9 * 32, 68), oracle.quantize_rows_two_stage(x))
    # the query and key sides produce the same record for the same row
    cache = np.zeros((10, 68), np.uint8)
    oracle.k_rope_pack_store_sglang(wl.q[:, 5], wl.positions, wl.cos_sin,
                                    np.arange(1, 10, dtype=np.int64), cache)
    assert np.array_equal(cache[1:], qrec[:, 5])
