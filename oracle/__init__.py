"""CPU oracle for the fused FP4 sparse-indexer producer.

TEST INFRASTRUCTURE ONLY: the plain scalar definition (``fp4idx_oracle.c``)
that the HIP kernels are checked against.  Only ``tests/``, the smoke check
and the CPU-baseline leg of ``bench.py`` may import this package.  It shares
no code with ``pack_token_amd`` and imports nothing from it.

Arrays are numpy, host memory.  bf16 tensors are passed as their uint16 bit
patterns.  Function arguments mean what the C-ABI arguments of the same name
mean (see ``include/fp4idx.h``).
"""
from __future__ import annotations

import ctypes
import os
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

_LIB = None
_LOCK = threading.Lock()

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            # FP4IDX_ORACLE_LIB: an alternative build of this oracle (used by the
            # mutation check, which loads deliberately broken copies)
            path = os.environ.get("FP4IDX_ORACLE_LIB") or _build.LIB
            if path == _build.LIB and not os.path.exists(path):
                _build.build()
            lib = ctypes.CDLL(path)
            lib.oracle_q_rope_pack.argtypes = [_p, _p, _i, _p, _i64, _p, _i64, _i, _i, _i, _i, _i,
                                               _i, _i, _f, _p, _p, _p]
            lib.oracle_q_rope_pack.restype = _i
            lib.oracle_k_rope_pack_store.argtypes = [_p, _p, _i, _p, _i64, _p, _p, _f, _i64, _i, _i,
                                                     _i, _i, _i, _i, _f, _p, _p, _i64, _i]
            lib.oracle_k_rope_pack_store.restype = _i
            lib.oracle_dequant.argtypes = [_i, _p, _p, _i64, _i, _p, _i64, _i, _p]
            lib.oracle_dequant.restype = _i
            lib.oracle_bf16_round.argtypes = [_p, _p, _i64]
            lib.oracle_bf16_round.restype = None
            lib.oracle_group_exponents.argtypes = [_p, _i64, _i, _f, _p]
            lib.oracle_group_exponents.restype = None
            lib.oracle_e2m1_nibbles.argtypes = [_p, _p, _i64, _p]
            lib.oracle_e2m1_nibbles.restype = None
            lib.oracle_quantize_rows.argtypes = [_p, _i64, _f, _p, _p]
            lib.oracle_quantize_rows.restype = None
            lib.oracle_rope_rows.argtypes = [_p, _p, _i64, _i, _i]
            lib.oracle_rope_rows.restype = None
            lib.oracle_fwht_rows.argtypes = [_p, _i64]
            lib.oracle_fwht_rows.restype = None
            lib.oracle_rmsnorm_rows.argtypes = [_p, _p, _f, _i64]
            lib.oracle_rmsnorm_rows.restype = None
            lib.oracle_paged_mqa_logits.argtypes = [_p, _p, _p, _f, _p, _p, _i64, _p, _i64, _p,
                                                    _i64, _i, _i, _i, _p, _i64, _p]
            lib.oracle_paged_mqa_logits.restype = _i
            lib.oracle_q_rope_pack_sglang.argtypes = [_p, _p, _i, _p, _i64, _i64, _i, _i, _i, _i,
                                                      _i, _i, _f, _f, _p]
            lib.oracle_q_rope_pack_sglang.restype = _i
            lib.oracle_k_rope_pack_store_sglang.argtypes = [_p, _p, _i, _p, _i64, _p, _p, _f, _i64,
                                                            _i, _i, _i, _i, _i, _i, _f, _f, _p,
                                                            _i64]
            lib.oracle_rope_fake_quant.argtypes = [_p, _i64, _i, _p, _i, _p, _i64, _i, _i, _i, _i,
                                                   _i, _i, _f, _p]
            lib.oracle_rope_fake_quant.restype = _i
            lib.oracle_fake_quant_rows.argtypes = [_p, _i64, _i, _f, _p]
            lib.oracle_fake_quant_rows.restype = None
            lib.oracle_k_rope_pack_store_sglang.restype = _i
            lib.oracle_quantize_rows_two_stage.argtypes = [_p, _i64, _f, _f, _p]
            lib.oracle_quantize_rows_two_stage.restype = None
            lib.oracle_q_rope_pack_fp8.argtypes = [_p, _p, _i, _p, _i64, _p, _f, _i64, _i, _i, _i,
                                                   _i, _i, _i, _i, _f, _p, _p]
            lib.oracle_q_rope_pack_fp8.restype = _i
            lib.oracle_k_rope_pack_store_fp8.argtypes = [_p, _p, _i, _p, _i64, _p, _p, _f, _i64,
                                                         _i, _i, _i, _i, _i, _i, _f, _p, _p, _i64,
                                                         _i]
            lib.oracle_k_rope_pack_store_fp8.restype = _i
            lib.oracle_e4m3_codes.argtypes = [_p, _i64, _p]
            lib.oracle_e4m3_codes.restype = None
            lib.oracle_fp8_scales.argtypes = [_p, _i64, _f, _i, _p]
            lib.oracle_fp8_scales.restype = None
            lib.oracle_quantize_rows_fp8.argtypes = [_p, _i64, _f, _i, _p, _p]
            lib.oracle_quantize_rows_fp8.restype = None
            lib.oracle_hadamard_scale.argtypes = []
            lib.oracle_hadamard_scale.restype = _f
            _LIB = lib
    return _LIB


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


HEAD_DIM = 128
ROPE_DIM = 64
KV_BLOCK = 64
DEFAULT_SCALE_FLOOR = float(np.float32(2.0 ** -126))


def q_scale_cols(H: int) -> int:
    """J = round_up(H/16, 4): last axis of the q-scale tensor."""
    return ((H // 16) + 3) // 4 * 4


def _split(T, threads):
    threads = max(1, int(threads))
    step = -(-T // threads) if T else 0
    return [(a, min(T, a + step)) for a in range(0, T, step)] if T else []


def q_rope_pack(q_bits, positions, cos_sin, weights=None, *, is_neox=True, rope_offset=64,
                apply_hadamard=False, scale_floor=DEFAULT_SCALE_FLOOR, threads=1):
    """Query path.  q_bits uint16 [T,H,128]; positions int32/int64 [T];
    cos_sin fp32 [max_pos,64]; weights fp32 [T,H] or None.
    Returns (q_out u8 [T,H,64], q_scale_out u8 [T,1,4,16,J], weights_out fp32 [T,H] or None)."""
    q_bits = _c(q_bits, np.uint16)
    T, H, D = q_bits.shape
    positions = np.ascontiguousarray(positions)
    pos64 = 1 if positions.dtype == np.int64 else 0
    if not pos64:
        positions = _c(positions, np.int32)
    cos_sin = _c(cos_sin, np.float32)
    max_pos = cos_sin.shape[0]
    J = q_scale_cols(H)
    # outputs start as a sentinel so bytes the oracle fails to write show up
    q_out = np.full((T, H, D // 2), 0xA5, np.uint8)
    q_scale = np.full((T, 1, 4, 16, J), 0xA5, np.uint8)
    w_out = None
    if weights is not None:
        weights = _c(weights, np.float32)
        w_out = np.full((T, H), np.nan, np.float32)
    lib = _lib()
    psz = positions.itemsize

    def run(rng):
        a, b = rng
        rc = lib.oracle_q_rope_pack(
            q_bits.ctypes.data + a * H * D * 2, positions.ctypes.data + a * psz, pos64,
            cos_sin.ctypes.data, max_pos,
            None if weights is None else weights.ctypes.data + a * H * 4,
            b - a, H, D, ROPE_DIM, rope_offset, 32, int(bool(is_neox)), int(bool(apply_hadamard)),
            scale_floor, q_out.ctypes.data + a * H * (D // 2), q_scale.ctypes.data + a * 64 * J,
            None if w_out is None else w_out.ctypes.data + a * H * 4)
        if rc != 0:
            raise ValueError(f"oracle_q_rope_pack rejected its arguments (rc={rc})")

    _run_ranges(run, _split(T, threads))
    return q_out, q_scale, w_out


def k_rope_pack_store(k_bits, positions, cos_sin, slot_mapping, kv_cache, kv_cache_scale, *,
                      k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                      apply_hadamard=False, scale_floor=DEFAULT_SCALE_FLOOR, threads=1):
    """Key path; writes kv_cache u8 [NB,1,4,64,16] and kv_cache_scale u8 [NB,1,4,64] in place."""
    k_bits = _c(k_bits, np.uint16)
    T, D = k_bits.shape
    positions = np.ascontiguousarray(positions)
    pos64 = 1 if positions.dtype == np.int64 else 0
    if not pos64:
        positions = _c(positions, np.int32)
    cos_sin = _c(cos_sin, np.float32)
    slot_mapping = _c(slot_mapping, np.int64)
    assert kv_cache.dtype == np.uint8 and kv_cache.flags.c_contiguous
    assert kv_cache_scale.dtype == np.uint8 and kv_cache_scale.flags.c_contiguous
    NB = kv_cache.shape[0]
    gamma = None if k_norm_gamma is None else _c(k_norm_gamma, np.uint16)
    lib = _lib()
    psz = positions.itemsize

    def run(rng):
        a, b = rng
        rc = lib.oracle_k_rope_pack_store(
            k_bits.ctypes.data + a * D * 2, positions.ctypes.data + a * psz, pos64,
            cos_sin.ctypes.data, cos_sin.shape[0], slot_mapping.ctypes.data + a * 8, _ptr(gamma),
            k_norm_eps, b - a, D, ROPE_DIM, rope_offset, 32, int(bool(is_neox)),
            int(bool(apply_hadamard)), scale_floor, kv_cache.ctypes.data, kv_cache_scale.ctypes.data,
            NB, KV_BLOCK)
        if rc != 0:
            raise ValueError(f"oracle_k_rope_pack_store rejected its arguments (rc={rc})")

    # slots are distinct by contract, so token ranges write disjoint bytes
    _run_ranges(run, _split(T, threads))
    return kv_cache, kv_cache_scale


def dequant_q(q_out, q_scale_out):
    T, H, _ = q_out.shape
    out = np.empty((T, H, HEAD_DIM), np.float32)
    rc = _lib().oracle_dequant(0, _c(q_out, np.uint8).ctypes.data, _c(q_scale_out, np.uint8).ctypes.data,
                               T, H, None, 0, KV_BLOCK, out.ctypes.data)
    assert rc == 0
    return out


def dequant_kcache(kv_cache, kv_cache_scale, slots=None):
    NB = kv_cache.shape[0]
    if slots is None:
        rows = NB * KV_BLOCK
        sp = None
    else:
        slots = _c(slots, np.int64)
        rows = slots.shape[0]
        sp = slots.ctypes.data
    out = np.empty((rows, HEAD_DIM), np.float32)
    rc = _lib().oracle_dequant(1, _c(kv_cache, np.uint8).ctypes.data,
                               _c(kv_cache_scale, np.uint8).ctypes.data, rows, 0, sp, NB, KV_BLOCK,
                               out.ctypes.data)
    assert rc == 0
    return out


def paged_mqa_logits(q_out, q_scale_out, weights, kv_cache, kv_cache_scale, block_table,
                     context_lens, next_n, *, weights_scale=1.0, apply_relu=True, stride=None,
                     logits=None, with_bound=False):
    """FP4 paged MQA logits.  q_out u8 [B*next_n,H,64], q_scale_out u8 [B*next_n,1,4,16,J],
    weights fp32 [B*next_n,H], kv cache u8 [NB,1,4,64,16] / [NB,1,4,64], block_table int32
    [B,max_blocks], context_lens int32 [B].  Returns logits fp32 [B*next_n, stride] (entries
    at or past a sequence's context length keep their initial value, NaN by default) and,
    with with_bound, the per-entry error scale abs_bound (float64, same shape)."""
    q_out = _c(q_out, np.uint8)
    T, H, _ = q_out.shape
    block_table = _c(block_table, np.int32)
    context_lens = _c(context_lens, np.int32)
    B, max_blocks = block_table.shape
    assert T == B * next_n
    if stride is None:
        stride = max(1, max_blocks * KV_BLOCK)
    if logits is None:
        logits = np.full((T, stride), np.nan, np.float32)
    bound = np.zeros((T, stride), np.float64) if with_bound else None
    rc = _lib().oracle_paged_mqa_logits(
        q_out.ctypes.data, _c(q_scale_out, np.uint8).ctypes.data, _c(weights, np.float32).ctypes.data,
        weights_scale, _c(kv_cache, np.uint8).ctypes.data, _c(kv_cache_scale, np.uint8).ctypes.data,
        kv_cache.shape[0], block_table.ctypes.data, max_blocks, context_lens.ctypes.data, B, next_n,
        H, int(bool(apply_relu)), logits.ctypes.data, stride, _ptr(bound))
    if rc != 0:
        raise ValueError(f"oracle_paged_mqa_logits rejected its arguments (rc={rc})")
    return (logits, bound) if with_bound else logits


SLOT68 = 68


def q_rope_pack_sglang(q_bits, positions, cos_sin, *, is_neox=True, rope_offset=64,
                       fake_quant_floor=DEFAULT_SCALE_FLOOR, pack_floor=DEFAULT_SCALE_FLOOR,
                       threads=1):
    """sglang-compatible query side: records u8 [T,H,68] (64 code bytes, 4 exponents).
    threads > 1 splits the tokens into ranges, each a separate call (tokens are
    independent)."""
    q_bits = _c(q_bits, np.uint16)
    T, H, D = q_bits.shape
    positions = np.ascontiguousarray(positions)
    pos64 = 1 if positions.dtype == np.int64 else 0
    if not pos64:
        positions = _c(positions, np.int32)
    cos_sin = _c(cos_sin, np.float32)
    out = np.full((T, H, SLOT68), 0xA5, np.uint8)
    lib = _lib()
    psz = positions.itemsize

    def run(rng):
        a, b = rng
        rc = lib.oracle_q_rope_pack_sglang(q_bits.ctypes.data + a * H * D * 2,
                                           positions.ctypes.data + a * psz, pos64,
                                           cos_sin.ctypes.data, cos_sin.shape[0], b - a, H, D,
                                           ROPE_DIM, rope_offset, 32, int(bool(is_neox)),
                                           fake_quant_floor, pack_floor,
                                           out.ctypes.data + a * H * SLOT68)
        if rc != 0:
            raise ValueError(f"oracle_q_rope_pack_sglang rejected its arguments (rc={rc})")

    _run_ranges(run, _split(T, threads))
    return out


def k_rope_pack_store_sglang(k_bits, positions, cos_sin, slot_mapping, index_k_cache, *,
                             k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                             compress_ratio=1, fake_quant_floor=DEFAULT_SCALE_FLOOR,
                             pack_floor=DEFAULT_SCALE_FLOOR):
    """sglang-compatible key side: writes 68-byte records into index_k_cache u8 [num_slots,68]."""
    k_bits = _c(k_bits, np.uint16)
    T, D = k_bits.shape
    positions = np.ascontiguousarray(positions)
    pos64 = 1 if positions.dtype == np.int64 else 0
    if not pos64:
        positions = _c(positions, np.int32)
    cos_sin = _c(cos_sin, np.float32)
    slot_mapping = _c(slot_mapping, np.int64)
    assert index_k_cache.dtype == np.uint8 and index_k_cache.flags.c_contiguous
    gamma = None if k_norm_gamma is None else _c(k_norm_gamma, np.uint16)
    rc = _lib().oracle_k_rope_pack_store_sglang(
        k_bits.ctypes.data, positions.ctypes.data, pos64, cos_sin.ctypes.data, cos_sin.shape[0],
        slot_mapping.ctypes.data, _ptr(gamma), k_norm_eps, T, D, ROPE_DIM, rope_offset, 32,
        int(bool(is_neox)), compress_ratio, fake_quant_floor, pack_floor,
        index_k_cache.ctypes.data, index_k_cache.shape[0])
    if rc != 0:
        raise ValueError(f"oracle_k_rope_pack_store_sglang rejected its arguments (rc={rc})")
    return index_k_cache


def quantize_rows_two_stage(x, floor1=DEFAULT_SCALE_FLOOR, floor2=DEFAULT_SCALE_FLOOR):
    x = _c(x, np.float32)
    n = x.shape[0]
    out = np.empty((n, SLOT68), np.uint8)
    _lib().oracle_quantize_rows_two_stage(x.ctypes.data, n, floor1, floor2, out.ctypes.data)
    return out


FP8_UE8M0, FP8_FP32 = 0, 1


def _positions(positions):
    positions = np.ascontiguousarray(positions)
    pos64 = 1 if positions.dtype == np.int64 else 0
    if not pos64:
        positions = _c(positions, np.int32)
    return positions, pos64


def q_rope_pack_fp8(q_bits, positions, cos_sin, weights, *, weights_scale=1.0, is_neox=True,
                    rope_offset=64, apply_hadamard=False, scale_fmt=FP8_UE8M0,
                    scale_floor=DEFAULT_SCALE_FLOOR, threads=1):
    """FP8 output mode, query side: (q_out u8 [T,H,128], weights_out bf16 bits u16 [T,H]).
    threads > 1 splits the tokens into ranges, each a separate call."""
    q_bits = _c(q_bits, np.uint16)
    T, H, D = q_bits.shape
    positions, pos64 = _positions(positions)
    cos_sin = _c(cos_sin, np.float32)
    weights = _c(weights, np.float32)
    q_out = np.full((T, H, D), 0xA5, np.uint8)
    w_out = np.full((T, H), 0xFFFF, np.uint16)
    lib = _lib()
    psz = positions.itemsize

    def run(rng):
        a, b = rng
        rc = lib.oracle_q_rope_pack_fp8(q_bits.ctypes.data + a * H * D * 2,
                                        positions.ctypes.data + a * psz, pos64,
                                        cos_sin.ctypes.data, cos_sin.shape[0],
                                        weights.ctypes.data + a * H * 4, weights_scale, b - a, H,
                                        D, ROPE_DIM, rope_offset, int(bool(is_neox)),
                                        int(bool(apply_hadamard)), scale_fmt, scale_floor,
                                        q_out.ctypes.data + a * H * D,
                                        w_out.ctypes.data + a * H * 2)
        if rc != 0:
            raise ValueError(f"oracle_q_rope_pack_fp8 rejected its arguments (rc={rc})")

    _run_ranges(run, _split(T, threads))
    return q_out, w_out


def k_rope_pack_store_fp8(k_bits, positions, cos_sin, slot_mapping, kv_cache, kv_cache_scale, *,
                          k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                          apply_hadamard=False, scale_fmt=FP8_UE8M0,
                          scale_floor=DEFAULT_SCALE_FLOOR):
    """FP8 output mode, key side: kv_cache u8 [NB,64,128], kv_cache_scale fp32 [NB,64]."""
    k_bits = _c(k_bits, np.uint16)
    T, D = k_bits.shape
    positions, pos64 = _positions(positions)
    cos_sin = _c(cos_sin, np.float32)
    slot_mapping = _c(slot_mapping, np.int64)
    assert kv_cache.dtype == np.uint8 and kv_cache.flags.c_contiguous
    assert kv_cache_scale.dtype == np.float32 and kv_cache_scale.flags.c_contiguous
    gamma = None if k_norm_gamma is None else _c(k_norm_gamma, np.uint16)
    rc = _lib().oracle_k_rope_pack_store_fp8(
        k_bits.ctypes.data, positions.ctypes.data, pos64, cos_sin.ctypes.data, cos_sin.shape[0],
        slot_mapping.ctypes.data, _ptr(gamma), k_norm_eps, T, D, ROPE_DIM, rope_offset,
        int(bool(is_neox)), int(bool(apply_hadamard)), scale_fmt, scale_floor,
        kv_cache.ctypes.data, kv_cache_scale.ctypes.data, kv_cache.shape[0], 64)
    if rc != 0:
        raise ValueError(f"oracle_k_rope_pack_store_fp8 rejected its arguments (rc={rc})")
    return kv_cache, kv_cache_scale


def e4m3_codes(y):
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    _lib().oracle_e4m3_codes(y.ctypes.data, y.size, out.ctypes.data)
    return out


def fp8_scales(amax, scale_floor=DEFAULT_SCALE_FLOOR, ue8m0=True):
    amax = _c(amax, np.float32)
    out = np.empty(amax.shape, np.float32)
    _lib().oracle_fp8_scales(amax.ctypes.data, amax.size, scale_floor, int(bool(ue8m0)),
                             out.ctypes.data)
    return out


def quantize_rows_fp8(x, scale_floor=DEFAULT_SCALE_FLOOR, ue8m0=True):
    x = _c(x, np.float32)
    n = x.shape[0]
    codes = np.empty((n, 128), np.uint8)
    scales = np.empty(n, np.float32)
    _lib().oracle_quantize_rows_fp8(x.ctypes.data, n, scale_floor, int(bool(ue8m0)),
                                    codes.ctypes.data, scales.ctypes.data)
    return codes, scales


FQ_UE8M0_32, FQ_E4M3_16 = 0, 1


def rope_fake_quant(x_bits, positions, cos_sin, *, rows_per_position=1, is_neox=True,
                    rope_offset=64, compress_ratio=1, mode=FQ_UE8M0_32,
                    scale_floor=DEFAULT_SCALE_FLOOR):
    """RoPE tail + FP4 fake quant: bf16 bits [..., 128] -> bf16 bits of the same shape."""
    x_bits = _c(x_bits, np.uint16)
    shape = x_bits.shape
    rows = x_bits.size // 128
    positions, pos64 = _positions(positions)
    cos_sin = _c(cos_sin, np.float32)
    y = np.full(shape, 0xFFFF, np.uint16)
    rc = _lib().oracle_rope_fake_quant(x_bits.ctypes.data, rows, rows_per_position,
                                       positions.ctypes.data, pos64, cos_sin.ctypes.data,
                                       cos_sin.shape[0], 128, ROPE_DIM, rope_offset,
                                       int(bool(is_neox)), compress_ratio, mode, scale_floor,
                                       y.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_rope_fake_quant rejected its arguments (rc={rc})")
    return y


def fake_quant_rows(x, mode=FQ_UE8M0_32, scale_floor=DEFAULT_SCALE_FLOOR):
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    _lib().oracle_fake_quant_rows(x.ctypes.data, x.shape[0], mode, scale_floor, y.ctypes.data)
    return y


# ---- step-level entry points (for the pins) ----

def bf16_round(x):
    x = _c(x, np.float32)
    out = np.empty_like(x)
    _lib().oracle_bf16_round(x.ctypes.data, out.ctypes.data, x.size)
    return out


def group_exponents(v, scale_floor=DEFAULT_SCALE_FLOOR):
    v = _c(v, np.float32)
    n, g = v.shape
    out = np.empty(n, np.int32)
    _lib().oracle_group_exponents(v.ctypes.data, n, g, scale_floor, out.ctypes.data)
    return out


def e2m1_nibbles(v, e):
    v = _c(v, np.float32)
    e = _c(np.broadcast_to(e, v.shape), np.int32)
    out = np.empty(v.shape, np.uint8)
    _lib().oracle_e2m1_nibbles(v.ctypes.data, e.ctypes.data, v.size, out.ctypes.data)
    return out


def quantize_rows(x, scale_floor=DEFAULT_SCALE_FLOOR):
    x = _c(x, np.float32)
    n = x.shape[0]
    b = np.empty((n, 64), np.uint8)
    e = np.empty((n, 4), np.uint8)
    _lib().oracle_quantize_rows(x.ctypes.data, n, scale_floor, b.ctypes.data, e.ctypes.data)
    return b, e


def rope_rows(x, cs, rope_offset=64, is_neox=True):
    x = _c(x, np.float32).copy()
    cs = _c(cs, np.float32)
    _lib().oracle_rope_rows(x.ctypes.data, cs.ctypes.data, x.shape[0], rope_offset, int(bool(is_neox)))
    return x


def fwht_rows(x):
    x = _c(x, np.float32).copy()
    _lib().oracle_fwht_rows(x.ctypes.data, x.shape[0])
    return x


def rmsnorm_rows(x, gamma_bits, eps):
    x = _c(x, np.float32).copy()
    g = _c(gamma_bits, np.uint16)
    _lib().oracle_rmsnorm_rows(x.ctypes.data, g.ctypes.data, eps, x.shape[0])
    return x


def hadamard_scale():
    return _lib().oracle_hadamard_scale()


def _run_ranges(fn, ranges):
    if len(ranges) <= 1:
        for r in ranges:
            fn(r)
        return
    with ThreadPoolExecutor(max_workers=len(ranges)) as ex:
        list(ex.map(fn, ranges))
