"""Thin ctypes binding of libfp4idx (C ABI in include/fp4idx.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfp4idx.so.  Tensors are torch tensors on the GPU; outputs the
caller does not pass are allocated with torch (device memory is torch's job
here).  Work is enqueued on torch's current stream unless `stream` is given.
The library must be built (``python -m pack_token_amd.build`` or
``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4idx.so")

OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
HEAD_DIM, ROPE_DIM, GROUP, KV_BLOCK = 128, 64, 32, 64
DEFAULT_SCALE_FLOOR = 2.0 ** -126

_lib = None
_lock = threading.Lock()

_p = ctypes.c_void_p
_i = ctypes.c_int
_i64 = ctypes.c_int64
_f = ctypes.c_float


class Fp4IdxError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[code {code}] {message}")
        self.code = code
        self.message = message


def lib():
    """Load libfp4idx.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m pack_token_amd.build` "
                    "(the FP4 indexer has no CPU or PyTorch fallback)")
            L = ctypes.CDLL(LIB_PATH)
            L.fp4idx_q_rope_pack.argtypes = [_p, _p, _i, _p, _i64, _p, _i64, _i, _i, _i, _i, _i, _i,
                                             _i, _f, _p, _p, _p, _p]
            L.fp4idx_q_rope_pack.restype = _i
            L.fp4idx_k_rope_pack_store.argtypes = [_p, _p, _i, _p, _i64, _p, _p, _f, _i64, _i, _i,
                                                   _i, _i, _i, _i, _f, _p, _p, _i64, _i, _p]
            L.fp4idx_k_rope_pack_store.restype = _i
            L.fp4idx_qk_rope_pack_store.argtypes = [_p, _p, _p, _i, _p, _i64, _p, _p, _p, _f,
                                                    _i64, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p,
                                                    _p, _p, _p, _i64, _i, _p]
            L.fp4idx_qk_rope_pack_store.restype = _i
            L.fp4idx_q_rope_pack_sglang.argtypes = [_p, _p, _i, _p, _i64, _i64, _i, _i, _i, _i,
                                                    _i, _i, _f, _f, _p, _p]
            L.fp4idx_q_rope_pack_sglang.restype = _i
            L.fp4idx_k_rope_pack_store_sglang.argtypes = [_p, _p, _i, _p, _i64, _p, _p, _f, _i64,
                                                          _i, _i, _i, _i, _i, _i, _f, _f, _p,
                                                          _i64, _p]
            L.fp4idx_rope_fake_quant.argtypes = [_p, _i64, _i64, _p, _i, _p, _i64, _i, _i, _i, _i,
                                                 _i, _i, _f, _p, _p]
            L.fp4idx_rope_fake_quant.restype = _i
            L.fp4idx_k_rope_pack_store_sglang.restype = _i
            L.fp4idx_q_rope_pack_fp8.argtypes = [_p, _p, _i, _p, _i64, _p, _f, _i64, _i, _i, _i, _i,
                                                 _i, _i, _i, _f, _p, _p, _p]
            L.fp4idx_q_rope_pack_fp8.restype = _i
            L.fp4idx_k_rope_pack_store_fp8.argtypes = [_p, _p, _i, _p, _i64, _p, _p, _f, _i64, _i,
                                                       _i, _i, _i, _i, _i, _f, _p, _p, _i64, _i,
                                                       _p]
            L.fp4idx_k_rope_pack_store_fp8.restype = _i
            L.fp4idx_paged_mqa_logits.argtypes = [_p, _p, _p, _f, _p, _p, _i64, _p, _i64, _p,
                                                  _i64, _i, _i, _i, _p, _i64, _p]
            L.fp4idx_paged_mqa_logits.restype = _i
            L.fp4idx_dequant_debug.argtypes = [_i, _p, _p, _i64, _i, _p, _i64, _i, _p, _p]
            L.fp4idx_dequant_debug.restype = _i
            L.fp4idx_ceiling_stream.argtypes = [_p, _i64, _p, _i64, _p]
            L.fp4idx_ceiling_stream.restype = _i
            L.fp4idx_ceiling_paged_gather.argtypes = [_p, _p, _i64, _p, _i64, _p, _i64, _i, _p,
                                                      _i64, _p]
            L.fp4idx_ceiling_paged_gather.restype = _i
            L.fp4idx_ceiling_valu.argtypes = [_i, _i64, _i64, _p, _p]
            L.fp4idx_ceiling_valu.restype = _i
            L.fp4idx_last_error.argtypes = []
            L.fp4idx_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def last_error() -> str:
    return lib().fp4idx_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise Fp4IdxError(rc, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def _require(t, name, dtypes, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t, name, shape):
    """Exact shape check (None entries match any size).  Runs before the device
    checks: the library sees only pointers, so a tensor of the wrong size would
    be read or written out of bounds on the GPU."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    got = tuple(t.shape)
    if len(got) != len(shape) or any(e is not None and g != e for g, e in zip(got, shape)):
        want = tuple("*" if e is None else e for e in shape)
        raise ValueError(f"{name} has shape {got}; expected {want}")


def _numel(t, name, n):
    """Element-count check for buffers whose layout the library defines."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.numel() != n:
        raise ValueError(f"{name} has {t.numel()} elements (shape {tuple(t.shape)}); expected {n}")


def _check_rows(T, positions, slot_mapping=None):
    _shape(positions, "positions", (T,))
    _shape(slot_mapping, "slot_mapping", (T,))


def _check_cos_sin(cos_sin):
    _shape(cos_sin, "cos_sin", (None, ROPE_DIM))


def _check_fp4_cache(kv_cache, kv_cache_scale):
    """kv_cache u8 [NB,1,4,64,16], kv_cache_scale u8 [NB,1,4,64] (any shapes with
    those element counts)."""
    if not isinstance(kv_cache, torch.Tensor):
        raise TypeError("kv_cache must be a torch.Tensor")
    NB = kv_cache.shape[0] if kv_cache.dim() else 0
    _numel(kv_cache, "kv_cache", NB * 4 * KV_BLOCK * 16)
    _numel(kv_cache_scale, "kv_cache_scale", NB * 4 * KV_BLOCK)
    return NB


def q_scale_cols(H: int) -> int:
    return ((H // 16) + 3) // 4 * 4


def q_rope_pack(q, positions, cos_sin, weights=None, *, q_out=None, q_scale_out=None,
                weights_out=None, is_neox=True, rope_offset=64, apply_hadamard=False,
                scale_floor=DEFAULT_SCALE_FLOOR, stream=None):
    """fp4idx_q_rope_pack.  q bf16 [T,H,128]; positions int32/int64 [T]; cos_sin fp32
    [max_pos,64]; weights fp32 [T,H] or None.  Returns (q_out, q_scale_out, weights_out)."""
    T, H, D = q.shape
    dev = q.device
    J = q_scale_cols(H)
    _check_rows(T, positions)
    _check_cos_sin(cos_sin)
    _shape(weights, "weights", (T, H))
    _numel(q_out, "q_out", T * H * (D // 2))
    _numel(q_scale_out, "q_scale_out", T * 4 * 16 * J)
    _numel(weights_out, "weights_out", T * H)
    _require(q, "q", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    _require(weights, "weights", (torch.float32,), dev)
    if q_out is None:
        q_out = torch.empty((T, H, D // 2), dtype=torch.uint8, device=dev)
    if q_scale_out is None:
        q_scale_out = torch.empty((T, D // 128 if D >= 128 else 1, 4, 16, J), dtype=torch.uint8,
                                  device=dev)
    if weights is not None and weights_out is None:
        weights_out = torch.empty_like(weights)
    _require(q_out, "q_out", (torch.uint8,), dev)
    _require(q_scale_out, "q_scale_out", (torch.uint8,), dev)
    _require(weights_out, "weights_out", (torch.float32,), dev)
    rc = lib().fp4idx_q_rope_pack(
        _ptr(q), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(weights), T, H, D, ROPE_DIM, rope_offset, GROUP, int(is_neox),
        int(apply_hadamard), scale_floor, _ptr(q_out), _ptr(q_scale_out), _ptr(weights_out),
        _stream_handle(stream))
    _check(rc)
    return q_out, q_scale_out, weights_out


def k_rope_pack_store(k, positions, cos_sin, slot_mapping, kv_cache, kv_cache_scale, *,
                      k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                      apply_hadamard=False, scale_floor=DEFAULT_SCALE_FLOOR, stream=None):
    """fp4idx_k_rope_pack_store.  k bf16 [T,128]; slot_mapping int64 [T]; kv_cache u8
    [NB,1,4,64,16] and kv_cache_scale u8 [NB,1,4,64] are updated in place."""
    T, D = k.shape
    dev = k.device
    _check_rows(T, positions, slot_mapping)
    _check_cos_sin(cos_sin)
    NB = _check_fp4_cache(kv_cache, kv_cache_scale)
    _numel(k_norm_gamma, "k_norm_gamma", D)
    _require(k, "k", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    _require(slot_mapping, "slot_mapping", (torch.int64,), dev)
    _require(kv_cache, "kv_cache", (torch.uint8,), dev)
    _require(kv_cache_scale, "kv_cache_scale", (torch.uint8,), dev)
    _require(k_norm_gamma, "k_norm_gamma", (torch.bfloat16, torch.int16, torch.uint16), dev)
    rc = lib().fp4idx_k_rope_pack_store(
        _ptr(k), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(slot_mapping), _ptr(k_norm_gamma), k_norm_eps, T, D, ROPE_DIM,
        rope_offset, GROUP, int(is_neox), int(apply_hadamard), scale_floor, _ptr(kv_cache),
        _ptr(kv_cache_scale), NB, KV_BLOCK, _stream_handle(stream))
    _check(rc)
    return kv_cache, kv_cache_scale


SCALE_UE8M0, SCALE_FP32 = 0, 1


def _scale_fmt(fmt):
    return {"ue8m0": SCALE_UE8M0, "fp32": SCALE_FP32}.get(fmt, fmt)


def q_rope_pack_fp8(q, positions, cos_sin, weights, *, weights_scale=1.0, q_out=None,
                    weights_out=None, is_neox=True, rope_offset=64, apply_hadamard=False,
                    scale_fmt="ue8m0", scale_floor=DEFAULT_SCALE_FLOOR, stream=None):
    """fp4idx_q_rope_pack_fp8.  Returns (q_out u8 [T,H,128] holding e4m3fn codes,
    weights_out bf16 [T,H] = (weights * q_scale) * weights_scale)."""
    T, H, D = q.shape
    dev = q.device
    _check_rows(T, positions)
    _check_cos_sin(cos_sin)
    _shape(weights, "weights", (T, H))
    _numel(q_out, "q_out", T * H * D)
    _numel(weights_out, "weights_out", T * H)
    _require(q, "q", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    _require(weights, "weights", (torch.float32,), dev)
    if q_out is None:
        q_out = torch.empty((T, H, D), dtype=torch.uint8, device=dev)
    if weights_out is None:
        weights_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _require(q_out, "q_out", (torch.uint8,), dev)
    _require(weights_out, "weights_out", (torch.bfloat16, torch.int16, torch.uint16), dev)
    rc = lib().fp4idx_q_rope_pack_fp8(
        _ptr(q), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(weights), weights_scale, T, H, D, ROPE_DIM, rope_offset,
        int(is_neox), int(apply_hadamard), _scale_fmt(scale_fmt), scale_floor, _ptr(q_out),
        _ptr(weights_out), _stream_handle(stream))
    _check(rc)
    return q_out, weights_out


def k_rope_pack_store_fp8(k, positions, cos_sin, slot_mapping, kv_cache, kv_cache_scale, *,
                          k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                          apply_hadamard=False, scale_fmt="ue8m0", scale_floor=DEFAULT_SCALE_FLOOR,
                          stream=None):
    """fp4idx_k_rope_pack_store_fp8.  kv_cache u8 [NB,64,128] (e4m3fn codes) and
    kv_cache_scale fp32 [NB,64] are updated in place."""
    T, D = k.shape
    dev = k.device
    _check_rows(T, positions, slot_mapping)
    _check_cos_sin(cos_sin)
    if not isinstance(kv_cache, torch.Tensor):
        raise TypeError("kv_cache must be a torch.Tensor")
    NB = kv_cache.shape[0] if kv_cache.dim() else 0
    _numel(kv_cache, "kv_cache", NB * KV_BLOCK * D)
    _numel(kv_cache_scale, "kv_cache_scale", NB * KV_BLOCK)
    _numel(k_norm_gamma, "k_norm_gamma", D)
    _require(k, "k", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    _require(slot_mapping, "slot_mapping", (torch.int64,), dev)
    _require(kv_cache, "kv_cache", (torch.uint8,), dev)
    _require(kv_cache_scale, "kv_cache_scale", (torch.float32,), dev)
    _require(k_norm_gamma, "k_norm_gamma", (torch.bfloat16, torch.int16, torch.uint16), dev)
    rc = lib().fp4idx_k_rope_pack_store_fp8(
        _ptr(k), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(slot_mapping), _ptr(k_norm_gamma), k_norm_eps, T, D, ROPE_DIM,
        rope_offset, int(is_neox), int(apply_hadamard), _scale_fmt(scale_fmt), scale_floor,
        _ptr(kv_cache), _ptr(kv_cache_scale), kv_cache.shape[0], KV_BLOCK,
        _stream_handle(stream))
    _check(rc)
    return kv_cache, kv_cache_scale


SGLANG_RECORD = 68
FQ_UE8M0_32, FQ_E4M3_16 = 0, 1


def rope_fake_quant(x, positions, cos_sin, *, y=None, rows_per_position=1, is_neox=True,
                    rope_offset=64, compress_ratio=1, mode="ue8m0_32",
                    scale_floor=DEFAULT_SCALE_FLOOR, stream=None):
    """fp4idx_rope_fake_quant.  x bf16 [..., 128]; returns y bf16 of the same shape
    (the fake-quantized values).  mode: "ue8m0_32" or "e4m3_16"."""
    dev = x.device
    if x.dim() == 0 or x.shape[-1] != HEAD_DIM:
        raise ValueError("x must end in a 128-dim axis")
    rows = x.numel() // HEAD_DIM
    if rows and positions.numel() * rows_per_position < rows:
        raise ValueError("positions has fewer than ceil(rows / rows_per_position) entries")
    _check_cos_sin(cos_sin)
    _numel(y, "y", x.numel())
    _require(x, "x", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    if y is None:
        y = torch.empty(x.shape, dtype=torch.bfloat16, device=dev)
    _require(y, "y", (torch.bfloat16, torch.int16, torch.uint16), dev)
    m = {"ue8m0_32": FQ_UE8M0_32, "e4m3_16": FQ_E4M3_16}.get(mode, mode)
    rc = lib().fp4idx_rope_fake_quant(
        _ptr(x), rows, rows_per_position, _ptr(positions), int(positions.dtype == torch.int64),
        _ptr(cos_sin), cos_sin.shape[0], HEAD_DIM, ROPE_DIM, rope_offset, int(is_neox),
        compress_ratio, m, scale_floor, _ptr(y), _stream_handle(stream))
    _check(rc)
    return y


def q_rope_pack_sglang(q, positions, cos_sin, *, q_packed=None, is_neox=True, rope_offset=64,
                       fake_quant_floor=DEFAULT_SCALE_FLOOR, pack_floor=DEFAULT_SCALE_FLOOR,
                       stream=None):
    """fp4idx_q_rope_pack_sglang.  q bf16 [T,H,128]; returns q_packed u8 [T,H,68]."""
    T, H, D = q.shape
    dev = q.device
    _check_rows(T, positions)
    _check_cos_sin(cos_sin)
    _require(q, "q", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    if q_packed is None:
        q_packed = torch.empty((T, H, SGLANG_RECORD), dtype=torch.uint8, device=dev)
    _require(q_packed, "q_packed", (torch.uint8,), dev)
    if q_packed.numel() != T * H * SGLANG_RECORD:
        raise ValueError(f"q_packed must hold [T, H, 68] = {T * H * SGLANG_RECORD} bytes")
    rc = lib().fp4idx_q_rope_pack_sglang(
        _ptr(q), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], T, H, D, ROPE_DIM, rope_offset, GROUP, int(is_neox), fake_quant_floor,
        pack_floor, _ptr(q_packed), _stream_handle(stream))
    _check(rc)
    return q_packed


def k_rope_pack_store_sglang(k, positions, cos_sin, slot_mapping, index_k_cache, *,
                             k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                             compress_ratio=1, fake_quant_floor=DEFAULT_SCALE_FLOOR,
                             pack_floor=DEFAULT_SCALE_FLOOR, stream=None):
    """fp4idx_k_rope_pack_store_sglang.  k bf16 [T,128]; index_k_cache u8 [num_slots,68] is
    updated in place (slot 0 publishes nothing)."""
    T, D = k.shape
    dev = k.device
    _check_rows(T, positions, slot_mapping)
    _check_cos_sin(cos_sin)
    _numel(k_norm_gamma, "k_norm_gamma", D)
    _require(k, "k", (torch.bfloat16, torch.int16, torch.uint16))
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    _require(slot_mapping, "slot_mapping", (torch.int64,), dev)
    _require(index_k_cache, "index_k_cache", (torch.uint8,), dev)
    _require(k_norm_gamma, "k_norm_gamma", (torch.bfloat16, torch.int16, torch.uint16), dev)
    if index_k_cache.dim() != 2 or index_k_cache.shape[1] != SGLANG_RECORD:
        raise ValueError("index_k_cache must be [num_slots, 68]")
    rc = lib().fp4idx_k_rope_pack_store_sglang(
        _ptr(k), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(slot_mapping), _ptr(k_norm_gamma), k_norm_eps, T, D, ROPE_DIM,
        rope_offset, GROUP, int(is_neox), compress_ratio, fake_quant_floor, pack_floor,
        _ptr(index_k_cache), index_k_cache.shape[0], _stream_handle(stream))
    _check(rc)
    return index_k_cache


def qk_rope_pack_store(q, k, positions, cos_sin, slot_mapping, kv_cache, kv_cache_scale,
                       weights=None, *, q_out=None, q_scale_out=None, weights_out=None,
                       k_norm_gamma=None, k_norm_eps=1e-6, is_neox=True, rope_offset=64,
                       apply_hadamard=False, scale_floor=DEFAULT_SCALE_FLOOR, stream=None):
    """fp4idx_qk_rope_pack_store: the query and key sides in one launch.
    Returns (q_out, q_scale_out, weights_out); the cache tensors are updated in place."""
    T, H, D = q.shape
    dev = q.device
    J = q_scale_cols(H)
    _shape(k, "k", (T, D))
    _check_rows(T, positions, slot_mapping)
    _check_cos_sin(cos_sin)
    _shape(weights, "weights", (T, H))
    _check_fp4_cache(kv_cache, kv_cache_scale)
    _numel(k_norm_gamma, "k_norm_gamma", D)
    _numel(q_out, "q_out", T * H * (D // 2))
    _numel(q_scale_out, "q_scale_out", T * 4 * 16 * J)
    _numel(weights_out, "weights_out", T * H)
    _require(q, "q", (torch.bfloat16, torch.int16, torch.uint16))
    _require(k, "k", (torch.bfloat16, torch.int16, torch.uint16), dev)
    _require(positions, "positions", (torch.int32, torch.int64), dev)
    _require(cos_sin, "cos_sin", (torch.float32,), dev)
    _require(weights, "weights", (torch.float32,), dev)
    _require(slot_mapping, "slot_mapping", (torch.int64,), dev)
    _require(kv_cache, "kv_cache", (torch.uint8,), dev)
    _require(kv_cache_scale, "kv_cache_scale", (torch.uint8,), dev)
    _require(k_norm_gamma, "k_norm_gamma", (torch.bfloat16, torch.int16, torch.uint16), dev)
    J = q_scale_cols(H)
    if q_out is None:
        q_out = torch.empty((T, H, D // 2), dtype=torch.uint8, device=dev)
    if q_scale_out is None:
        q_scale_out = torch.empty((T, 1, 4, 16, J), dtype=torch.uint8, device=dev)
    if weights is not None and weights_out is None:
        weights_out = torch.empty_like(weights)
    _require(q_out, "q_out", (torch.uint8,), dev)
    _require(q_scale_out, "q_scale_out", (torch.uint8,), dev)
    _require(weights_out, "weights_out", (torch.float32,), dev)
    rc = lib().fp4idx_qk_rope_pack_store(
        _ptr(q), _ptr(k), _ptr(positions), int(positions.dtype == torch.int64), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(weights), _ptr(slot_mapping), _ptr(k_norm_gamma), k_norm_eps, T,
        H, D, ROPE_DIM, rope_offset, GROUP, int(is_neox), int(apply_hadamard), scale_floor,
        _ptr(q_out), _ptr(q_scale_out), _ptr(weights_out), _ptr(kv_cache), _ptr(kv_cache_scale),
        kv_cache.shape[0], KV_BLOCK, _stream_handle(stream))
    _check(rc)
    return q_out, q_scale_out, weights_out


def paged_mqa_logits(q_out, q_scale_out, weights, kv_cache, kv_cache_scale, block_table,
                     context_lens, next_n, *, weights_scale=1.0, apply_relu=True, logits=None,
                     stride=None, stream=None):
    """fp4idx_paged_mqa_logits.  Returns logits fp32 [B*next_n, stride]; entries at or past
    a sequence's context length keep their previous contents (uninitialised if allocated
    here)."""
    T, H, _ = q_out.shape
    dev = q_out.device
    B, max_blocks = block_table.shape
    if T != B * next_n:
        raise ValueError(f"q_out has {T} tokens, expected B*next_n = {B * next_n}")
    _shape(q_out, "q_out", (T, H, HEAD_DIM // 2))
    _numel(q_scale_out, "q_scale_out", T * 4 * 16 * q_scale_cols(H))
    _shape(weights, "weights", (T, H))
    _check_fp4_cache(kv_cache, kv_cache_scale)
    _shape(context_lens, "context_lens", (B,))
    if logits is not None:
        _shape(logits, "logits", (T, None))
        if stride is not None and stride != logits.shape[1]:
            raise ValueError(f"stride {stride} differs from logits.shape[1] = {logits.shape[1]}")
    _require(q_out, "q_out", (torch.uint8,))
    _require(q_scale_out, "q_scale_out", (torch.uint8,), dev)
    _require(weights, "weights", (torch.float32,), dev)
    _require(kv_cache, "kv_cache", (torch.uint8,), dev)
    _require(kv_cache_scale, "kv_cache_scale", (torch.uint8,), dev)
    _require(block_table, "block_table", (torch.int32,), dev)
    _require(context_lens, "context_lens", (torch.int32,), dev)
    if stride is None:
        stride = logits.shape[1] if logits is not None else max(1, max_blocks * KV_BLOCK)
    if logits is None:
        logits = torch.empty((T, stride), dtype=torch.float32, device=dev)
    _require(logits, "logits", (torch.float32,), dev)
    _check(lib().fp4idx_paged_mqa_logits(
        _ptr(q_out), _ptr(q_scale_out), _ptr(weights), weights_scale, _ptr(kv_cache),
        _ptr(kv_cache_scale), kv_cache.shape[0], _ptr(block_table), max_blocks,
        _ptr(context_lens), B, next_n, H, int(bool(apply_relu)), _ptr(logits), stride,
        _stream_handle(stream)))
    return logits


def dequant_q(q_out, q_scale_out, *, out=None, stream=None):
    """fp4idx_dequant_debug(which=0): fp32 [T,H,128]."""
    T, H, _ = q_out.shape
    _shape(q_out, "q_out", (T, H, HEAD_DIM // 2))
    _numel(q_scale_out, "q_scale_out", T * 4 * 16 * q_scale_cols(H))
    _numel(out, "out", T * H * HEAD_DIM)
    if out is None:
        out = torch.empty((T, H, HEAD_DIM), dtype=torch.float32, device=q_out.device)
    _require(q_out, "q_out", (torch.uint8,))
    _require(q_scale_out, "q_scale_out", (torch.uint8,), q_out.device)
    _require(out, "out", (torch.float32,), q_out.device)
    _check(lib().fp4idx_dequant_debug(0, _ptr(q_out), _ptr(q_scale_out), T, H, None, 0, KV_BLOCK,
                                      _ptr(out), _stream_handle(stream)))
    return out


def dequant_kcache(kv_cache, kv_cache_scale, slots=None, *, out=None, stream=None):
    """fp4idx_dequant_debug(which=1): fp32 [rows,128] for the given slots (or all slots)."""
    NB = _check_fp4_cache(kv_cache, kv_cache_scale)
    if slots is not None:
        _shape(slots, "slots", (None,))
    rows = NB * KV_BLOCK if slots is None else slots.shape[0]
    _numel(out, "out", rows * HEAD_DIM)
    if out is None:
        out = torch.empty((rows, HEAD_DIM), dtype=torch.float32, device=kv_cache.device)
    _require(kv_cache, "kv_cache", (torch.uint8,))
    _require(kv_cache_scale, "kv_cache_scale", (torch.uint8,), kv_cache.device)
    _require(slots, "slots", (torch.int64,), kv_cache.device)
    _require(out, "out", (torch.float32,), kv_cache.device)
    _check(lib().fp4idx_dequant_debug(1, _ptr(kv_cache), _ptr(kv_cache_scale), rows, 0,
                                      _ptr(slots), NB, KV_BLOCK, _ptr(out), _stream_handle(stream)))
    return out


# ---- measurement entry points (include/fp4idx_ceiling.h) ---------------------

def ceiling_stream(src, read_bytes: int, dst, write_bytes: int, *, stream=None):
    """Plain stream: read read_bytes of src, write write_bytes of dst (writes
    spread over the reads).  A measurement of the HBM rate of that traffic."""
    for t, name, n in ((src, "src", read_bytes), (dst, "dst", max(write_bytes, 1024))):
        _require(t, name, (torch.uint8,))
        if t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} bytes, needs {n}")
    rc = lib().fp4idx_ceiling_stream(_ptr(src), read_bytes, _ptr(dst), write_bytes,
                                     _stream_handle(stream))
    if rc != OK:
        raise Fp4IdxError(rc, "fp4idx_ceiling_stream failed")


def ceiling_paged_gather(kv_cache, kv_cache_scale, block_table, context_lens, next_n, logits, *,
                         stream=None):
    """The decode scorer's reads and writes without its arithmetic."""
    _check_fp4_cache(kv_cache, kv_cache_scale)
    _require(block_table, "block_table", (torch.int32,))
    _require(context_lens, "context_lens", (torch.int32,))
    _require(logits, "logits", (torch.float32,))
    B, max_blocks = block_table.shape
    _numel(context_lens, "context_lens", B)
    if logits.dim() != 2 or logits.shape[0] != B * next_n:
        raise ValueError("logits must be [B * next_n, stride]")
    rc = lib().fp4idx_ceiling_paged_gather(_ptr(kv_cache), _ptr(kv_cache_scale), kv_cache.shape[0],
                                           _ptr(block_table), max_blocks, _ptr(context_lens), B,
                                           next_n, _ptr(logits), logits.shape[1],
                                           _stream_handle(stream))
    if rc != OK:
        raise Fp4IdxError(rc, "fp4idx_ceiling_paged_gather failed")


VALU_KINDS = {"fp32_add": 0, "fp32_fma": 1, "fp32_max": 2, "bf16_pack": 3, "fp4_convert": 4}


def ceiling_valu(kind: str, workgroups: int, iterations: int, out, *, stream=None):
    """VALU issue rate of one instruction kind: workgroups x 256 threads, 8
    independent chains of `iterations` steps per lane (workgroups * 256 *
    iterations * 8 lane operations); out (int32, workgroups * 256 elements)
    receives one value per thread."""
    if kind not in VALU_KINDS:
        raise ValueError(f"kind must be one of {sorted(VALU_KINDS)}")
    if out is None:
        raise ValueError("out is required")
    _require(out, "out", (torch.int32,))
    if out.numel() < workgroups * 256:
        raise ValueError(f"out holds {out.numel()} elements, needs {workgroups * 256}")
    rc = lib().fp4idx_ceiling_valu(VALU_KINDS[kind], workgroups, iterations, _ptr(out),
                                   _stream_handle(stream))
    if rc != OK:
        raise Fp4IdxError(rc, "fp4idx_ceiling_valu failed")
