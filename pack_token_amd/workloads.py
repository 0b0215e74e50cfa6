"""Seeded synthetic inputs for the fused FP4 indexer producer.

This module only makes inputs: random bf16 queries and keys, positions, the
fp32 cos/sin table, slot mappings, head weights and the key-norm gamma.  It
holds none of the method's arithmetic, and both the HIP path and the CPU
oracle consume what it returns.  bf16 values are produced by torch's CPU
float32 -> bfloat16 cast and handled as their uint16 bit patterns.

Random draws use numpy's PCG64 with a fixed order per workload, so a
workload is a pure function of (recipe, seed, sizes).

Recipes (shapes and value structure follow the verification matrices on the
pages: tokens x heads x is_neox sweeps in ROCm/aiter PR 5484 "Verification",
and rows {1,5,64,300}, scales {1,40,1e-3} plus zero, subnormal and half-way
rows, int32/int64 positions in sgl-project/sglang PR 39656 "Verification"):

  tiny        T=8, H=32, neox, q,k ~ N(0,1), positions 0..7, 1 block, slot = t
  edge_mix    T=300, H=64, interleaved; rows x {1,40,1e-3}; ~5% all-zero,
              ~5% subnormal-only, exact-midpoint groups (in groups 0-1);
              positions U[0,32768); slots = a permutation of 512 over 8
              blocks with 15 tokens (5%) at -1
  decode      64 seqs x 4 = 256 tokens, H=32, neox, positions base..base+3
              with base U[0,131068]; 4096 blocks, filled first by 262,144
              background keys at contiguous slots, then the 256 keys go to
              distinct random slots
  prefill_norm_rotate  T=16384, H=64, neox, key RMSNorm (eps 1e-6,
              gamma ~ N(1,0.1)), RoPE, Hadamard on q and k; contiguous slots
  large_prefill  T=131072, H=64, neox, q,k ~ 2 N(0,1) with 1% of token rows
              x100; positions 0..T-1; contiguous slots into T/64 blocks
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

HEAD_DIM = 128
ROPE_DIM = 64
KV_BLOCK = 64
ROPE_BASE = 10000.0
SENTINEL = 0xA5


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns via torch's CPU cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> float32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cos_sin_table(max_pos: int, base: float = ROPE_BASE) -> np.ndarray:
    """fp32 [max_pos, 64]: cols 0..31 = cos(p * f_i), cols 32..63 = sin(p * f_i),
    f_i = base^(-2i/64), evaluated in float64 and rounded once to fp32."""
    i = np.arange(ROPE_DIM // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * i / ROPE_DIM)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    out = np.empty((max_pos, ROPE_DIM), np.float32)
    out[:, : ROPE_DIM // 2] = np.cos(ang)
    out[:, ROPE_DIM // 2:] = np.sin(ang)
    return out


def q_scale_cols(H: int) -> int:
    return ((H // 16) + 3) // 4 * 4


@dataclass
class Workload:
    name: str
    T: int
    H: int
    q: np.ndarray               # uint16 [T,H,128]
    k: np.ndarray               # uint16 [T,128]
    positions: np.ndarray       # int64 or int32 [T]
    cos_sin: np.ndarray         # fp32 [max_pos,64]
    weights: np.ndarray         # fp32 [T,H]
    slot_mapping: np.ndarray    # int64 [T]
    NB: int
    is_neox: bool = True
    rope_offset: int = 64
    apply_hadamard: bool = False
    k_norm_gamma: Optional[np.ndarray] = None   # uint16 [128]
    k_norm_eps: float = 1e-6
    scale_floor: float = float(np.float32(2.0 ** -126))
    # keys written before the timed/tested call (decode recipe)
    background: Optional[dict] = field(default=None)

    @property
    def max_pos(self) -> int:
        return int(self.cos_sin.shape[0])

    @property
    def J(self) -> int:
        return q_scale_cols(self.H)

    def empty_cache(self):
        kv = np.full((self.NB, 1, 4, KV_BLOCK, 16), SENTINEL, np.uint8)
        ks = np.full((self.NB, 1, 4, KV_BLOCK), SENTINEL, np.uint8)
        return kv, ks


def _normal_bf16(rng, shape, std=1.0, chunk_rows=None):
    """bf16 bits of std * N(0,1), generated in row chunks to bound peak memory."""
    shape = tuple(shape)
    out = np.empty(shape, np.uint16)
    n0 = shape[0]
    step = chunk_rows or n0 or 1
    for a in range(0, n0, step):
        b = min(n0, a + step)
        x = rng.standard_normal((b - a,) + shape[1:], dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[a:b] = to_bf16_bits(x)
    return out


def tiny(seed: int = 0, T: int = 8, H: int = 32) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal_bf16(rng, (T, H, HEAD_DIM))
    k = _normal_bf16(rng, (T, HEAD_DIM))
    weights = rng.random((T, H), dtype=np.float32)
    positions = np.arange(T, dtype=np.int64)
    NB = max(1, -(-T // KV_BLOCK))
    return Workload("tiny", T, H, q, k, positions, cos_sin_table(max(T, 1)), weights,
                    np.arange(T, dtype=np.int64), NB, is_neox=True)


def sweep_case(seed: int, T: int, H: int, is_neox: bool, rope_offset: int,
               positions_int32: bool = False) -> Workload:
    """One point of the tokens x heads x is_neox x rope-slice sweep."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal_bf16(rng, (T, H, HEAD_DIM))
    k = _normal_bf16(rng, (T, HEAD_DIM))
    weights = rng.random((T, H), dtype=np.float32)
    max_pos = 4096
    positions = rng.integers(0, max_pos, T, dtype=np.int64)
    if positions_int32:
        positions = positions.astype(np.int32)
    NB = max(1, -(-2 * T // KV_BLOCK))
    slots = rng.permutation(NB * KV_BLOCK)[:T].astype(np.int64)
    return Workload(f"sweep_T{T}_H{H}_{'neox' if is_neox else 'inter'}_o{rope_offset}", T, H, q, k,
                    positions, cos_sin_table(max_pos), weights, slots, NB, is_neox=is_neox,
                    rope_offset=rope_offset)


def _plant_overflow_pairs(rng, rows_bits: np.ndarray, rope_offset: int, is_neox: bool):
    """rows_bits: uint16 [n,128] modified in place.  About half of the rows get
    one RoPE pair of the slice at rope_offset whose two elements have the
    largest finite bf16 magnitude (0x7F7F) with random signs, so that the
    rotated value of the pair can exceed the fp32 range.  One pair per row:
    the rotation sends at most one of its two outputs past the range."""
    n = rows_bits.shape[0]
    rows = np.nonzero(rng.random(n) < 0.5)[0]
    pair = rng.integers(0, ROPE_DIM // 2, rows.size)
    if is_neox:
        ia, ib = pair, pair + ROPE_DIM // 2
    else:
        ia, ib = 2 * pair, 2 * pair + 1
    signs = rng.integers(0, 2, (rows.size, 2)).astype(np.uint16) << 15
    rows_bits[rows, rope_offset + ia] = 0x7F7F | signs[:, 0]
    rows_bits[rows, rope_offset + ib] = 0x7F7F | signs[:, 1]


def overflow_case(seed: int, T: int, H: int, is_neox: bool, rope_offset: int,
                  apply_hadamard: bool) -> Workload:
    """A sweep point whose rows carry pairs of largest-magnitude bf16 values in
    the rotated slice (see _plant_overflow_pairs), positions U[0,4096)."""
    wl = sweep_case(seed, T, H, is_neox, rope_offset)
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    _plant_overflow_pairs(rng, wl.q.reshape(T * H, HEAD_DIM), rope_offset, is_neox)
    _plant_overflow_pairs(rng, wl.k, rope_offset, is_neox)
    wl.name = f"overflow_T{T}_H{H}_{'neox' if is_neox else 'inter'}_o{rope_offset}" + (
        "_had" if apply_hadamard else "")
    wl.apply_hadamard = apply_hadamard
    return wl


_MID_MULTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0],
                      np.float32)


def _plant_special_groups(rng, rows_bits: np.ndarray, frac: float = 0.05):
    """rows_bits: uint16 [n,128] modified in place.  Each (row, group) unit is
    independently made all-zero (mixed +-0), subnormal-only (bf16 patterns
    0x0001..0x007F with random signs) or, in groups 0-1 only, an exact-midpoint
    group (one element +-6*2^k, the rest +-{grid points and midpoints}*2^k,
    k in [-20,20])."""
    n = rows_bits.shape[0]
    u = rng.random((n, 4))
    g3 = rows_bits.reshape(n, 4, 32)
    zero = u < frac
    sub = (u >= frac) & (u < 2 * frac)
    mid = (u >= 2 * frac) & (u < 3 * frac)
    mid[:, 2:] = False
    # all-zero
    zi = np.nonzero(zero)
    zsign = rng.integers(0, 2, (len(zi[0]), 32)).astype(np.uint16) << 15
    g3[zi] = zsign
    # subnormal-only
    si = np.nonzero(sub)
    mag = rng.integers(1, 0x80, (len(si[0]), 32)).astype(np.uint16)
    ssign = rng.integers(0, 2, (len(si[0]), 32)).astype(np.uint16) << 15
    g3[si] = mag | ssign
    # exact midpoints
    mi = np.nonzero(mid)
    m = len(mi[0])
    kexp = rng.integers(-20, 21, m)
    idx = rng.integers(0, len(_MID_MULTS), (m, 32))
    vals = _MID_MULTS[idx]
    where6 = rng.integers(0, 32, m)
    vals[np.arange(m), where6] = 6.0
    signs = np.where(rng.integers(0, 2, (m, 32)) == 1, -1.0, 1.0).astype(np.float32)
    vals = vals * signs * np.ldexp(np.float32(1.0), kexp)[:, None].astype(np.float32)
    g3[mi] = to_bf16_bits(vals.astype(np.float32))


def edge_mix(seed: int = 1, T: int = 300, H: int = 64, positions_int32: bool = False) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    scales = np.array([1.0, 40.0, 1e-3], np.float32)[np.arange(T) % 3]
    qf = rng.standard_normal((T, H, HEAD_DIM), dtype=np.float32) * scales[:, None, None]
    kf = rng.standard_normal((T, HEAD_DIM), dtype=np.float32) * scales[:, None]
    q = to_bf16_bits(qf)
    k = to_bf16_bits(kf)
    _plant_special_groups(rng, q.reshape(T * H, HEAD_DIM))
    _plant_special_groups(rng, k)
    weights = rng.random((T, H), dtype=np.float32)
    max_pos = 32768
    positions = rng.integers(0, max_pos, T, dtype=np.int64)
    if positions_int32:
        positions = positions.astype(np.int32)
    NB = 8 if T <= 8 * KV_BLOCK else -(-T // KV_BLOCK) + 1
    slots = rng.permutation(NB * KV_BLOCK)[:T].astype(np.int64)
    n_skip = max(1, round(0.05 * T)) if T else 0
    if n_skip:
        slots[rng.choice(T, n_skip, replace=False)] = -1
    return Workload("edge_mix", T, H, q, k, positions, cos_sin_table(max_pos), weights, slots, NB,
                    is_neox=False)


def decode(seed: int = 2, n_seq: int = 64, next_n: int = 4, H: int = 32, NB: int = 4096,
           max_pos: int = 131072) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    T = n_seq * next_n
    q = _normal_bf16(rng, (T, H, HEAD_DIM))
    k = _normal_bf16(rng, (T, HEAD_DIM))
    weights = rng.random((T, H), dtype=np.float32)
    base = rng.integers(0, max_pos - next_n + 1, n_seq, dtype=np.int64)
    positions = (base[:, None] + np.arange(next_n, dtype=np.int64)[None, :]).reshape(-1)
    n_bg = NB * KV_BLOCK
    k_bg = _normal_bf16(rng, (n_bg, HEAD_DIM), chunk_rows=65536)
    pos_bg = rng.integers(0, max_pos, n_bg, dtype=np.int64)
    slots_bg = np.arange(n_bg, dtype=np.int64)
    slots = rng.choice(n_bg, T, replace=False).astype(np.int64)
    return Workload("decode", T, H, q, k, positions, cos_sin_table(max_pos), weights, slots, NB,
                    is_neox=True, background={"k": k_bg, "positions": pos_bg, "slots": slots_bg})


def prefill_norm_rotate(seed: int = 3, T: int = 16384, H: int = 64) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal_bf16(rng, (T, H, HEAD_DIM), chunk_rows=4096)
    k = _normal_bf16(rng, (T, HEAD_DIM))
    weights = rng.random((T, H), dtype=np.float32)
    gamma = to_bf16_bits((1.0 + 0.1 * rng.standard_normal(HEAD_DIM)).astype(np.float32))
    positions = np.arange(T, dtype=np.int64)
    NB = max(1, -(-T // KV_BLOCK))
    return Workload("prefill_norm_rotate", T, H, q, k, positions, cos_sin_table(max(T, 1)), weights,
                    np.arange(T, dtype=np.int64), NB, is_neox=True, apply_hadamard=True,
                    k_norm_gamma=gamma, k_norm_eps=1e-6)


def large_prefill(seed: int = 4, T: int = 131072, H: int = 64) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    n_out = max(1, round(0.01 * T))
    outliers = np.sort(rng.choice(T, n_out, replace=False))
    q = np.empty((T, H, HEAD_DIM), np.uint16)
    k = np.empty((T, HEAD_DIM), np.uint16)
    is_out = np.zeros(T, bool)
    is_out[outliers] = True
    step = 4096
    for a in range(0, T, step):
        b = min(T, a + step)
        qf = rng.standard_normal((b - a, H, HEAD_DIM), dtype=np.float32) * np.float32(2.0)
        kf = rng.standard_normal((b - a, HEAD_DIM), dtype=np.float32) * np.float32(2.0)
        sel = is_out[a:b]
        qf[sel] *= np.float32(100.0)
        kf[sel] *= np.float32(100.0)
        q[a:b] = to_bf16_bits(qf)
        k[a:b] = to_bf16_bits(kf)
    weights = rng.random((T, H), dtype=np.float32)
    positions = np.arange(T, dtype=np.int64)
    NB = max(1, -(-T // KV_BLOCK))
    return Workload("large_prefill", T, H, q, k, positions, cos_sin_table(max(T, 1)), weights,
                    np.arange(T, dtype=np.int64), NB, is_neox=True)


RECIPES = {
    "tiny": tiny,
    "edge_mix": edge_mix,
    "decode": decode,
    "prefill_norm_rotate": prefill_norm_rotate,
    "large_prefill": large_prefill,
}


@dataclass
class ScorerCase:
    """Inputs of the paged MQA-logits scorer: FP4 query rows with their q-scale rows,
    head weights, a paged FP4 key cache, block tables and context lengths."""
    name: str
    B: int
    next_n: int
    H: int
    q_out: np.ndarray           # u8 [B*next_n, H, 64]
    q_scale_out: np.ndarray     # u8 [B*next_n, 1, 4, 16, J]
    weights: np.ndarray         # fp32 [B*next_n, H]
    kv_cache: np.ndarray        # u8 [NB, 1, 4, 64, 16]
    kv_cache_scale: np.ndarray  # u8 [NB, 1, 4, 64]
    block_table: np.ndarray     # int32 [B, max_blocks]
    context_lens: np.ndarray    # int32 [B]

    @property
    def NB(self) -> int:
        return int(self.kv_cache.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])


def scorer_case(seed: int, B: int, next_n: int, H: int, ctx_lo: int, ctx_hi: int,
                max_context: Optional[int] = None, exp_lo: int = 118, exp_hi: int = 130,
                signed_weights: bool = False, spare_blocks: int = 0) -> ScorerCase:
    """Random FP4 bytes: uniform nibbles, e8m0 exponents U[exp_lo, exp_hi]; context
    lengths U[ctx_lo, ctx_hi]; every sequence owns distinct cache blocks, assigned in
    a random order; unused block-table entries are -1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = B * next_n
    J = q_scale_cols(H)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, B).astype(np.int32)
    if max_context is None:
        max_context = int(ctx.max()) if B else 1
    max_blocks = max(1, -(-max_context // KV_BLOCK))
    need = [-(-int(c) // KV_BLOCK) for c in ctx]
    NB = sum(need) + spare_blocks
    perm = rng.permutation(NB).astype(np.int32)
    table = np.full((B, max_blocks), -1, np.int32)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    q_out = rng.integers(0, 256, (T, H, 64), dtype=np.uint8)
    qs = np.zeros((T, 1, 4, 16, J), np.uint8)
    qs[..., : H // 16] = rng.integers(exp_lo, exp_hi + 1, (T, 1, 4, 16, H // 16), dtype=np.uint8)
    if signed_weights:
        weights = rng.uniform(-1.0, 1.0, (T, H)).astype(np.float32)
    else:
        weights = rng.random((T, H), dtype=np.float32)
    kv = rng.integers(0, 256, (NB, 1, 4, KV_BLOCK, 16), dtype=np.uint8)
    ks = rng.integers(exp_lo, exp_hi + 1, (NB, 1, 4, KV_BLOCK), dtype=np.uint8)
    return ScorerCase(f"scorer_B{B}_n{next_n}_H{H}", B, next_n, H, q_out, qs, weights, kv, ks,
                      table, ctx)
