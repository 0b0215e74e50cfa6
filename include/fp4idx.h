/*
 * fp4idx.h -- C ABI of libfp4idx, the fused FP4 sparse-indexer producer for
 * AMD Instinct MI355X (gfx950).
 *
 * Per token the library rotates the 64-dim RoPE slice of every 128-dim query
 * head and of the single index key (optionally RMS-normalising the key and
 * applying a 128-point Hadamard transform), quantizes each 32-element group
 * to E2M1 with a UE8M0 block exponent, packs two codes per byte, and
 * scatters the key into a paged FP4 index cache.
 *
 * Sources (web pages):
 *   ROCm/aiter PR 5484 "[HIP] Add FP4 output mode to
 *     indexer_qk_rope_quant_and_cache" -- sections "API", "Verification",
 *     "One deliberate deviation";
 *   sgl-project/sglang PR 39656 "dsv4.1: RoPE and FP4 packing kernels" --
 *     "Summary" and the review by @BBuf;
 *   ROCm/aiter PR 4029 "DeepSeek-V4 FP4: fused_compress FP4 scatter +
 *     rmsnorm_rope_rotate FP4 KV-cache kernel" -- "Changes" and the review
 *     by @zufayu.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer (memory from hipMalloc, e.g. a
 *   torch tensor on the GPU) unless stated otherwise.  The caller allocates
 *   and owns all buffers; the library allocates nothing, keeps no state other
 *   than a thread-local error message, and never synchronizes.
 * - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *   Work is enqueued on that stream only; outputs are valid once the caller
 *   has synchronized with it.  Calls on different streams or threads are
 *   independent (they must not share output buffers).
 * - All tensors are dense and row-major (C-contiguous).
 * - bf16 tensors hold IEEE bfloat16 bit patterns (uint16).
 * - Supported shapes are exactly head_dim D = 128, rope_dim R = 64,
 *   group_size = 32, kv block size BS = 64, and n_heads H a positive multiple
 *   of 16 up to 2048 (ROCm/aiter PR 5484 "API": anything else is rejected on
 *   the host with a specific message).
 * - Block exponent of a 32-group: e = clamp(max(E(amax/6), E(scale_floor)),
 *   1, 254) where E(x) is the biased exponent of x rounded up to a power of
 *   two, (bits >> 23) + (mantissa != 0) (sgl-project/sglang PR 39656,
 *   review).  `scale_floor` is the eps floor applied after the divide; 2^-126
 *   (FLT_MIN) makes it coincide with the lower clamp.  A finite input that the
 *   rotation, RMSNorm or Hadamard carries past the fp32 range is +-inf: its
 *   group's amax / 6 is infinite, E = 255 clamps to e = 254, and the
 *   infinite values take code 7 with their sign.
 * - Codes: each value v of the group becomes the E2M1 code of v * 2^(127-e)
 *   rounded to nearest, ties to even, with the sign bit of v kept even when
 *   the magnitude code is 0 (ROCm/aiter PR 5484 "One deliberate deviation").
 *   Element 2b goes to the low nibble of byte b.
 *
 * Return codes
 * ------------
 *   FP4IDX_OK (0); FP4IDX_EINVAL (1): null or misaligned pointer, negative
 *   size, flag outside {0,1}, inconsistent optional arguments, non-finite or
 *   negative floor/eps; FP4IDX_EUNSUPPORTED (2): a shape outside the list
 *   above, the message names the argument and its value; FP4IDX_EHIP (3): a
 *   HIP launch error, the message carries the HIP error string.  One call is
 *   one launch, and a launch covers at most 2^32 - 1 work-items (the grid size
 *   of a dispatch is 32-bit): a call past that (about 53 M query tokens,
 *   268 M keys or key rows, or dequant_debug of more than 2^28 - 1 rows x H
 *   query heads) returns FP4IDX_EHIP ("invalid configuration") with nothing
 *   enqueued.
 *   All validation happens before anything is enqueued: on a non-zero return
 *   nothing has been written.  T == 0 (rows == 0) is a successful no-op once
 *   the shape arguments are valid.  fp4idx_last_error() describes the last
 *   non-zero return on the calling thread.
 *
 * Caller errors that are NOT checked on the device
 *   duplicate non-negative slots in one call (which writer wins is
 *   unspecified); non-finite inputs.  Positions outside [0, max_pos) are
 *   clamped into that range and slots outside [0, NB*BS) are skipped, so no
 *   input value can make the library read or write out of bounds.
 */
#ifndef FP4IDX_H
#define FP4IDX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4IDX_OK 0
#define FP4IDX_EINVAL 1
#define FP4IDX_EUNSUPPORTED 2
#define FP4IDX_EHIP 3

/* fake-quant modes */
#define FP4IDX_FQ_UE8M0_32 0
#define FP4IDX_FQ_E4M3_16 1

/* FP8 scale formats */
#define FP4IDX_SCALE_UE8M0 0
#define FP4IDX_SCALE_FP32 1

/*
 * fp4idx_q_rope_pack -- query side of the producer (ROCm/aiter PR 5484 "API":
 * q_out u8 [num_tokens, n_heads, head_dim/2], q_scale_out u8
 * [num_tokens, k_tiles, 4, 16, round_up(H/16, 4)], weights_out with the plain
 * weight and nothing folded in).
 *
 *   q            bf16 [T, H, 128], 16-byte aligned.
 *   positions    [T] int64 (positions_int64 = 1) or int32 (= 0), naturally
 *                aligned.  Each is clamped to [0, max_pos).
 *   cos_sin      fp32 [max_pos, 64], 16-byte aligned: columns 0..31 are
 *                cos(p*f_i), 32..63 sin(p*f_i); pair i uses column i.
 *   weights      fp32 [T, H] or NULL, 4-byte aligned.
 *   T, H         tokens (>= 0), heads (multiple of 16, <= 2048).
 *   D, R, group_size   must be 128, 64, 32.
 *   rope_offset  first rotated dim: 64 (the tail of the row) or 0.
 *   is_neox      1: pairs (i, i+32) of the slice; 0: pairs (2i, 2i+1).
 *                Rotation a' = bf16(a*c - b*s), b' = bf16(b*c + a*s), each
 *                product rounded to fp32 separately (no fused multiply-add).
 *   apply_hadamard  1: after RoPE, a 128-point Walsh-Hadamard transform in
 *                natural (Sylvester) order, butterflies of stride 1..64 in
 *                fp32, then x * fp32(1/sqrt(128)) rounded to bf16.
 *   scale_floor  eps floor of the block scale (>= 0, finite); 2^-126 default.
 *   q_out        u8 [T, H, 64], 16-byte aligned.  Row (t,h) holds the codes
 *                of the four 32-groups, 16 bytes each.
 *   q_scale_out  u8 [T, 1, 4, 16, J], J = round_up(H/16, 4), 4-byte aligned.
 *                Entry [t, 0, g, h % 16, h / 16] = e of group g of head h;
 *                entries with h/16 >= H/16 are written as 0.
 *   weights_out  fp32 [T, H] or NULL (must be NULL iff weights is NULL):
 *                bit copy of weights.
 */
int fp4idx_q_rope_pack(const void* q, const void* positions, int positions_int64,
                       const float* cos_sin, int64_t max_pos, const float* weights,
                       int64_t T, int H, int D, int R, int rope_offset, int group_size,
                       int is_neox, int apply_hadamard, float scale_floor,
                       uint8_t* q_out, uint8_t* q_scale_out, float* weights_out, void* stream);

/*
 * fp4idx_k_rope_pack_store -- key side: optional RMSNorm, RoPE, optional
 * Hadamard, quantize, and scatter into the paged index cache (ROCm/aiter PR
 * 5484 "API": kv_cache u8 [num_blocks, k_tiles, 4, kv_block_size, 16],
 * kv_cache_scale u8 [num_blocks, k_tiles, 4, kv_block_size]; ROCm/aiter PR
 * 4029 "Changes": scales interleaved at (pos%16)*(kv_block_size/16)+pos/16;
 * sgl-project/sglang PR 39656 "Summary": RMSNorm, RoPE, quantize and store
 * fused in one launch).
 *
 *   k            bf16 [T, 128], 16-byte aligned.
 *   positions, positions_int64, cos_sin, max_pos, rope_offset, is_neox,
 *   apply_hadamard, scale_floor, D, R, group_size: as for the query call.
 *   slot_mapping int64 [T], 8-byte aligned.  Token t goes to block
 *                slot/64, position slot%64; a slot outside [0, NB*64)
 *                (e.g. -1) writes nothing for that token.
 *   k_norm_gamma bf16 [128] (16-byte aligned) or NULL = no RMSNorm.  With it:
 *                ss = sum of x_i^2 folded by halves (i with i+64, then +32,
 *                ..., +1), r = 1/sqrt(ss/128 + k_norm_eps) with correctly
 *                rounded sqrt and divide, x_i = bf16((x_i*r)*gamma_i).
 *   k_norm_eps   >= 0 and finite when k_norm_gamma is given.
 *   kv_cache     u8 [NB, 1, 4, 64, 16], 16-byte aligned:
 *                [blk, 0, g, pos, :] = the 16 code bytes of group g.
 *   kv_cache_scale u8 [NB, 1, 4, 64], 4-byte aligned:
 *                [blk, 0, g, (pos%16)*4 + pos/16] = e of group g.
 *   NB, BS       number of blocks (>= 0) and block size (must be 64).
 * Bytes of slots that no token maps to are left untouched.
 */
int fp4idx_k_rope_pack_store(const void* k, const void* positions, int positions_int64,
                             const float* cos_sin, int64_t max_pos, const int64_t* slot_mapping,
                             const void* k_norm_gamma, float k_norm_eps,
                             int64_t T, int D, int R, int rope_offset, int group_size,
                             int is_neox, int apply_hadamard, float scale_floor,
                             uint8_t* kv_cache, uint8_t* kv_cache_scale, int64_t NB, int BS,
                             void* stream);

/*
 * fp4idx_qk_rope_pack_store -- both sides of the producer in one launch, as
 * the pages' producer writes all five outputs from one kernel (ROCm/aiter PR
 * 5484 "Verification" compares all five outputs of that kernel).
 * Arguments mean what they mean for fp4idx_q_rope_pack and
 * fp4idx_k_rope_pack_store (q and k share T, positions, cos_sin, rope_offset,
 * is_neox, apply_hadamard and scale_floor); every check of both calls
 * applies.  The outputs are byte-identical to calling the two entry points
 * one after the other; positions and cos/sin rows are read once.
 */
int fp4idx_qk_rope_pack_store(const void* q, const void* k, const void* positions,
                              int positions_int64, const float* cos_sin, int64_t max_pos,
                              const float* weights, const int64_t* slot_mapping,
                              const void* k_norm_gamma, float k_norm_eps, int64_t T, int H, int D,
                              int R, int rope_offset, int group_size, int is_neox,
                              int apply_hadamard, float scale_floor, uint8_t* q_out,
                              uint8_t* q_scale_out, float* weights_out, uint8_t* kv_cache,
                              uint8_t* kv_cache_scale, int64_t NB, int BS, void* stream);

/*
 * fp4idx_q_rope_pack_sglang / fp4idx_k_rope_pack_store_sglang -- the
 * sglang-compatible mode (sgl-project/sglang PR 39656 "Summary": RoPE and
 * FP4 packing into the 68-byte index-K format, 64 E2M1 bytes plus four block
 * exponents; review: the packer's sign rule and separate stage floors).
 * Per 128-row, after the optional key RMSNorm and the RoPE (as for the calls
 * above; there is no Hadamard in this mode), each 32-group is quantized twice:
 *   stage 1 (fake quant): e1 from fake_quant_floor by the block-exponent
 *     rule above, y_i = E2M1(v_i * 2^(127-e1)) * 2^(e1-127) in fp32 (a y of
 *     magnitude >= 2^128 is +-inf);
 *   stage 2 (packer): e2 from the y's with pack_floor by the same rule, codes
 *     of y_i * 2^(127-e2) rounded to nearest even, and the sign bit set only
 *     when the magnitude code is nonzero (no -0 codes).
 * Record (68 bytes): byte g*16+b holds the codes of elements 32g+2b (low
 * nibble) and 32g+2b+1 (high nibble); bytes 64..67 hold e2 of groups 0..3.
 * Both floors: finite and >= 0.  No weights are passed through.
 *
 * fp4idx_q_rope_pack_sglang
 *   q, positions, positions_int64, cos_sin, max_pos, T, H, D, R, rope_offset,
 *   group_size, is_neox: as for fp4idx_q_rope_pack.
 *   q_packed     u8 [T, H, 68], 16-byte aligned: record of head h of token t.
 *
 * fp4idx_k_rope_pack_store_sglang
 *   k, positions, positions_int64, cos_sin, max_pos, slot_mapping,
 *   k_norm_gamma, k_norm_eps, T, D, R, rope_offset, group_size, is_neox: as
 *   for fp4idx_k_rope_pack_store.
 *   index_k_cache u8 [num_slots, 68], 4-byte aligned: token t's record goes
 *                to row slot_mapping[t] when 1 <= slot < num_slots; slot 0
 *                (and any slot outside that range) publishes nothing.
 *   compress_ratio 1, 2 or 4: each key row stands for that many consecutive
 *                tokens (a compressed KV entry) and is rotated at the first
 *                position of its group, pos - pos % compress_ratio
 *                (sgl-project/sglang PR 39656 "Summary": RoPE at the group's
 *                first position; "Verification": ratios 1, 2, 4).
 *   num_slots    >= 0.  Rows that no token maps to are left untouched.
 */
int fp4idx_q_rope_pack_sglang(const void* q, const void* positions, int positions_int64,
                              const float* cos_sin, int64_t max_pos, int64_t T, int H, int D,
                              int R, int rope_offset, int group_size, int is_neox,
                              float fake_quant_floor, float pack_floor, uint8_t* q_packed,
                              void* stream);

int fp4idx_k_rope_pack_store_sglang(const void* k, const void* positions, int positions_int64,
                                    const float* cos_sin, int64_t max_pos,
                                    const int64_t* slot_mapping, const void* k_norm_gamma,
                                    float k_norm_eps, int64_t T, int D, int R, int rope_offset,
                                    int group_size, int is_neox, int compress_ratio,
                                    float fake_quant_floor, float pack_floor,
                                    uint8_t* index_k_cache, int64_t num_slots, void* stream);

/*
 * fp4idx_q_rope_pack_fp8 / fp4idx_k_rope_pack_store_fp8 -- the FP8 output
 * mode of the same producer (ROCm/aiter PR 5484 "API": the FP8 contract folds
 * its per-(token, head) q scale, and weights_scale, into weights_out of
 * dtype q.dtype; scale_fmt ue8m0 or fp32.  ROCm/aiter PR 4029 review: the
 * gfx950 FP8 format is e4m3fn, largest value 448).  The rotation, key
 * RMSNorm and optional Hadamard are those of the FP4 calls above; then each
 * 128-row (a query head, a key token) gets one scale
 *     s = max(amax / 448, scale_floor)                  (fp32, scale_fmt = 1)
 *     s = 2^(E - 127), E = clamp(E(amax / 448 floored), 1, 254)   (ue8m0 = 0)
 * with E() the block-exponent rule above, and every element the e4m3fn code
 * nearest to x / s (x / s rounded to fp32 first; ties to even; the sign kept
 * on zero; every magnitude at or beyond 448, infinities included, saturates
 * to 448).  Codes 0x7F/0xFF are never produced, except 0x7F for inf / inf
 * when an infinite value makes an fp32 scale infinite (its other elements
 * are then signed zeros).  The preshuffled cache layout is not provided.
 *
 * fp4idx_q_rope_pack_fp8
 *   q, positions, positions_int64, cos_sin, max_pos, T, H, D, R,
 *   rope_offset, is_neox, apply_hadamard: as for fp4idx_q_rope_pack.
 *   weights      fp32 [T, H], 4-byte aligned (required: it carries the scale).
 *   weights_scale finite fp32 scalar.
 *   scale_fmt    FP4IDX_SCALE_UE8M0 or FP4IDX_SCALE_FP32.
 *   scale_floor  >= 0; >= 2^-126 with fp32 scales.
 *   q_out        e4m3fn [T, H, 128] (bytes), 16-byte aligned.
 *   weights_out  bf16 [T, H], 2-byte aligned:
 *                bf16((weights[t,h] * s_{t,h}) * weights_scale), round to
 *                nearest even, products rounded separately.
 *
 * fp4idx_k_rope_pack_store_fp8
 *   k, positions, positions_int64, cos_sin, max_pos, slot_mapping,
 *   k_norm_gamma, k_norm_eps, T, D, R, rope_offset, is_neox,
 *   apply_hadamard, NB, BS: as for fp4idx_k_rope_pack_store; scale_fmt and
 *   scale_floor as above.
 *   kv_cache       e4m3fn [NB, 64, 128], 16-byte aligned: row slot = the
 *                  token's 128 codes.
 *   kv_cache_scale fp32 [NB, 64], 4-byte aligned: [slot] = the token's s.
 *   A slot outside [0, NB*64) writes nothing.
 */
int fp4idx_q_rope_pack_fp8(const void* q, const void* positions, int positions_int64,
                           const float* cos_sin, int64_t max_pos, const float* weights,
                           float weights_scale, int64_t T, int H, int D, int R, int rope_offset,
                           int is_neox, int apply_hadamard, int scale_fmt, float scale_floor,
                           uint8_t* q_out, uint16_t* weights_out, void* stream);

int fp4idx_k_rope_pack_store_fp8(const void* k, const void* positions, int positions_int64,
                                 const float* cos_sin, int64_t max_pos,
                                 const int64_t* slot_mapping, const void* k_norm_gamma,
                                 float k_norm_eps, int64_t T, int D, int R, int rope_offset,
                                 int is_neox, int apply_hadamard, int scale_fmt,
                                 float scale_floor, uint8_t* kv_cache, float* kv_cache_scale,
                                 int64_t NB, int BS, void* stream);

/*
 * fp4idx_rope_fake_quant -- RoPE tail plus FP4 fake quant for the
 * torch-shaped path (sgl-project/sglang PR 39656 "Summary": per-32 UE8M0
 * scales by default and per-16 E4M3 scales for compressed KV, keeping the
 * bf16 round trip after RoPE and rounding half to even).  Returns the bf16
 * values of the quantized rows, not codes.
 *
 *   x            bf16 [rows, 128], 16-byte aligned (e.g. q [T, H, 128] with
 *                rows = T*H, or compressed keys [N, 128]).
 *   rows_per_position  row r uses positions[r / rows_per_position] (H for
 *                queries, 1 for keys); positions holds
 *                ceil(rows / rows_per_position) entries.
 *   positions, positions_int64, cos_sin, max_pos, D, R, rope_offset,
 *   is_neox: as for fp4idx_q_rope_pack (RoPE on the 64-dim slice, bf16).
 *   compress_ratio 1, 2 or 4: the rotation uses pos - pos % compress_ratio.
 *   mode         FP4IDX_FQ_UE8M0_32: per 32-group, e by the block-exponent
 *                rule with scale_floor, value = E2M1(code) * 2^(e-127) as an
 *                fp32 product (+-inf when it reaches 2^128), then bf16;
 *                FP4IDX_FQ_E4M3_16: per 16-group, s = the e4m3fn value nearest
 *                to max(amax/6, scale_floor) (448 at most), code = E2M1
 *                value nearest to fl(x/s) (ties to even, 6 at most),
 *                value = code value * s with the sign of x; s = 0 gives
 *                signed zeros.
 *   scale_floor  finite, >= 0.
 *   y            bf16 [rows, 128], 16-byte aligned (may not alias x).
 */
int fp4idx_rope_fake_quant(const void* x, int64_t rows, int64_t rows_per_position,
                           const void* positions, int positions_int64, const float* cos_sin,
                           int64_t max_pos, int D, int R, int rope_offset, int is_neox,
                           int compress_ratio, int mode, float scale_floor, void* y,
                           void* stream);

/*
 * fp4idx_dequant_debug -- reader side, for tests and debugging: expands
 * codes back to fp32, value = E2M1(nibble) * 2^(e-127) with E2M1 magnitudes
 * {0, .5, 1, 1.5, 2, 3, 4, 6} and bit 3 the sign; e = 0 gives 2^-127 and
 * e = 255 gives NaN (OCP MX e8m0).
 *
 *   which = 0 (Q):      packed = q_out [rows=T, H, 64], scales = q_scale_out
 *                       [T, 1, 4, 16, J]; out fp32 [T, H, 128].
 *   which = 1 (KCACHE): packed = kv_cache [NB, 1, 4, 64, 16], scales =
 *                       kv_cache_scale [NB, 1, 4, 64]; slots int64 [rows]
 *                       (or NULL: row r reads slot r); out fp32 [rows, 128];
 *                       a slot outside [0, NB*64) gives a row of zeros.
 *   H is used only for which = 0; NB and BS (= 64) only for which = 1.
 *   out must be 16-byte aligned.
 */
int fp4idx_dequant_debug(int which, const uint8_t* packed, const uint8_t* scales, int64_t rows,
                         int H, const int64_t* slots, int64_t NB, int BS, float* out, void* stream);

/*
 * fp4idx_paged_mqa_logits -- the scorer that consumes the producer's bytes
 * (ROCm/aiter PR 5484, intro: flydsl_pa_mqa_logits_fp4 scores the FP4 keys
 * directly from the paged cache; "API": the MFMA consumes the per-group
 * e8m0 scales directly and the scorer applies its own fp32 weights_scale).
 * Runs on the gfx950 scaled-FP4 matrix cores.
 *
 * For sequence b (0 <= b < B) with context length ctx_b and query token
 * t = b*next_n + j (position ctx_b - next_n + j), and key s < ctx_b stored at
 * slot block_table[b, s/64]*64 + s%64:
 *     logits[t, s] = weights_scale * sum_h weights[t,h] * R(q_h . k_s)
 * where q_h and k_s are the dequantized 128-vectors (E2M1 x 2^(e-127)) and R
 * is ReLU (apply_relu = 1) or the identity (0).  Keys after the query's
 * position, and keys whose block-table entry is outside [0, NB), get -inf.
 * Entries s >= ctx_b are not written.  Products and sums are fp32 (matrix-core
 * accumulation, then fused multiply-adds): results match an exact evaluation
 * to within a few fp32 roundings of sum_h |w| sum_d |q_d k_d|.
 *
 *   q_out, q_scale_out  as written by fp4idx_q_rope_pack for T = B*next_n
 *                       tokens (16- and 4-byte aligned).
 *   weights      fp32 [T, H], 16-byte aligned (the plain weights_out).
 *   kv_cache, kv_cache_scale, NB   as written by fp4idx_k_rope_pack_store.
 *   block_table  int32 [B, max_blocks]; only entries s/64 < ctx_b are read.
 *   context_lens int32 [B]; clamped to [0, min(max_blocks*64, stride)].
 *   H            16, 32, 48 or 64;  B <= 65535.
 *   next_n       1..131070.  1..4: decode, one tile of next_n query tokens per
 *                sequence (multi-token prediction).  Larger: chunked prefill,
 *                the next_n queries in tiles of 4 (H = 32) or 2 (other H);
 *                a key block that lies entirely after a tile's last position
 *                is written as -inf without being read.
 *   logits       fp32 [T, stride].
 */
int fp4idx_paged_mqa_logits(const uint8_t* q_out, const uint8_t* q_scale_out, const float* weights,
                            float weights_scale, const uint8_t* kv_cache,
                            const uint8_t* kv_cache_scale, int64_t NB, const int32_t* block_table,
                            int64_t max_blocks, const int32_t* context_lens, int64_t B,
                            int next_n, int H, int apply_relu, float* logits, int64_t stride,
                            void* stream);

/* Message describing the last non-zero return on the calling thread
 * (thread-local; "" if there was none).  Owned by the library. */
const char* fp4idx_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4IDX_H */
