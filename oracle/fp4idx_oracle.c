/*
 * fp4idx_oracle.c -- CPU oracle for the fused FP4 sparse-indexer producer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, scalar definition
 * that the HIP kernels are checked against.  Only the test-suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it; the product
 * path never does.  It shares no code, header, table or constant with the
 * GPU library.
 *
 * Sources (the four web pages this method is described on):
 *   [aiter-5484]  ROCm/aiter PR 5484 "[HIP] Add FP4 output mode to
 *                 indexer_qk_rope_quant_and_cache": API, Verification,
 *                 "One deliberate deviation".
 *   [sglang-39656] sgl-project/sglang PR 39656 "dsv4.1: RoPE and FP4 packing
 *                 kernels": Summary, review by @BBuf.
 *   [aiter-4029]  ROCm/aiter PR 4029 "DeepSeek-V4 FP4: fused_compress FP4
 *                 scatter + rmsnorm_rope_rotate FP4 KV-cache kernel":
 *                 Changes, review by @zufayu.
 *
 * Arithmetic: every floating-point step is one IEEE-754 binary32 operation
 * with round-to-nearest-even and denormals preserved.  Build with
 * -O2 -fno-fast-math -ffp-contract=off (no FMA contraction, no FTZ/DAZ).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - RoPE acts on dims [rope_offset, rope_offset+64) of a 128-dim row
 *     (sglang's kernel rotates the tail of the row, so the default
 *     offset is 64).
 *   - cos/sin table: fp32 [max_pos, 64], cols 0..31 cos, 32..63 sin; pair i
 *     uses column i.  neox pairs (i, i+32); interleaved pairs (2i, 2i+1).
 *   - RoPE: a' = bf16(a*c - b*s), b' = bf16(b*c + a*s), products rounded
 *     separately (no FMA).
 *   - key RMSNorm: squares summed by folding halves (n = 64, 32, ..., 1),
 *     r = 1 / sqrt(ss/128 + eps) as two correctly rounded ops,
 *     y = bf16((x*r)*gamma).
 *   - Hadamard: natural (Sylvester) order, butterflies with stride 1, 2, ...,
 *     64, then one multiply by fp32(1/sqrt(128)) and a bf16 rounding.
 *   - eps floor of the block scale: an ABI parameter, default 2^-126.
 *   - E2M1 code: round half to even, sign kept on zero codes (hardware
 *     semantics as stated in [aiter-5484] "One deliberate deviation").
 *   - nibble order: element 2b in the low nibble of byte b.
 *   - positions outside [0, max_pos) are clamped into it; slots outside
 *     [0, num_blocks*block_size) write nothing.
 *
 * Parity pins: see tests/test_oracle_*.py.  The exact rounding order of the
 * RoPE, RMSNorm and Hadamard steps is a reading, not a page fact: parity
 * unpinned for those orders (their results are pinned only to tolerance).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1

#define HEAD_DIM 128
#define ROPE_DIM 64
#define GROUP 32
#define NGROUPS (HEAD_DIM / GROUP)
#define KV_BLOCK 64

/* ------------------------------------------------------------------ */
/* bit helpers                                                         */
/* ------------------------------------------------------------------ */
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32. */
static float bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* fp32 -> bf16, round to nearest, ties to even (finite inputs). */
static uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = f2u(f);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* bf16(x): the value after the bf16 round trip, as fp32. */
static float round_bf16(float f) { return bf16_to_f32(f32_to_bf16_bits(f)); }

/* ------------------------------------------------------------------ */
/* step 5: UE8M0 block exponent of one 32-group                        */
/* [sglang-39656] review: biased exponent of ceil_pow2(amax / 6) is     */
/* (bits >> 23) + (mantissa != 0), with a post-divide floor and the     */
/* clamp min(max(e, 1), 254).  [aiter-4029] review: all-zero groups get */
/* an eps floor.                                                        */
/* ------------------------------------------------------------------ */
static int group_exponent(const float* v, int n, float scale_floor) {
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    float q = amax / 6.0f;
    if (q < scale_floor) q = scale_floor;
    uint32_t b = f2u(q);
    int e = (int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0);
    if (e < 1) e = 1;
    if (e > 254) e = 254;
    return e;
}

/* ------------------------------------------------------------------ */
/* step 6: one E2M1 nibble of v under block exponent e                  */
/* value grid {0, .5, 1, 1.5, 2, 3, 4, 6} = codes 0..7; a value exactly */
/* half-way between two grid points goes to the even code; magnitudes   */
/* above 6 saturate to code 7.  Bit 3 is the sign of v, kept on zero    */
/* codes ([aiter-5484] "One deliberate deviation").                      */
/* ------------------------------------------------------------------ */
/* magnitude code of m >= 0: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to
   the even code, anything above 6 saturating to 6 */
static int e2m1_magnitude_code(float m) {
    int code;
    if (m <= 0.25f) code = 0;
    else if (m < 0.75f) code = 1;
    else if (m <= 1.25f) code = 2;
    else if (m < 1.75f) code = 3;
    else if (m <= 2.5f) code = 4;
    else if (m < 3.5f) code = 5;
    else if (m <= 5.0f) code = 6;
    else code = 7;
    return code;
}

static uint8_t e2m1_nibble(float v, int e) {
    float inv = ldexpf(1.0f, 127 - e); /* exact power of two */
    int code = e2m1_magnitude_code(fabsf(v * inv));
    int sign = signbit(v) ? 1 : 0;
    return (uint8_t)((sign << 3) | code);
}

/* steps 5-7 on a 128-row: exponents e[4], packed bytes out[64]. */
static void quantize_row(const float* x, float scale_floor, uint8_t* e_out, uint8_t* bytes) {
    for (int g = 0; g < NGROUPS; ++g) {
        const float* v = x + g * GROUP;
        int e = group_exponent(v, GROUP, scale_floor);
        e_out[g] = (uint8_t)e;
        for (int b = 0; b < GROUP / 2; ++b) {
            uint8_t lo = e2m1_nibble(v[2 * b], e);
            uint8_t hi = e2m1_nibble(v[2 * b + 1], e);
            bytes[g * (GROUP / 2) + b] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* ------------------------------------------------------------------ */
/* step 3: RoPE on the 64-wide slice S, then bf16                       */
/* ------------------------------------------------------------------ */
static void rope_slice(float* S, const float* cs_row, int is_neox) {
    for (int i = 0; i < ROPE_DIM / 2; ++i) {
        int ia = is_neox ? i : 2 * i;
        int ib = is_neox ? i + ROPE_DIM / 2 : 2 * i + 1;
        float a = S[ia], b = S[ib];
        float c = cs_row[i], s = cs_row[ROPE_DIM / 2 + i];
        float ac = a * c;
        float bs = b * s;
        float bc = b * c;
        float as = a * s;
        S[ia] = round_bf16(ac - bs);
        S[ib] = round_bf16(bc + as);
    }
}

/* ------------------------------------------------------------------ */
/* step 4: 128-point Walsh-Hadamard transform, orthonormal scale, bf16 */
/* ------------------------------------------------------------------ */
static float hadamard_scale(void) { return (float)(1.0 / sqrt((double)HEAD_DIM)); }

static void fwht128(float* x) {
    for (int h = 1; h < HEAD_DIM; h <<= 1) {
        for (int j = 0; j < HEAD_DIM; ++j) {
            if (j & h) continue;
            float u = x[j], w = x[j + h];
            x[j] = u + w;
            x[j + h] = u - w;
        }
    }
    float sc = hadamard_scale();
    for (int i = 0; i < HEAD_DIM; ++i) x[i] = round_bf16(x[i] * sc);
}

/* ------------------------------------------------------------------ */
/* step 2: key RMSNorm                                                  */
/* ------------------------------------------------------------------ */
static void rmsnorm128(float* x, const uint16_t* gamma, float eps) {
    float p[HEAD_DIM];
    for (int i = 0; i < HEAD_DIM; ++i) p[i] = x[i] * x[i];
    for (int n = HEAD_DIM / 2; n >= 1; n >>= 1)
        for (int i = 0; i < n; ++i) p[i] = p[i] + p[i + n];
    float mean = p[0] / (float)HEAD_DIM;
    float den = sqrtf(mean + eps);
    float r = 1.0f / den;
    for (int i = 0; i < HEAD_DIM; ++i) {
        float y = x[i] * r;
        x[i] = round_bf16(y * bf16_to_f32(gamma[i]));
    }
}

/* ------------------------------------------------------------------ */
/* shared per-token helpers                                             */
/* ------------------------------------------------------------------ */
static int64_t read_position(const void* positions, int positions_int64, int64_t t, int64_t max_pos) {
    int64_t p = positions_int64 ? ((const int64_t*)positions)[t] : (int64_t)((const int32_t*)positions)[t];
    if (p < 0) p = 0;
    if (p >= max_pos) p = max_pos - 1;
    return p;
}

/* one 128-row through steps 1, 3, 4 (RMSNorm is applied by the caller). */
static void rope_hadamard_row(float* x, const float* cs_row, int rope_offset, int is_neox, int apply_hadamard) {
    rope_slice(x + rope_offset, cs_row, is_neox);
    if (apply_hadamard) fwht128(x);
}

static int check_shape(int D, int R, int rope_offset, int group_size) {
    if (D != HEAD_DIM || R != ROPE_DIM || group_size != GROUP) return ORC_EINVAL;
    if (rope_offset != 0 && rope_offset != HEAD_DIM - ROPE_DIM) return ORC_EINVAL;
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* public: query path                                                   */
/* q_out [T,H,64]; q_scale_out [T,1,4,16,J], J = round_up(H/16, 4),     */
/* entry [t,0,g,h%16,h/16] = e, pad entries 0 ([aiter-5484] API and     */
/* Verification, which tests the zero padding); weights_out = plain.    */
/* ------------------------------------------------------------------ */
int oracle_q_rope_pack(const uint16_t* q, const void* positions, int positions_int64,
                       const float* cos_sin, int64_t max_pos, const float* weights,
                       int64_t T, int H, int D, int R, int rope_offset, int group_size,
                       int is_neox, int apply_hadamard, float scale_floor,
                       uint8_t* q_out, uint8_t* q_scale_out, float* weights_out) {
    if (check_shape(D, R, rope_offset, group_size) != ORC_OK) return ORC_EINVAL;
    if (H <= 0 || H % 16 != 0 || T < 0 || max_pos <= 0) return ORC_EINVAL;
    const int J = ((H / 16) + 3) / 4 * 4;
    for (int64_t t = 0; t < T; ++t) {
        int64_t pos = read_position(positions, positions_int64, t, max_pos);
        const float* cs_row = cos_sin + pos * ROPE_DIM;
        uint8_t* qs = q_scale_out + t * (int64_t)NGROUPS * 16 * J;
        memset(qs, 0, (size_t)NGROUPS * 16 * J);
        for (int h = 0; h < H; ++h) {
            const uint16_t* src = q + (t * H + h) * HEAD_DIM;
            float x[HEAD_DIM];
            for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_f32(src[i]);
            rope_hadamard_row(x, cs_row, rope_offset, is_neox, apply_hadamard);
            uint8_t e[NGROUPS];
            quantize_row(x, scale_floor, e, q_out + (t * H + h) * (HEAD_DIM / 2));
            for (int g = 0; g < NGROUPS; ++g) qs[(g * 16 + h % 16) * J + h / 16] = e[g];
        }
        if (weights && weights_out)
            for (int h = 0; h < H; ++h) weights_out[t * H + h] = weights[t * H + h];
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* public: key path with paged scatter                                  */
/* kv_cache [NB,1,4,BS,16]: kv_cache[blk,0,g,pos,:] = the 16 bytes of   */
/* group g ([aiter-5484] API); kv_cache_scale [NB,1,4,BS] with the       */
/* exponent of group g at (pos%16)*(BS/16) + pos/16 ([aiter-4029]       */
/* Changes: the interleaved KV scale layout).                          */
/* ------------------------------------------------------------------ */
int oracle_k_rope_pack_store(const uint16_t* k, const void* positions, int positions_int64,
                             const float* cos_sin, int64_t max_pos, const int64_t* slot_mapping,
                             const uint16_t* k_norm_gamma, float k_norm_eps,
                             int64_t T, int D, int R, int rope_offset, int group_size,
                             int is_neox, int apply_hadamard, float scale_floor,
                             uint8_t* kv_cache, uint8_t* kv_cache_scale, int64_t NB, int BS) {
    if (check_shape(D, R, rope_offset, group_size) != ORC_OK) return ORC_EINVAL;
    if (BS != KV_BLOCK || NB < 0 || T < 0 || max_pos <= 0) return ORC_EINVAL;
    const int64_t nslots = NB * BS;
    for (int64_t t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= nslots) continue;
        int64_t pos = read_position(positions, positions_int64, t, max_pos);
        const float* cs_row = cos_sin + pos * ROPE_DIM;
        float x[HEAD_DIM];
        for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_f32(k[t * HEAD_DIM + i]);
        if (k_norm_gamma) rmsnorm128(x, k_norm_gamma, k_norm_eps);
        rope_hadamard_row(x, cs_row, rope_offset, is_neox, apply_hadamard);
        uint8_t e[NGROUPS];
        uint8_t bytes[HEAD_DIM / 2];
        quantize_row(x, scale_floor, e, bytes);
        int64_t blk = slot / BS;
        int64_t p = slot % BS;
        for (int g = 0; g < NGROUPS; ++g) {
            uint8_t* dst = kv_cache + (((blk * 1 + 0) * NGROUPS + g) * BS + p) * 16;
            memcpy(dst, bytes + g * 16, 16);
            kv_cache_scale[((blk * 1 + 0) * NGROUPS + g) * BS + (p % 16) * (BS / 16) + p / 16] = e[g];
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* public: dequantization (reader side), fp32                           */
/* value = E2M1(nibble) * 2^(e - 127); e = 255 gives NaN (OCP e8m0).    */
/* which = 0: q_out/q_scale_out rows [T,H,128] -> out [T,H,128].        */
/* which = 1: cache slots -> out [rows,128]; slots NULL = slot r for    */
/* row r; a slot outside the cache gives a row of zeros.                */
/* ------------------------------------------------------------------ */
static float e2m1_value(uint8_t nib) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float v = mag[nib & 7];
    return (nib & 8) ? -v : v;
}

static float e8m0_value(uint8_t e) {
    if (e == 255) return u2f(0x7FC00000u);
    return ldexpf(1.0f, (int)e - 127);
}

int oracle_dequant(int which, const uint8_t* packed, const uint8_t* scales, int64_t rows, int H,
                   const int64_t* slots, int64_t NB, int BS, float* out) {
    if (rows < 0) return ORC_EINVAL;
    if (which == 0) {
        if (H <= 0 || H % 16 != 0) return ORC_EINVAL;
        const int J = ((H / 16) + 3) / 4 * 4;
        for (int64_t t = 0; t < rows; ++t)
            for (int h = 0; h < H; ++h)
                for (int d = 0; d < HEAD_DIM; ++d) {
                    int g = d / GROUP;
                    uint8_t byte = packed[(t * H + h) * (HEAD_DIM / 2) + d / 2];
                    uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                    uint8_t e = scales[t * (int64_t)NGROUPS * 16 * J + (g * 16 + h % 16) * J + h / 16];
                    out[(t * H + h) * HEAD_DIM + d] = e2m1_value(nib) * e8m0_value(e);
                }
        return ORC_OK;
    }
    if (which == 1) {
        if (BS != KV_BLOCK || NB < 0) return ORC_EINVAL;
        for (int64_t r = 0; r < rows; ++r) {
            int64_t slot = slots ? slots[r] : r;
            float* o = out + r * HEAD_DIM;
            if (slot < 0 || slot >= NB * BS) {
                for (int d = 0; d < HEAD_DIM; ++d) o[d] = 0.0f;
                continue;
            }
            int64_t blk = slot / BS, p = slot % BS;
            for (int d = 0; d < HEAD_DIM; ++d) {
                int g = d / GROUP;
                uint8_t byte = packed[((blk * NGROUPS + g) * BS + p) * 16 + (d % GROUP) / 2];
                uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                uint8_t e = scales[(blk * NGROUPS + g) * BS + (p % 16) * (BS / 16) + p / 16];
                o[d] = e2m1_value(nib) * e8m0_value(e);
            }
        }
        return ORC_OK;
    }
    return ORC_EINVAL;
}

/* ------------------------------------------------------------------ */
/* step-level entry points, exported so the pins can test each step    */
/* ------------------------------------------------------------------ */
void oracle_bf16_round(const float* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(in[i]);
}

/* v: [n_groups, gsize] fp32; e_out: [n_groups] */
void oracle_group_exponents(const float* v, int64_t n_groups, int gsize, float scale_floor, int32_t* e_out) {
    for (int64_t g = 0; g < n_groups; ++g) e_out[g] = group_exponent(v + g * gsize, gsize, scale_floor);
}

/* nibble of v[i] under exponent e[i] */
void oracle_e2m1_nibbles(const float* v, const int32_t* e, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e2m1_nibble(v[i], e[i]);
}

/* x: [n,128] fp32 (bf16 values), in place: quantize rows -> bytes [n,64], e [n,4] */
void oracle_quantize_rows(const float* x, int64_t n, float scale_floor, uint8_t* bytes, uint8_t* e) {
    for (int64_t r = 0; r < n; ++r) quantize_row(x + r * HEAD_DIM, scale_floor, e + r * NGROUPS, bytes + r * (HEAD_DIM / 2));
}

/* x: [n,128] fp32 in place; RoPE on the slice at rope_offset with cos/sin row cs [n,64] */
void oracle_rope_rows(float* x, const float* cs, int64_t n, int rope_offset, int is_neox) {
    for (int64_t r = 0; r < n; ++r) rope_slice(x + r * HEAD_DIM + rope_offset, cs + r * ROPE_DIM, is_neox);
}

void oracle_fwht_rows(float* x, int64_t n) {
    for (int64_t r = 0; r < n; ++r) fwht128(x + r * HEAD_DIM);
}

void oracle_rmsnorm_rows(float* x, const uint16_t* gamma, float eps, int64_t n) {
    for (int64_t r = 0; r < n; ++r) rmsnorm128(x + r * HEAD_DIM, gamma, eps);
}

float oracle_hadamard_scale(void) { return hadamard_scale(); }

/* ------------------------------------------------------------------ */
/* public: FP4 paged MQA logits (the scorer that reads the producer's  */
/* bytes; [aiter-5484] intro and Verification: flydsl_pa_mqa_logits_fp4 */
/* scores q_out/q_scale_out against the paged cache, with the plain     */
/* weights and a separate fp32 scalar weights_scale).                   */
/* Readings (not stated on the pages): the logit of key s for query     */
/* token t is weights_scale * sum_h weights[t,h] * ReLU(q_h . k_s)      */
/* (ReLU optional); query j of a sequence with context length ctx sits  */
/* at position ctx - next_n + j and sees keys s <= that position, the   */
/* others get -inf; entries s >= ctx are not written; a block-table     */
/* entry outside [0, NB) gives -inf for its keys.                       */
/* Values are dequantized exactly and accumulated in double; abs_bound  */
/* (optional) receives |weights_scale| * sum_h |w| * sum_d |q_d k_d|,   */
/* the scale of any rounding error of an fp32 evaluation.               */
/* ------------------------------------------------------------------ */
int oracle_paged_mqa_logits(const uint8_t* q_out, const uint8_t* q_scale_out, const float* weights,
                            float weights_scale, const uint8_t* kv_cache,
                            const uint8_t* kv_cache_scale, int64_t NB, const int32_t* block_table,
                            int64_t max_blocks, const int32_t* context_lens, int64_t B, int next_n,
                            int H, int apply_relu, float* logits, int64_t stride,
                            double* abs_bound) {
    if (H <= 0 || H % 16 != 0 || next_n <= 0 || B < 0 || max_blocks < 0 || stride <= 0 || NB < 0)
        return ORC_EINVAL;
    const int J = ((H / 16) + 3) / 4 * 4;
    double kd[HEAD_DIM];
    /* the dequantized query heads of one token */
    double* qd = (double*)malloc(sizeof(double) * (size_t)H * HEAD_DIM);
    if (!qd) return ORC_EINVAL;
    for (int64_t b = 0; b < B; ++b) {
        int64_t ctx = context_lens[b];
        if (ctx < 0) ctx = 0;
        if (ctx > max_blocks * KV_BLOCK) ctx = max_blocks * KV_BLOCK;
        if (ctx > stride) ctx = stride;
        for (int j = 0; j < next_n; ++j) {
            const int64_t t = b * next_n + j;
            const int64_t pos = ctx - next_n + j;
            for (int h = 0; h < H; ++h)
                for (int d = 0; d < HEAD_DIM; ++d) {
                    int g = d / GROUP;
                    uint8_t byte = q_out[(t * H + h) * (HEAD_DIM / 2) + d / 2];
                    uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                    uint8_t e = q_scale_out[t * (int64_t)NGROUPS * 16 * J + (g * 16 + h % 16) * J + h / 16];
                    qd[h * HEAD_DIM + d] = (double)e2m1_value(nib) * (double)e8m0_value(e);
                }
            for (int64_t s = 0; s < ctx; ++s) {
                float* out = logits + t * stride + s;
                double* bnd = abs_bound ? abs_bound + t * stride + s : (double*)0;
                int32_t blk = block_table[b * max_blocks + s / KV_BLOCK];
                if (s > pos || blk < 0 || blk >= NB) {
                    *out = -INFINITY;
                    if (bnd) *bnd = 0.0;
                    continue;
                }
                const int64_t p = s % KV_BLOCK;
                for (int d = 0; d < HEAD_DIM; ++d) {
                    int g = d / GROUP;
                    uint8_t byte = kv_cache[(((int64_t)blk * NGROUPS + g) * KV_BLOCK + p) * 16 + (d % GROUP) / 2];
                    uint8_t nib = (d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                    uint8_t e = kv_cache_scale[((int64_t)blk * NGROUPS + g) * KV_BLOCK + (p % 16) * (KV_BLOCK / 16) + p / 16];
                    kd[d] = (double)e2m1_value(nib) * (double)e8m0_value(e);
                }
                double acc = 0.0, abs_acc = 0.0;
                for (int h = 0; h < H; ++h) {
                    double dot = 0.0, abs_dot = 0.0;
                    for (int d = 0; d < HEAD_DIM; ++d) {
                        double pr = qd[h * HEAD_DIM + d] * kd[d];
                        dot += pr;
                        abs_dot += fabs(pr);
                    }
                    double score = (apply_relu && dot < 0.0) ? 0.0 : dot;
                    double w = (double)weights[t * H + h];
                    acc += w * score;
                    abs_acc += fabs(w) * abs_dot;
                }
                *out = (float)((double)weights_scale * acc);
                if (bnd) *bnd = fabs((double)weights_scale) * abs_acc;
            }
        }
    }
    free(qd);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* sglang-compatible mode ([sglang-39656] Summary and review).          */
/* Two quantization stages with their own floors: stage 1 fake-quantizes */
/* each 32-group to the UE8M0 E2M1 grid (values, not codes); stage 2     */
/* (the packer) recomputes the exponent from the fake-quant            */
/* values with its own floor and packs codes whose sign bit is set only  */
/* when the magnitude code is nonzero (sign = (x < 0) & (idx != 0)).     */
/* Record: 64 code bytes then the 4 stage-2 exponents = 68 bytes.        */
/* ------------------------------------------------------------------ */
#define SLOT68 68

static void quantize_row_two_stage(const float* x, float floor1, float floor2, uint8_t* record) {
    for (int g = 0; g < NGROUPS; ++g) {
        const float* v = x + g * GROUP;
        int e1 = group_exponent(v, GROUP, floor1);
        float y[GROUP];
        for (int i = 0; i < GROUP; ++i) y[i] = e2m1_value(e2m1_nibble(v[i], e1)) * e8m0_value((uint8_t)e1);
        int e2 = group_exponent(y, GROUP, floor2);
        for (int b = 0; b < GROUP / 2; ++b) {
            uint8_t n[2];
            for (int q = 0; q < 2; ++q) {
                float yv = y[2 * b + q];
                uint8_t code = (uint8_t)(e2m1_nibble(yv, e2) & 7);
                uint8_t sign = (yv < 0.0f && code != 0) ? 1 : 0;
                n[q] = (uint8_t)((sign << 3) | code);
            }
            record[g * 16 + b] = (uint8_t)(n[0] | (n[1] << 4));
        }
        record[64 + g] = (uint8_t)e2;
    }
}

/* query side: record [t, h, 0:68] = two-stage codes of head h, then its 4 exponents */
int oracle_q_rope_pack_sglang(const uint16_t* q, const void* positions, int positions_int64,
                              const float* cos_sin, int64_t max_pos, int64_t T, int H, int D,
                              int R, int rope_offset, int group_size, int is_neox,
                              float fake_quant_floor, float pack_floor, uint8_t* q_packed) {
    if (check_shape(D, R, rope_offset, group_size) != ORC_OK) return ORC_EINVAL;
    if (H <= 0 || H % 16 != 0 || T < 0 || max_pos <= 0) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        int64_t pos = read_position(positions, positions_int64, t, max_pos);
        const float* cs_row = cos_sin + pos * ROPE_DIM;
        for (int h = 0; h < H; ++h) {
            float x[HEAD_DIM];
            for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_f32(q[(t * H + h) * HEAD_DIM + i]);
            rope_slice(x + rope_offset, cs_row, is_neox);
            quantize_row_two_stage(x, fake_quant_floor, pack_floor, q_packed + (t * H + h) * SLOT68);
        }
    }
    return ORC_OK;
}

/* key side: optional RMSNorm, RoPE, two stages, 68-byte record at slot; slot 0
   (and any slot outside [1, num_slots)) publishes nothing.  A compressed key
   row stands for compress_ratio consecutive tokens and is rotated at the
   first position of that group ([sglang-39656] Summary):
   pos - pos % compress_ratio. */
int oracle_k_rope_pack_store_sglang(const uint16_t* k, const void* positions, int positions_int64,
                                    const float* cos_sin, int64_t max_pos,
                                    const int64_t* slot_mapping, const uint16_t* k_norm_gamma,
                                    float k_norm_eps, int64_t T, int D, int R, int rope_offset,
                                    int group_size, int is_neox, int compress_ratio,
                                    float fake_quant_floor, float pack_floor,
                                    uint8_t* index_k_cache, int64_t num_slots) {
    if (check_shape(D, R, rope_offset, group_size) != ORC_OK) return ORC_EINVAL;
    if (num_slots < 0 || T < 0 || max_pos <= 0) return ORC_EINVAL;
    if (compress_ratio != 1 && compress_ratio != 2 && compress_ratio != 4) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        int64_t slot = slot_mapping[t];
        if (slot <= 0 || slot >= num_slots) continue;
        int64_t pos = read_position(positions, positions_int64, t, max_pos);
        pos -= pos % compress_ratio;    /* RoPE at the group's first position */
        float x[HEAD_DIM];
        for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_f32(k[t * HEAD_DIM + i]);
        if (k_norm_gamma) rmsnorm128(x, k_norm_gamma, k_norm_eps);
        rope_slice(x + rope_offset, cos_sin + pos * ROPE_DIM, is_neox);
        quantize_row_two_stage(x, fake_quant_floor, pack_floor, index_k_cache + slot * SLOT68);
    }
    return ORC_OK;
}

/* step-level: two-stage records of n rows of 128 (for the pins) */
void oracle_quantize_rows_two_stage(const float* x, int64_t n, float floor1, float floor2,
                                    uint8_t* records) {
    for (int64_t r = 0; r < n; ++r) quantize_row_two_stage(x + r * HEAD_DIM, floor1, floor2, records + r * SLOT68);
}

/* ------------------------------------------------------------------ */
/* FP8 output mode ([aiter-5484] API: the FP8 contract of the same op   */
/* folds its per-(token, head) q scale into weights_out, together with  */
/* weights_scale, which then rounds through q.dtype = bf16; scale_fmt   */
/* is ue8m0 or fp32.  [aiter-4029] review: the gfx950 FP8 format is     */
/* e4m3fn with a largest value of 448).                                 */
/* Readings: one scale per 128-row (a query head, a key token); scale   */
/* s = max(amax / 448, floor), under ue8m0 raised to a power of two by  */
/* the same (bits >> 23) + (mantissa != 0) rule as the FP4 exponent;    */
/* codes are the e4m3fn values nearest to x / s (ties to even, sign     */
/* kept on zero); keys go to kv_cache[slot, 0:128] with the fp32 scale  */
/* at kv_cache_scale[slot].                                             */
/* ------------------------------------------------------------------ */
#define FP8_MAX 448.0f

/* e4m3fn code of y.  Magnitudes: k * 2^-9 for codes k < 8 (subnormals),
   (8 + m) * 2^(E - 10) for code (E << 3) | m, E = 1..15, except code 0x7F
   (NaN).  Nearest value, ties to the even code; anything at or beyond 448,
   infinities included, saturates to 448 (0x7E).  A NaN y (inf / inf, when
   an infinite amax makes an fp32 scale infinite) is the format's NaN
   pattern with the sign bit clear, 0x7F: IEEE arithmetic leaves the sign of
   that NaN unspecified. */
static uint8_t e4m3_code(float y) {
    if (isnan(y)) return 0x7F;
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int code;
    if (a < ldexp(1.0, -6)) {
        const double k = a * 512.0;              /* exact */
        const double fk = floor(k);
        int ki = (int)fk;
        const double r = k - fk;
        if (r > 0.5 || (r == 0.5 && (ki & 1))) ki += 1;
        code = ki;                               /* 8 is the smallest normal */
    } else {
        int e;
        const double m = frexp(a, &e);           /* a = m * 2^e, m in [0.5, 1) */
        const double s = m * 16.0;               /* exact, in [8, 16) */
        const double fs = floor(s);
        int si = (int)fs;
        const double r = s - fs;
        if (r > 0.5 || (r == 0.5 && (si & 1))) si += 1;
        int E = e - 1 + 7;
        if (si == 16) { si = 8; E += 1; }
        code = (E << 3) | (si - 8);
    }
    return (uint8_t)(sign | code);
}

static float fp8_scale(float amax, float scale_floor, int ue8m0) {
    float s = amax / FP8_MAX;
    if (s < scale_floor) s = scale_floor;
    if (ue8m0) {
        uint32_t b = f2u(s);
        int e = (int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0);
        if (e < 1) e = 1;
        if (e > 254) e = 254;
        s = u2f((uint32_t)e << 23);
    }
    return s;
}

/* one 128-row: scale and the 128 codes */
static float quantize_row_fp8(const float* x, float scale_floor, int ue8m0, uint8_t* codes) {
    float amax = 0.0f;
    for (int i = 0; i < HEAD_DIM; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    const float s = fp8_scale(amax, scale_floor, ue8m0);
    for (int i = 0; i < HEAD_DIM; ++i) codes[i] = e4m3_code(x[i] / s);
    return s;
}

static int check_fp8_args(int scale_fmt, float scale_floor) {
    if (scale_fmt != 0 && scale_fmt != 1) return ORC_EINVAL;
    if (!(scale_floor >= 0.0f)) return ORC_EINVAL;
    if (scale_fmt == 1 && !(scale_floor > 0.0f)) return ORC_EINVAL;  /* s must be > 0 */
    return ORC_OK;
}

/* scale_fmt: 0 = ue8m0, 1 = fp32.  q_out u8 [T, H, 128]; weights_out bf16
   [T, H] = bf16((weights * s_q) * weights_scale). */
int oracle_q_rope_pack_fp8(const uint16_t* q, const void* positions, int positions_int64,
                           const float* cos_sin, int64_t max_pos, const float* weights,
                           float weights_scale, int64_t T, int H, int D, int R, int rope_offset,
                           int is_neox, int apply_hadamard, int scale_fmt, float scale_floor,
                           uint8_t* q_out, uint16_t* weights_out) {
    if (check_shape(D, R, rope_offset, GROUP) != ORC_OK) return ORC_EINVAL;
    if (check_fp8_args(scale_fmt, scale_floor) != ORC_OK) return ORC_EINVAL;
    if (H <= 0 || H % 16 != 0 || T < 0 || max_pos <= 0) return ORC_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        int64_t pos = read_position(positions, positions_int64, t, max_pos);
        const float* cs_row = cos_sin + pos * ROPE_DIM;
        for (int h = 0; h < H; ++h) {
            float x[HEAD_DIM];
            for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_f32(q[(t * H + h) * HEAD_DIM + i]);
            rope_hadamard_row(x, cs_row, rope_offset, is_neox, apply_hadamard);
            const float s = quantize_row_fp8(x, scale_floor, scale_fmt == 0,
                                             q_out + (t * H + h) * HEAD_DIM);
            const float w = weights[t * H + h] * s;
            weights_out[t * H + h] = f32_to_bf16_bits(w * weights_scale);
        }
    }
    return ORC_OK;
}

/* kv_cache u8 [NB, BS, 128]: token -> kv_cache[slot, :]; kv_cache_scale fp32
   [NB, BS]: its scale at [slot].  Slots outside [0, NB*BS) write nothing. */
int oracle_k_rope_pack_store_fp8(const uint16_t* k, const void* positions, int positions_int64,
                                 const float* cos_sin, int64_t max_pos,
                                 const int64_t* slot_mapping, const uint16_t* k_norm_gamma,
                                 float k_norm_eps, int64_t T, int D, int R, int rope_offset,
                                 int is_neox, int apply_hadamard, int scale_fmt,
                                 float scale_floor, uint8_t* kv_cache, float* kv_cache_scale,
                                 int64_t NB, int BS) {
    if (check_shape(D, R, rope_offset, GROUP) != ORC_OK) return ORC_EINVAL;
    if (check_fp8_args(scale_fmt, scale_floor) != ORC_OK) return ORC_EINVAL;
    if (BS != KV_BLOCK || NB < 0 || T < 0 || max_pos <= 0) return ORC_EINVAL;
    const int64_t nslots = NB * BS;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0 || slot >= nslots) continue;
        int64_t pos = read_position(positions, positions_int64, t, max_pos);
        float x[HEAD_DIM];
        for (int i = 0; i < HEAD_DIM; ++i) x[i] = bf16_to_f32(k[t * HEAD_DIM + i]);
        if (k_norm_gamma) rmsnorm128(x, k_norm_gamma, k_norm_eps);
        rope_hadamard_row(x, cos_sin + pos * ROPE_DIM, rope_offset, is_neox, apply_hadamard);
        kv_cache_scale[slot] = quantize_row_fp8(x, scale_floor, scale_fmt == 0,
                                                kv_cache + slot * HEAD_DIM);
    }
    return ORC_OK;
}

/* step-level, for the pins */
void oracle_e4m3_codes(const float* y, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = e4m3_code(y[i]);
}

void oracle_fp8_scales(const float* amax, int64_t n, float scale_floor, int ue8m0, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = fp8_scale(amax[i], scale_floor, ue8m0);
}

void oracle_quantize_rows_fp8(const float* x, int64_t n, float scale_floor, int ue8m0,
                              uint8_t* codes, float* scales) {
    for (int64_t r = 0; r < n; ++r)
        scales[r] = quantize_row_fp8(x + r * HEAD_DIM, scale_floor, ue8m0, codes + r * HEAD_DIM);
}

/* ------------------------------------------------------------------ */
/* RoPE tail + FP4 fake quant ([sglang-39656] Summary: the torch-shaped */
/* path rotates the tail, keeps the bf16 round trip, and fake-quantizes */
/* with per-32 UE8M0 scales by default or per-16 E4M3 scales for        */
/* compressed KV, rounding half to even).  Output: the bf16 values of   */
/* the quantized rows (code value times scale).                         */
/* Readings: row r uses positions[r / rows_per_position], rounded down  */
/* to a multiple of compress_ratio; the E4M3 scale of a 16-group is the */
/* e4m3fn value nearest to max(amax / 6, floor) (saturating at 448); a  */
/* zero scale gives signed zeros; codes are the E2M1 values nearest to  */
/* fl(x / s), ties to even, saturating at 6.                            */
/* ------------------------------------------------------------------ */
#define FQ_UE8M0_32 0
#define FQ_E4M3_16 1

static float e4m3_value(uint8_t c) {
    const int E = (c >> 3) & 15, m = c & 7;
    const float v = E == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), E - 10);
    return (c & 0x80) ? -v : v;
}

static void fake_quant_row(const float* x, int mode, float scale_floor, uint16_t* y) {
    if (mode == FQ_UE8M0_32) {
        for (int g = 0; g < NGROUPS; ++g) {
            const float* v = x + g * GROUP;
            const int e = group_exponent(v, GROUP, scale_floor);
            for (int i = 0; i < GROUP; ++i) {
                const float q = e2m1_value(e2m1_nibble(v[i], e)) * e8m0_value((uint8_t)e);
                y[g * GROUP + i] = f32_to_bf16_bits(q);
            }
        }
        return;
    }
    for (int g = 0; g < HEAD_DIM / 16; ++g) {
        const float* v = x + g * 16;
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) {
            float a = fabsf(v[i]);
            if (a > amax) amax = a;
        }
        float q = amax / 6.0f;
        if (q < scale_floor) q = scale_floor;
        const float s = e4m3_value(e4m3_code(q));
        for (int i = 0; i < 16; ++i) {
            float out;
            if (s == 0.0f) {
                out = copysignf(0.0f, v[i]);
            } else {
                const int code = e2m1_magnitude_code(fabsf(v[i] / s));
                out = copysignf(e2m1_value((uint8_t)code) * s, v[i]);
            }
            y[g * 16 + i] = f32_to_bf16_bits(out);
        }
    }
}

int oracle_rope_fake_quant(const uint16_t* x, int64_t rows, int rows_per_position,
                           const void* positions, int positions_int64, const float* cos_sin,
                           int64_t max_pos, int D, int R, int rope_offset, int is_neox,
                           int compress_ratio, int mode, float scale_floor, uint16_t* y) {
    if (check_shape(D, R, rope_offset, GROUP) != ORC_OK) return ORC_EINVAL;
    if (rows < 0 || rows_per_position <= 0 || max_pos <= 0) return ORC_EINVAL;
    if (compress_ratio != 1 && compress_ratio != 2 && compress_ratio != 4) return ORC_EINVAL;
    if (mode != FQ_UE8M0_32 && mode != FQ_E4M3_16) return ORC_EINVAL;
    if (!(scale_floor >= 0.0f)) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t pos = read_position(positions, positions_int64, r / rows_per_position, max_pos);
        pos -= pos % compress_ratio;
        float v[HEAD_DIM];
        for (int i = 0; i < HEAD_DIM; ++i) v[i] = bf16_to_f32(x[r * HEAD_DIM + i]);
        rope_slice(v + rope_offset, cos_sin + pos * ROPE_DIM, is_neox);
        fake_quant_row(v, mode, scale_floor, y + r * HEAD_DIM);
    }
    return ORC_OK;
}

/* step-level: fake quant of n rows of 128 (for the pins) */
void oracle_fake_quant_rows(const float* x, int64_t n, int mode, float scale_floor, uint16_t* y) {
    for (int64_t r = 0; r < n; ++r) fake_quant_row(x + r * HEAD_DIM, mode, scale_floor, y + r * HEAD_DIM);
}
