// fp4idx_modes.hip -- gfx950 kernels of the producer's other output modes:
// the sglang-compatible two-stage records (sgl-project/sglang PR 39656), the
// FP8 output mode (ROCm/aiter PR 5484 "API"), and the RoPE tail + FP4 fake
// quant of the torch-shaped path (sgl-project/sglang PR 39656 "Summary").
// The register layout and the shared helpers are in fp4idx_device.h.
#include "fp4idx_device.h"

namespace fp4idx {
namespace {

// ---- sglang-compatible mode --------------------------------------------------
// (sgl-project/sglang PR 39656 "Summary" and review.)  Each 32-group is
// quantized twice.  Stage 1 fake-quantizes to the UE8M0 E2M1 grid with its own
// floor: codes c1 under exponent e1, standing for the values
// y = val(c1) * 2^(e1-127).  Stage 2 (the packer) takes the exponent of the
// y's with the packer floor and packs their codes with the sign bit kept
// only on a nonzero magnitude (+0 codes).
//
// Stage 2 works on the codes, not on the y's.  The largest |y| is
// val(cmax) * 2^(e1-127) where cmax is the code of the stage-1 amax, and
// ceil_pow2(val/6) is 2^((cmax >> 1) - 3) for every nonzero code, so
//     e2 = max(e1 + (cmax >> 1) - 3, e_lo2)     (cmax > 0),   e_lo2 otherwise,
// and the stage-2 code of y is RNE(val(c1) / 2^(e2-e1)) on the E2M1 grid:
// the scaled converter applied to val(c1) (exact in bf16) with the
// power-of-two scale 2^(e2-e1).  One corner differs: for e1 >= 253 a y of
// magnitude >= 2^128 is +-inf in fp32, which makes the packer's amax infinite
// (e2 = 254) and its code 7.
__device__ __forceinline__ Q8 quant8_two_stage(uint4 v, int e_lo1, int e_lo2) {
    const u16x2_t a0 = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
    const u16x2_t a1 = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
    const u16x2_t a2 = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
    const u16x2_t a3 = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                 __builtin_elementwise_max(a2, a3));
    uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    const int e1 = m >= 0x7F80u ? 254 : max((int)((m + 0x3Fu) >> 7) - 2, e_lo1);
    const float scale1 = __uint_as_float((uint32_t)e1 << 23);
    // each converter writes one byte of its first operand; the four calls
    // overwrite all of it, so any dead value may seed the chain
    uint32_t c1 = v.x;
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c1, __builtin_bit_cast(bf16x2_t, v.x), scale1, 0);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c1, __builtin_bit_cast(bf16x2_t, v.y), scale1, 1);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c1, __builtin_bit_cast(bf16x2_t, v.z), scale1, 2);
    c1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(c1, __builtin_bit_cast(bf16x2_t, v.w), scale1, 3);
    const uint32_t cmax = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                              m, __builtin_bit_cast(bf16x2_t, m), scale1, 0) & 7u;
    // t = e1 + (cmax >> 1) - 3 for a nonzero cmax; -3 (below every floor)
    // when the whole group is zero.  A y overflows iff t >= 253.
    const int t = (cmax ? e1 : 0) + (int)(cmax >> 1) - 3;
    const bool ovf = t >= 253;
    const int e2 = max(ovf ? 254 : t, e_lo2);
    const int d = min(max(e2 - e1, -3), 8);  // beyond 8 every code is 0 either way
    const float scale2 = __uint_as_float((uint32_t)(127 + d) << 23);
    bf16x2_t y = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1, 1.0f, 0);
    uint32_t p = __builtin_bit_cast(uint32_t, y);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, y, scale2, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1, 1.0f, 1), scale2, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1, 1.0f, 2), scale2, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c1, 1.0f, 3), scale2, 3);
    if (ovf) {
        // nibbles whose y is infinite: (c >> 1) >= 3 for e1 = 253, >= 2 for e1 = 254
        const uint32_t hi = (c1 >> 2) & 0x11111111u;
        const uint32_t inf = (e1 >= 254) ? hi : (hi & (c1 >> 1));
        p = (p & ~(inf * 0xFu)) | (inf * 7u) | (c1 & (inf << 3));
    }
    // +0 codes: bit 4k of nz is set iff nibble k has a nonzero magnitude
    const uint32_t nz = (p | (p >> 1) | (p >> 2)) & 0x11111111u;
    p &= 0x77777777u | (nz << 3);
    return {p, e2};
}

// Query records [T, H, 68]: head h of token t is 64 code bytes, then its four
// stage-2 exponents as one dword.  Lane and load layout as q_split_token; the
// exponents of a head's four groups sit on the two quads of its 8 lanes and
// are merged into lane 0 of the 8 with one half-row mirror.  A 68-byte record
// never fills whole lines from one store instruction (streaming stores of the
// pieces measured ~18% slower than default-policy ones, which L2 merges), so
// the records of 64 heads are assembled in the wavefront's 4,352 bytes of
// LDS and written as 34 whole 128-byte lines with 16-byte streaming stores
// (a run of 64 records starts at a multiple of 64 x 68 bytes, and q_packed is
// 16-byte aligned): 505-511 -> 494-496 us at 131072 x 64 (497-499 with runs
// of 32; default-policy stores of the staged lines: 538-541).
template <bool NEOX>
__device__ __forceinline__ void q_sglang_token(const SQArgs& a, int64_t t, int lane,
                                               const float C[8], const float S[8],
                                               uint32_t* stage) {
    const int H = a.H;
    const int c = chunk_of(lane & 7);
    const int hsub = lane >> 3;
    const int ro = a.rope_offset;
    const int nro = 64 - ro;
    const int sh_rot = 8 * (ro / 32 + (c >> 2));
    const int sh_pln = 8 * (nro / 32 + (c >> 2));
    const bool writer = (lane & 7) == 0;
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    uint8_t* ot = reinterpret_cast<uint8_t*>(stage) + hsub * kSglangRecord + 4 * c;
    uint8_t* const out = a.q_packed + t * (int64_t)H * kSglangRecord;

    // one 16-head step: quantize the four loaded chunks, stage the records,
    // flush a full run of 64 heads (or the last 16-48)
    auto step = [&](int hb, uint4 p0, uint4 r0, uint4 p1, uint4 r1) {
        const Q8 qp0 = quant8_two_stage(p0, a.e_lo1, a.e_lo2);
        const Q8 qr0 = quant8_two_stage(rope8<NEOX>(r0, C, S), a.e_lo1, a.e_lo2);
        const Q8 qp1 = quant8_two_stage(p1, a.e_lo1, a.e_lo2);
        const Q8 qr1 = quant8_two_stage(rope8<NEOX>(r1, C, S), a.e_lo1, a.e_lo2);
        uint8_t* o = ot + (hb & 48) * kSglangRecord;
        store4_plain(o + nro / 2, qp0.codes);
        store4_plain(o + ro / 2, qr0.codes);
        store4_plain(o + 8 * kSglangRecord + nro / 2, qp1.codes);
        store4_plain(o + 8 * kSglangRecord + ro / 2, qr1.codes);
        uint32_t x0 = ((uint32_t)qp0.e << sh_pln) | ((uint32_t)qr0.e << sh_rot);
        uint32_t x1 = ((uint32_t)qp1.e << sh_pln) | ((uint32_t)qr1.e << sh_rot);
        x0 |= dpp<kDppHalfMirror>(x0);
        x1 |= dpp<kDppHalfMirror>(x1);
        if (writer) {  // c == 0 here, so o is the start of the head's record
            store4_plain(o + 64, x0);
            store4_plain(o + 8 * kSglangRecord + 64, x1);
        }
        if ((hb & 48) == 48 || hb + 16 >= H) {  // 64 heads (or the last 16-48) are staged
            wave_sync();
            const int h0 = hb & ~63;
            const int n16 = (hb + 16 - h0) * kSglangRecord / 16;  // 272, 204, 136 or 68
            const uint4* src = reinterpret_cast<const uint4*>(stage);
            for (int i = lane; i < n16; i += 64)
                store16_stream(out + h0 * kSglangRecord + 16 * i, src[i]);
            wave_sync();
        }
    };
    // Two register sets take turns: set A is computed while set B loads the
    // next 16 heads, then the roles swap.  (A single set copied from the
    // prefetch registers each step cost 16 moves per step.)
    auto load = [&](int hb, uint4& p0, uint4& r0, uint4& p1, uint4& r1) {
        const uint16_t* nx = qt + hb * 128;
        p0 = load16_stream(nx + nro);
        r0 = load16_stream(nx + ro);
        p1 = load16_stream(nx + 8 * 128 + nro);
        r1 = load16_stream(nx + 8 * 128 + ro);
    };
    uint4 ap0, ar0, ap1, ar1, bp0, br0, bp1, br1;
    load(0, ap0, ar0, ap1, ar1);
    for (int hb = 0; hb < H; hb += 32) {
        if (hb + 16 < H) load(hb + 16, bp0, br0, bp1, br1);
        step(hb, ap0, ar0, ap1, ar1);
        if (hb + 16 >= H) break;
        if (hb + 32 < H) load(hb + 32, ap0, ar0, ap1, ar1);
        step(hb + 16, bp0, br0, bp1, br1);
    }
}

// Registers held to 80 (the bound of six wavefronts per SIMD): the neox build
// would take 82; at 80 the compiler keeps one 8-byte value in scratch (reloaded
// twice per 32 heads).  With the launcher's four resident workgroups per CU the
// kernel ran at 425-427 us at 131072 x 64 against 489-492 without the bound
// (at full occupancy: 475.6 against 489.6; seven wavefronts, 72 VGPRs: 481).
template <bool NEOX>
__global__ __launch_bounds__(kBlock, 6) void q_sglang_kernel(SQArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= a.T) return;
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
    __shared__ __attribute__((aligned(16))) uint32_t stage[kWavesPerBlock][64 * kSglangRecord / 4];
    q_sglang_token<NEOX>(a, t, lane, C, S, stage[wave]);
}

// Key records [num_slots, 68]: 16 lanes per token as k_row_kernel.  Slot 0,
// like any slot outside [1, num_slots), publishes nothing.  A compressed key
// row (compress_ratio consecutive tokens) is rotated at the first position of
// its group.  The four group
// exponents are merged into lane 0 of the row (half-row mirror, then ror 8).
template <bool NEOX, bool NORM>
__global__ __launch_bounds__(kBlock) void k_sglang_kernel(SKArgs a) {
    const int lane16 = threadIdx.x & 15;
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4);
    if (t >= a.T) return;
    const int c = chunk_of(lane16);
    uint4 v = load16_stream(a.k + t * 128 + 8 * c);
    const int64_t slot = a.slot_mapping[t];
    // a compressed row is rotated at its group's first position (ratio 1, 2 or 4)
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos) &
                        ~(int64_t)(a.compress_ratio - 1);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, c & 7, C, S);
    if (slot <= 0 || slot >= a.nslots) return;
    if (NORM) {
        float G[8];
        unpack8(load16(a.gamma + 8 * c), G);
        v = rmsnorm8(v, G, a.eps);
    }
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    v = select4(rot_lane, rope8<NEOX>(v, C, S), v);
    const Q8 q = quant8_two_stage(v, a.e_lo1, a.e_lo2);
    uint8_t* rec = a.index_k_cache + slot * kSglangRecord;
    *reinterpret_cast<uint32_t*>(rec + 4 * c) = q.codes;
    uint32_t x = (uint32_t)q.e << (8 * (c >> 2));
    x |= dpp<kDppHalfMirror>(x);
    x |= dpp<kDppRor8>(x);
    if (lane16 == 0) *reinterpret_cast<uint32_t*>(rec + 64) = x;
}

// ---- FP8 output mode ----------------------------------------------------------
// (ROCm/aiter PR 5484 "API": the FP8 contract of the same op, with its
// per-(token, head) q scale folded into weights_out together with
// weights_scale; scale_fmt ue8m0 or fp32.  ROCm/aiter PR 4029 review: e4m3fn,
// largest value 448, on gfx950.)  One scale per 128-row (a query head, a key
// token): s = max(amax / 448, floor), raised to a power of two under ue8m0;
// codes are the e4m3fn values nearest to x / s, ties to even, sign kept on
// zero.  A row is the 16 lanes of a DPP row (lane chunk c = chunk_of(lane16)),
// so its amax takes four DPP steps.
//
// ue8m0: the scaled converter divides by the power-of-two scale exactly.
// fp32: x / s rounded to fp32 first (the value the converter then rounds),
// computed as y0 = x * r, y = fma(fma(-y0, s, x), r, y0) with r = RN(1/s)
// (the correctly rounded fp32 reciprocal);
// for every bf16 x and normal fp32 s this equals RN(x / s) -- checked
// exhaustively over all 2^30 significand pairs on the CPU.
__device__ __forceinline__ void store8_stream(void* p, uint2 v) {
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
    return pack_bf16x2(x, 0.0f) & 0xFFFFu;
}

// A row whose amax is infinite (a rotated or normalised value past the fp32
// range) has an infinite amax / 448 (the division sequence below would give
// NaN), so under fp32 scales s = inf and under ue8m0 s = 2^127 (e = 254).
// Its codes:
//   ue8m0: the converter turns +-inf into the NaN code (0x7F / 0xFF) while
//     every value at or beyond 448 saturates to 448, so bytes 0x7F / 0xFF
//     become 0x7E / 0xFE.  A finite x never meets the NaN code here (s >=
//     amax / 448 keeps |x| / s <= 448), so rows with s = 2^127 are patched
//     whether or not they hold an infinity.  (t + 1 reaches bit 7 of a byte
//     exactly when its low seven bits are all set, with no carry into the
//     next byte.)
//   fp32: x / inf is +-0 for a finite x (0x00 / 0x80) and NaN for an infinite
//     one (0x7F); w0, w1 hold four bf16 values, the result their codes.
constexpr uint32_t kUe8m0MaxScaleBits = 254u << 23;  // 2^127

__device__ __forceinline__ uint32_t saturate_nan_codes(uint32_t d) {
    const uint32_t t = d & 0x7F7F7F7Fu;
    return d ^ (((t + 0x01010101u) & 0x80808080u) >> 7);
}

__device__ __forceinline__ uint32_t infinite_scale_codes(uint32_t w0, uint32_t w1) {
    const uint32_t h[4] = {w0 & 0xFFFFu, w0 >> 16, w1 & 0xFFFFu, w1 >> 16};
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r |= ((h[i] & 0x7FFFu) >= 0x7F80u ? 0x7Fu : (h[i] >> 8) & 0x80u) << (8 * i);
    return r;
}

__device__ __forceinline__ float fp8_amax_over_448(uint32_t m) {
    return m >= 0x7F80u ? __builtin_huge_valf()
                        : div_const_rn(__uint_as_float(m << 16), 448.0f, kRcp448);
}

template <bool FP32>
__device__ __forceinline__ uint2 quant_fp8_row(uint4 v, float scale_floor, float& s_out) {
    const u16x2_t a0 = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
    const u16x2_t a1 = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
    const u16x2_t a2 = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
    const u16x2_t a3 = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                 __builtin_elementwise_max(a2, a3));
    uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    m = max(m, dpp<kDppHalfMirror>(m));
    m = max(m, dpp<kDppRor8>(m));
    float s = fp8_amax_over_448(m);
    s = s < scale_floor ? scale_floor : s;
    s16x2_t lo = {0, 0}, hi = {0, 0};
    if (!FP32) {
        const uint32_t b = __float_as_uint(s);
        const int e = min(max((int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0), 1), 254);
        s = __uint_as_float((uint32_t)e << 23);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, v.x), s, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, v.y), s, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, v.z), s, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, v.w), s, true);
        if (__float_as_uint(s) == kUe8m0MaxScaleBits) {
            lo = __builtin_bit_cast(s16x2_t, saturate_nan_codes(__builtin_bit_cast(uint32_t, lo)));
            hi = __builtin_bit_cast(s16x2_t, saturate_nan_codes(__builtin_bit_cast(uint32_t, hi)));
        }
    } else if (s == __builtin_huge_valf()) {
        lo = __builtin_bit_cast(s16x2_t, infinite_scale_codes(v.x, v.y));
        hi = __builtin_bit_cast(s16x2_t, infinite_scale_codes(v.z, v.w));
    } else {
        const float r = __frcp_rn(s);  // RN(1/s)
        float x[8], y[8];
        unpack8(v, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float y0 = x[e] * r;
            const float err = __builtin_fmaf(-y0, s, x[e]);
            // s > 0, so the quotient has the sign of x; the correction alone
            // would turn -0 into +0
            y[e] = __builtin_copysignf(__builtin_fmaf(err, r, y0), x[e]);
        }
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[0], y[1], 1.0f, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], 1.0f, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[4], y[5], 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[6], y[7], 1.0f, true);
    }
    s_out = s;
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Query: one token per wavefront, 16 lanes per head, 16 heads per step (four
// 16-byte loads per lane, all issued before any compute: 533 -> 517 us at
// 131072 x 64 against 8 heads per step; 32 heads per step measured slower).
// q_out rows are 128 bytes, written by the 16 lanes of the head with 8-byte
// streaming stores; lane 0 of each head writes the folded weight.
template <bool NEOX, bool HAD, bool FP32>
__global__ __launch_bounds__(kBlock) void q_fp8_kernel(FQArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= a.T) return;
    const int H = a.H;
    const int c = chunk_of(lane & 15);
    const int hsub = lane >> 4;
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, c & 7, C, S);
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    uint8_t* ot = a.q_out + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    const float* wt = a.weights + t * H;
    uint16_t* wo = a.weights_out + t * H;
    for (int hb = 0; hb < H; hb += 16) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = load16_stream(qt + (hb + 4 * u) * 128);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint4 w = select4(rot_lane, rope8<NEOX>(v[u], C, S), v[u]);
            if (HAD) w = hadamard8(w, c);
            float s;
            const uint2 q = quant_fp8_row<FP32>(w, a.scale_floor, s);
            store8_stream(ot + (hb + 4 * u) * 128, q);
            if ((lane & 15) == 0) {
                const int h = hb + 4 * u + hsub;
                wo[h] = (uint16_t)bf16_bits((wt[h] * s) * a.weights_scale);
            }
        }
    }
}

// Query with fp32 scales and no Hadamard: the split layout of the FP4 query kernel -- 8
// lanes per half-head, lane chunk c = chunk_of(lane & 7), the plain and the
// rotated halves in separate registers (no lane computes a RoPE it discards),
// 16 heads per step with the next step's loads in flight.  A head's amax is
// the in-lane max of both halves, then quad xor 1, xor 2 and the half-row
// mirror.  Each half goes out as 64 bytes per head (8-byte streaming stores).
template <bool FP32>
__device__ __forceinline__ float fp8_head_scale(uint4 p, uint4 r, float scale_floor) {
    const u16x2_t a0 = __builtin_bit_cast(u16x2_t, p.x & 0x7FFF7FFFu);
    const u16x2_t a1 = __builtin_bit_cast(u16x2_t, p.y & 0x7FFF7FFFu);
    const u16x2_t a2 = __builtin_bit_cast(u16x2_t, p.z & 0x7FFF7FFFu);
    const u16x2_t a3 = __builtin_bit_cast(u16x2_t, p.w & 0x7FFF7FFFu);
    const u16x2_t b0 = __builtin_bit_cast(u16x2_t, r.x & 0x7FFF7FFFu);
    const u16x2_t b1 = __builtin_bit_cast(u16x2_t, r.y & 0x7FFF7FFFu);
    const u16x2_t b2 = __builtin_bit_cast(u16x2_t, r.z & 0x7FFF7FFFu);
    const u16x2_t b3 = __builtin_bit_cast(u16x2_t, r.w & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_elementwise_max(
        __builtin_elementwise_max(__builtin_elementwise_max(a0, a1), __builtin_elementwise_max(a2, a3)),
        __builtin_elementwise_max(__builtin_elementwise_max(b0, b1), __builtin_elementwise_max(b2, b3)));
    uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    m = max(m, dpp<kDppHalfMirror>(m));
    float s = fp8_amax_over_448(m);
    s = s < scale_floor ? scale_floor : s;
    if (!FP32) {
        const uint32_t b = __float_as_uint(s);
        const int e = min(max((int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0), 1), 254);
        s = __uint_as_float((uint32_t)e << 23);
    }
    return s;
}

template <bool FP32>
__device__ __forceinline__ uint2 fp8_codes8(uint4 v, float s, float r) {
    s16x2_t lo = {0, 0}, hi = {0, 0};
    if (!FP32) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, v.x), s, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, __builtin_bit_cast(bf16x2_t, v.y), s, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, v.z), s, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, __builtin_bit_cast(bf16x2_t, v.w), s, true);
        if (__float_as_uint(s) == kUe8m0MaxScaleBits) {
            lo = __builtin_bit_cast(s16x2_t, saturate_nan_codes(__builtin_bit_cast(uint32_t, lo)));
            hi = __builtin_bit_cast(s16x2_t, saturate_nan_codes(__builtin_bit_cast(uint32_t, hi)));
        }
    } else if (s == __builtin_huge_valf()) {
        lo = __builtin_bit_cast(s16x2_t, infinite_scale_codes(v.x, v.y));
        hi = __builtin_bit_cast(s16x2_t, infinite_scale_codes(v.z, v.w));
    } else {
        float x[8], y[8];
        unpack8(v, x);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float y0 = x[e] * r;
            const float err = __builtin_fmaf(-y0, s, x[e]);
            y[e] = __builtin_copysignf(__builtin_fmaf(err, r, y0), x[e]);
        }
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[0], y[1], 1.0f, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, y[2], y[3], 1.0f, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[4], y[5], 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, y[6], y[7], 1.0f, true);
    }
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

template <bool NEOX, bool FP32>
__device__ __forceinline__ void fp8_split_head(const FQArgs& a, uint4 p, uint4 r, int64_t t, int h,
                                               int c, const float C[8], const float S[8]) {
    const int ro = a.rope_offset;
    const uint4 x = rope8<NEOX>(r, C, S);
    const float s = fp8_head_scale<FP32>(p, x, a.scale_floor);
    const float rc = FP32 ? __frcp_rn(s) : 0.0f;
    uint8_t* o = a.q_out + (t * a.H + h) * 128 + 8 * c;
    store8_stream(o + 64 - ro, fp8_codes8<FP32>(p, s, rc));
    store8_stream(o + ro, fp8_codes8<FP32>(x, s, rc));
    if (c == 0)
        a.weights_out[t * a.H + h] = (uint16_t)bf16_bits((a.weights[t * a.H + h] * s) * a.weights_scale);
}

template <bool NEOX>
__global__ __launch_bounds__(kBlock) void q_fp8_split_kernel(FQArgs a) {
    constexpr bool FP32 = true;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= a.T) return;
    const int H = a.H;
    const int c = chunk_of(lane & 7);
    const int hsub = lane >> 3;
    const int ro = a.rope_offset;
    const int nro = 64 - ro;
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, c, C, S);
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    // two load-register sets take turns (no per-step copy of a prefetch set)
    auto load = [&](int hb, uint4& p0, uint4& r0, uint4& p1, uint4& r1) {
        const uint16_t* nx = qt + hb * 128;
        p0 = load16_stream(nx + nro);
        r0 = load16_stream(nx + ro);
        p1 = load16_stream(nx + 8 * 128 + nro);
        r1 = load16_stream(nx + 8 * 128 + ro);
    };
    auto step = [&](int hb, uint4 p0, uint4 r0, uint4 p1, uint4 r1) {
        fp8_split_head<NEOX, FP32>(a, p0, r0, t, hb + hsub, c, C, S);
        fp8_split_head<NEOX, FP32>(a, p1, r1, t, hb + 8 + hsub, c, C, S);
    };
    uint4 ap0, ar0, ap1, ar1, bp0, br0, bp1, br1;
    load(0, ap0, ar0, ap1, ar1);
    for (int hb = 0; hb < H; hb += 32) {
        if (hb + 16 < H) load(hb + 16, bp0, br0, bp1, br1);
        step(hb, ap0, ar0, ap1, ar1);
        if (hb + 16 >= H) break;
        if (hb + 32 < H) load(hb + 32, ap0, ar0, ap1, ar1);
        step(hb + 16, bp0, br0, bp1, br1);
    }
}

// Key: 16 lanes per row as k_row_kernel; the row's 128 code bytes go to
// kv_cache[slot] and its scale to kv_cache_scale[slot].
template <bool NEOX, bool NORM, bool HAD, bool FP32>
__global__ __launch_bounds__(kBlock) void k_fp8_kernel(FKArgs a) {
    const int lane16 = threadIdx.x & 15;
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4);
    if (t >= a.T) return;
    const int c = chunk_of(lane16);
    uint4 v = load16_stream(a.k + t * 128 + 8 * c);
    const int64_t slot = a.slot_mapping[t];
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, c & 7, C, S);
    if (slot < 0 || slot >= a.nslots) return;
    if (NORM) {
        float G[8];
        unpack8(load16(a.gamma + 8 * c), G);
        v = rmsnorm8(v, G, a.eps);
    }
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    v = select4(rot_lane, rope8<NEOX>(v, C, S), v);
    if (HAD) v = hadamard8(v, c);
    float s;
    const uint2 q = quant_fp8_row<FP32>(v, a.scale_floor, s);
    *reinterpret_cast<uint2*>(a.kv_cache + slot * 128 + 8 * c) = q;
    if (lane16 == 0) a.kv_cache_scale[slot] = s;
}

// ---- RoPE tail + FP4 fake quant ----------------------------------------------
// (sgl-project/sglang PR 39656 "Summary": the torch-shaped path rotates the
// tail with the bf16 round trip and fake-quantizes with per-32 UE8M0 scales
// by default or per-16 E4M3 scales for compressed KV, round half to even.)
// Output: the bf16 values of the quantized rows.  16 lanes per 128-row
// (lane chunk c = chunk_of(lane16)), 16 rows per block.
//   UE8M0/32: the main quantizer, then code value * 2^(e-127) in fp32 (a
//     product of magnitude >= 2^128 is inf, as in fp32) and bf16 (exact).
//   E4M3/16: a 16-group is chunks 2j, 2j+1 = lanes L, L^1.  s = e4m3fn(
//     max(amax/6, floor)) through the FP8 converter (saturated at 448 first);
//     codes of fl(x/s) (reciprocal + FMA correction, exact as in the FP8
//     path), clamped to 6 before the FP4 converter; value = code value * s,
//     exact in fp32 and in bf16.  A zero scale gives signed zeros.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t E = (c >> 3) & 15u, m = c & 7u;
    return E == 0 ? (float)m * 0.001953125f  // m * 2^-9
                  : __uint_as_float(((E + 120u) << 23) | (m << 20));
}

// value of code byte B's two nibbles (exact bf16 grid values at scale 1), times
// `scale` in fp32
template <int B>
__device__ __forceinline__ void scaled_pair(uint32_t codes, float scale, float* out) {
    const uint32_t g = __builtin_bit_cast(uint32_t,
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, 1.0f, B));
    out[2 * B] = __uint_as_float(g << 16) * scale;
    out[2 * B + 1] = __uint_as_float(g & 0xFFFF0000u) * scale;
}

__device__ __forceinline__ void scaled_codes(uint32_t codes, float scale, float out[8]) {
    scaled_pair<0>(codes, scale, out);
    scaled_pair<1>(codes, scale, out);
    scaled_pair<2>(codes, scale, out);
    scaled_pair<3>(codes, scale, out);
}

template <int MODE>
__device__ __forceinline__ uint4 fake_quant8(uint4 v, int e_lo, float scale_floor) {
    float val[8];
    if (MODE == 0) {
        const Q8 q = quant8(v, e_lo);
        const float sc = __uint_as_float((uint32_t)q.e << 23);
        scaled_codes(q.codes, sc, val);
    } else {
        const u16x2_t a0 = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
        const u16x2_t a1 = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
        const u16x2_t a2 = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
        const u16x2_t a3 = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
        const u16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                     __builtin_elementwise_max(a2, a3));
        uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
        m = max(m, dpp<kDppXor1>(m));
        float qs = div_const_rn(__uint_as_float(m << 16), 6.0f, kRcp6);
        qs = qs < scale_floor ? scale_floor : qs;
        qs = qs < 448.0f ? qs : 448.0f;
        const s16x2_t sc8 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2_t{0, 0}, qs, qs, 1.0f,
                                                                     false);
        const float s = e4m3_to_f32(__builtin_bit_cast(uint32_t, sc8) & 0xFFu);
        float x[8];
        unpack8(v, x);
        if (s == 0.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) val[e] = __builtin_copysignf(0.0f, x[e]);
        } else {
            // RN(1/s): s is an e4m3fn value (at most 4 significant bits); one
            // Newton step from any reciprocal within 2 ulp of RN(1/s) lands on
            // it (checked on the CPU for every positive finite e4m3fn value),
            // and the hardware reciprocal is within 1 ulp
            const float r0 = __builtin_amdgcn_rcpf(s);
            const float r = __builtin_fmaf(r0, __builtin_fmaf(-s, r0, 1.0f), r0);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y0 = x[e] * r;
                const float err = __builtin_fmaf(-y0, s, x[e]);
                const float q = __builtin_fmaf(err, r, y0);
                y[e] = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(q), 6.0f), x[e]);
            }
            uint32_t codes = __float_as_uint(y[0]);  // all four bytes are overwritten
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[0], y[1], 1.0f, 0);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[2], y[3], 1.0f, 1);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[4], y[5], 1.0f, 2);
            codes = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(codes, y[6], y[7], 1.0f, 3);
            scaled_codes(codes, s, val);
        }
    }
    return pack8(val);
}

// One row per 16 lanes, for rows_per_position < 4 (keys: one row per position).
template <bool NEOX, int MODE>
__global__ __launch_bounds__(kBlock) void fake_quant_kernel(FakeQArgs a) {
    const int lane16 = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4);
    if (row >= a.rows) return;
    const int c = chunk_of(lane16);
    const uint4 v = load16_stream(a.x + row * 128 + 8 * c);
    const int64_t pidx = a.rows_per_position == 1 ? row : row / a.rows_per_position;
    const int64_t pos = clamped_position(a.positions, a.pos64, pidx, a.max_pos) &
                        ~(int64_t)(a.compress_ratio - 1);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, c & 7, C, S);
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    const uint4 w = select4(rot_lane, rope8<NEOX>(v, C, S), v);
    const uint4 y = fake_quant8<MODE>(w, a.e_lo, a.scale_floor);
    store16_stream(a.y + row * 128 + 8 * c, y);
}

// One position per wavefront for rows_per_position >= 4 (queries: the H heads
// of a token): the RoPE coefficients are formed once.  Each step handles 16
// rows while they fit (four 16-byte loads per lane, lanes 16k..16k+15 on rows
// k, k+4, k+8, k+12: 798 -> 787 us at 8.4 M rows against 8 rows per step),
// then 8 rows (rows k and k+4).  A row past the token's last leaves as a
// whole 16-lane group, so every DPP pattern still reads lanes of its own row.
template <bool NEOX, int MODE>
__global__ __launch_bounds__(kBlock) void fake_quant_token_kernel(FakeQArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t r0 = t * a.rows_per_position;
    if (r0 >= a.rows) return;
    const int64_t r_end = min(r0 + a.rows_per_position, a.rows);
    const int c = chunk_of(lane & 15);
    const int rsub = lane >> 4;
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos) &
                        ~(int64_t)(a.compress_ratio - 1);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, c & 7, C, S);
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    int64_t rb = r0;
    for (; rb + 16 <= r_end; rb += 16) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = load16_stream(a.x + (rb + rsub + 4 * u) * 128 + 8 * c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint4 y = fake_quant8<MODE>(select4(rot_lane, rope8<NEOX>(v[u], C, S), v[u]),
                                              a.e_lo, a.scale_floor);
            store16_stream(a.y + (rb + rsub + 4 * u) * 128 + 8 * c, y);
        }
    }
    for (; rb < r_end; rb += 8) {
        const int64_t ra = rb + rsub, rc = ra + 4;
        if (rc < r_end) {
            const uint4 v0 = load16_stream(a.x + ra * 128 + 8 * c);
            const uint4 v1 = load16_stream(a.x + rc * 128 + 8 * c);
            const uint4 y0 = fake_quant8<MODE>(select4(rot_lane, rope8<NEOX>(v0, C, S), v0),
                                               a.e_lo, a.scale_floor);
            const uint4 y1 = fake_quant8<MODE>(select4(rot_lane, rope8<NEOX>(v1, C, S), v1),
                                               a.e_lo, a.scale_floor);
            store16_stream(a.y + ra * 128 + 8 * c, y0);
            store16_stream(a.y + rc * 128 + 8 * c, y1);
        } else if (ra < r_end) {
            const uint4 v0 = load16_stream(a.x + ra * 128 + 8 * c);
            const uint4 y0 = fake_quant8<MODE>(select4(rot_lane, rope8<NEOX>(v0, C, S), v0),
                                               a.e_lo, a.scale_floor);
            store16_stream(a.y + ra * 128 + 8 * c, y0);
        }
    }
}

}  // namespace

hipError_t launch_q_rope_pack_sglang(const SQArgs& a, bool is_neox, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kWavesPerBlock - 1) / kWavesPerBlock;
    // four workgroups per compute unit: 421-427 against 474-478 us at 131072 x 64
    // with the six that the registers allow (three: 429-438, two: 540)
    if (is_neox)
        return launch(q_sglang_kernel<true>, blocks,
                      resident_cap_lds(reinterpret_cast<const void*>(q_sglang_kernel<true>), 0, 4),
                      stream, a);
    return launch(q_sglang_kernel<false>, blocks,
                  resident_cap_lds(reinterpret_cast<const void*>(q_sglang_kernel<false>), 0, 4),
                  stream, a);
}

hipError_t launch_k_rope_pack_store_sglang(const SKArgs& a, bool is_neox, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kBlock / 16 - 1) / (kBlock / 16);
    const bool norm = a.gamma != nullptr;
    if (is_neox)
        return norm ? launch(k_sglang_kernel<true, true>, blocks, 0, stream, a)
                    : launch(k_sglang_kernel<true, false>, blocks, 0, stream, a);
    return norm ? launch(k_sglang_kernel<false, true>, blocks, 0, stream, a)
                : launch(k_sglang_kernel<false, false>, blocks, 0, stream, a);
}

hipError_t launch_q_rope_pack_fp8(const FQArgs& a, bool is_neox, bool hadamard, bool fp32_scale,
                                  hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kWavesPerBlock - 1) / kWavesPerBlock;
    // fp32 scales without the Hadamard: the split layout, whose saved RoPE work
    // pays for the per-element division (599 -> 565 us at 131072 x 64); with
    // ue8m0 scales the 16-lane layout's 512-byte store runs win (530 vs 538 us)
    if (!hadamard && fp32_scale)
        return is_neox ? launch(q_fp8_split_kernel<true>, blocks, 0, stream, a)
                       : launch(q_fp8_split_kernel<false>, blocks, 0, stream, a);
    const int sel = (is_neox ? 4 : 0) | (hadamard ? 2 : 0) | (fp32_scale ? 1 : 0);
    switch (sel) {
        case 0: return launch(q_fp8_kernel<false, false, false>, blocks, 0, stream, a);
        case 1: return launch(q_fp8_kernel<false, false, true>, blocks, 0, stream, a);
        case 2: return launch(q_fp8_kernel<false, true, false>, blocks, 0, stream, a);
        case 3: return launch(q_fp8_kernel<false, true, true>, blocks, 0, stream, a);
        case 4: return launch(q_fp8_kernel<true, false, false>, blocks, 0, stream, a);
        case 5: return launch(q_fp8_kernel<true, false, true>, blocks, 0, stream, a);
        case 6: return launch(q_fp8_kernel<true, true, false>, blocks, 0, stream, a);
        default: return launch(q_fp8_kernel<true, true, true>, blocks, 0, stream, a);
    }
}

template <bool NEOX, bool NORM>
hipError_t launch_k_fp8(const FKArgs& a, bool hadamard, bool fp32_scale, int64_t blocks,
                        hipStream_t stream) {
    if (hadamard)
        return fp32_scale ? launch(k_fp8_kernel<NEOX, NORM, true, true>, blocks, 0, stream, a)
                          : launch(k_fp8_kernel<NEOX, NORM, true, false>, blocks, 0, stream, a);
    return fp32_scale ? launch(k_fp8_kernel<NEOX, NORM, false, true>, blocks, 0, stream, a)
                      : launch(k_fp8_kernel<NEOX, NORM, false, false>, blocks, 0, stream, a);
}

hipError_t launch_k_rope_pack_store_fp8(const FKArgs& a, bool is_neox, bool hadamard,
                                        bool fp32_scale, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kBlock / 16 - 1) / (kBlock / 16);
    const bool norm = a.gamma != nullptr;
    if (is_neox)
        return norm ? launch_k_fp8<true, true>(a, hadamard, fp32_scale, blocks, stream)
                    : launch_k_fp8<true, false>(a, hadamard, fp32_scale, blocks, stream);
    return norm ? launch_k_fp8<false, true>(a, hadamard, fp32_scale, blocks, stream)
                : launch_k_fp8<false, false>(a, hadamard, fp32_scale, blocks, stream);
}

hipError_t launch_rope_fake_quant(const FakeQArgs& a, bool is_neox, int mode, hipStream_t stream) {
    if (a.rows == 0) return hipSuccess;
    if (a.rows_per_position >= 4) {
        const int64_t npos = (a.rows + a.rows_per_position - 1) / a.rows_per_position;
        const int64_t blocks = (npos + kWavesPerBlock - 1) / kWavesPerBlock;
        if (mode == 0)
            return is_neox ? launch(fake_quant_token_kernel<true, 0>, blocks, 0, stream, a)
                           : launch(fake_quant_token_kernel<false, 0>, blocks, 0, stream, a);
        return is_neox ? launch(fake_quant_token_kernel<true, 1>, blocks, 0, stream, a)
                       : launch(fake_quant_token_kernel<false, 1>, blocks, 0, stream, a);
    }
    const int64_t blocks = (a.rows + kBlock / 16 - 1) / (kBlock / 16);
    if (mode == 0)
        return is_neox ? launch(fake_quant_kernel<true, 0>, blocks, 0, stream, a)
                       : launch(fake_quant_kernel<false, 0>, blocks, 0, stream, a);
    return is_neox ? launch(fake_quant_kernel<true, 1>, blocks, 0, stream, a)
                   : launch(fake_quant_kernel<false, 1>, blocks, 0, stream, a);
}

}  // namespace fp4idx
