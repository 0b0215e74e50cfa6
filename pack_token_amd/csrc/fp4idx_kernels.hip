// fp4idx_kernels.hip -- gfx950 kernels of the fused FP4 indexer producer.
//
// What is computed (per token; ROCm/aiter PR 5484 "API" and "One deliberate
// deviation", sgl-project/sglang PR 39656 "Summary" and review, ROCm/aiter
// PR 4029 "Changes"):
//   optional key RMSNorm -> RoPE on a 64-wide slice (bf16 round trip) ->
//   optional 128-point Hadamard (bf16) -> per 32-group UE8M0 exponent ->
//   E2M1 codes (RNE, sign kept on zero) -> two codes per byte -> q_out /
//   q_scale_out / weights_out, or the paged key cache and its interleaved
//   scale row.
//
// Data layout in registers.  A 128-dim bf16 row is 16 chunks of 8 values
// (16 bytes).  Every lane loads one chunk with a 16-byte load.  Lanes are
// mapped to chunks so that every cross-lane step of the method is a single
// DPP lane pattern that can be fused into the consuming VALU op:
//     chunk(L) = L ^ (bit2(L) ? 3 : 0)          (L = lane within 16)
// so chunk c ^ 1 sits at lane L ^ 1 (DPP quad_perm), c ^ 2 at L ^ 2
// (quad_perm), c ^ 4 at L ^ 7 (row_half_mirror) and c ^ 8 at L ^ 8
// (row_ror:8).  The 4 chunks of a 32-group are always one quad of lanes,
// the neox RoPE partner (slice element i <-> i+32, i.e. chunk c ^ 4) is the
// half-row mirror, and the Hadamard strides 8/16/32/64 and the RMSNorm
// fold-by-halves steps map to the four patterns above.
//
// Nothing here is a dense contraction, so there is no MFMA: the path is
// bound by HBM bandwidth, and the kernels are written to stream q once with
// 16-byte loads and to issue no more VALU work than the stream can hide.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4idx_internal.h"

namespace fp4idx {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x2_t __attribute__((ext_vector_type(2)));

// DPP lane patterns (CDNA data-parallel primitives).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]: lane i <- i ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]: lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141; // row_half_mirror: lane i <- i ^ 7 (within 8)
constexpr int kDppRor8 = 0x128;       // row_ror:8: lane i <- i ^ 8 (within 16)

constexpr int kWavesPerBlock = 4;
constexpr int kBlock = 64 * kWavesPerBlock;

// fp32(1/sqrt(128)), the orthonormal Hadamard scale.
constexpr uint32_t kHadamardScaleBits = 0x3DB504F3u;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __uint_as_float(dpp<CTRL>(__float_as_uint(v)));
}

__device__ __forceinline__ int chunk_of(int lane16) {
    return lane16 ^ (((lane16 >> 2) & 1) * 3);
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint4 load16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Streaming (non-temporal) accesses for data touched exactly once: q, k and
// the query code bytes.  They set the nt cache-policy bit so the lines do not
// displace anything in L2; on MI355X this raises the query kernel from
// ~5.4 to ~6.5 TB/s.  The small per-token rows (weights, scales) and the key
// cache writes keep the default policy, which measured faster for them.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load16_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store16_stream(void* p, uint4 v) {
    const u32x4_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ void store4_plain(void* p, uint32_t v) {
    *reinterpret_cast<uint32_t*>(p) = v;
}

__device__ __forceinline__ void store4_stream(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ---- bf16 <-> fp32 ---------------------------------------------------------

__device__ __forceinline__ void unpack8(uint4 v, float x[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// two fp32 -> packed bf16x2 (a in the low half), round to nearest even
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint4 pack8(const float x[8]) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                      pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}

__device__ __forceinline__ uint4 select4(bool c, uint4 a, uint4 b) {
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// ---- quantizer ---------------------------------------------------------------
// UE8M0 exponent of a group whose largest |value| is the bf16 number with
// magnitude bits m: the least e with amax <= 6 * 2^(e-127), which equals the
// biased exponent of ceil_pow2(fl(amax / 6)) for every bf16 amax, i.e.
// ((m + 0x3F) >> 7) - 2, then raised to the floor's exponent e_lo >= 1.
// Codes come from the gfx950 scaled converter, which divides by the
// power-of-two scale 2^(e-127) exactly and rounds to the E2M1 grid with ties
// to even, keeping the sign of zero.

struct Q8 {
    uint32_t codes;  // 8 nibbles: element 2b low, 2b+1 high nibble of byte b
    int e;
};

__device__ __forceinline__ Q8 quant8(uint4 v, int e_lo) {
    const u16x2_t a0 = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
    const u16x2_t a1 = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
    const u16x2_t a2 = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
    const u16x2_t a3 = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                 __builtin_elementwise_max(a2, a3));
    uint32_t m = max((uint32_t)m2.x, (uint32_t)m2.y);
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    const int e = max((int)((m + 0x3Fu) >> 7) - 2, e_lo);
    const float scale = __uint_as_float((uint32_t)e << 23);
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.x), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.y), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.z), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.w), scale, 3);
    return {r, e};
}

// ---- RoPE ------------------------------------------------------------------
// Slice chunk j (0..7) of the 64-wide rotated slice holds slice elements
// 8j..8j+7.  Every element is updated as x' = bf16(fl(x*C) + fl(p*S)) where p
// is its pair partner; with S = -s for the first element of a pair this is
// a' = a*c - b*s and b' = b*c + a*s exactly (negation is exact).
//   neox:        pair (i, i+32): chunk j <-> j ^ 4, same element, C = cos[i],
//                S = -+sin[i] with i = 8 (j & 3) + e
//   interleaved: pair (2i, 2i+1) inside the lane, i = 4j + e/2
template <bool NEOX>
__device__ __forceinline__ void rope_coeffs(const float* cs_row, int j, float C[8], float S[8]) {
    if (NEOX) {
        const int i0 = 8 * (j & 3);
        const float4 c0 = *reinterpret_cast<const float4*>(cs_row + i0);
        const float4 c1 = *reinterpret_cast<const float4*>(cs_row + i0 + 4);
        const float4 s0 = *reinterpret_cast<const float4*>(cs_row + 32 + i0);
        const float4 s1 = *reinterpret_cast<const float4*>(cs_row + 32 + i0 + 4);
        const uint32_t neg = (j < 4) ? 0x80000000u : 0u;
        const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            C[e] = c[e];
            S[e] = __uint_as_float(__float_as_uint(s[e]) ^ neg);
        }
    } else {
        const int i0 = 4 * j;
        const float4 c4 = *reinterpret_cast<const float4*>(cs_row + i0);
        const float4 s4 = *reinterpret_cast<const float4*>(cs_row + 32 + i0);
        const float c[4] = {c4.x, c4.y, c4.z, c4.w};
        const float s[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            C[2 * p] = c[p];
            C[2 * p + 1] = c[p];
            S[2 * p] = -s[p];
            S[2 * p + 1] = s[p];
        }
    }
}

template <bool NEOX>
__device__ __forceinline__ uint4 rope8(uint4 v, const float C[8], const float S[8]) {
    float x[8], p[8];
    unpack8(v, x);
    if (NEOX) {
        const uint4 pv = make_uint4(dpp<kDppHalfMirror>(v.x), dpp<kDppHalfMirror>(v.y),
                                    dpp<kDppHalfMirror>(v.z), dpp<kDppHalfMirror>(v.w));
        unpack8(pv, p);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = x[e ^ 1];
    }
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float xc = x[e] * C[e];
        const float ps = p[e] * S[e];
        y[e] = xc + ps;
    }
    return pack8(y);
}

// ---- Hadamard (row of 16 lanes) ----------------------------------------------
// Natural-order FWHT: butterflies of stride 1, 2, 4 inside the lane, then
// strides 8, 16, 32, 64 across lanes (chunk bits 0..3).  The lower element
// of a pair becomes u + w and the upper u - w; the upper lane computes it as
// partner + (-mine), which is the same IEEE operation.
template <int CTRL>
__device__ __forceinline__ void fwht_cross(float x[8], bool upper) {
    const uint32_t neg = upper ? 0x80000000u : 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = dppf<CTRL>(x[e]);
        const float m = __uint_as_float(__float_as_uint(x[e]) ^ neg);
        x[e] = p + m;
    }
}

__device__ __forceinline__ uint4 hadamard8(uint4 v, int c) {
    float x[8];
    unpack8(v, x);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j & h) continue;
            const float u = x[j], w = x[j + h];
            x[j] = u + w;
            x[j + h] = u - w;
        }
    }
    fwht_cross<kDppXor1>(x, (c & 1) != 0);
    fwht_cross<kDppXor2>(x, (c & 2) != 0);
    fwht_cross<kDppHalfMirror>(x, (c & 4) != 0);
    fwht_cross<kDppRor8>(x, (c & 8) != 0);
    const float sc = __uint_as_float(kHadamardScaleBits);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = x[e] * sc;
    return pack8(x);
}

// ---- key RMSNorm (row of 16 lanes) -------------------------------------------
// Correctly rounded fp32 sqrt and reciprocal: a float64 candidate, then an
// exact check against the midpoints to the neighbouring floats (products of
// <= 25-bit significands are exact in float64).
__device__ __forceinline__ float sqrt_rn(float v) {
    if (!(v > 0.0f)) return __builtin_sqrtf(v);
    float s = (float)__builtin_sqrt((double)v);
    const uint32_t b = __float_as_uint(s);
    const double hi = 0.5 * ((double)s + (double)__uint_as_float(b + 1));
    const double lo = 0.5 * ((double)s + (double)__uint_as_float(b - 1));
    if ((double)v > hi * hi) s = __uint_as_float(b + 1);
    else if ((double)v < lo * lo) s = __uint_as_float(b - 1);
    return s;
}

__device__ __forceinline__ float rcp_rn(float d) {
    float r = (float)(1.0 / (double)d);
    const uint32_t b = __float_as_uint(r);
    if (!(r > 0.0f) || b >= 0x7F800000u) return r;
    const double hi = 0.5 * ((double)r + (double)__uint_as_float(b + 1));
    const double lo = 0.5 * ((double)r + (double)__uint_as_float(b - 1));
    if ((double)d * hi < 1.0) r = __uint_as_float(b + 1);
    else if ((double)d * lo > 1.0) r = __uint_as_float(b - 1);
    return r;
}

// Sum of squares folded by halves (element i with i+64, then +32, +16, +8
// across lanes, +4, +2, +1 inside the lane).  Both lanes of every cross-lane
// pair compute the same sum, so every lane of the row ends with the same ss.
__device__ __forceinline__ uint4 rmsnorm8(uint4 v, const float G[8], float eps) {
    float x[8], p[8];
    unpack8(v, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = x[e] * x[e];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = p[e] + dppf<kDppRor8>(p[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = p[e] + dppf<kDppHalfMirror>(p[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = p[e] + dppf<kDppXor2>(p[e]);
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = p[e] + dppf<kDppXor1>(p[e]);
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = p[e] + p[e + 4];
    p[0] = p[0] + p[2];
    p[1] = p[1] + p[3];
    p[0] = p[0] + p[1];
    const float mean = p[0] * 0.0078125f;  // ss / 128, exact scaling
    const float r = rcp_rn(sqrt_rn(mean + eps));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float y = x[e] * r;
        x[e] = y * G[e];
    }
    return pack8(x);
}

__device__ __forceinline__ int64_t clamped_position(const void* positions, int pos64, int64_t t,
                                                    int64_t max_pos) {
    int64_t p = pos64 ? reinterpret_cast<const int64_t*>(positions)[t]
                      : (int64_t) reinterpret_cast<const int32_t*>(positions)[t];
    p = p < 0 ? 0 : p;
    return p >= max_pos ? max_pos - 1 : p;
}

// ---- query side ----------------------------------------------------------------
// One wavefront per token.  The token's scale bytes are gathered in LDS
// ([4][16][J] bytes, pads zero) and written out as whole dwords at the end.

__device__ __forceinline__ void q_token_prologue(const QArgs& a, int64_t t, int lane,
                                                 uint32_t* sc) {
    for (int i = lane; i < 16 * a.J; i += 64) sc[i] = 0u;
    if (a.weights != nullptr) {
        const float* w = a.weights + t * a.H;
        float* wo = a.weights_out + t * a.H;
        for (int h = lane; h < a.H; h += 64) wo[h] = w[h];
    }
}

__device__ __forceinline__ void q_token_epilogue(const QArgs& a, int64_t t, int lane,
                                                 const uint32_t* sc) {
    wave_sync();
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.q_scale_out + t * 64 * (int64_t)a.J);
    for (int i = lane; i < 16 * a.J; i += 64) dst[i] = sc[i];
}

// Without the Hadamard, the rotated and the plain halves of a head never mix,
// so every 16-byte load of a wave covers one half (128 bytes) of 8 heads:
// lanes 8k..8k+7 take head hb+k, lane chunk c = chunk_of(lane & 7).  Rotated
// and plain halves go through separate instruction streams and no lane
// computes a RoPE it throws away.  Each step handles 16 heads (4 loads) and
// issues the next step's loads before it computes.
template <bool NEOX>
__device__ __forceinline__ void q_split_token(const QArgs& a, int64_t t, int lane, uint8_t* scb,
                                              const float C[8], const float S[8]) {
    const int H = a.H;
    const int J = a.J;
    const int c = chunk_of(lane & 7);
    const int hsub = lane >> 3;
    const int ro = a.rope_offset;
    const int nro = 64 - ro;
    const int g_rot = ro / 32 + (c >> 2);
    const int g_pln = nro / 32 + (c >> 2);
    const bool writer = (lane & 3) == 0;
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    uint8_t* ot = a.q_out + t * (int64_t)H * 64 + hsub * 64 + 4 * c;

    uint4 np0 = load16_stream(qt + nro), nr0 = load16_stream(qt + ro);
    uint4 np1 = load16_stream(qt + 8 * 128 + nro), nr1 = load16_stream(qt + 8 * 128 + ro);
    for (int hb = 0; hb < H; hb += 16) {
        const uint4 p0 = np0, r0 = nr0, p1 = np1, r1 = nr1;
        if (hb + 16 < H) {
            const uint16_t* nx = qt + (hb + 16) * 128;
            np0 = load16_stream(nx + nro);
            nr0 = load16_stream(nx + ro);
            np1 = load16_stream(nx + 8 * 128 + nro);
            nr1 = load16_stream(nx + 8 * 128 + ro);
        }
        const Q8 qp0 = quant8(p0, a.e_lo);
        const Q8 qr0 = quant8(rope8<NEOX>(r0, C, S), a.e_lo);
        const Q8 qp1 = quant8(p1, a.e_lo);
        const Q8 qr1 = quant8(rope8<NEOX>(r1, C, S), a.e_lo);
        uint8_t* o = ot + hb * 64;
        store4_stream(o + nro / 2, qp0.codes);
        store4_stream(o + ro / 2, qr0.codes);
        store4_stream(o + 8 * 64 + nro / 2, qp1.codes);
        store4_stream(o + 8 * 64 + ro / 2, qr1.codes);
        if (writer) {
            const int h0 = hb + hsub, h1 = h0 + 8;
            scb[(g_pln * 16 + (h0 & 15)) * J + (h0 >> 4)] = (uint8_t)qp0.e;
            scb[(g_rot * 16 + (h0 & 15)) * J + (h0 >> 4)] = (uint8_t)qr0.e;
            scb[(g_pln * 16 + (h1 & 15)) * J + (h1 >> 4)] = (uint8_t)qp1.e;
            scb[(g_rot * 16 + (h1 & 15)) * J + (h1 >> 4)] = (uint8_t)qr1.e;
        }
    }
}

// With the Hadamard every output mixes the whole 128-row, so a wave-load is 4
// full heads (16 lanes each, lane chunk c = chunk_of(lane & 15)); RoPE is
// computed on every lane and kept only on the lanes of the rotated slice.
template <bool NEOX>
__device__ __forceinline__ void q_row_token(const QArgs& a, int64_t t, int lane, uint8_t* scb,
                                            const float C[8], const float S[8]) {
    const int H = a.H;
    const int J = a.J;
    const int c = chunk_of(lane & 15);
    const int hsub = lane >> 4;
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    const int g = c >> 2;
    const bool writer = (lane & 3) == 0;
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    uint8_t* ot = a.q_out + t * (int64_t)H * 64 + hsub * 64 + 4 * c;

    for (int hb = 0; hb < H; hb += 8) {
        const uint4 v0 = load16_stream(qt + hb * 128);
        const uint4 v1 = load16_stream(qt + (hb + 4) * 128);
        const uint4 w0 = hadamard8(select4(rot_lane, rope8<NEOX>(v0, C, S), v0), c);
        const uint4 w1 = hadamard8(select4(rot_lane, rope8<NEOX>(v1, C, S), v1), c);
        const Q8 q0 = quant8(w0, a.e_lo);
        const Q8 q1 = quant8(w1, a.e_lo);
        store4_stream(ot + hb * 64, q0.codes);
        store4_stream(ot + (hb + 4) * 64, q1.codes);
        if (writer) {
            const int h0 = hb + hsub, h1 = h0 + 4;
            scb[(g * 16 + (h0 & 15)) * J + (h0 >> 4)] = (uint8_t)q0.e;
            scb[(g * 16 + (h1 & 15)) * J + (h1 >> 4)] = (uint8_t)q1.e;
        }
    }
}

// ---- key side ---------------------------------------------------------------------
// One key row on the 16 lanes of a DPP row (lane chunk c = chunk_of(lane16)).
// v holds the row's raw bf16 chunk, already loaded.  C/S are the RoPE
// coefficients of slice chunk c & 7.  A slot outside the cache writes nothing.
template <bool NEOX, bool NORM, bool HAD>
__device__ __forceinline__ void k_row(const KArgs& a, uint4 v, int64_t slot, int lane16,
                                      const float C[8], const float S[8]) {
    const int c = chunk_of(lane16);
    if (NORM) {
        float G[8];
        unpack8(load16(a.gamma + 8 * c), G);
        v = rmsnorm8(v, G, a.eps);
    }
    const bool rot_lane = (c >> 3) == (a.rope_offset >> 6);
    v = select4(rot_lane, rope8<NEOX>(v, C, S), v);
    if (HAD) v = hadamard8(v, c);
    const Q8 q = quant8(v, a.e_lo);
    const int64_t blk = slot >> 6;
    const int p = (int)(slot & 63);
    const int g = c >> 2;
    const int64_t row = blk * 4 + g;
    // default cache policy: a block's 64 B pieces of a 64-slot row are written by
    // several workgroups, and L2 merges them before the line goes to HBM
    *reinterpret_cast<uint32_t*>(a.kv_cache + (row * 64 + p) * 16 + 4 * (c & 3)) = q.codes;
    if ((c & 3) == 0) a.kv_cache_scale[row * 64 + (p & 15) * 4 + (p >> 4)] = (uint8_t)q.e;
}

// ---- kernels ----------------------------------------------------------------------

template <bool NEOX>
__global__ __launch_bounds__(kBlock) void q_split_kernel(QArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= a.T) return;
    uint32_t* sc = smem + wave * 16 * a.J;
    q_token_prologue(a, t, lane, sc);
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
    q_split_token<NEOX>(a, t, lane, reinterpret_cast<uint8_t*>(sc), C, S);
    q_token_epilogue(a, t, lane, sc);
}

template <bool NEOX>
__global__ __launch_bounds__(kBlock) void q_row_kernel(QArgs a) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= a.T) return;
    uint32_t* sc = smem + wave * 16 * a.J;
    q_token_prologue(a, t, lane, sc);
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
    q_row_token<NEOX>(a, t, lane, reinterpret_cast<uint8_t*>(sc), C, S);
    q_token_epilogue(a, t, lane, sc);
}

// 16 lanes per token, 4 tokens per wavefront.  The row's loads are issued
// before its slot is inspected; a token whose slot is outside the cache then
// leaves as a whole row of 16 lanes, so the DPP patterns (all within a row)
// only ever read lanes of the same token.
template <bool NEOX, bool NORM, bool HAD>
__global__ __launch_bounds__(kBlock) void k_row_kernel(KArgs a) {
    const int lane16 = threadIdx.x & 15;
    const int64_t t = (int64_t)blockIdx.x * (kBlock / 16) + (threadIdx.x >> 4);
    if (t >= a.T) return;
    const uint4 v = load16_stream(a.k + t * 128 + 8 * chunk_of(lane16));
    const int64_t slot = a.slot_mapping[t];
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, chunk_of(lane16) & 7, C, S);
    if (slot < 0 || slot >= a.nslots) return;
    k_row<NEOX, NORM, HAD>(a, v, slot, lane16, C, S);
}

// Both sides of a token in one launch (ROCm/aiter PR 5484: one kernel writes
// all five outputs).  One wavefront per token for the query heads as above;
// wavefront 0 of each block also does the key rows of the block's 4 tokens,
// one per 16-lane row (rather than every wavefront doing its own key on a
// quarter of its lanes).  The key loads are issued before the query work.
// The RoPE coefficients of lane L for a key row are those of slice chunk
// chunk_of(L & 15) & 7 = chunk_of(L & 7).
template <bool NEOX, bool HAD, bool NORM>
__global__ __launch_bounds__(kBlock) void qk_kernel(QArgs qa, KArgs ka) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= qa.T) return;
    uint32_t* sc = smem + wave * 16 * qa.J;
    // key row of token tk on the 16-lane row lane / 16 of wavefront 0; rows past
    // T and rows whose slot is outside the cache leave as a whole row
    const int64_t tk = (int64_t)blockIdx.x * kWavesPerBlock + (lane >> 4);
    const bool krow = wave == 0 && tk < ka.T;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
    int64_t kslot = -1;
    float KC[8], KS[8];
    if (krow) {
        kv = load16_stream(ka.k + tk * 128 + 8 * chunk_of(lane & 15));
        kslot = ka.slot_mapping[tk];
        const int64_t kpos = clamped_position(ka.positions, ka.pos64, tk, ka.max_pos);
        rope_coeffs<NEOX>(ka.cos_sin + kpos * 64, chunk_of(lane & 7), KC, KS);
    }
    q_token_prologue(qa, t, lane, sc);
    const int64_t pos = clamped_position(qa.positions, qa.pos64, t, qa.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(qa.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
    if (HAD) q_row_token<NEOX>(qa, t, lane, reinterpret_cast<uint8_t*>(sc), C, S);
    else q_split_token<NEOX>(qa, t, lane, reinterpret_cast<uint8_t*>(sc), C, S);
    q_token_epilogue(qa, t, lane, sc);
    if (krow && kslot >= 0 && kslot < ka.nslots)
        k_row<NEOX, NORM, HAD>(ka, kv, kslot, lane & 15, KC, KS);
}

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
    const int e1 = max((int)((m + 0x3Fu) >> 7) - 2, e_lo1);
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
// are merged into lane 0 of the 8 with one half-row mirror.  The records are
// written with the default cache policy: a 68-byte record never fills whole
// 32-byte sectors from one store instruction, and streaming stores of such
// pieces measured ~18% slower (partial lines leave L2 before they complete).
template <bool NEOX>
__device__ __forceinline__ void q_sglang_token(const SQArgs& a, int64_t t, int lane,
                                               const float C[8], const float S[8]) {
    const int H = a.H;
    const int c = chunk_of(lane & 7);
    const int hsub = lane >> 3;
    const int ro = a.rope_offset;
    const int nro = 64 - ro;
    const int sh_rot = 8 * (ro / 32 + (c >> 2));
    const int sh_pln = 8 * (nro / 32 + (c >> 2));
    const bool writer = (lane & 7) == 0;
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hsub * 128 + 8 * c;
    uint8_t* ot = a.q_packed + t * (int64_t)H * kSglangRecord + hsub * kSglangRecord + 4 * c;

    uint4 np0 = load16_stream(qt + nro), nr0 = load16_stream(qt + ro);
    uint4 np1 = load16_stream(qt + 8 * 128 + nro), nr1 = load16_stream(qt + 8 * 128 + ro);
    for (int hb = 0; hb < H; hb += 16) {
        const uint4 p0 = np0, r0 = nr0, p1 = np1, r1 = nr1;
        if (hb + 16 < H) {
            const uint16_t* nx = qt + (hb + 16) * 128;
            np0 = load16_stream(nx + nro);
            nr0 = load16_stream(nx + ro);
            np1 = load16_stream(nx + 8 * 128 + nro);
            nr1 = load16_stream(nx + 8 * 128 + ro);
        }
        const Q8 qp0 = quant8_two_stage(p0, a.e_lo1, a.e_lo2);
        const Q8 qr0 = quant8_two_stage(rope8<NEOX>(r0, C, S), a.e_lo1, a.e_lo2);
        const Q8 qp1 = quant8_two_stage(p1, a.e_lo1, a.e_lo2);
        const Q8 qr1 = quant8_two_stage(rope8<NEOX>(r1, C, S), a.e_lo1, a.e_lo2);
        uint8_t* o = ot + hb * kSglangRecord;
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
    }
}

template <bool NEOX>
__global__ __launch_bounds__(kBlock) void q_sglang_kernel(SQArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= a.T) return;
    const int64_t pos = clamped_position(a.positions, a.pos64, t, a.max_pos);
    float C[8], S[8];
    rope_coeffs<NEOX>(a.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
    q_sglang_token<NEOX>(a, t, lane, C, S);
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
// exhaustively over all 2^31 significand pairs on the CPU.
__device__ __forceinline__ void store8_stream(void* p, uint2 v) {
    const u32x2_t w = {v.x, v.y};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}

__device__ __forceinline__ uint32_t bf16_bits(float x) {
    return pack_bf16x2(x, 0.0f) & 0xFFFFu;
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
    float s = __uint_as_float(m << 16) / 448.0f;
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

// Query: one token per wavefront, 16 lanes per head, 8 heads per step (two
// 16-byte loads per lane).  q_out rows are 128 bytes, written by the 16
// lanes of the head with 8-byte streaming stores; lane 0 of each head writes
// the folded weight.
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
    for (int hb = 0; hb < H; hb += 8) {
        const uint4 v0 = load16_stream(qt + hb * 128);
        const uint4 v1 = load16_stream(qt + (hb + 4) * 128);
        uint4 w0 = select4(rot_lane, rope8<NEOX>(v0, C, S), v0);
        uint4 w1 = select4(rot_lane, rope8<NEOX>(v1, C, S), v1);
        if (HAD) {
            w0 = hadamard8(w0, c);
            w1 = hadamard8(w1, c);
        }
        float s0, s1;
        const uint2 q0 = quant_fp8_row<FP32>(w0, a.scale_floor, s0);
        const uint2 q1 = quant_fp8_row<FP32>(w1, a.scale_floor, s1);
        store8_stream(ot + hb * 128, q0);
        store8_stream(ot + (hb + 4) * 128, q1);
        if ((lane & 15) == 0) {
            const int h0 = hb + hsub, h1 = h0 + 4;
            wo[h0] = (uint16_t)bf16_bits((wt[h0] * s0) * a.weights_scale);
            wo[h1] = (uint16_t)bf16_bits((wt[h1] * s1) * a.weights_scale);
        }
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
        float qs = __uint_as_float(m << 16) / 6.0f;
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
            const float r = __frcp_rn(s);  // RN(1/s)
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y0 = x[e] * r;
                const float err = __builtin_fmaf(-y0, s, x[e]);
                const float q = __builtin_fmaf(err, r, y0);
                y[e] = __builtin_copysignf(__builtin_fminf(__builtin_fabsf(q), 6.0f), x[e]);
            }
            uint32_t codes = 0;
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
// of a token): the RoPE coefficients are formed once, and each step handles 8
// rows (two 16-byte loads per lane, lanes 16k..16k+15 on rows k and k+4).  A
// row past the token's last leaves as a whole 16-lane group, so every DPP
// pattern still reads lanes of its own row.
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
    for (int64_t rb = r0; rb < r_end; rb += 8) {
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

// ---- dequantization (debug reader) -------------------------------------------
// One thread per 8 consecutive values (4 code bytes).
__device__ __forceinline__ float e2m1_value(uint32_t nib) {
    // magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} in half units: 0,1,2,3,4,6,8,12
    const uint32_t half_units = (0xC8643210u >> (4 * (nib & 7))) & 0xF;
    const float v = (float)half_units * 0.5f;
    return (nib & 8) ? -v : v;
}

__device__ __forceinline__ float e8m0_value(uint32_t e) {
    if (e == 255u) return __uint_as_float(0x7FC00000u);
    if (e == 0u) return __uint_as_float(0x00400000u);  // 2^-127
    return __uint_as_float(e << 23);
}

__global__ __launch_bounds__(256) void dequant_kernel(DArgs a) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t chunks_per_row = (a.which == 0) ? (int64_t)a.H * 16 : 16;
    if (i >= a.rows * chunks_per_row) return;
    const int64_t row = i / chunks_per_row;
    const int c = (int)(i % 16);
    const int g = c >> 2;
    uint32_t codes = 0, e = 0;
    bool zero = false;
    float* out;
    if (a.which == 0) {
        const int h = (int)((i / 16) % a.H);
        const int64_t t = row;
        codes = *reinterpret_cast<const uint32_t*>(a.packed + (t * a.H + h) * 64 + 4 * c);
        e = a.scales[t * 64 * (int64_t)a.J + (g * 16 + (h & 15)) * a.J + (h >> 4)];
        out = a.out + (t * a.H + h) * 128 + 8 * c;
    } else {
        const int64_t slot = a.slots ? a.slots[row] : row;
        out = a.out + row * 128 + 8 * c;
        if (slot < 0 || slot >= a.nslots) {
            zero = true;
        } else {
            const int64_t r = (slot >> 6) * 4 + g;
            const int p = (int)(slot & 63);
            codes = *reinterpret_cast<const uint32_t*>(a.packed + (r * 64 + p) * 16 + 4 * (c & 3));
            e = a.scales[r * 64 + (p & 15) * 4 + (p >> 4)];
        }
    }
    float y[8];
    const float s = e8m0_value(e);
#pragma unroll
    for (int k = 0; k < 8; ++k) y[k] = zero ? 0.0f : e2m1_value(codes >> (4 * k)) * s;
    reinterpret_cast<float4*>(out)[0] = make_float4(y[0], y[1], y[2], y[3]);
    reinterpret_cast<float4*>(out)[1] = make_float4(y[4], y[5], y[6], y[7]);
}

template <typename K, typename A>
hipError_t launch(K kernel, int64_t blocks, size_t lds, hipStream_t stream, const A& a) {
    A copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks),
                           dim3(kBlock), args, lds, stream);
}

template <typename K>
hipError_t launch2(K kernel, int64_t blocks, size_t lds, hipStream_t stream, const QArgs& qa,
                   const KArgs& ka) {
    QArgs q = qa;
    KArgs k = ka;
    void* args[] = {&q, &k};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks),
                           dim3(kBlock), args, lds, stream);
}

}  // namespace

hipError_t launch_q_rope_pack(const QArgs& a, bool is_neox, bool hadamard, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = (size_t)kWavesPerBlock * 16 * a.J * sizeof(uint32_t);
    if (hadamard)
        return is_neox ? launch(q_row_kernel<true>, blocks, lds, stream, a)
                       : launch(q_row_kernel<false>, blocks, lds, stream, a);
    return is_neox ? launch(q_split_kernel<true>, blocks, lds, stream, a)
                   : launch(q_split_kernel<false>, blocks, lds, stream, a);
}

hipError_t launch_k_rope_pack_store(const KArgs& a, bool is_neox, bool hadamard,
                                    hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kBlock / 16 - 1) / (kBlock / 16);
    const bool norm = a.gamma != nullptr;
    const int sel = (is_neox ? 4 : 0) | (norm ? 2 : 0) | (hadamard ? 1 : 0);
    switch (sel) {
        case 0: return launch(k_row_kernel<false, false, false>, blocks, 0, stream, a);
        case 1: return launch(k_row_kernel<false, false, true>, blocks, 0, stream, a);
        case 2: return launch(k_row_kernel<false, true, false>, blocks, 0, stream, a);
        case 3: return launch(k_row_kernel<false, true, true>, blocks, 0, stream, a);
        case 4: return launch(k_row_kernel<true, false, false>, blocks, 0, stream, a);
        case 5: return launch(k_row_kernel<true, false, true>, blocks, 0, stream, a);
        case 6: return launch(k_row_kernel<true, true, false>, blocks, 0, stream, a);
        default: return launch(k_row_kernel<true, true, true>, blocks, 0, stream, a);
    }
}

hipError_t launch_qk_rope_pack_store(const QArgs& qa, const KArgs& ka, bool is_neox, bool hadamard,
                                     hipStream_t stream) {
    if (qa.T == 0) return hipSuccess;
    const int64_t blocks = (qa.T + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = (size_t)kWavesPerBlock * 16 * qa.J * sizeof(uint32_t);
    const bool norm = ka.gamma != nullptr;
    const int sel = (is_neox ? 4 : 0) | (hadamard ? 2 : 0) | (norm ? 1 : 0);
    switch (sel) {
        case 0: return launch2(qk_kernel<false, false, false>, blocks, lds, stream, qa, ka);
        case 1: return launch2(qk_kernel<false, false, true>, blocks, lds, stream, qa, ka);
        case 2: return launch2(qk_kernel<false, true, false>, blocks, lds, stream, qa, ka);
        case 3: return launch2(qk_kernel<false, true, true>, blocks, lds, stream, qa, ka);
        case 4: return launch2(qk_kernel<true, false, false>, blocks, lds, stream, qa, ka);
        case 5: return launch2(qk_kernel<true, false, true>, blocks, lds, stream, qa, ka);
        case 6: return launch2(qk_kernel<true, true, false>, blocks, lds, stream, qa, ka);
        default: return launch2(qk_kernel<true, true, true>, blocks, lds, stream, qa, ka);
    }
}

hipError_t launch_q_rope_pack_sglang(const SQArgs& a, bool is_neox, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    const int64_t blocks = (a.T + kWavesPerBlock - 1) / kWavesPerBlock;
    return is_neox ? launch(q_sglang_kernel<true>, blocks, 0, stream, a)
                   : launch(q_sglang_kernel<false>, blocks, 0, stream, a);
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

hipError_t launch_dequant(const DArgs& a, hipStream_t stream) {
    const int64_t chunks = a.rows * (a.which == 0 ? (int64_t)a.H * 16 : 16);
    if (chunks == 0) return hipSuccess;
    return launch(dequant_kernel, (chunks + 255) / 256, 0, stream, a);
}

}  // namespace fp4idx
