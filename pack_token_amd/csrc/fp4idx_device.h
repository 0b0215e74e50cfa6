// fp4idx_device.h -- device helpers shared by the gfx950 kernels of libfp4idx
// (fp4idx_kernels.hip: the FP4 producer; fp4idx_modes.hip: the sglang-
// compatible, FP8 and fake-quant modes).  Not installed.
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
#pragma once

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

// Rows and banks all enabled, and a lane whose source is invalid gets 0
// (bound_ctrl) -- the result the form with an explicit old value of 0 gives,
// without zeroing a register first.  (Every pattern used here reads an active
// lane of the same row for every lane anyway.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
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
// biased exponent of ceil_pow2(fl(amax / 6)) for every finite bf16 amax, i.e.
// ((m + 0x3F) >> 7) - 2, then raised to the floor's exponent e_lo >= 1.  An
// infinite amax (a rotated or normalised value past the fp32 range) makes
// amax / 6 infinite, whose exponent field 255 clamps to 254.
// Codes come from the gfx950 scaled converter, which divides by the
// power-of-two scale 2^(e-127) exactly and rounds to the E2M1 grid with ties
// to even, keeping the sign of zero.

struct Q8 {
    uint32_t codes;  // 8 nibbles: element 2b low, 2b+1 high nibble of byte b
    int e;
};

// The group's 8 values (a lane's share of a 32-group spread over a quad of
// lanes) as packed bf16 in v, with m the bf16 magnitude bits of the lane's own
// largest |value|: the quad's maximum, the exponent and the codes.
__device__ __forceinline__ Q8 quant8_m(uint4 v, uint32_t m, int e_lo) {
    m = max(m, dpp<kDppXor1>(m));
    m = max(m, dpp<kDppXor2>(m));
    const int e = m >= 0x7F80u ? 254 : max((int)((m + 0x3Fu) >> 7) - 2, e_lo);
    const float scale = __uint_as_float((uint32_t)e << 23);
    // each converter writes one byte of its first operand and the four calls
    // cover all of it, so a dead value seeds the chain (no zeroing move)
    uint32_t r = v.x;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.x), scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.y), scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.z), scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2_t, v.w), scale, 3);
    return {r, e};
}

// Values already in bf16: the lane's amax from the magnitude bits.
__device__ __forceinline__ Q8 quant8(uint4 v, int e_lo) {
    const u16x2_t a0 = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
    const u16x2_t a1 = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
    const u16x2_t a2 = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
    const u16x2_t a3 = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(a0, a1),
                                                 __builtin_elementwise_max(a2, a3));
    return quant8_m(v, max((uint32_t)m2.x, (uint32_t)m2.y), e_lo);
}

// fp32 values that the method rounds to bf16 before quantizing: the lane's
// amax from the fp32 magnitudes (three-operand maxima, the abs free), rounded
// once.  Rounding to nearest is monotonic, so bf16(max |x|) = max |bf16(x)|:
// the same m as from the rounded values, in fewer issue cycles (Hadamard
// query path, 59.2-60.4 against 59.7-61.0 us at T = 16384, H = 64).
__device__ __forceinline__ Q8 quant8_f(const float x[8], int e_lo) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(x[i]));
    return quant8_m(pack8(x), pack_bf16x2(a, 0.0f), e_lo);
}

// ---- division by a constant ---------------------------------------------------
// RN(x / d) for a non-negative bf16 x and the constants d = 6 and 448, from
// the reciprocal rc = RN(1/d) and one FMA correction instead of the IEEE
// division sequence.  Checked on the CPU for every finite bf16 x, subnormal
// quotients included (0 mismatches for either d).
constexpr float kRcp6 = 0x1.555556p-3f;    // RN(1/6)
constexpr float kRcp448 = 0x1.24924ap-9f;  // RN(1/448)

__device__ __forceinline__ float div_const_rn(float x, float d, float rc) {
    const float y0 = x * rc;
    return __builtin_fmaf(__builtin_fmaf(-y0, d, x), rc, y0);
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

// A dispatch's grid size is a 32-bit work-item count: a launch past it would
// wrap, so it is refused before anything is enqueued.
inline bool grid_fits(int64_t blocks, int64_t threads) {
    return blocks >= 0 && blocks <= (int64_t)0xFFFFFFFF / threads;
}

// Dynamic LDS for a launch that keeps at most `per_cu` of its workgroups
// resident on a compute unit: the launch reserves about 1/per_cu of the unit's
// LDS (the part beyond `dyn` and the kernel's static LDS is not used).  The
// streaming kernels move their bytes faster with fewer wavefronts resident
// (fewer concurrent DRAM streams); the cap is chosen per kernel by measurement.
// If the device cannot give a workgroup that much LDS, or reading its limits
// fails, the launch keeps `dyn` and its occupancy.
inline size_t resident_cap_lds(const void* fn, size_t dyn, int per_cu) {
    int dev = 0, lds_cu = 0, lds_wg = 0;
    hipFuncAttributes fa;
    if (per_cu <= 0 || hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&lds_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        hipFuncGetAttributes(&fa, fn) != hipSuccess)
        return dyn;
    // per_cu workgroups fit and per_cu + 1 do not
    const size_t total = (size_t)lds_cu / (size_t)per_cu - 1024;
    if (total > (size_t)lds_wg || total <= fa.sharedSizeBytes + dyn) return dyn;
    return total - fa.sharedSizeBytes;
}

template <typename K, typename A>
hipError_t launch(K kernel, int64_t blocks, size_t lds, hipStream_t stream, const A& a) {
    if (!grid_fits(blocks, kBlock)) return hipErrorInvalidConfiguration;
    A copy = a;
    void* args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks),
                           dim3(kBlock), args, lds, stream);
}

template <typename K>
hipError_t launch2(K kernel, int64_t blocks, size_t lds, hipStream_t stream, const QArgs& qa,
                   const KArgs& ka, unsigned threads = kBlock) {
    if (!grid_fits(blocks, threads)) return hipErrorInvalidConfiguration;
    QArgs q = qa;
    KArgs k = ka;
    void* args[] = {&q, &k};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)blocks),
                           dim3(threads), args, lds, stream);
}

}  // namespace
}  // namespace fp4idx
