// fp4idx_kernels.hip -- gfx950 kernels of the fused FP4 indexer producer.
//
// What is computed (per token; ROCm/aiter PR 5484 "API" and "One deliberate
// deviation", sgl-project/sglang PR 39656 "Summary" and review, ROCm/aiter
// PR 4029 "Changes"):
//   optional key RMSNorm -> RoPE on a 64-wide slice (bf16 round trip) ->
//   optional 128-point Hadamard (bf16) -> per 32-group UE8M0 exponent ->
//   E2M1 codes (RNE, sign kept on zero) -> two codes per byte -> q_out /
//   q_scale_out / weights_out, or the paged key cache and its interleaved
//   scale row.  The register layout and the shared helpers are in
//   fp4idx_device.h.
//
// Nothing here is a dense contraction, so there is no MFMA.  Without the
// Hadamard the path is bound by HBM bandwidth, and the kernels stream q once
// with 16-byte loads and issue no more VALU work than the stream can hide;
// with it the query side is bound by VALU issue, and its layout (a quad of
// lanes per head) is chosen to minimise VALU instructions.
#include "fp4idx_device.h"

namespace fp4idx {
namespace {

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
// issues the next step's loads before it computes; its codes meet in the
// wave's 1 KB of LDS and leave as one 16-byte store per lane (the 16 heads'
// 1,024 output bytes, whole lines: 413 against 416 us at 131072 x 64 with the
// four 4-byte stores per lane that write half lines).
template <bool NEOX>
__device__ __forceinline__ void q_split_token(const QArgs& a, int64_t t, int lane, uint8_t* scb,
                                              const float C[8], const float S[8], uint32_t* stage) {
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

    auto step = [&](int hb, uint4 p0, uint4 r0, uint4 p1, uint4 r1) {
        const Q8 qp0 = quant8(p0, a.e_lo);
        const Q8 qr0 = quant8(rope8<NEOX>(r0, C, S), a.e_lo);
        const Q8 qp1 = quant8(p1, a.e_lo);
        const Q8 qr1 = quant8(rope8<NEOX>(r1, C, S), a.e_lo);
        const int so = hsub * 16 + c;  // dword of the lane's 4 bytes in a head row pair
        stage[so + nro / 8] = qp0.codes;
        stage[so + ro / 8] = qr0.codes;
        stage[so + 128 + nro / 8] = qp1.codes;
        stage[so + 128 + ro / 8] = qr1.codes;
        wave_sync();
        store16_stream(a.q_out + (t * (int64_t)H + hb) * 64 + 16 * lane,
                       *reinterpret_cast<const uint4*>(stage + 4 * lane));
        wave_sync();
        if (writer) {
            const int h0 = hb + hsub, h1 = h0 + 8;
            scb[(g_pln * 16 + (h0 & 15)) * J + (h0 >> 4)] = (uint8_t)qp0.e;
            scb[(g_rot * 16 + (h0 & 15)) * J + (h0 >> 4)] = (uint8_t)qr0.e;
            scb[(g_pln * 16 + (h1 & 15)) * J + (h1 >> 4)] = (uint8_t)qp1.e;
            scb[(g_rot * 16 + (h1 & 15)) * J + (h1 >> 4)] = (uint8_t)qr1.e;
        }
    };
    // Two register sets take turns: one is computed while the other loads the
    // next 16 heads (a single set refilled from prefetch registers costs 16
    // register moves per step).
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

// With the Hadamard the query side is bound by VALU issue, not by HBM (with
// every access made L2-resident it runs in about the same time), so its layout
// minimises VALU work: a quad of lanes holds one head, lane r = lane & 3 of the
// quad holding chunks r, r+4, r+8, r+12, i.e. element 32j + 8r + e in x[j][e].
// Index bits 0-2 (e) and 5-6 (j) are inside the lane and bits 3-4 (r) across
// the quad, so the neox RoPE partner (slice element + 32) and five of the
// seven FWHT strides (1, 2, 4, 32, 64) need no lane exchange, RoPE runs only
// on the two rotated chunks, and each 32-group (row j) is one quad, as quant8
// expects.  Against 16 lanes per head (RoPE on every lane, four of the seven
// strides across lanes) this is 2208 instead of 2952 VALU instructions per
// token at H = 64.

// RoPE coefficients of quad lane r: neox pairs (s, s + 32) with s = 8r + e;
// interleaved pairs (2i, 2i + 1) with i = 16q + 4r + p for rotated chunk q.
template <bool NEOX>
__device__ __forceinline__ void rope_coeffs_quad(const float* cs_row, int r, float C[8],
                                                 float S[8]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int i0 = NEOX ? 8 * r + 4 * q : 16 * q + 4 * r;
        const float4 c4 = *reinterpret_cast<const float4*>(cs_row + i0);
        const float4 s4 = *reinterpret_cast<const float4*>(cs_row + 32 + i0);
        C[4 * q] = c4.x, C[4 * q + 1] = c4.y, C[4 * q + 2] = c4.z, C[4 * q + 3] = c4.w;
        S[4 * q] = s4.x, S[4 * q + 1] = s4.y, S[4 * q + 2] = s4.z, S[4 * q + 3] = s4.w;
    }
}

// RoPE of the rotated chunks lo (slice elements 8r + e) and hi (32 + 8r + e),
// then the bf16 round trip: a' = a c - b s, b' = b c + a s.
template <bool NEOX>
__device__ __forceinline__ void rope_quad(float lo[8], float hi[8], const float C[8],
                                          const float S[8]) {
    float y[16];
    if (NEOX) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[e] = lo[e] * C[e] - hi[e] * S[e];
            y[8 + e] = hi[e] * C[e] + lo[e] * S[e];
        }
    } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const float* x = q ? hi : lo;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const float c = C[4 * q + p], sn = S[4 * q + p];
                y[8 * q + 2 * p] = x[2 * p] * c - x[2 * p + 1] * sn;
                y[8 * q + 2 * p + 1] = x[2 * p + 1] * c + x[2 * p] * sn;
            }
        }
    }
    unpack8(pack8(y), lo);
    unpack8(pack8(y + 8), hi);
}

// A cross-lane FWHT butterfly stage for a quad of lanes holding N chunks each,
// with the partner fetched through the LDS crossbar (ds_swizzle in quad-permute mode,
// which takes no VALU issue slot) and one fused multiply-add per element:
// x' = x * s + p with s = +1 on the lower lane (x + p) and -1 on the upper
// (p - x).  The product by +-1 is exact, so the FMA rounds p + s*x once, the
// IEEE add or subtract itself, signed zeros included.  All of a stage's
// swizzles are issued before its first FMA.
constexpr int kSwzXor1 = 0x8000 | kDppXor1;  // ds_swizzle quad_perm [1,0,3,2]
constexpr int kSwzXor2 = 0x8000 | kDppXor2;  // ds_swizzle quad_perm [2,3,0,1]

template <int PAT, int N>
__device__ __forceinline__ void fwht_cross_swz(float (*x)[8], float s) {
    float p[N][8];
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            p[j][e] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x[j][e]), PAT));
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = __builtin_fmaf(x[j][e], s, p[j][e]);
}

// Natural-order FWHT of the quad's head: strides 1, 2, 4 inside each chunk,
// 8 and 16 across the quad (quad lanes r ^ 1, r ^ 2), 32 and 64 between the
// lane's chunks; then the orthonormal scale.
__device__ __forceinline__ void hadamard_quad(float x[4][8], int r) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if (e & h) continue;
                const float u = x[j][e], w = x[j][e + h];
                x[j][e] = u + w;
                x[j][e + h] = u - w;
            }
        }
    }
    fwht_cross_swz<kSwzXor1, 4>(x, (r & 1) ? -1.0f : 1.0f);
    fwht_cross_swz<kSwzXor2, 4>(x, (r & 2) ? -1.0f : 1.0f);
#pragma unroll
    for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j & h) continue;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float u = x[j][e], w = x[j + h][e];
                x[j][e] = u + w;
                x[j + h][e] = u - w;
            }
        }
    }
    const float sc = __uint_as_float(kHadamardScaleBits);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[j][e] = x[j][e] * sc;
}

// 16 heads per wave step.  Each lane loads its four 16-byte chunks with the
// default cache policy: one load instruction covers 64 bytes of every head, the
// other half of each 128-byte line comes from the next instruction, and L2
// joins them (streaming loads measured ~12% slower here).  The code bytes go
// through the wave's 1 KB LDS `stage` so that one 16-byte store per lane writes
// the 16 heads' 1024 output bytes contiguously.  TAIL: rope_offset == 64 (a
// template parameter, so the rotated chunks are fixed registers).
template <bool NEOX, bool TAIL>
__device__ __forceinline__ void q_quad_token(const QArgs& a, int64_t t, int lane, uint8_t* scb,
                                             const float C[8], const float S[8], uint32_t* stage) {
    const int H = a.H;
    const int J = a.J;
    const int r = lane & 3;
    const int hs = lane >> 2;
    const uint16_t* qt = a.q + t * (int64_t)H * 128 + hs * 128 + 8 * r;
    for (int hb = 0; hb < H; hb += 16) {
        uint4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = load16(qt + hb * 128 + 32 * j);
        float x[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) unpack8(v[j], x[j]);
        rope_quad<NEOX>(x[TAIL ? 2 : 0], x[TAIL ? 3 : 1], C, S);
        hadamard_quad(x, r);
        const int h = hb + hs;
        int eg[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const Q8 q = quant8_f(x[g], a.e_lo);
            stage[hs * 16 + 4 * g + r] = q.codes;  // bytes 16g + 4r of head hs
            eg[g] = q.e;
        }
        wave_sync();
        store16_stream(a.q_out + (t * (int64_t)H + hb) * 64 + 16 * lane,
                       *reinterpret_cast<const uint4*>(stage + 4 * lane));
        wave_sync();
        if (r == 0) {
#pragma unroll
            for (int g = 0; g < 4; ++g) scb[(g * 16 + (h & 15)) * J + (h >> 4)] = (uint8_t)eg[g];
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
    __shared__ __attribute__((aligned(16))) uint32_t qst[kWavesPerBlock * 256];
    q_split_token<NEOX>(a, t, lane, reinterpret_cast<uint8_t*>(sc), C, S, qst + wave * 256);
    q_token_epilogue(a, t, lane, sc);
}

// Query side with the Hadamard: one token per wavefront, a quad of lanes per
// head (q_quad_token), 1 KB of static LDS per wavefront for the code staging
// beside the dynamic scale rows.
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
    rope_coeffs_quad<NEOX>(a.cos_sin + pos * 64, lane & 3, C, S);
    __shared__ __attribute__((aligned(16))) uint32_t qstage[kWavesPerBlock * 256];
    if (a.rope_offset != 0)
        q_quad_token<NEOX, true>(a, t, lane, reinterpret_cast<uint8_t*>(sc), C, S, qstage + wave * 256);
    else
        q_quad_token<NEOX, false>(a, t, lane, reinterpret_cast<uint8_t*>(sc), C, S, qstage + wave * 256);
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
// all five outputs).  One wavefront per token for the query heads as above,
// and the key rows of the block's 4 tokens one per 16-lane row:
//   without the Hadamard, on a fifth wavefront of the block (the query side is
//     memory-bound and the extra wavefront fills idle issue slots: 443 -> 436
//     us at 131072 x 64);
//   with it, on wavefront 0 after its query token (a fifth wavefront competes
//     for the VALU there: 66.8 -> 68.4 us at 16384 x 64).  The key loads are
//     issued only then: held across the query loop, the key row's registers
//     took the kernel from 78 to 115 VGPRs (6 -> 4 wavefronts per SIMD) and
//     the launch from 69-71 to 74-76 us.
// The RoPE coefficients of lane L for a key row are those of slice chunk
// chunk_of(L & 15) & 7 = chunk_of(L & 7).  Rows past T and rows whose slot is
// outside the cache leave as a whole 16-lane row.
template <bool NEOX, bool HAD, bool NORM>
__global__ __launch_bounds__(HAD ? kBlock : kBlock + 64) void qk_kernel(QArgs qa, KArgs ka) {
    extern __shared__ uint32_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tk = (int64_t)blockIdx.x * kWavesPerBlock + (lane >> 4);
    if (!HAD && wave == kWavesPerBlock) {
        if (tk >= ka.T) return;
        const uint4 kv = load16_stream(ka.k + tk * 128 + 8 * chunk_of(lane & 15));
        const int64_t kslot = ka.slot_mapping[tk];
        const int64_t kpos = clamped_position(ka.positions, ka.pos64, tk, ka.max_pos);
        float KC[8], KS[8];
        rope_coeffs<NEOX>(ka.cos_sin + kpos * 64, chunk_of(lane & 7), KC, KS);
        if (kslot < 0 || kslot >= ka.nslots) return;
        k_row<NEOX, NORM, HAD>(ka, kv, kslot, lane & 15, KC, KS);
        return;
    }
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= qa.T) return;
    uint32_t* sc = smem + wave * 16 * qa.J;
    q_token_prologue(qa, t, lane, sc);
    const int64_t pos = clamped_position(qa.positions, qa.pos64, t, qa.max_pos);
    float C[8], S[8];
    if (HAD) {
        rope_coeffs_quad<NEOX>(qa.cos_sin + pos * 64, lane & 3, C, S);
        __shared__ __attribute__((aligned(16))) uint32_t qstage[kWavesPerBlock * 256];
        if (qa.rope_offset != 0)
            q_quad_token<NEOX, true>(qa, t, lane, reinterpret_cast<uint8_t*>(sc), C, S,
                                     qstage + wave * 256);
        else
            q_quad_token<NEOX, false>(qa, t, lane, reinterpret_cast<uint8_t*>(sc), C, S,
                                      qstage + wave * 256);
    } else {
        rope_coeffs<NEOX>(qa.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
        __shared__ __attribute__((aligned(16))) uint32_t qst[kWavesPerBlock * 256];
        q_split_token<NEOX>(qa, t, lane, reinterpret_cast<uint8_t*>(sc), C, S, qst + wave * 256);
    }
    q_token_epilogue(qa, t, lane, sc);
    if (HAD && wave == 0 && tk < ka.T) {
        const uint4 kv = load16_stream(ka.k + tk * 128 + 8 * chunk_of(lane & 15));
        const int64_t kslot = ka.slot_mapping[tk];
        const int64_t kpos = clamped_position(ka.positions, ka.pos64, tk, ka.max_pos);
        float KC[8], KS[8];
        rope_coeffs<NEOX>(ka.cos_sin + kpos * 64, chunk_of(lane & 7), KC, KS);
        if (kslot >= 0 && kslot < ka.nslots) k_row<NEOX, NORM, HAD>(ka, kv, kslot, lane & 15, KC, KS);
    }
}

// ---- small batches -------------------------------------------------------------
// Below kSmallBatchTokens tokens the per-token kernels leave fewer than two
// wavefronts per CU.  Here one wavefront takes a (token, group of 8 heads), so
// a decode batch spreads over H/8 times as many wavefronts and each carries
// one step of work (measured: 256 tokens x 32 heads, 5.4 -> 5.1 us, and with
// key RMSNorm + Hadamard 8.9 -> 5.9 us; from 1024 tokens on the per-token
// kernels are faster).  The group's scale bytes go
// straight to q_scale_out (each byte has one writer; group 0 writes the zero
// pads); group 0 also copies the token's weights and, with WITH_KEY, does the
// token's key row on lanes 0..15, its loads issued first.
template <bool NEOX, bool HAD, bool NORM, bool WITH_KEY>
__global__ __launch_bounds__(kBlock) void qk_small_kernel(QArgs qa, KArgs ka) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int groups = qa.H >> 3;
    const int64_t wid = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    const int64_t t = wid / groups;
    if (t >= qa.T) return;
    const int g8 = (int)(wid - t * groups);
    const int H = qa.H;
    const int J = qa.J;
    // The token's position is read first: it heads the only chain of dependent
    // reads (position, then the cos/sin row).  The key row shares the query's
    // position and table (one call, one positions and one cos_sin argument) and,
    // on lanes 0..15, its RoPE coefficients C/S, so it adds no round trip.
    const int64_t pos = clamped_position(qa.positions, qa.pos64, t, qa.max_pos);
    const bool krow = WITH_KEY && g8 == 0 && lane < 16;
    uint4 kv = make_uint4(0u, 0u, 0u, 0u);
    int64_t kslot = -1;
    if (krow) {
        kv = load16_stream(ka.k + t * 128 + 8 * chunk_of(lane));
        kslot = ka.slot_mapping[t];
    }
    uint8_t* qs = qa.q_scale_out + t * 64 * (int64_t)J;
    if (g8 == 0) {
        if (qa.weights != nullptr)
            for (int h = lane; h < H; h += 64) qa.weights_out[t * H + h] = qa.weights[t * H + h];
        const int used = H >> 4;
        for (int i = lane; i < 64 * J; i += 64)
            if ((i % J) >= used) qs[i] = 0;
    }
    float C[8], S[8];
    rope_coeffs<NEOX>(qa.cos_sin + pos * 64, chunk_of(lane & 7), C, S);
    const int ro = qa.rope_offset;
    if (!HAD) {
        const int c = chunk_of(lane & 7);
        const int h = 8 * g8 + (lane >> 3);
        const uint16_t* qt = qa.q + (t * H + h) * 128 + 8 * c;
        const uint4 p = load16_stream(qt + 64 - ro);
        const uint4 r = load16_stream(qt + ro);
        const Q8 qp = quant8(p, qa.e_lo);
        const Q8 qr = quant8(rope8<NEOX>(r, C, S), qa.e_lo);
        uint8_t* o = qa.q_out + (t * H + h) * 64 + 4 * c;
        store4_stream(o + (64 - ro) / 2, qp.codes);
        store4_stream(o + ro / 2, qr.codes);
        if ((lane & 3) == 0) {
            const int gp = (64 - ro) / 32 + (c >> 2), gr = ro / 32 + (c >> 2);
            qs[(gp * 16 + (h & 15)) * J + (h >> 4)] = (uint8_t)qp.e;
            qs[(gr * 16 + (h & 15)) * J + (h >> 4)] = (uint8_t)qr.e;
        }
    } else {
        const int c = chunk_of(lane & 15);
        const bool rot_lane = (c >> 3) == (ro >> 6);
        const int h0 = 8 * g8 + (lane >> 4), h1 = h0 + 4;
        const uint4 v0 = load16_stream(qa.q + (t * H + h0) * 128 + 8 * c);
        const uint4 v1 = load16_stream(qa.q + (t * H + h1) * 128 + 8 * c);
        const Q8 q0 = quant8(hadamard8(select4(rot_lane, rope8<NEOX>(v0, C, S), v0), c), qa.e_lo);
        const Q8 q1 = quant8(hadamard8(select4(rot_lane, rope8<NEOX>(v1, C, S), v1), c), qa.e_lo);
        store4_stream(qa.q_out + (t * H + h0) * 64 + 4 * c, q0.codes);
        store4_stream(qa.q_out + (t * H + h1) * 64 + 4 * c, q1.codes);
        if ((lane & 3) == 0) {
            const int g = c >> 2;
            qs[(g * 16 + (h0 & 15)) * J + (h0 >> 4)] = (uint8_t)q0.e;
            qs[(g * 16 + (h1 & 15)) * J + (h1 >> 4)] = (uint8_t)q1.e;
        }
    }
    if (krow && kslot >= 0 && kslot < ka.nslots) k_row<NEOX, NORM, HAD>(ka, kv, kslot, lane, C, S);
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

}  // namespace


// a small batch goes to qk_small_kernel (see there)
constexpr int64_t kSmallBatchTokens = 512;

template <bool WITH_KEY>
hipError_t launch_small(const QArgs& qa, const KArgs& ka, bool is_neox, bool hadamard,
                        hipStream_t stream) {
    const int64_t waves = qa.T * (int64_t)(qa.H / 8);
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    const bool norm = WITH_KEY && ka.gamma != nullptr;
    const int sel = (is_neox ? 4 : 0) | (hadamard ? 2 : 0) | (norm ? 1 : 0);
    switch (sel) {
        case 0: return launch2(qk_small_kernel<false, false, false, WITH_KEY>, blocks, 0, stream, qa, ka);
        case 1: return launch2(qk_small_kernel<false, false, true, WITH_KEY>, blocks, 0, stream, qa, ka);
        case 2: return launch2(qk_small_kernel<false, true, false, WITH_KEY>, blocks, 0, stream, qa, ka);
        case 3: return launch2(qk_small_kernel<false, true, true, WITH_KEY>, blocks, 0, stream, qa, ka);
        case 4: return launch2(qk_small_kernel<true, false, false, WITH_KEY>, blocks, 0, stream, qa, ka);
        case 5: return launch2(qk_small_kernel<true, false, true, WITH_KEY>, blocks, 0, stream, qa, ka);
        case 6: return launch2(qk_small_kernel<true, true, false, WITH_KEY>, blocks, 0, stream, qa, ka);
        default: return launch2(qk_small_kernel<true, true, true, WITH_KEY>, blocks, 0, stream, qa, ka);
    }
}

hipError_t launch_q_rope_pack(const QArgs& a, bool is_neox, bool hadamard, hipStream_t stream) {
    if (a.T == 0) return hipSuccess;
    if (a.T < kSmallBatchTokens) return launch_small<false>(a, KArgs{}, is_neox, hadamard, stream);
    const int64_t blocks = (a.T + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = (size_t)kWavesPerBlock * 16 * a.J * sizeof(uint32_t);
    if (hadamard)
        return is_neox ? launch(q_row_kernel<true>, blocks, lds, stream, a)
                       : launch(q_row_kernel<false>, blocks, lds, stream, a);
    // two workgroups per compute unit: 409 against 431 us at 131072 x 64 with
    // the five that the registers allow
    if (is_neox)
        return launch(q_split_kernel<true>, blocks,
                      resident_cap_lds(reinterpret_cast<const void*>(q_split_kernel<true>), lds, 2),
                      stream, a);
    return launch(q_split_kernel<false>, blocks,
                  resident_cap_lds(reinterpret_cast<const void*>(q_split_kernel<false>), lds, 2),
                  stream, a);
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
    if (qa.T < kSmallBatchTokens) return launch_small<true>(qa, ka, is_neox, hadamard, stream);
    const int64_t blocks = (qa.T + kWavesPerBlock - 1) / kWavesPerBlock;
    const size_t lds = (size_t)kWavesPerBlock * 16 * qa.J * sizeof(uint32_t);
    const bool norm = ka.gamma != nullptr;
    const int sel = (is_neox ? 4 : 0) | (hadamard ? 2 : 0) | (norm ? 1 : 0);
    const unsigned kw = kBlock + 64;  // a fifth wavefront for the key rows (no Hadamard)
    // without the Hadamard, two workgroups per compute unit: 416 against 427 us
    // at 131072 x 64 with the four that the registers allow (three: 426 us)
    auto cap = [&](const void* fn) { return resident_cap_lds(fn, lds, 2); };
    switch (sel) {
        case 0: return launch2(qk_kernel<false, false, false>, blocks,
                               cap(reinterpret_cast<const void*>(qk_kernel<false, false, false>)),
                               stream, qa, ka, kw);
        case 1: return launch2(qk_kernel<false, false, true>, blocks,
                               cap(reinterpret_cast<const void*>(qk_kernel<false, false, true>)),
                               stream, qa, ka, kw);
        case 2: return launch2(qk_kernel<false, true, false>, blocks, lds, stream, qa, ka);
        case 3: return launch2(qk_kernel<false, true, true>, blocks, lds, stream, qa, ka);
        case 4: return launch2(qk_kernel<true, false, false>, blocks,
                               cap(reinterpret_cast<const void*>(qk_kernel<true, false, false>)),
                               stream, qa, ka, kw);
        case 5: return launch2(qk_kernel<true, false, true>, blocks,
                               cap(reinterpret_cast<const void*>(qk_kernel<true, false, true>)),
                               stream, qa, ka, kw);
        case 6: return launch2(qk_kernel<true, true, false>, blocks, lds, stream, qa, ka);
        default: return launch2(qk_kernel<true, true, true>, blocks, lds, stream, qa, ka);
    }
}

hipError_t launch_dequant(const DArgs& a, hipStream_t stream) {
    const int64_t chunks = a.rows * (a.which == 0 ? (int64_t)a.H * 16 : 16);
    if (chunks == 0) return hipSuccess;
    return launch(dequant_kernel, (chunks + 255) / 256, 0, stream, a);
}

}  // namespace fp4idx
