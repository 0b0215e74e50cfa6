// fp4idx_scorer.hip -- FP4 paged MQA logits on gfx950 scaled-FP4 MFMA.
//
// The consumer of the producer's bytes (ROCm/aiter PR 5484, intro and
// "Verification": flydsl_pa_mqa_logits_fp4 scores q_out/q_scale_out straight
// out of the paged cache; "API": the MFMA consumes the per-group e8m0 scales
// directly, and the scorer applies its own fp32 weights_scale).  For query
// token t of sequence b (t = b*next_n + j, position ctx_b - next_n + j) and
// key s of that sequence:
//     logits[t, s] = weights_scale * sum_h weights[t, h] * ReLU(q_h . k_s)
// with -inf where s is past the query's position or its block-table entry is
// outside the cache; entries s >= ctx_b are left untouched.
//
// Mapping onto v_mfma_scale_f32_16x16x128_f8f6f4 (E2M1 x E2M1, K = 128 in one
// instruction, one e8m0 scale per 32 K-values per row/column):
//   A = 16 query heads x 128 dims: lane L holds head (L % 16), dims
//       32 (L / 16) .. +32 = 16 bytes of q_out; its scale byte is byte
//       (head tile % 4) of the q_scale_out dword [t, 0, L / 16, L % 16, :],
//       which is why that tensor's last axis is round_up(H/16, 4).
//   B = 16 keys x 128 dims: lane L holds key 16 kt + (L % 16) of a 64-slot
//       block, group L / 16 = kv_cache[blk, 0, L/16, 16 kt + L%16, :]; its scale
//       is byte kt of the dword kv_cache_scale[blk, 0, L/16, 4 (L%16) .. +4],
//       the interleaved (pos%16)*4 + pos/16 order of ROCm/aiter PR 4029.
//   C = 16 heads x 16 keys: lane L holds heads 4 (L/16) + i, key L % 16.
// Each lane folds its 4 heads (weighted ReLU) for each of the block's four
// key tiles, then a transpose-reduce over the four 16-lane row groups leaves
// lane L with the total of key 64 blk + L, stored as one coalesced row.
// The library is built with the VGPR form of MFMA so results are read by the
// epilogue without accumulator-register copies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4idx_internal.h"

namespace fp4idx {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
// 64-slot cache blocks per wavefront: 4 for decode, 8 with query tiles, where
// the next block's fetch hides under a longer epilogue (measured at 4,096 x
// 65,536, H = 64: 1.62 -> 1.56 ms; decode at 4.6 M keys: 101 -> 106 us with 8)
template <bool TILED>
constexpr int blocks_per_wave() { return TILED ? 8 : 4; }

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// E2M1 operands occupy the low 4 dwords of the 8-dword operand; the upper 4
// are not read, so they are left undefined (no register moves to clear them).
__device__ __forceinline__ i32x8_t as_operand(u32x4_t v) {
    const i32x4_t w = __builtin_bit_cast(i32x4_t, v);
    return __builtin_shufflevector(w, w, 0, 1, 2, 3, -1, -1, -1, -1);
}

// C = A x B with scale bytes selected by the immediates SA_SEL / SB_SEL.
template <int SA_SEL, int SB_SEL>
__device__ __forceinline__ f32x4_t mma(i32x8_t a, i32x8_t b, int sa, int sb) {
    const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 4, 4, SA_SEL, sa, SB_SEL,
                                                            sb);
}

// ReLU on the bit pattern: every negative float (and -0) is a negative
// integer.  One integer max instead of a float max that the compiler would
// precede with a NaN-quieting canonicalize of each matrix-core result.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// acc += sum_i w_i * ReLU(c_i) for the lane's 4 heads
__device__ __forceinline__ float fold4(f32x4_t c, float4 w, float acc) {
    acc = __builtin_fmaf(w.x, relu(c[0]), acc);
    acc = __builtin_fmaf(w.y, relu(c[1]), acc);
    acc = __builtin_fmaf(w.z, relu(c[2]), acc);
    acc = __builtin_fmaf(w.w, relu(c[3]), acc);
    return acc;
}

__device__ __forceinline__ float fold4_linear(f32x4_t c, float4 w, float acc) {
    acc = __builtin_fmaf(w.x, c[0], acc);
    acc = __builtin_fmaf(w.y, c[1], acc);
    acc = __builtin_fmaf(w.z, c[2], acc);
    acc = __builtin_fmaf(w.w, c[3], acc);
    return acc;
}

// Static loop over the head tiles and key tiles of one query token.
template <int HT, int I, bool RELU>
struct HeadLoop {
    __device__ __forceinline__ static void run(const i32x8_t* A, const int* SA, const float4* W,
                                               const i32x8_t* Bk, int sb, float* acc) {
        const i32x8_t a = A[I];
        const int sa = SA[I / 4];
        const float4 w = W[I];
        const f32x4_t c0 = mma<I % 4, 0>(a, Bk[0], sa, sb);
        const f32x4_t c1 = mma<I % 4, 1>(a, Bk[1], sa, sb);
        const f32x4_t c2 = mma<I % 4, 2>(a, Bk[2], sa, sb);
        const f32x4_t c3 = mma<I % 4, 3>(a, Bk[3], sa, sb);
        if (RELU) {
            acc[0] = fold4(c0, w, acc[0]);
            acc[1] = fold4(c1, w, acc[1]);
            acc[2] = fold4(c2, w, acc[2]);
            acc[3] = fold4(c3, w, acc[3]);
        } else {
            acc[0] = fold4_linear(c0, w, acc[0]);
            acc[1] = fold4_linear(c1, w, acc[1]);
            acc[2] = fold4_linear(c2, w, acc[2]);
            acc[3] = fold4_linear(c3, w, acc[3]);
        }
        HeadLoop<HT, I + 1, RELU>::run(A, SA, W, Bk, sb, acc);
    }
};
template <int HT, bool RELU>
struct HeadLoop<HT, HT, RELU> {
    __device__ __forceinline__ static void run(const i32x8_t*, const int*, const float4*,
                                               const i32x8_t*, int, float*) {}
};

// acc[kt] (this lane's partial sums of key 16 kt + L%16) -> the total of key
// tile L/16 summed over the four 16-lane row groups, with the gfx950 lane
// swaps: permlane32_swap(a, b) returns ([a.lo, b.lo], [a.hi, b.hi]) and
// permlane16_swap(a, b) returns ([a.r0, b.r0, a.r2, b.r2], [a.r1, b.r1, a.r3,
// b.r3]) in 32-lane halves / 16-lane rows, so the sum of the two outputs is,
// per lane, exactly the partner total it needs (no selects, no LDS).
__device__ __forceinline__ float transpose_reduce(const float acc[4]) {
    const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[0]),
                                                      __float_as_uint(acc[2]), false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[1]),
                                                      __float_as_uint(acc[3]), false, false);
    const float n0 = __uint_as_float(p02[0]) + __uint_as_float(p02[1]);
    const float n1 = __uint_as_float(p13[0]) + __uint_as_float(p13[1]);
    const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(n0), __float_as_uint(n1),
                                                    false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Key blocks are fetched one ahead with the gfx950 LDS-DMA loads
// (global_load_lds: each lane's 16 or 4 bytes land at base + lane * size), so
// a wavefront has the next block's 4,352 bytes in flight while it scores the
// current one, without spending registers on them.  Lane L fetches bytes
// 16 L + 1024 i of the block (i = 0..3) and its scale dword 4 L, so the two
// buffers of a wavefront hold the block's codes and scale row verbatim:
//   kbuf[p][wave]: kv_cache[blk, 0, :, :, :] (4,096 bytes),
//   sbuf[p][wave]: kv_cache_scale[blk, 0, :, :] (256 bytes),
// and each lane reads its matrix-core operand at the offset it has in the
// block (group g = L / 16, key 16 kt + L % 16).
// The compiler cannot tell the two buffers apart and would wait for every
// load in flight before any read of either, so the wait is explicit (vmcnt
// counts only this wavefront's vector memory operations, which complete in
// issue order: after the next block's 5 loads are issued, vmcnt(5) means the
// current block has landed) and the reads are one asm block that waits for
// its own LDS reads before it ends.
constexpr int kBlockBytes = 64 * 4 * 16;  // one 64-slot block of codes

constexpr int waitcnt_vmcnt(int n) {  // s_waitcnt with only vmcnt limited (gfx9 encoding)
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void fetch_block(const LArgs& a, int32_t blk, int lane, uint8_t* kl,
                                            uint32_t* sl) {
    const uint8_t* base = a.kv_cache + (int64_t)blk * kBlockBytes + 16 * lane;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
        __builtin_amdgcn_global_load_lds(base + kt * 1024, (lds_ptr_t)(kl + kt * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(a.kv_cache_scale + (int64_t)blk * 256 + 4 * lane,
                                     (lds_ptr_t)sl, 4, 0, 0);
}

// The lane's four code pieces and scale dword of a fetched block.
__device__ __forceinline__ void read_block(const uint8_t* kl, const uint32_t* sl, int lane,
                                           u32x4_t v[4], int& sb) {
    const uint32_t ka = (uint32_t)(uintptr_t)(lds_ptr_t)kl + 1024 * (lane >> 4) + 16 * (lane & 15);
    const uint32_t sa = (uint32_t)(uintptr_t)(lds_ptr_t)sl + 4 * lane;
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:256\n\t"
        "ds_read_b128 %2, %5 offset:512\n\t"
        "ds_read_b128 %3, %5 offset:768\n\t"
        "ds_read_b32 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(sb)
        : "v"(ka), "v"(sa)
        : "memory");
}

// Query tokens come in tiles of NQ: with next_n <= 4 one tile of next_n
// tokens (decode with multi-token prediction; TILED = false, everything known
// at compile time), with larger next_n (chunked prefill; TILED = true) tiles
// of NQ = 2 or 4 on blockIdx.z and a last tile of next_n % NQ.  A key block that lies
// entirely after the tile's last position holds -inf for every query of the
// tile and is not read.
template <int NQ, int HT, bool RELU, bool TILED>
__global__ __launch_bounds__(64 * kWaves) void mqa_logits_kernel(LArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t b = blockIdx.y;
    const int j0 = TILED ? (int)blockIdx.z * NQ : 0;  // first query of the tile
    const int nq = TILED ? min(NQ, a.next_n - j0) : NQ;  // queries in the tile (>= 1)
    int64_t ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : ctx;
    ctx = ctx > a.max_blocks * 64 ? a.max_blocks * 64 : ctx;
    ctx = ctx > a.stride ? a.stride : ctx;
    const int64_t nblk = (ctx + 63) >> 6;
    constexpr int BPW = blocks_per_wave<TILED>();
    const int64_t kb0 = ((int64_t)blockIdx.x * kWaves + wave) * BPW;
    if (kb0 >= nblk) return;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int H = HT * 16;
    const int J = a.J;
    const int64_t t0 = b * a.next_n + j0;            // token row of the tile's first query
    const int64_t p_last = ctx - a.next_n + j0 + nq - 1;

    // query operands of the tile's tokens, kept in registers (zeros past nq)
    i32x8_t A[NQ][HT];
    int SA[NQ][(HT + 3) / 4];
    float4 W[NQ][HT];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int64_t t = t0 + j;
        const bool live = j < nq;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            A[j][ht] = live ? as_operand(*reinterpret_cast<const u32x4_t*>(
                                  a.q_out + ((t * H + 16 * ht + n) * 64 + 16 * g)))
                            : i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
            W[j][ht] = live ? *reinterpret_cast<const float4*>(a.weights + t * H + 16 * ht + 4 * g)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int d = 0; d < (HT + 3) / 4; ++d)
            SA[j][d] = live ? *reinterpret_cast<const int*>(a.q_scale_out + t * 64 * (int64_t)J +
                                                            (g * 16 + n) * J + 4 * d)
                            : 0;
    }

    const int64_t kb_end = kb0 + BPW < nblk ? kb0 + BPW : nblk;
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kWaves][kBlockBytes];
    __shared__ __attribute__((aligned(16))) uint32_t sbuf[2][kWaves][64];
    const int32_t* table = a.block_table + b * a.max_blocks;
    // a block is read when some query of the tile sees it and its entry is valid
    auto fetched = [&](int64_t kb, int32_t blk) {
        return !(TILED && kb * 64 > p_last) && blk >= 0 && (int64_t)blk < a.nblocks;
    };
    // the wavefront's block-table entries, read before any fetch is in flight
    int32_t blks[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i) blks[i] = kb0 + i < kb_end ? table[kb0 + i] : -1;
    // the query operands are in registers before the first block is fetched, so
    // no wait inside the loop has to cover them
    __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
    bool has_next = fetched(kb0, blks[0]);
    if (has_next) fetch_block(a, blks[0], lane, kbuf[0][wave], sbuf[0][wave]);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int64_t kb = kb0 + i;
        if (kb >= kb_end) break;
        const int p = i & 1;
        const int64_t s = kb * 64 + lane;
        const bool valid = has_next;  // this block was fetched
        // issue the next block's loads, then wait for this block's (uniform branches)
        has_next = i + 1 < BPW && kb + 1 < kb_end && fetched(kb + 1, blks[i + 1]);
        if (has_next) {
            fetch_block(a, blks[i + 1], lane, kbuf[p ^ 1][wave], sbuf[p ^ 1][wave]);
            // at most the next block's 5 loads may still be in flight: this
            // block's loads, and everything issued before them, have landed
            // (whatever else the previous block issued)
            __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(5));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
        }
        if (TILED && kb * 64 > p_last) {  // after every query of the tile
#pragma unroll
            for (int j = 0; j < NQ; ++j)
                if (j < nq && s < ctx)
                    __builtin_nontemporal_store(-__builtin_huge_valf(),
                                                a.logits + (t0 + j) * a.stride + s);
            continue;
        }
        i32x8_t Bk[4];
        int sb = 0;
        if (valid) {
            u32x4_t v[4];
            read_block(kbuf[p][wave], sbuf[p][wave], lane, v, sb);
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) Bk[kt] = as_operand(v[kt]);
        } else {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) Bk[kt] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if (j < nq) {  // uniform: the tile's token count
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
                HeadLoop<HT, 0, RELU>::run(A[j], SA[j], W[j], Bk, sb, acc);
                const float v = transpose_reduce(acc);
                const int64_t pos = p_last - (nq - 1) + j;
                const float out =
                    (!valid || s > pos) ? -__builtin_huge_valf() : a.weights_scale * v;
                if (s < ctx) __builtin_nontemporal_store(out, a.logits + (t0 + j) * a.stride + s);
            }
        }
    }
}

// ---- decode over a flat, balanced list of block quads ----------------------------
// Decode (next_n <= 4) with B <= kFlatMaxB sequences.  A sequence's key blocks
// are taken in quads (blocks 4q .. 4q+3, the last quad of a sequence possibly
// short); the quads of all sequences form one flat list and every wavefront of
// the grid takes an equal contiguous range of it, so no wavefront idles on a
// short sequence and none exits without work.  Each workgroup first builds the
// inclusive prefix of the per-sequence quad counts in LDS; a wavefront maps the
// blocks of a window of 16 quads to (sequence, block index) by binary search
// with one lane per block, reads their block-table entries with one load per
// lane, and walks them with each block fetched one ahead into a ring of two
// LDS buffers (fetching two ahead into three buffers measured 2% slower: 80-82
// against 79-80 us on the 4.6 M-key decode batch).  The query operands of a
// sequence are loaded when the walk enters it.
//
// Key order inside a block: matrix-core tile kt takes keys 4n + kt (n = lane %
// 16), so after the cross-row reduce lane 16r + m holds key 4m + r.  Four such
// results (the quad's blocks) go through a 4 x 4 exchange of 16-lane rows
// across registers, after which lane 16r' + m' holds keys 4m' .. 4m' + 3 of
// block r' of the quad: each query token's logits of the quad (1 KB) leave in
// one 16-byte-per-lane store.  The scale byte of key 4n + kt in its group row
// (interleaved order (p % 16) * 4 + p / 16) is byte n / 4 of dword
// 4 (n % 4) + kt, so a lane reads the 16 bytes at 16 (n % 4) and picks byte
// n / 4 of each dword with byte permutes.
constexpr int kFlatMaxB = 1024;
constexpr int kRing = 2;

__device__ __forceinline__ void wait_prefetch(int n_after) {
    // n_after blocks (5 loads each) were fetched after the block that is needed:
    // once at most their loads are in flight, that block and everything issued
    // before it has landed (vector memory operations complete in issue order),
    // whatever else was issued in between
    if (n_after >= 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(5));
    else
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
}

// The lane's four code pieces (keys 4n + kt, group g) and the scale dword whose
// byte kt belongs to key 4n + kt.
__device__ __forceinline__ void read_block_strided(const uint8_t* kl, const uint32_t* sl, int lane,
                                                   uint32_t sel, u32x4_t v[4], int& sb) {
    const uint32_t ka = (uint32_t)(uintptr_t)(lds_ptr_t)kl + 1024 * (lane >> 4) + 64 * (lane & 15);
    const uint32_t sa = (uint32_t)(uintptr_t)(lds_ptr_t)sl + 64 * (lane >> 4) + 16 * (lane & 3);
    u32x4_t d;
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:16\n\t"
        "ds_read_b128 %2, %5 offset:32\n\t"
        "ds_read_b128 %3, %5 offset:48\n\t"
        "ds_read_b128 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(d)
        : "v"(ka), "v"(sa)
        : "memory");
    const uint32_t x01 = __builtin_amdgcn_perm(d[1], d[0], sel);
    const uint32_t x23 = __builtin_amdgcn_perm(d[3], d[2], sel);
    sb = (int)__builtin_amdgcn_perm(x23, x01, 0x05040100u);
}

// rows (16 lanes) r of E[b] -> row b of T[r]: T[i] lane 16 r' + m' = E[r'] lane 16 i + m'
__device__ __forceinline__ void exchange4x4(const float E[4], float T[4]) {
    const auto p02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(E[0]), __float_as_uint(E[2]),
                                                      false, false);
    const auto p13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(E[1]), __float_as_uint(E[3]),
                                                      false, false);
    const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
    const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
    T[0] = __uint_as_float(q01[0]);
    T[1] = __uint_as_float(q01[1]);
    T[2] = __uint_as_float(q23[0]);
    T[3] = __uint_as_float(q23[1]);
}

template <int NQ, int HT, bool RELU>
__global__ __launch_bounds__(64 * kWaves, HT <= 2 ? 3 : 2) void mqa_logits_flat_kernel(LArgs a) {
    extern __shared__ int32_t prefix[];  // [B] inclusive quad counts
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[kRing][kWaves][kBlockBytes];
    __shared__ __attribute__((aligned(16))) uint32_t sbuf[kRing][kWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int B = (int)a.B;
    const int64_t ctx_cap = a.max_blocks * 64 < a.stride ? a.max_blocks * 64 : a.stride;
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < B; base += 64) {
            int v = 0;
            if (base + lane < B) {
                int64_t c = a.context_lens[base + lane];
                c = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
                v = (int)((c + 255) >> 8);
            }
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int u = __shfl_up(v, d, 64);
                if (lane >= d) v += u;
            }
            if (base + lane < B) prefix[base + lane] = carry + v;
            carry += __shfl(v, 63, 64);
        }
    }
    __syncthreads();
    const int64_t nquads = prefix[B - 1];
    const int64_t W = (int64_t)gridDim.x * kWaves;
    const int64_t w = (int64_t)blockIdx.x * kWaves + wave;
    const int64_t lo = w * nquads / W;
    const int64_t hi = (w + 1) * nquads / W;
    if (lo >= hi) return;

    const int n = lane & 15;
    const int g = lane >> 4;
    const int H = HT * 16;
    const int J = a.J;
    // byte n/4 of two dwords: selector bytes (n/4, 4 + n/4, zero, zero)
    const uint32_t sel = (uint32_t)(n >> 2) | ((uint32_t)(4 + (n >> 2)) << 8) | 0x0C0C0000u;
    // key of this lane's reduced result inside a block, and of its stored values
    const int key_red = 4 * n + g;
    i32x8_t A[NQ][HT];
    int SA[NQ][(HT + 3) / 4];
    float4 W4[NQ][HT];
    int cur_b = -1;
    int64_t ctx = 0;
    float E[NQ][4];  // the quad's reduced results per query token, block by block

    for (int64_t win = lo; win < hi; win += 16) {
        const int nq_win = (int)(hi - win < 16 ? hi - win : 16);
        const int cnt = 4 * nq_win;  // block slots of the window, 4 per quad
        // lane i: block i % 4 of quad win + i / 4 -> sequence, block index, entry
        int bi = 0, kbi = 0, blki = -1, live = 0;
        if (lane < cnt) {
            const int qf = (int)(win + (lane >> 2));
            int l = 0, r = B;  // first sequence whose inclusive quad count exceeds qf
            while (l < r) {
                const int m = (l + r) >> 1;
                if (prefix[m] > qf) r = m; else l = m + 1;
            }
            bi = l;
            kbi = 4 * (qf - (l ? prefix[l - 1] : 0)) + (lane & 3);
            int64_t c = a.context_lens[l];
            c = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
            live = (int64_t)kbi * 64 < c;  // the quad's last blocks may lie past the context
            if (live) blki = a.block_table[(int64_t)bi * a.max_blocks + kbi];
        }
        // the previous window's blocks were all consumed; the table entries land
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
        auto fetched = [&](int j) {
            if (j >= cnt) return false;
            const int32_t blk = __builtin_amdgcn_readlane(blki, j);
            return blk >= 0 && (int64_t)blk < a.nblocks;
        };
        auto fetch = [&](int j) {
            const int32_t blk = __builtin_amdgcn_readlane(blki, j);
            fetch_block(a, blk, lane, kbuf[j % kRing][wave], sbuf[j % kRing][wave]);
        };
        bool f1 = fetched(0);
        if (f1) fetch(0);
        int b = 0;
        int64_t kb = 0;
        for (int qi = 0; qi < nq_win; ++qi) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 4 * qi + r;
                const bool f0 = f1;  // block slot j was fetched
                f1 = fetched(j + 1);
                if (f1) fetch(j + 1);  // into the ring slot block j - 1 left
                b = __builtin_amdgcn_readlane(bi, j);
                kb = __builtin_amdgcn_readlane(kbi, j);
                if (__builtin_amdgcn_readlane(live, j) == 0) continue;  // past the context
                wait_prefetch((int)f1);
                if (b != cur_b) {  // entering a sequence: its query operands
                    cur_b = b;
                    int64_t c = a.context_lens[b];
                    ctx = c < 0 ? 0 : (c > ctx_cap ? ctx_cap : c);
                    const int64_t t0 = (int64_t)b * NQ;
#pragma unroll
                    for (int jj = 0; jj < NQ; ++jj) {
                        const int64_t t = t0 + jj;
#pragma unroll
                        for (int ht = 0; ht < HT; ++ht) {
                            A[jj][ht] = as_operand(*reinterpret_cast<const u32x4_t*>(
                                a.q_out + ((t * H + 16 * ht + n) * 64 + 16 * g)));
                            W4[jj][ht] = *reinterpret_cast<const float4*>(
                                a.weights + t * H + 16 * ht + 4 * g);
                        }
#pragma unroll
                        for (int d = 0; d < (HT + 3) / 4; ++d)
                            SA[jj][d] = *reinterpret_cast<const int*>(
                                a.q_scale_out + t * 64 * (int64_t)J + (g * 16 + n) * J + 4 * d);
                    }
                    __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
                }
                i32x8_t Bk[4];
                int sb = 0;
                if (f0) {
                    u32x4_t v[4];
                    read_block_strided(kbuf[j % kRing][wave], sbuf[j % kRing][wave], lane, sel, v,
                                       sb);
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) Bk[kt] = as_operand(v[kt]);
                } else {
#pragma unroll
                    for (int kt = 0; kt < 4; ++kt) Bk[kt] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
                }
                const int64_t s = kb * 64 + key_red;
#pragma unroll
                for (int jj = 0; jj < NQ; ++jj) {
                    float acc[4] = {0.f, 0.f, 0.f, 0.f};
                    HeadLoop<HT, 0, RELU>::run(A[jj], SA[jj], W4[jj], Bk, sb, acc);
                    const float v = transpose_reduce(acc);
                    const int64_t pos = ctx - NQ + jj;
                    E[jj][r] = (!f0 || s > pos) ? -__builtin_huge_valf() : a.weights_scale * v;
                }
            }
            // The quad's logits leave: lane 16 r' + m' holds keys 4 m' .. 4 m' + 3 of
            // block r'.  The quad's first block always lies inside the context, so b
            // and ctx are the quad's sequence; blocks past the context (their E
            // entries are stale) have every key >= ctx and store nothing.
            const int64_t s0 = (kb - 3 + g) * 64 + 4 * n;
#pragma unroll
            for (int jj = 0; jj < NQ; ++jj) {
                float T[4];
                exchange4x4(E[jj], T);
                float* row = a.logits + ((int64_t)b * NQ + jj) * a.stride;
                if (a.logits_vec4 && s0 + 4 <= ctx) {
                    const f32x4_t q4 = {T[0], T[1], T[2], T[3]};
                    __builtin_nontemporal_store(q4, reinterpret_cast<f32x4_t*>(row + s0));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (s0 + i < ctx) __builtin_nontemporal_store(T[i], row + s0 + i);
                }
            }
        }
    }
}

template <int NQ, int HT, bool RELU>
const void* kernel_for(bool tiled) {
    if constexpr (NQ == 2 || NQ == 4)
        if (tiled) return reinterpret_cast<const void*>(mqa_logits_kernel<NQ, HT, RELU, true>);
    return reinterpret_cast<const void*>(mqa_logits_kernel<NQ, HT, RELU, false>);
}

template <int NQ, int HT>
hipError_t launch_nq_ht(const LArgs& a, hipStream_t stream) {
    // the grid must match the kernel kernel_for picks (its blocks per wavefront)
    const bool tiled = (NQ == 2 || NQ == 4) && a.next_n > NQ;
    const int64_t per_wg =
        (int64_t)kWaves * (tiled ? blocks_per_wave<true>() : blocks_per_wave<false>());
    dim3 grid((unsigned)((a.max_blocks + per_wg - 1) / per_wg), (unsigned)a.B,
              (unsigned)((a.next_n + NQ - 1) / NQ));
    LArgs copy = a;
    void* args[] = {&copy};
    const void* fn = a.apply_relu ? kernel_for<NQ, HT, true>(tiled)
                                  : kernel_for<NQ, HT, false>(tiled);
    return hipLaunchKernel(fn, grid, dim3(64 * kWaves), args, 0, stream);
}

// Workgroups the flat decode grid keeps resident: compute units x the
// kernel's occupancy (looked up once per device and kernel).
template <int NQ, int HT>
hipError_t launch_flat(const LArgs& a, hipStream_t stream) {
    const void* fn = a.apply_relu
                         ? reinterpret_cast<const void*>(mqa_logits_flat_kernel<NQ, HT, true>)
                         : reinterpret_cast<const void*>(mqa_logits_flat_kernel<NQ, HT, false>);
    const size_t lds = (size_t)a.B * sizeof(int32_t);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 64 * kWaves, lds);
    if (e != hipSuccess) return e;
    // no more wavefronts than quads to score (bounded by B x max_blocks / 4)
    const int64_t most = (a.B * ((a.max_blocks + 3) / 4) + kWaves - 1) / kWaves;
    int64_t wgs = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    wgs = wgs < most ? wgs : most;
    LArgs copy = a;
    copy.logits_vec4 = ((uintptr_t)a.logits % 16 == 0) && (a.stride % 4 == 0);
    void* args[] = {&copy};
    return hipLaunchKernel(fn, dim3((unsigned)wgs), dim3(64 * kWaves), args, lds, stream);
}

template <int NQ>
hipError_t launch_nq(const LArgs& a, hipStream_t stream) {
    if (a.next_n <= 4 && a.B <= kFlatMaxB && a.B * a.max_blocks < ((int64_t)1 << 31)) {
        switch (a.H / 16) {
            case 1: return launch_flat<NQ, 1>(a, stream);
            case 2: return launch_flat<NQ, 2>(a, stream);
            case 3: return launch_flat<NQ, 3>(a, stream);
            default: return launch_flat<NQ, 4>(a, stream);
        }
    }
    switch (a.H / 16) {
        case 1: return launch_nq_ht<NQ, 1>(a, stream);
        case 2: return launch_nq_ht<NQ, 2>(a, stream);
        case 3: return launch_nq_ht<NQ, 3>(a, stream);
        default: return launch_nq_ht<NQ, 4>(a, stream);
    }
}

}  // namespace

hipError_t launch_paged_mqa_logits(const LArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.max_blocks == 0) return hipSuccess;
    // Above 4 query tokens (chunked prefill), tiles of 4 at H = 32 and of 2
    // otherwise: at H = 48 and 64, four tokens' query operands and weights take
    // ~180 VGPRs (2 wavefronts per SIMD) and tiles of 2 ran 13% faster at
    // 4096 x 65536, H = 64 (1 token per tile was 8% slower than 2); at H = 32
    // tiles of 4 were 5% faster, at H = 16 tiles of 2 were 9% faster.
    if (a.next_n > 4) return a.H == 32 ? launch_nq<4>(a, stream) : launch_nq<2>(a, stream);
    switch (a.next_n) {
        case 1: return launch_nq<1>(a, stream);
        case 2: return launch_nq<2>(a, stream);
        case 3: return launch_nq<3>(a, stream);
        default: return launch_nq<4>(a, stream);
    }
}

}  // namespace fp4idx
