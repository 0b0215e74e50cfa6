// fp4idx_ceiling.hip -- measurement kernels: the HBM rate that plain traffic of
// a given shape reaches on this GPU, with none of the method's arithmetic.
// They set the ceilings the producer and scorer kernels are compared with:
//   - a stream that reads R bytes and writes W bytes, the writes spread evenly
//     over the reads (read-only: W = 0; the producer's 79:21 mix; a 1:1 copy);
//   - a gather of whole paged-cache blocks (4,096 code bytes and the 256-byte
//     scale row of each block named by a block table) with the scorer's flat,
//     balanced decomposition, writing next_n fp32 values per key as the scorer
//     writes its logits.
//   - a VALU issue-rate kernel: independent chains of one instruction kind,
//     the rate the ALU-bound kernels are set against.
// Every load feeds a store, so no access is dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4idx_ceiling.h"

namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld_nt(const u32x4_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4_t* p, u32x4_t v) { __builtin_nontemporal_store(v, p); }

// The stream works in units of 1 KB (64 lanes x 16 bytes), U consecutive
// units per wavefront step: a wavefront takes steps s = w, w + W, ... (W
// wavefronts in the grid), issues the loads of units U s .. U s + U - 1
// together, and after unit u, whenever the running write count (u + 1) * ratio
// crosses an integer, writes the next 1 KB write unit with that unit's data, so
// writes follow reads evenly at the ratio nw:nr (ratio = nw / nr in 32.32 fixed
// point, nw <= nr).  Units past the mixed part are written by a write-only
// loop.  A read-only stream folds its data into one value per lane and stores
// it only if every bit of it is set, which zero-filled buffers never produce.
// Shapes by measurement: read-only, U = 4 on two workgroups per compute unit
// (7.2-7.3 TB/s, against 6.95 with U = 1 at full occupancy); with writes, U = 1
// at full occupancy (a 1:1 copy ran at 5.4 TB/s, at 4.9 with U = 4 on the
// smaller grid).
template <int U>
__global__ __launch_bounds__(kThreads) void stream_kernel(const u32x4_t* __restrict__ src,
                                                          u32x4_t* __restrict__ dst, int64_t nr,
                                                          uint64_t ratio, int64_t nw_mixed,
                                                          int64_t nw) {
    const int lane = threadIdx.x & 63;
    const int64_t W = (int64_t)gridDim.x * (kThreads / 64);
    const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    u32x4_t acc = {0u, 0u, 0u, 0u};
    for (int64_t st = w; st * U < nr; st += W) {
        u32x4_t v[U];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t u = st * U + i;
            v[i] = u < nr ? ld_nt(src + u * 64 + lane) : (u32x4_t){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int64_t u = st * U + i;
            if (u >= nr) break;
            acc ^= v[i];
            const int64_t k0 = (int64_t)(((uint64_t)u * ratio) >> 32);
            const int64_t k1 = (int64_t)(((uint64_t)(u + 1) * ratio) >> 32);
            if (k1 > k0 && k0 < nw_mixed) st_nt(dst + k0 * 64 + lane, v[i]);
        }
    }
    for (int64_t k = nw_mixed + w; k < nw; k += W) st_nt(dst + k * 64 + lane, acc);
    if (acc.x == 0xFFFFFFFFu && acc.y == 0xFFFFFFFFu && acc.z == 0xFFFFFFFFu &&
        acc.w == 0xFFFFFFFFu)
        dst[lane] = acc;
}

// ---- paged gather with the decode scorer's decomposition --------------------
// Quads of blocks (4q .. 4q+3 of one sequence) in one flat list, equal
// contiguous ranges per wavefront, as the decode scorer takes them, and the
// scorer's kind of data movement: each block's 4,096 code bytes and 256-byte
// scale row come in through LDS-DMA loads (global_load_lds: lane L's 16 or 4
// bytes land at the slot base + 16 L or 4 L) into a ring of slots per
// wavefront, here three slots two blocks ahead of the one being read (the
// fastest depth for the reads alone; the scorer, with its arithmetic between
// reads, keeps one block ahead in two).  A block is read out of LDS and
// folded into one value per lane; each quad's next_n logit rows leave as 1 KB
// stores, lane 16 r + m covering keys 4 m .. 4 m + 3 of the quad's block r.
// (A ring of four register sets, three blocks ahead, at five wavefronts per
// SIMD moved the same bytes 8% slower.)
constexpr int kGatherMaxB = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRing = 3;
constexpr int kBlockBytes = 4096;

struct GatherArgs {
    const uint8_t* kv_cache;
    const uint8_t* kv_cache_scale;
    const int32_t* block_table;
    const int32_t* context_lens;
    float* logits;
    int64_t nblocks;
    int64_t max_blocks;
    int64_t B;
    int64_t stride;
    int next_n;
    int vec4;
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int waitcnt_vmcnt(int n) {  // s_waitcnt with only vmcnt limited (gfx9 encoding)
    return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// Block blk's codes and scale row into one ring slot: five loads.
__device__ __forceinline__ void fetch_block(const GatherArgs& a, int32_t blk, int lane, uint8_t* kl,
                                            uint32_t* sl) {
    const uint8_t* base = a.kv_cache + (int64_t)blk * kBlockBytes + 16 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds(base + 1024 * i, (lds_ptr_t)(kl + 1024 * i), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(a.kv_cache_scale + (int64_t)blk * 256 + 4 * lane,
                                     (lds_ptr_t)sl, 4, 0, 0);
}

// Vector memory operations complete in issue order: with the loads of n_after
// later blocks (5 each) allowed in flight, every earlier block has landed.
__device__ __forceinline__ void wait_landed(int n_after) {
    if (n_after >= 2)
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(10));
    else if (n_after == 1)
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(5));
    else
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
}

// The lane's 64 bytes of a landed slot and its scale dword, folded to 32 bits;
// the reads wait for themselves before the block ends.
__device__ __forceinline__ uint32_t fold_slot(const uint8_t* kl, const uint32_t* sl, int lane) {
    const uint32_t ka = (uint32_t)(uintptr_t)(lds_ptr_t)kl + 16 * lane;
    const uint32_t sa = (uint32_t)(uintptr_t)(lds_ptr_t)sl + 4 * lane;
    u32x4_t v0, v1, v2, v3;
    uint32_t sc;
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:1024\n\t"
        "ds_read_b128 %2, %5 offset:2048\n\t"
        "ds_read_b128 %3, %5 offset:3072\n\t"
        "ds_read_b32 %4, %6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(sc)
        : "v"(ka), "v"(sa)
        : "memory");
    const u32x4_t x = v0 ^ v1 ^ v2 ^ v3;
    return x.x ^ x.y ^ x.z ^ x.w ^ sc;
}

__global__ __launch_bounds__(kThreads) void gather_kernel(GatherArgs a) {
    extern __shared__ int32_t prefix[];  // [B] inclusive quad counts
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[kRing][kWaves][kBlockBytes];
    __shared__ __attribute__((aligned(16))) uint32_t sbuf[kRing][kWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int B = (int)a.B;
    const int64_t cap = a.max_blocks * 64 < a.stride ? a.max_blocks * 64 : a.stride;
    if (wave == 0) {
        int carry = 0;
        for (int base = 0; base < B; base += 64) {
            int v = 0;
            if (base + lane < B) {
                int64_t c = a.context_lens[base + lane];
                c = c < 0 ? 0 : (c > cap ? cap : c);
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
    const int64_t lo = w * nquads / W, hi = (w + 1) * nquads / W;
    const int g = lane >> 4, n = lane & 15;
    int cur_b = -1;
    int64_t ctx = 0;
    for (int64_t win = lo; win < hi; win += 16) {
        const int nq_win = (int)(hi - win < 16 ? hi - win : 16);
        const int cnt = 4 * nq_win;
        int bi = 0, kbi = 0, blki = -1;
        if (lane < cnt) {
            const int qf = (int)(win + (lane >> 2));
            int l = 0, r = B;
            while (l < r) {
                const int m = (l + r) >> 1;
                if (prefix[m] > qf) r = m; else l = m + 1;
            }
            bi = l;
            kbi = 4 * (qf - (l ? prefix[l - 1] : 0)) + (lane & 3);
            int64_t c = a.context_lens[l];
            c = c < 0 ? 0 : (c > cap ? cap : c);
            if ((int64_t)kbi * 64 < c) blki = a.block_table[(int64_t)bi * a.max_blocks + kbi];
        }
        // the previous window's blocks were all read; the entries land
        __builtin_amdgcn_s_waitcnt(waitcnt_vmcnt(0));
        auto fetched = [&](int j) {
            if (j >= cnt) return false;
            const int32_t blk = __builtin_amdgcn_readlane(blki, j);
            return blk >= 0 && (int64_t)blk < a.nblocks;
        };
        auto fetch = [&](int j) {
            fetch_block(a, __builtin_amdgcn_readlane(blki, j), lane, kbuf[j % kRing][wave],
                        sbuf[j % kRing][wave]);
        };
        bool f1 = fetched(0), f2 = fetched(1);
        if (f1) fetch(0);
        if (f2) fetch(1);
        for (int qi = 0; qi < nq_win; ++qi) {
            const int b = __builtin_amdgcn_readlane(bi, 4 * qi);
            const int64_t kb0 = __builtin_amdgcn_readlane(kbi, 4 * qi);
            if (b != cur_b) {
                cur_b = b;
                int64_t c = a.context_lens[b];
                ctx = c < 0 ? 0 : (c > cap ? cap : c);
            }
            uint32_t u = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int j = 4 * qi + r;
                const bool f0 = f1;  // block slot j was fetched
                f1 = f2;
                f2 = fetched(j + 2);
                if (f2) fetch(j + 2);  // into the slot block j - 1 left
                wait_landed((int)f1 + (int)f2);
                const uint32_t x = f0 ? fold_slot(kbuf[j % kRing][wave], sbuf[j % kRing][wave], lane)
                                      : 0u;
                if (g == r) u = x & 0x3FFFFFFFu;
            }
            const f32x4_t o = {__uint_as_float(u), __uint_as_float(u ^ 1u), __uint_as_float(u ^ 2u),
                               __uint_as_float(u ^ 3u)};
            const int64_t s0 = (kb0 + g) * 64 + 4 * n;
            for (int jj = 0; jj < a.next_n; ++jj) {
                float* row = a.logits + ((int64_t)b * a.next_n + jj) * a.stride;
                if (a.vec4 && s0 + 4 <= ctx) {
                    __builtin_nontemporal_store(o, reinterpret_cast<f32x4_t*>(row + s0));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (s0 + i < ctx) __builtin_nontemporal_store(o[i], row + s0 + i);
                }
            }
        }
    }
}

// VALU issue rate of one instruction kind: every lane runs 8 independent chains
// of `iterations` steps (8 wave instructions per step, so the issue rate, not
// the latency of one chain, limits a SIMD holding several wavefronts) and
// stores one dword that depends on all of them.
//   0  fp32 add              v_add_f32           f = f + y
//   1  fp32 fused mul-add    v_fma_f32 / fmac    f = fma(f, y, z)
//   2  fp32 max              v_max_f32           f = max(f, y)
//   3  fp32 -> packed bf16   v_cvt_pk_bf16_f32   u = bf16x2(u, u')
//   4  bf16 -> E2M1 scaled   v_cvt_scalef32_pk_fp4_bf16, one byte of u
typedef __bf16 ceil_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float ceil_f32x2_t __attribute__((ext_vector_type(2)));

template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_kernel(uint32_t* out, int64_t iterations, float y,
                                                       float z) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    float f[8];
    uint32_t u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        f[i] = (float)(tid & 1023) * 0.001f + (float)i;
        u[i] = (uint32_t)tid * 2654435761u + 0x3F803F80u * (uint32_t)i;
    }
    // the step operands in vector registers, as the kernels measured against
    // hold theirs (an operand read from a scalar register measured slower)
    float yv, zv;
    asm("v_mov_b32 %0, %1" : "=v"(yv) : "s"(y));
    asm("v_mov_b32 %0, %1" : "=v"(zv) : "s"(z));
    auto step = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (KIND == 0) f[i] = f[i] + yv;
            if (KIND == 1) f[i] = __builtin_fmaf(f[i], yv, zv);
            // written out: fmaxf would first quiet signalling NaNs with a
            // second max of the operand with itself
            if (KIND == 2) asm("v_max_f32_e32 %0, %0, %1" : "+v"(f[i]) : "v"(yv));
            if (KIND == 3) {
                const ceil_f32x2_t v = {__uint_as_float(u[i]), __uint_as_float(u[(i + 1) & 7])};
                u[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, ceil_bf16x2_t));
            }
            if (KIND == 4)
                u[i] = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    u[i], __builtin_bit_cast(ceil_bf16x2_t, u[(i + 3) & 7]), yv, 0);
        }
    };
    // four steps per trip, so the loop's scalar bookkeeping is a small share
    int64_t it = 0;
    for (; it + 4 <= iterations; it += 4) {
        step();
        step();
        step();
        step();
    }
    for (; it < iterations; ++it) step();
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) r ^= u[i] ^ __float_as_uint(f[i]);
    out[tid] = r;
}

int device_wgs(const void* fn, size_t lds, int* wgs) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 3;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 3;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess)
        return 3;
    *wgs = cus * (per_cu > 0 ? per_cu : 1);
    return 0;
}

}  // namespace

extern "C" int fp4idx_ceiling_stream(const void* src, int64_t read_bytes, void* dst,
                                     int64_t write_bytes, void* stream) {
    if (read_bytes < 0 || write_bytes < 0 || read_bytes % 1024 || write_bytes % 1024) return 1;
    if ((read_bytes && !src) || !dst) return 1;
    if (((uintptr_t)src | (uintptr_t)dst) & 15) return 1;
    if (read_bytes > ((int64_t)1 << 40) || write_bytes > ((int64_t)1 << 40)) return 1;
    int64_t nr = read_bytes / 1024, nw = write_bytes / 1024;  // 1 KB units
    if (nr == 0 && nw == 0) return 0;
    // writes up to the read count are spread over the reads, the rest follow
    int64_t nw_mixed = nw < nr ? nw : nr;
    uint64_t ratio = nr ? (uint64_t)(((unsigned __int128)nw_mixed << 32) / (uint64_t)nr) : 0;
    // (u + 1) * ratio >> 32 may fall short of nw_mixed by rounding: the
    // write-only loop covers from the last unit the mixed part reaches
    nw_mixed = nr ? (int64_t)(((unsigned __int128)nr * ratio) >> 32) : 0;
    const bool read_only = nw == 0;
    const void* fn = read_only ? reinterpret_cast<const void*>(stream_kernel<4>)
                               : reinterpret_cast<const void*>(stream_kernel<1>);
    int wgs = 0;
    if (read_only) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 3;
        wgs = 2 * cus;
    } else if (device_wgs(fn, 0, &wgs)) {
        return 3;
    }
    const u32x4_t* s = static_cast<const u32x4_t*>(src);
    u32x4_t* d = static_cast<u32x4_t*>(dst);
    void* args[] = {&s, &d, &nr, &ratio, &nw_mixed, &nw};
    return hipLaunchKernel(fn, dim3(wgs), dim3(kThreads), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 3;
}

extern "C" int fp4idx_ceiling_paged_gather(const uint8_t* kv_cache, const uint8_t* kv_cache_scale,
                                           int64_t NB, const int32_t* block_table,
                                           int64_t max_blocks, const int32_t* context_lens,
                                           int64_t B, int next_n, float* logits, int64_t stride,
                                           void* stream) {
    if (B < 1 || B > kGatherMaxB || max_blocks < 1 || NB < 0 || stride < 1 || next_n < 1 ||
        next_n > 64 || B * max_blocks >= ((int64_t)1 << 31))
        return 1;
    if (!kv_cache || !kv_cache_scale || !block_table || !context_lens || !logits) return 1;
    if (((uintptr_t)kv_cache & 15) || ((uintptr_t)kv_cache_scale & 3)) return 1;
    GatherArgs a{kv_cache, kv_cache_scale, block_table, context_lens, logits, NB, max_blocks, B,
                 stride, next_n, ((uintptr_t)logits % 16 == 0) && (stride % 4 == 0)};
    const size_t lds = (size_t)B * sizeof(int32_t);
    int wgs = 0;
    if (device_wgs(reinterpret_cast<const void*>(gather_kernel), lds, &wgs)) return 3;
    const int64_t most = (B * ((max_blocks + 3) / 4) + kWaves - 1) / kWaves;
    if (wgs > most) wgs = (int)most;
    void* args[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(gather_kernel), dim3(wgs), dim3(kThreads),
                           args, lds, static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 3;
}

extern "C" int fp4idx_ceiling_valu(int kind, int64_t workgroups, int64_t iterations, uint32_t* out,
                                   void* stream) {
    if (kind < 0 || kind > 4 || workgroups < 1 || workgroups > ((int64_t)1 << 20) ||
        iterations < 0 || iterations > ((int64_t)1 << 32) || !out || ((uintptr_t)out & 3))
        return 1;
    const void* fns[] = {reinterpret_cast<const void*>(valu_kernel<0>),
                         reinterpret_cast<const void*>(valu_kernel<1>),
                         reinterpret_cast<const void*>(valu_kernel<2>),
                         reinterpret_cast<const void*>(valu_kernel<3>),
                         reinterpret_cast<const void*>(valu_kernel<4>)};
    // y, z: a step that keeps add and fma chains finite and non-constant
    float y = 1.0001f, z = 0.25f;
    void* args[] = {&out, &iterations, &y, &z};
    return hipLaunchKernel(fns[kind], dim3((unsigned)workgroups), dim3(kThreads), args, 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess ? 0 : 3;
}
