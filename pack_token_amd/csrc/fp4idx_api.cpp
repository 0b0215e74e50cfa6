// fp4idx_api.cpp -- extern "C" entry points of libfp4idx (declared and
// documented in include/fp4idx.h): argument validation, error reporting and
// kernel launch on the caller's stream.
//
// Host-side rejection follows ROCm/aiter PR 5484 "API": anything outside
// head_dim 128, rope_dim 64, group 32, kv block 64 and n_heads % 16 == 0 is
// refused with a message that names the argument.  Every check runs before
// anything is enqueued, so a rejected call writes nothing and makes no HIP
// call at all.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "fp4idx.h"
#include "fp4idx_internal.h"

namespace {

thread_local std::string g_last_error;

constexpr int kHeadDim = 128;
constexpr int kRopeDim = 64;
constexpr int kGroup = 32;
constexpr int kKvBlock = 64;
constexpr int kMaxHeads = 2048;
// query tiles of 2 tokens (4 at H = 32) on the third grid dimension (at most 65535)
constexpr int kMaxNextN = 2 * 65535;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_flag(int v) { return v == 0 || v == 1; }

// biased exponent of ceil_pow2(x) for x >= 0: (bits >> 23) + (mantissa != 0)
int ceil_pow2_exponent(float x) {
    uint32_t b;
    std::memcpy(&b, &x, 4);
    return (int)(b >> 23) + ((b & 0x7FFFFFu) != 0u ? 1 : 0);
}

int floor_exponent(float scale_floor) {
    int e = ceil_pow2_exponent(scale_floor);
    return e < 1 ? 1 : (e > 254 ? 254 : e);
}

// Shape checks shared by the q and k calls.
int check_common(const char* fn, int D, int R, int group_size, int rope_offset, int positions_int64,
                 int is_neox, int apply_hadamard, float scale_floor, int64_t T, int64_t max_pos) {
    if (D != kHeadDim)
        return fail(FP4IDX_EUNSUPPORTED, "%s: head_dim D must be 128 (got %d)", fn, D);
    if (R != kRopeDim)
        return fail(FP4IDX_EUNSUPPORTED, "%s: rope_dim R must be 64 (got %d)", fn, R);
    if (group_size != kGroup)
        return fail(FP4IDX_EUNSUPPORTED, "%s: group_size must be 32 (got %d)", fn, group_size);
    if (rope_offset != 0 && rope_offset != kHeadDim - kRopeDim)
        return fail(FP4IDX_EUNSUPPORTED, "%s: rope_offset must be 0 or 64 (got %d)", fn,
                    rope_offset);
    if (!is_flag(positions_int64))
        return fail(FP4IDX_EINVAL, "%s: positions_int64 must be 0 or 1 (got %d)", fn,
                    positions_int64);
    if (!is_flag(is_neox))
        return fail(FP4IDX_EINVAL, "%s: is_neox must be 0 or 1 (got %d)", fn, is_neox);
    if (!is_flag(apply_hadamard))
        return fail(FP4IDX_EINVAL, "%s: apply_hadamard must be 0 or 1 (got %d)", fn,
                    apply_hadamard);
    if (!std::isfinite(scale_floor) || scale_floor < 0.0f)
        return fail(FP4IDX_EINVAL, "%s: scale_floor must be finite and >= 0 (got %g)", fn,
                    (double)scale_floor);
    if (T < 0) return fail(FP4IDX_EINVAL, "%s: T must be >= 0 (got %lld)", fn, (long long)T);
    if (max_pos <= 0)
        return fail(FP4IDX_EINVAL, "%s: max_pos must be > 0 (got %lld)", fn, (long long)max_pos);
    if (max_pos > INT64_MAX / (kRopeDim * 4))
        return fail(FP4IDX_EINVAL, "%s: max_pos too large (%lld)", fn, (long long)max_pos);
    return FP4IDX_OK;
}

int check_floor(const char* fn, const char* name, float v) {
    if (!std::isfinite(v) || v < 0.0f)
        return fail(FP4IDX_EINVAL, "%s: %s must be finite and >= 0 (got %g)", fn, name, (double)v);
    return FP4IDX_OK;
}

// FP8 scale format; an fp32 scale must stay a normal number (its reciprocal
// is taken), so that format needs scale_floor >= 2^-126.
int check_fp8_scale(const char* fn, int scale_fmt, float scale_floor) {
    if (scale_fmt != FP4IDX_SCALE_UE8M0 && scale_fmt != FP4IDX_SCALE_FP32)
        return fail(FP4IDX_EINVAL, "%s: scale_fmt must be 0 (ue8m0) or 1 (fp32) (got %d)", fn,
                    scale_fmt);
    if (scale_fmt == FP4IDX_SCALE_FP32 && !(scale_floor >= 1.17549435e-38f))
        return fail(FP4IDX_EINVAL, "%s: scale_floor must be >= 2^-126 with fp32 scales (got %g)",
                    fn, (double)scale_floor);
    return FP4IDX_OK;
}

int check_ratio(const char* fn, int compress_ratio) {
    if (compress_ratio != 1 && compress_ratio != 2 && compress_ratio != 4)
        return fail(FP4IDX_EUNSUPPORTED, "%s: compress_ratio must be 1, 2 or 4 (got %d)", fn,
                    compress_ratio);
    return FP4IDX_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, uintptr_t align) {
    if (p == nullptr) return fail(FP4IDX_EINVAL, "%s: %s must not be NULL", fn, name);
    if (!aligned(p, align))
        return fail(FP4IDX_EINVAL, "%s: %s must be %u-byte aligned (got %p)", fn, name,
                    (unsigned)align, p);
    return FP4IDX_OK;
}

#define FP4IDX_TRY(expr)                   \
    do {                                   \
        int rc_ = (expr);                  \
        if (rc_ != FP4IDX_OK) return rc_;  \
    } while (0)

int hip_fail(const char* fn, hipError_t err) {
    return fail(FP4IDX_EHIP, "%s: kernel launch failed: %s (%d)", fn, hipGetErrorString(err),
                (int)err);
}

}  // namespace

namespace {

int prepare_q(const char* fn, const void* q, const void* positions, int positions_int64,
              const float* cos_sin, int64_t max_pos, const float* weights, int64_t T, int H,
              int D, int R, int rope_offset, int group_size, int is_neox, int apply_hadamard,
              float scale_floor, uint8_t* q_out, uint8_t* q_scale_out, float* weights_out,
              fp4idx::QArgs& a) {
    FP4IDX_TRY(check_common(fn, D, R, group_size, rope_offset, positions_int64, is_neox,
                            apply_hadamard, scale_floor, T, max_pos));
    if (H <= 0 || H % 16 != 0 || H > kMaxHeads)
        return fail(FP4IDX_EUNSUPPORTED,
                    "%s: n_heads H must be a positive multiple of 16 and <= %d (got %d)", fn,
                    kMaxHeads, H);
    if ((weights == nullptr) != (weights_out == nullptr))
        return fail(FP4IDX_EINVAL, "%s: weights and weights_out must both be given or both NULL",
                    fn);
    if (T > INT64_MAX / ((int64_t)H * kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: T too large (%lld)", fn, (long long)T);
    a = fp4idx::QArgs{};
    a.T = T;
    if (T == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "q", q, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "q_out", q_out, 16));
    FP4IDX_TRY(check_ptr(fn, "q_scale_out", q_scale_out, 4));
    if (weights != nullptr) {
        FP4IDX_TRY(check_ptr(fn, "weights", weights, 4));
        FP4IDX_TRY(check_ptr(fn, "weights_out", weights_out, 4));
    }
    a.q = static_cast<const uint16_t*>(q);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.weights = weights;
    a.q_out = q_out;
    a.q_scale_out = q_scale_out;
    a.weights_out = weights_out;
    a.max_pos = max_pos;
    a.H = H;
    a.J = ((H / 16) + 3) / 4 * 4;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.e_lo = floor_exponent(scale_floor);
    return FP4IDX_OK;
}

int prepare_k(const char* fn, const void* k, const void* positions, int positions_int64,
              const float* cos_sin, int64_t max_pos, const int64_t* slot_mapping,
              const void* k_norm_gamma, float k_norm_eps, int64_t T, int D, int R,
              int rope_offset, int group_size, int is_neox, int apply_hadamard, float scale_floor,
              uint8_t* kv_cache, uint8_t* kv_cache_scale, int64_t NB, int BS, fp4idx::KArgs& a) {
    FP4IDX_TRY(check_common(fn, D, R, group_size, rope_offset, positions_int64, is_neox,
                            apply_hadamard, scale_floor, T, max_pos));
    if (BS != kKvBlock)
        return fail(FP4IDX_EUNSUPPORTED, "%s: kv_block_size BS must be 64 (got %d)", fn, BS);
    if (NB < 0) return fail(FP4IDX_EINVAL, "%s: NB must be >= 0 (got %lld)", fn, (long long)NB);
    if (NB > INT64_MAX / ((int64_t)kKvBlock * kHeadDim))
        return fail(FP4IDX_EINVAL, "%s: NB too large (%lld)", fn, (long long)NB);
    if (k_norm_gamma != nullptr && (!std::isfinite(k_norm_eps) || k_norm_eps < 0.0f))
        return fail(FP4IDX_EINVAL, "%s: k_norm_eps must be finite and >= 0 (got %g)", fn,
                    (double)k_norm_eps);
    if (T > INT64_MAX / (kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: T too large (%lld)", fn, (long long)T);
    a = fp4idx::KArgs{};
    a.T = T;
    if (T == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "k", k, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "slot_mapping", slot_mapping, 8));
    if (k_norm_gamma != nullptr) FP4IDX_TRY(check_ptr(fn, "k_norm_gamma", k_norm_gamma, 16));
    if (NB > 0) {
        FP4IDX_TRY(check_ptr(fn, "kv_cache", kv_cache, 16));
        FP4IDX_TRY(check_ptr(fn, "kv_cache_scale", kv_cache_scale, 4));
    }
    a.k = static_cast<const uint16_t*>(k);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.slot_mapping = slot_mapping;
    a.gamma = static_cast<const uint16_t*>(k_norm_gamma);
    a.kv_cache = kv_cache;
    a.kv_cache_scale = kv_cache_scale;
    a.max_pos = max_pos;
    a.nslots = NB * kKvBlock;
    a.eps = k_norm_eps;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.e_lo = floor_exponent(scale_floor);
    return FP4IDX_OK;
}

}  // namespace

extern "C" {

int fp4idx_q_rope_pack(const void* q, const void* positions, int positions_int64,
                       const float* cos_sin, int64_t max_pos, const float* weights, int64_t T,
                       int H, int D, int R, int rope_offset, int group_size, int is_neox,
                       int apply_hadamard, float scale_floor, uint8_t* q_out,
                       uint8_t* q_scale_out, float* weights_out, void* stream) {
    static const char* fn = "fp4idx_q_rope_pack";
    fp4idx::QArgs a;
    FP4IDX_TRY(prepare_q(fn, q, positions, positions_int64, cos_sin, max_pos, weights, T, H, D, R,
                         rope_offset, group_size, is_neox, apply_hadamard, scale_floor, q_out,
                         q_scale_out, weights_out, a));
    if (T == 0) return FP4IDX_OK;
    hipError_t err = fp4idx::launch_q_rope_pack(a, is_neox != 0, apply_hadamard != 0,
                                                static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_k_rope_pack_store(const void* k, const void* positions, int positions_int64,
                             const float* cos_sin, int64_t max_pos, const int64_t* slot_mapping,
                             const void* k_norm_gamma, float k_norm_eps, int64_t T, int D, int R,
                             int rope_offset, int group_size, int is_neox, int apply_hadamard,
                             float scale_floor, uint8_t* kv_cache, uint8_t* kv_cache_scale,
                             int64_t NB, int BS, void* stream) {
    static const char* fn = "fp4idx_k_rope_pack_store";
    fp4idx::KArgs a;
    FP4IDX_TRY(prepare_k(fn, k, positions, positions_int64, cos_sin, max_pos, slot_mapping,
                         k_norm_gamma, k_norm_eps, T, D, R, rope_offset, group_size, is_neox,
                         apply_hadamard, scale_floor, kv_cache, kv_cache_scale, NB, BS, a));
    if (T == 0) return FP4IDX_OK;
    hipError_t err = fp4idx::launch_k_rope_pack_store(a, is_neox != 0, apply_hadamard != 0,
                                                      static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_qk_rope_pack_store(const void* q, const void* k, const void* positions,
                              int positions_int64, const float* cos_sin, int64_t max_pos,
                              const float* weights, const int64_t* slot_mapping,
                              const void* k_norm_gamma, float k_norm_eps, int64_t T, int H, int D,
                              int R, int rope_offset, int group_size, int is_neox,
                              int apply_hadamard, float scale_floor, uint8_t* q_out,
                              uint8_t* q_scale_out, float* weights_out, uint8_t* kv_cache,
                              uint8_t* kv_cache_scale, int64_t NB, int BS, void* stream) {
    static const char* fn = "fp4idx_qk_rope_pack_store";
    fp4idx::QArgs qa;
    fp4idx::KArgs ka;
    FP4IDX_TRY(prepare_q(fn, q, positions, positions_int64, cos_sin, max_pos, weights, T, H, D, R,
                         rope_offset, group_size, is_neox, apply_hadamard, scale_floor, q_out,
                         q_scale_out, weights_out, qa));
    FP4IDX_TRY(prepare_k(fn, k, positions, positions_int64, cos_sin, max_pos, slot_mapping,
                         k_norm_gamma, k_norm_eps, T, D, R, rope_offset, group_size, is_neox,
                         apply_hadamard, scale_floor, kv_cache, kv_cache_scale, NB, BS, ka));
    if (T == 0) return FP4IDX_OK;
    hipError_t err = fp4idx::launch_qk_rope_pack_store(qa, ka, is_neox != 0, apply_hadamard != 0,
                                                       static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_q_rope_pack_sglang(const void* q, const void* positions, int positions_int64,
                              const float* cos_sin, int64_t max_pos, int64_t T, int H, int D,
                              int R, int rope_offset, int group_size, int is_neox,
                              float fake_quant_floor, float pack_floor, uint8_t* q_packed,
                              void* stream) {
    static const char* fn = "fp4idx_q_rope_pack_sglang";
    FP4IDX_TRY(check_floor(fn, "fake_quant_floor", fake_quant_floor));
    FP4IDX_TRY(check_floor(fn, "pack_floor", pack_floor));
    FP4IDX_TRY(check_common(fn, D, R, group_size, rope_offset, positions_int64, is_neox, 0,
                            fake_quant_floor, T, max_pos));
    if (H <= 0 || H % 16 != 0 || H > kMaxHeads)
        return fail(FP4IDX_EUNSUPPORTED,
                    "%s: n_heads H must be a positive multiple of 16 and <= %d (got %d)", fn,
                    kMaxHeads, H);
    if (T > INT64_MAX / ((int64_t)H * kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: T too large (%lld)", fn, (long long)T);
    if (T == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "q", q, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "q_packed", q_packed, 16));
    fp4idx::SQArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.q_packed = q_packed;
    a.T = T;
    a.max_pos = max_pos;
    a.H = H;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.e_lo1 = floor_exponent(fake_quant_floor);
    a.e_lo2 = floor_exponent(pack_floor);
    hipError_t err = fp4idx::launch_q_rope_pack_sglang(a, is_neox != 0,
                                                       static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_k_rope_pack_store_sglang(const void* k, const void* positions, int positions_int64,
                                    const float* cos_sin, int64_t max_pos,
                                    const int64_t* slot_mapping, const void* k_norm_gamma,
                                    float k_norm_eps, int64_t T, int D, int R, int rope_offset,
                                    int group_size, int is_neox, int compress_ratio,
                                    float fake_quant_floor, float pack_floor,
                                    uint8_t* index_k_cache, int64_t num_slots, void* stream) {
    static const char* fn = "fp4idx_k_rope_pack_store_sglang";
    FP4IDX_TRY(check_ratio(fn, compress_ratio));
    FP4IDX_TRY(check_floor(fn, "fake_quant_floor", fake_quant_floor));
    FP4IDX_TRY(check_floor(fn, "pack_floor", pack_floor));
    FP4IDX_TRY(check_common(fn, D, R, group_size, rope_offset, positions_int64, is_neox, 0,
                            fake_quant_floor, T, max_pos));
    if (num_slots < 0 || num_slots > INT64_MAX / fp4idx::kSglangRecord)
        return fail(FP4IDX_EINVAL, "%s: num_slots out of range (%lld)", fn, (long long)num_slots);
    if (k_norm_gamma != nullptr && (!std::isfinite(k_norm_eps) || k_norm_eps < 0.0f))
        return fail(FP4IDX_EINVAL, "%s: k_norm_eps must be finite and >= 0 (got %g)", fn,
                    (double)k_norm_eps);
    if (T > INT64_MAX / (kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: T too large (%lld)", fn, (long long)T);
    if (T == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "k", k, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "slot_mapping", slot_mapping, 8));
    if (k_norm_gamma != nullptr) FP4IDX_TRY(check_ptr(fn, "k_norm_gamma", k_norm_gamma, 16));
    if (num_slots > 0) FP4IDX_TRY(check_ptr(fn, "index_k_cache", index_k_cache, 4));
    fp4idx::SKArgs a{};
    a.k = static_cast<const uint16_t*>(k);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.slot_mapping = slot_mapping;
    a.gamma = static_cast<const uint16_t*>(k_norm_gamma);
    a.index_k_cache = index_k_cache;
    a.T = T;
    a.max_pos = max_pos;
    a.nslots = num_slots;
    a.eps = k_norm_eps;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.compress_ratio = compress_ratio;
    a.e_lo1 = floor_exponent(fake_quant_floor);
    a.e_lo2 = floor_exponent(pack_floor);
    hipError_t err = fp4idx::launch_k_rope_pack_store_sglang(a, is_neox != 0,
                                                             static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_q_rope_pack_fp8(const void* q, const void* positions, int positions_int64,
                           const float* cos_sin, int64_t max_pos, const float* weights,
                           float weights_scale, int64_t T, int H, int D, int R, int rope_offset,
                           int is_neox, int apply_hadamard, int scale_fmt, float scale_floor,
                           uint8_t* q_out, uint16_t* weights_out, void* stream) {
    static const char* fn = "fp4idx_q_rope_pack_fp8";
    FP4IDX_TRY(check_common(fn, D, R, kGroup, rope_offset, positions_int64, is_neox,
                            apply_hadamard, scale_floor, T, max_pos));
    FP4IDX_TRY(check_fp8_scale(fn, scale_fmt, scale_floor));
    if (!std::isfinite(weights_scale))
        return fail(FP4IDX_EINVAL, "%s: weights_scale must be finite", fn);
    if (H <= 0 || H % 16 != 0 || H > kMaxHeads)
        return fail(FP4IDX_EUNSUPPORTED,
                    "%s: n_heads H must be a positive multiple of 16 and <= %d (got %d)", fn,
                    kMaxHeads, H);
    if (T > INT64_MAX / ((int64_t)H * kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: T too large (%lld)", fn, (long long)T);
    if (T == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "q", q, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "weights", weights, 4));
    FP4IDX_TRY(check_ptr(fn, "q_out", q_out, 16));
    FP4IDX_TRY(check_ptr(fn, "weights_out", weights_out, 2));
    fp4idx::FQArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.weights = weights;
    a.q_out = q_out;
    a.weights_out = weights_out;
    a.T = T;
    a.max_pos = max_pos;
    a.H = H;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.scale_floor = scale_floor;
    a.weights_scale = weights_scale;
    hipError_t err = fp4idx::launch_q_rope_pack_fp8(a, is_neox != 0, apply_hadamard != 0,
                                                    scale_fmt == FP4IDX_SCALE_FP32,
                                                    static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_k_rope_pack_store_fp8(const void* k, const void* positions, int positions_int64,
                                 const float* cos_sin, int64_t max_pos,
                                 const int64_t* slot_mapping, const void* k_norm_gamma,
                                 float k_norm_eps, int64_t T, int D, int R, int rope_offset,
                                 int is_neox, int apply_hadamard, int scale_fmt,
                                 float scale_floor, uint8_t* kv_cache, float* kv_cache_scale,
                                 int64_t NB, int BS, void* stream) {
    static const char* fn = "fp4idx_k_rope_pack_store_fp8";
    FP4IDX_TRY(check_common(fn, D, R, kGroup, rope_offset, positions_int64, is_neox,
                            apply_hadamard, scale_floor, T, max_pos));
    FP4IDX_TRY(check_fp8_scale(fn, scale_fmt, scale_floor));
    if (BS != kKvBlock)
        return fail(FP4IDX_EUNSUPPORTED, "%s: kv_block_size BS must be 64 (got %d)", fn, BS);
    if (NB < 0 || NB > INT64_MAX / ((int64_t)kKvBlock * kHeadDim))
        return fail(FP4IDX_EINVAL, "%s: NB out of range (%lld)", fn, (long long)NB);
    if (k_norm_gamma != nullptr && (!std::isfinite(k_norm_eps) || k_norm_eps < 0.0f))
        return fail(FP4IDX_EINVAL, "%s: k_norm_eps must be finite and >= 0 (got %g)", fn,
                    (double)k_norm_eps);
    if (T > INT64_MAX / (kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: T too large (%lld)", fn, (long long)T);
    if (T == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "k", k, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "slot_mapping", slot_mapping, 8));
    if (k_norm_gamma != nullptr) FP4IDX_TRY(check_ptr(fn, "k_norm_gamma", k_norm_gamma, 16));
    if (NB > 0) {
        FP4IDX_TRY(check_ptr(fn, "kv_cache", kv_cache, 16));
        FP4IDX_TRY(check_ptr(fn, "kv_cache_scale", kv_cache_scale, 4));
    }
    fp4idx::FKArgs a{};
    a.k = static_cast<const uint16_t*>(k);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.slot_mapping = slot_mapping;
    a.gamma = static_cast<const uint16_t*>(k_norm_gamma);
    a.kv_cache = kv_cache;
    a.kv_cache_scale = kv_cache_scale;
    a.T = T;
    a.max_pos = max_pos;
    a.nslots = NB * kKvBlock;
    a.eps = k_norm_eps;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.scale_floor = scale_floor;
    hipError_t err = fp4idx::launch_k_rope_pack_store_fp8(a, is_neox != 0, apply_hadamard != 0,
                                                          scale_fmt == FP4IDX_SCALE_FP32,
                                                          static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_rope_fake_quant(const void* x, int64_t rows, int64_t rows_per_position,
                           const void* positions, int positions_int64, const float* cos_sin,
                           int64_t max_pos, int D, int R, int rope_offset, int is_neox,
                           int compress_ratio, int mode, float scale_floor, void* y,
                           void* stream) {
    static const char* fn = "fp4idx_rope_fake_quant";
    if (mode != FP4IDX_FQ_UE8M0_32 && mode != FP4IDX_FQ_E4M3_16)
        return fail(FP4IDX_EINVAL, "%s: mode must be 0 (per-32 UE8M0) or 1 (per-16 E4M3) (got %d)",
                    fn, mode);
    FP4IDX_TRY(check_ratio(fn, compress_ratio));
    FP4IDX_TRY(check_common(fn, D, R, kGroup, rope_offset, positions_int64, is_neox, 0,
                            scale_floor, rows, max_pos));
    if (rows_per_position < 1)
        return fail(FP4IDX_EINVAL, "%s: rows_per_position must be >= 1 (got %lld)", fn,
                    (long long)rows_per_position);
    if (rows > INT64_MAX / (kHeadDim * 2))
        return fail(FP4IDX_EINVAL, "%s: rows too large (%lld)", fn, (long long)rows);
    if (rows == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "x", x, 16));
    FP4IDX_TRY(check_ptr(fn, "positions", positions, positions_int64 ? 8 : 4));
    FP4IDX_TRY(check_ptr(fn, "cos_sin", cos_sin, 16));
    FP4IDX_TRY(check_ptr(fn, "y", y, 16));
    fp4idx::FakeQArgs a{};
    a.x = static_cast<const uint16_t*>(x);
    a.positions = positions;
    a.cos_sin = cos_sin;
    a.y = static_cast<uint16_t*>(y);
    a.rows = rows;
    a.max_pos = max_pos;
    // past `rows` every row maps to position 0 either way; the clamp keeps the
    // kernel's row arithmetic (token index x rows_per_position) inside int64
    a.rows_per_position = rows_per_position > rows ? rows : rows_per_position;
    a.pos64 = positions_int64;
    a.rope_offset = rope_offset;
    a.compress_ratio = compress_ratio;
    a.e_lo = floor_exponent(scale_floor);
    a.scale_floor = scale_floor;
    hipError_t err = fp4idx::launch_rope_fake_quant(a, is_neox != 0, mode,
                                                    static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_dequant_debug(int which, const uint8_t* packed, const uint8_t* scales, int64_t rows,
                         int H, const int64_t* slots, int64_t NB, int BS, float* out,
                         void* stream) {
    static const char* fn = "fp4idx_dequant_debug";
    if (which != 0 && which != 1)
        return fail(FP4IDX_EINVAL, "%s: which must be 0 (Q) or 1 (KCACHE) (got %d)", fn, which);
    if (rows < 0) return fail(FP4IDX_EINVAL, "%s: rows must be >= 0 (got %lld)", fn, (long long)rows);
    fp4idx::DArgs a{};
    a.which = which;
    a.rows = rows;
    if (which == 0) {
        if (H <= 0 || H % 16 != 0 || H > kMaxHeads)
            return fail(FP4IDX_EUNSUPPORTED,
                        "%s: n_heads H must be a positive multiple of 16 and <= %d (got %d)", fn,
                        kMaxHeads, H);
        if (rows > INT64_MAX / ((int64_t)H * kHeadDim * 4))
            return fail(FP4IDX_EINVAL, "%s: rows too large (%lld)", fn, (long long)rows);
        a.H = H;
        a.J = ((H / 16) + 3) / 4 * 4;
    } else {
        if (BS != kKvBlock)
            return fail(FP4IDX_EUNSUPPORTED, "%s: kv_block_size BS must be 64 (got %d)", fn, BS);
        if (NB < 0 || NB > INT64_MAX / ((int64_t)kKvBlock * kHeadDim))
            return fail(FP4IDX_EINVAL, "%s: NB out of range (%lld)", fn, (long long)NB);
        if (rows > INT64_MAX / (kHeadDim * 4))
            return fail(FP4IDX_EINVAL, "%s: rows too large (%lld)", fn, (long long)rows);
        a.nslots = NB * kKvBlock;
    }
    if (rows == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "out", out, 16));
    // with an empty cache every slot is out of range and no code byte is read
    if (which == 0 || NB > 0) {
        FP4IDX_TRY(check_ptr(fn, "packed", packed, 4));
        FP4IDX_TRY(check_ptr(fn, "scales", scales, 1));
    }
    if (slots != nullptr) FP4IDX_TRY(check_ptr(fn, "slots", slots, 8));
    a.packed = packed;
    a.scales = scales;
    a.slots = which == 1 ? slots : nullptr;
    a.out = out;
    hipError_t err = fp4idx::launch_dequant(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

int fp4idx_paged_mqa_logits(const uint8_t* q_out, const uint8_t* q_scale_out, const float* weights,
                            float weights_scale, const uint8_t* kv_cache,
                            const uint8_t* kv_cache_scale, int64_t NB, const int32_t* block_table,
                            int64_t max_blocks, const int32_t* context_lens, int64_t B,
                            int next_n, int H, int apply_relu, float* logits, int64_t stride,
                            void* stream) {
    static const char* fn = "fp4idx_paged_mqa_logits";
    if (H <= 0 || H % 16 != 0 || H > 64)
        return fail(FP4IDX_EUNSUPPORTED,
                    "%s: n_heads H must be 16, 32, 48 or 64 (got %d)", fn, H);
    if (next_n < 1 || next_n > kMaxNextN)
        return fail(FP4IDX_EUNSUPPORTED, "%s: next_n must be 1..%d (got %d)", fn, kMaxNextN,
                    next_n);
    if (!is_flag(apply_relu))
        return fail(FP4IDX_EINVAL, "%s: apply_relu must be 0 or 1 (got %d)", fn, apply_relu);
    if (!std::isfinite(weights_scale))
        return fail(FP4IDX_EINVAL, "%s: weights_scale must be finite", fn);
    if (B < 0 || B > 65535)
        return fail(FP4IDX_EINVAL, "%s: B must be in [0, 65535] (got %lld)", fn, (long long)B);
    if (NB < 0 || NB > INT32_MAX)
        return fail(FP4IDX_EINVAL, "%s: NB out of range (%lld)", fn, (long long)NB);
    if (max_blocks < 0 || max_blocks > (int64_t)1 << 24)
        return fail(FP4IDX_EINVAL, "%s: max_blocks out of range (%lld)", fn, (long long)max_blocks);
    if (stride <= 0 || stride > ((int64_t)1 << 40) / (B * next_n + 1))
        return fail(FP4IDX_EINVAL, "%s: stride out of range (%lld)", fn, (long long)stride);
    if (B == 0 || max_blocks == 0) return FP4IDX_OK;
    FP4IDX_TRY(check_ptr(fn, "q_out", q_out, 16));
    FP4IDX_TRY(check_ptr(fn, "q_scale_out", q_scale_out, 4));
    FP4IDX_TRY(check_ptr(fn, "weights", weights, 16));
    FP4IDX_TRY(check_ptr(fn, "block_table", block_table, 4));
    FP4IDX_TRY(check_ptr(fn, "context_lens", context_lens, 4));
    FP4IDX_TRY(check_ptr(fn, "logits", logits, 4));
    if (NB > 0) {
        FP4IDX_TRY(check_ptr(fn, "kv_cache", kv_cache, 16));
        FP4IDX_TRY(check_ptr(fn, "kv_cache_scale", kv_cache_scale, 4));
    }
    fp4idx::LArgs a{};
    a.q_out = q_out;
    a.q_scale_out = q_scale_out;
    a.weights = weights;
    a.kv_cache = kv_cache;
    a.kv_cache_scale = kv_cache_scale;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.logits = logits;
    a.nblocks = NB;
    a.max_blocks = max_blocks;
    a.B = B;
    a.stride = stride;
    a.weights_scale = weights_scale;
    a.next_n = next_n;
    a.H = H;
    a.J = ((H / 16) + 3) / 4 * 4;
    a.apply_relu = apply_relu;
    hipError_t err = fp4idx::launch_paged_mqa_logits(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(fn, err);
    return FP4IDX_OK;
}

const char* fp4idx_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
