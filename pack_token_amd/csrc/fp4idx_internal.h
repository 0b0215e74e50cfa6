// fp4idx_internal.h -- launch descriptors shared by the C-ABI layer
// (fp4idx_api.cpp) and the kernels (fp4idx_kernels.hip, fp4idx_modes.hip,
// fp4idx_scorer.hip).  Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fp4idx {

// Arguments of one query launch.  All pointers are device pointers that the
// C-ABI layer has already validated (non-null, aligned, sizes consistent).
struct QArgs {
    const uint16_t* q;          // bf16 [T, H, 128]
    const void* positions;      // int32 or int64 [T]
    const float* cos_sin;       // fp32 [max_pos, 64]
    const float* weights;       // fp32 [T, H] or nullptr
    uint8_t* q_out;             // u8 [T, H, 64]
    uint8_t* q_scale_out;       // u8 [T, 1, 4, 16, J]
    float* weights_out;         // fp32 [T, H] or nullptr
    int64_t T;
    int64_t max_pos;
    int H;
    int J;                      // round_up(H/16, 4)
    int pos64;                  // positions are int64
    int rope_offset;            // 0 or 64
    int e_lo;                   // clamp(E(scale_floor), 1, 254)
};

struct KArgs {
    const uint16_t* k;          // bf16 [T, 128]
    const void* positions;
    const float* cos_sin;
    const int64_t* slot_mapping;  // [T]
    const uint16_t* gamma;      // bf16 [128] or nullptr
    uint8_t* kv_cache;          // u8 [NB, 1, 4, 64, 16]
    uint8_t* kv_cache_scale;    // u8 [NB, 1, 4, 64]
    int64_t T;
    int64_t max_pos;
    int64_t nslots;             // NB * 64
    float eps;
    int pos64;
    int rope_offset;
    int e_lo;
};

struct DArgs {
    const uint8_t* packed;
    const uint8_t* scales;
    const int64_t* slots;       // KCACHE only, may be nullptr
    float* out;
    int64_t rows;
    int64_t nslots;             // KCACHE: NB * 64
    int which;                  // 0 = Q, 1 = KCACHE
    int H;
    int J;
};

// sglang-compatible mode: two quantization stages, 68-byte records.
constexpr int kSglangRecord = 68;   // 64 code bytes + 4 exponent bytes

struct SQArgs {
    const uint16_t* q;          // bf16 [T, H, 128]
    const void* positions;
    const float* cos_sin;
    uint8_t* q_packed;          // u8 [T, H, 68]
    int64_t T;
    int64_t max_pos;
    int H;
    int pos64;
    int rope_offset;
    int e_lo1;                  // clamp(E(fake_quant_floor), 1, 254)
    int e_lo2;                  // clamp(E(pack_floor), 1, 254)
};

struct SKArgs {
    const uint16_t* k;          // bf16 [T, 128]
    const void* positions;
    const float* cos_sin;
    const int64_t* slot_mapping;  // [T]
    const uint16_t* gamma;      // bf16 [128] or nullptr
    uint8_t* index_k_cache;     // u8 [num_slots, 68]
    int64_t T;
    int64_t max_pos;
    int64_t nslots;             // num_slots
    float eps;
    int pos64;
    int rope_offset;
    int compress_ratio;         // 1, 2 or 4: RoPE at pos & ~(ratio - 1)
    int e_lo1;
    int e_lo2;
};

// RoPE tail + FP4 fake quant (bf16 in, bf16 out).
struct FakeQArgs {
    const uint16_t* x;          // bf16 [rows, 128]
    const void* positions;      // [ceil(rows / rows_per_position)]
    const float* cos_sin;
    uint16_t* y;                // bf16 [rows, 128]
    int64_t rows;
    int64_t max_pos;
    int64_t rows_per_position;
    int pos64;
    int rope_offset;
    int compress_ratio;
    int e_lo;                   // clamp(E(scale_floor), 1, 254), UE8M0 mode
    float scale_floor;          // E4M3 mode
};

// FP8 output mode: one e4m3fn scale per 128-row.
struct FQArgs {
    const uint16_t* q;          // bf16 [T, H, 128]
    const void* positions;
    const float* cos_sin;
    const float* weights;       // fp32 [T, H]
    uint8_t* q_out;             // e4m3fn [T, H, 128]
    uint16_t* weights_out;      // bf16 [T, H]: (weights * s) * weights_scale
    int64_t T;
    int64_t max_pos;
    int H;
    int pos64;
    int rope_offset;
    float scale_floor;
    float weights_scale;
};

struct FKArgs {
    const uint16_t* k;          // bf16 [T, 128]
    const void* positions;
    const float* cos_sin;
    const int64_t* slot_mapping;  // [T]
    const uint16_t* gamma;      // bf16 [128] or nullptr
    uint8_t* kv_cache;          // e4m3fn [NB, 64, 128]
    float* kv_cache_scale;      // fp32 [NB, 64]
    int64_t T;
    int64_t max_pos;
    int64_t nslots;             // NB * 64
    float eps;
    int pos64;
    int rope_offset;
    float scale_floor;
};

// FP4 paged MQA logits (scorer).
struct LArgs {
    const uint8_t* q_out;         // u8 [B*next_n, H, 64]
    const uint8_t* q_scale_out;   // u8 [B*next_n, 1, 4, 16, J]
    const float* weights;         // fp32 [B*next_n, H]
    const uint8_t* kv_cache;      // u8 [NB, 1, 4, 64, 16]
    const uint8_t* kv_cache_scale;  // u8 [NB, 1, 4, 64]
    const int32_t* block_table;   // int32 [B, max_blocks]
    const int32_t* context_lens;  // int32 [B]
    float* logits;                // fp32 [B*next_n, stride]
    int64_t nblocks;              // NB
    int64_t max_blocks;
    int64_t B;
    int64_t stride;
    float weights_scale;
    int next_n;
    int H;
    int J;
    int apply_relu;
    int logits_vec4;              // set by the launcher: logits rows allow 16-byte stores
};

hipError_t launch_q_rope_pack(const QArgs& a, bool is_neox, bool hadamard, hipStream_t stream);
hipError_t launch_k_rope_pack_store(const KArgs& a, bool is_neox, bool hadamard,
                                    hipStream_t stream);
hipError_t launch_qk_rope_pack_store(const QArgs& qa, const KArgs& ka, bool is_neox, bool hadamard,
                                     hipStream_t stream);
hipError_t launch_q_rope_pack_sglang(const SQArgs& a, bool is_neox, hipStream_t stream);
hipError_t launch_k_rope_pack_store_sglang(const SKArgs& a, bool is_neox, hipStream_t stream);
hipError_t launch_q_rope_pack_fp8(const FQArgs& a, bool is_neox, bool hadamard, bool fp32_scale,
                                  hipStream_t stream);
hipError_t launch_k_rope_pack_store_fp8(const FKArgs& a, bool is_neox, bool hadamard,
                                        bool fp32_scale, hipStream_t stream);
hipError_t launch_rope_fake_quant(const FakeQArgs& a, bool is_neox, int mode, hipStream_t stream);
hipError_t launch_dequant(const DArgs& a, hipStream_t stream);
hipError_t launch_paged_mqa_logits(const LArgs& a, hipStream_t stream);

}  // namespace fp4idx
