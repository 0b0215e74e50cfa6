// Runs the C-ABI argument validation of libfp4idx on the CPU, with the kernel
// launchers replaced by recorders (api_host_stubs.cpp), under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Every pointer is a fake,
// well-aligned address that nothing dereferences.  Extreme sizes exercise the
// overflow guards; valid calls check the descriptors handed to the launchers.
// Prints "ok N" and exits 0, or names the failing check and exits 1.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fp4idx.h"
#include "api_host_stubs.h"

static int g_checks = 0;
#define CHECK(cond)                                                                   \
    do {                                                                              \
        ++g_checks;                                                                   \
        if (!(cond)) {                                                                \
            std::printf("FAILED line %d: %s (last error: %s)\n", __LINE__, #cond,     \
                        fp4idx_last_error());                                         \
            return 1;                                                                 \
        }                                                                             \
    } while (0)

static void* const P = reinterpret_cast<void*>(uintptr_t(1) << 20);
static const float FMIN = 1.17549435e-38f;

static int q(int64_t T, int H, float floor_, int64_t max_pos = 16) {
    return fp4idx_q_rope_pack(P, P, 1, (const float*)P, max_pos, (const float*)P, T, H, 128, 64,
                              64, 32, 1, 0, floor_, (uint8_t*)P, (uint8_t*)P, (float*)P, nullptr);
}
static int k(int64_t T, int64_t NB, int64_t max_pos = 16) {
    return fp4idx_k_rope_pack_store(P, P, 1, (const float*)P, max_pos, (const int64_t*)P, P,
                                    1e-6f, T, 128, 64, 64, 32, 1, 1, FMIN, (uint8_t*)P,
                                    (uint8_t*)P, NB, 64, nullptr);
}

int main() {
    // valid calls reach the launcher with the expected descriptors
    CHECK(q(10, 48, FMIN) == FP4IDX_OK && g_stub.q.J == 4 && g_stub.q.e_lo == 1);
    CHECK(q(10, 2048, 1e-10f) == FP4IDX_OK && g_stub.q.J == 128 && g_stub.q.e_lo == 94);
    CHECK(q(10, 16, 0.0f) == FP4IDX_OK && g_stub.q.e_lo == 1);
    CHECK(q(10, 16, 3.0e38f) == FP4IDX_OK && g_stub.q.e_lo == 254);
    CHECK(k(7, 3) == FP4IDX_OK && g_stub.k.nslots == 192 && g_stub.k.gamma != nullptr);
    // extreme sizes are refused, not overflowed
    CHECK(q(INT64_MAX, 64, FMIN) == FP4IDX_EINVAL);
    CHECK(q(INT64_MAX / 4096, 2048, FMIN) == FP4IDX_EINVAL);
    CHECK(q(4, INT_MAX, FMIN) == FP4IDX_EUNSUPPORTED);
    CHECK(q(4, INT_MIN, FMIN) == FP4IDX_EUNSUPPORTED);
    CHECK(q(4, 64, FMIN, INT64_MAX) == FP4IDX_EINVAL);
    CHECK(q(-1, 64, FMIN) == FP4IDX_EINVAL);
    CHECK(q(4, 64, NAN) == FP4IDX_EINVAL && q(4, 64, -INFINITY) == FP4IDX_EINVAL);
    CHECK(k(INT64_MAX, 4) == FP4IDX_EINVAL);
    CHECK(k(4, INT64_MAX) == FP4IDX_EINVAL);
    CHECK(k(4, INT64_MAX / 8192 + 1) == FP4IDX_EINVAL);
    CHECK(k(4, -5) == FP4IDX_EINVAL);
    // fused call
    CHECK(fp4idx_qk_rope_pack_store(P, P, P, 0, (const float*)P, 8, nullptr, (const int64_t*)P,
                                    nullptr, 0.0f, 3, 32, 128, 64, 0, 32, 0, 1, FMIN, (uint8_t*)P,
                                    (uint8_t*)P, nullptr, (uint8_t*)P, (uint8_t*)P, 5, 64,
                                    nullptr) == FP4IDX_OK &&
          std::strcmp(g_stub.last, "qk") == 0 && g_stub.k.nslots == 320 && g_stub.q.pos64 == 0);
    // sglang mode
    CHECK(fp4idx_q_rope_pack_sglang(P, P, 1, (const float*)P, 8, 5, 64, 128, 64, 64, 32, 1, 1e-4f,
                                    1e-10f, (uint8_t*)P, nullptr) == FP4IDX_OK &&
          g_stub.sq.e_lo1 == 114 && g_stub.sq.e_lo2 == 94);
    CHECK(fp4idx_k_rope_pack_store_sglang(P, P, 1, (const float*)P, 8, (const int64_t*)P, nullptr,
                                          0.0f, 5, 128, 64, 64, 32, 1, 4, FMIN, FMIN,
                                          (uint8_t*)P, 100, nullptr) == FP4IDX_OK &&
          g_stub.sk.compress_ratio == 4 && g_stub.sk.nslots == 100);
    CHECK(fp4idx_k_rope_pack_store_sglang(P, P, 1, (const float*)P, 8, (const int64_t*)P, nullptr,
                                          0.0f, 5, 128, 64, 64, 32, 1, 1, FMIN, FMIN,
                                          (uint8_t*)P, INT64_MAX, nullptr) == FP4IDX_EINVAL);
    // FP8 mode
    CHECK(fp4idx_q_rope_pack_fp8(P, P, 1, (const float*)P, 8, (const float*)P, 0.5f, 5, 32, 128,
                                 64, 64, 1, 1, FP4IDX_SCALE_FP32, 1e-3f, (uint8_t*)P,
                                 (uint16_t*)P, nullptr) == FP4IDX_OK &&
          g_stub.fp32 && g_stub.fq.weights_scale == 0.5f && g_stub.fq.scale_floor == 1e-3f);
    CHECK(fp4idx_k_rope_pack_store_fp8(P, P, 1, (const float*)P, 8, (const int64_t*)P, nullptr,
                                       0.0f, 5, 128, 64, 64, 1, 0, FP4IDX_SCALE_UE8M0, 0.0f,
                                       (uint8_t*)P, (float*)P, 2, 64, nullptr) == FP4IDX_OK &&
          !g_stub.fp32 && g_stub.fk.nslots == 128);
    CHECK(fp4idx_k_rope_pack_store_fp8(P, P, 1, (const float*)P, 8, (const int64_t*)P, nullptr,
                                       0.0f, 5, 128, 64, 64, 1, 0, FP4IDX_SCALE_UE8M0, 0.0f,
                                       (uint8_t*)P, (float*)P, INT64_MAX, 64,
                                       nullptr) == FP4IDX_EINVAL);
    // fake quant
    CHECK(fp4idx_rope_fake_quant(P, 640, 64, P, 1, (const float*)P, 8, 128, 64, 64, 1, 2,
                                 FP4IDX_FQ_E4M3_16, 1e-3f, P, nullptr) == FP4IDX_OK &&
          g_stub.mode == 1 && g_stub.fake.compress_ratio == 2 && g_stub.fake.e_lo == 118);
    CHECK(fp4idx_rope_fake_quant(P, INT64_MAX, 1, P, 1, (const float*)P, 8, 128, 64, 64, 1, 1,
                                 0, 0.0f, P, nullptr) == FP4IDX_EINVAL);
    CHECK(fp4idx_rope_fake_quant(P, 64, INT64_MIN, P, 1, (const float*)P, 8, 128, 64, 64, 1, 1,
                                 0, 0.0f, P, nullptr) == FP4IDX_EINVAL);
    // rows_per_position beyond rows (all rows on position 0) reaches the kernel clamped
    CHECK(fp4idx_rope_fake_quant(P, 64, INT64_MAX, P, 1, (const float*)P, 8, 128, 64, 64, 1, 1,
                                 0, 0.0f, P, nullptr) == FP4IDX_OK &&
          g_stub.fake.rows_per_position == 64);
    CHECK(fp4idx_rope_fake_quant(P, 640, 64, P, 1, (const float*)P, 8, 128, 64, 64, 1, 1,
                                 0, 0.0f, P, nullptr) == FP4IDX_OK &&
          g_stub.fake.rows_per_position == 64);
    // dequant reader
    CHECK(fp4idx_dequant_debug(0, (const uint8_t*)P, (const uint8_t*)P, 4, 32, nullptr, 0, 64,
                               (float*)P, nullptr) == FP4IDX_OK && g_stub.d.J == 4);
    CHECK(fp4idx_dequant_debug(1, (const uint8_t*)P, (const uint8_t*)P, INT64_MAX, 32, nullptr, 2,
                               64, (float*)P, nullptr) == FP4IDX_EINVAL);
    CHECK(fp4idx_dequant_debug(0, (const uint8_t*)P, (const uint8_t*)P, INT64_MAX / 16384, 2048,
                               nullptr, 0, 64, (float*)P, nullptr) == FP4IDX_EINVAL);
    // scorer
    CHECK(fp4idx_paged_mqa_logits((const uint8_t*)P, (const uint8_t*)P, (const float*)P, 1.0f,
                                  (const uint8_t*)P, (const uint8_t*)P, 4, (const int32_t*)P, 8,
                                  (const int32_t*)P, 2, 4, 32, 1, (float*)P, 512,
                                  nullptr) == FP4IDX_OK &&
          g_stub.l.J == 4 && g_stub.l.B == 2);
    CHECK(fp4idx_paged_mqa_logits((const uint8_t*)P, (const uint8_t*)P, (const float*)P, 1.0f,
                                  (const uint8_t*)P, (const uint8_t*)P, 4, (const int32_t*)P, 8,
                                  (const int32_t*)P, 65535, 4, 32, 1, (float*)P, INT64_MAX,
                                  nullptr) == FP4IDX_EINVAL);
    CHECK(fp4idx_paged_mqa_logits((const uint8_t*)P, (const uint8_t*)P, (const float*)P, 1.0f,
                                  (const uint8_t*)P, (const uint8_t*)P, INT64_MAX,
                                  (const int32_t*)P, 8, (const int32_t*)P, 2, 4, 32, 1, (float*)P,
                                  512, nullptr) == FP4IDX_EINVAL);
    // a failing launch is reported with the HIP error string; nothing else changes
    g_stub.status = hipErrorInvalidValue;
    CHECK(q(4, 64, FMIN) == FP4IDX_EHIP && std::strstr(fp4idx_last_error(), "stub error"));
    g_stub.status = hipSuccess;
    // a rejected call never reaches a launcher
    const int before = g_stub.calls;
    CHECK(q(4, 24, FMIN) == FP4IDX_EUNSUPPORTED && g_stub.calls == before);
    std::printf("ok %d\n", g_checks);
    return 0;
}
