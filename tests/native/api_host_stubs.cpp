// Host-only stand-ins for the kernel launchers of libfp4idx (test
// infrastructure): they record the launch descriptor the C-ABI layer built and
// return a configurable status, so the argument validation in fp4idx_api.cpp
// can be run on the CPU under AddressSanitizer / UndefinedBehaviorSanitizer.
#include <hip/hip_runtime_api.h>

#include "fp4idx_internal.h"
#include "api_host_stubs.h"

StubRecord g_stub;

const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }

namespace fp4idx {

static hipError_t rec(const char* which) {
    g_stub.calls += 1;
    g_stub.last = which;
    return g_stub.status;
}

hipError_t launch_q_rope_pack(const QArgs& a, bool, bool, hipStream_t) {
    g_stub.q = a;
    return rec("q");
}
hipError_t launch_k_rope_pack_store(const KArgs& a, bool, bool, hipStream_t) {
    g_stub.k = a;
    return rec("k");
}
hipError_t launch_qk_rope_pack_store(const QArgs& qa, const KArgs& ka, bool, bool, hipStream_t) {
    g_stub.q = qa;
    g_stub.k = ka;
    return rec("qk");
}
hipError_t launch_q_rope_pack_sglang(const SQArgs& a, bool, hipStream_t) {
    g_stub.sq = a;
    return rec("sq");
}
hipError_t launch_k_rope_pack_store_sglang(const SKArgs& a, bool, hipStream_t) {
    g_stub.sk = a;
    return rec("sk");
}
hipError_t launch_q_rope_pack_fp8(const FQArgs& a, bool, bool, bool fp32, hipStream_t) {
    g_stub.fq = a;
    g_stub.fp32 = fp32;
    return rec("fq");
}
hipError_t launch_k_rope_pack_store_fp8(const FKArgs& a, bool, bool, bool fp32, hipStream_t) {
    g_stub.fk = a;
    g_stub.fp32 = fp32;
    return rec("fk");
}
hipError_t launch_rope_fake_quant(const FakeQArgs& a, bool, int mode, hipStream_t) {
    g_stub.fake = a;
    g_stub.mode = mode;
    return rec("fake");
}
hipError_t launch_dequant(const DArgs& a, hipStream_t) {
    g_stub.d = a;
    return rec("d");
}
hipError_t launch_paged_mqa_logits(const LArgs& a, hipStream_t) {
    g_stub.l = a;
    return rec("l");
}

}  // namespace fp4idx
