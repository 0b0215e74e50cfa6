// Shared between the host-only launcher stand-ins and the sanitizer driver.
#pragma once
#include "fp4idx_internal.h"

struct StubRecord {
    int calls = 0;
    const char* last = "";
    hipError_t status = hipSuccess;
    fp4idx::QArgs q{};
    fp4idx::KArgs k{};
    fp4idx::SQArgs sq{};
    fp4idx::SKArgs sk{};
    fp4idx::FQArgs fq{};
    fp4idx::FKArgs fk{};
    fp4idx::FakeQArgs fake{};
    fp4idx::DArgs d{};
    fp4idx::LArgs l{};
    bool fp32 = false;
    int mode = -1;
};

extern StubRecord g_stub;
