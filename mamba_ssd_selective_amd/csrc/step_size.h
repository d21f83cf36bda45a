// The step size of the selective scan from the raw in-projection value:
// dt = softplus(raw + bias[h]) (page "Nemotron-H", section 4.1 "Mamba2 SSM
// layer": the decay takes softplus of dt plus the per-head ssm_dt.bias).
#pragma once

#include <hip/hip_runtime.h>

namespace m2 {

// log(1 + e^v) written as max(v, 0) + log1p(e^-|v|): the exponent is never
// positive, so neither end overflows, and log1p keeps the small tail exact.
__device__ __forceinline__ float softplus(float v) {
    return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v)));
}

}  // namespace m2
