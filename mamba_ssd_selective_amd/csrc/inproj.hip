// Ingestion of the packed in-projection row for gfx950.
//
// A Mamba-2 layer's in-projection emits one row per token holding z, xBC and
// the raw step size, in that order (page "feat(#1311 A2-D1): NemotronH decodes
// on the single-step recurrent kernels ...": in_proj -> QkvSplit(z | xBC | dt),
// three outputs of widths (I, conv_dim, num_heads) from the head, middle and
// tail of the row).  z and xBC are read where they lie, as row-strided views;
// only the step size needs a kernel of its own: dt = softplus(raw + bias[h])
// (page "Nemotron-H", section 4.1), written as fp32 [T, nheads] for the scan.
// The same file rebases the row offsets of a mixed batch's prefill part.

#include "device_common.h"
#include "kernels.h"
#include "step_size.h"

namespace m2 {
namespace {

constexpr int NT = 256;

// One thread per (token, head): the raw values of a row are nheads consecutive
// elements, so a wave reads whole runs of them; the output is one contiguous array.
template <typename Tin>
__global__ __launch_bounds__(NT) void step_size_kernel(const Tin* raw, int64_t ld_raw,
                                                       const float* bias, int nheads,
                                                       int64_t n, float* dt) {
    const int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (i >= n) return;
    const int64_t t = i / nheads;
    const int h = (int)(i - t * nheads);
    const float b = bias ? bias[h] : 0.f;
    dt[i] = softplus(Act<Tin>::load(raw + t * ld_raw + h) + b);
}

// Row offsets of sequences first .. first+count of a batch whose rows before
// sequence `first` are one per sequence: out[i] = cu[first + i] - first, clamped
// into [0, rows] so that offsets outside the contract still index in bounds.
// With slot_out set, also the identity slot map of those sequences (slot first + i).
__global__ __launch_bounds__(NT) void rebase_kernel(const int32_t* cu, int first, int count,
                                                    int32_t rows, int32_t* out,
                                                    int32_t* slot_out) {
    const int i = blockIdx.x * NT + threadIdx.x;
    if (i <= count) out[i] = min(max(cu[first + i] - first, 0), rows);
    if (slot_out && i < count) slot_out[i] = first + i;
}

}  // namespace

hipError_t launch_step_size(const void* raw, int64_t ld_raw, int act_dtype, const float* bias,
                            int nheads, int64_t total_tokens, float* dt, hipStream_t stream) {
    const int64_t n = total_tokens * nheads;
    if (n <= 0) return hipSuccess;
    const dim3 grid((unsigned)((n + NT - 1) / NT));
    if (act_dtype == kBF16)
        hipLaunchKernelGGL(step_size_kernel<uint16_t>, grid, dim3(NT), 0, stream,
                           static_cast<const uint16_t*>(raw), ld_raw, bias, nheads, n, dt);
    else
        hipLaunchKernelGGL(step_size_kernel<float>, grid, dim3(NT), 0, stream,
                           static_cast<const float*>(raw), ld_raw, bias, nheads, n, dt);
    return hipGetLastError();
}

hipError_t launch_rebase(const int32_t* cu, int first, int count, int32_t rows, int32_t* out,
                         int32_t* slot_out, hipStream_t stream) {
    const dim3 grid((unsigned)((count + 1 + NT - 1) / NT));
    hipLaunchKernelGGL(rebase_kernel, grid, dim3(NT), 0, stream, cu, first, count, rows, out,
                       slot_out);
    return hipGetLastError();
}

}  // namespace m2
