// Grouped gated RMSNorm with the SiLU(z) gate, for gfx950.
//
// Page "Nemotron-H", section 4.1: the scan output is RMS-normalized group by
// group with the ssm_norm weight and multiplied by SiLU(z) (norm first, the
// default here); the other order (gate, then norm) is selected by a flag.  The
// NemotronH decode page names the op RmsNormGatedGroup(n_groups).
//
// HBM-bound: one wavefront per (token, group); lanes stride over the group's
// channels (4 per load when the group width allows), a butterfly reduction
// gives the group's mean square, and the same lanes write the result.

#include "device_common.h"
#include "kernels.h"

namespace m2 {
namespace {

constexpr int BLOCK = 256;
constexpr int MAXV = 32;   // values per lane: group width up to 2048

template <typename Tz, typename Tout>
__global__ __launch_bounds__(BLOCK) void gated_norm_kernel(NormArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * (BLOCK / 64) + (threadIdx.x >> 6);
    const int gs = a.d_inner / a.ngroups;
    if (item >= a.total_tokens * a.ngroups) return;
    const int64_t t = item / a.ngroups;
    const int j = (int)(item % a.ngroups);
    const int cbase = j * gs;
    const float* yr = a.y + t * a.ld_y + cbase;
    const Tz* zr = static_cast<const Tz*>(a.z) + t * a.ld_z + cbase;

    float v[MAXV], gate[MAXV];
    const int nv = (gs + 63) / 64;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        if (k < nv) {
            const int c = k * 64 + lane;
            float yv = 0.f, g = 0.f;
            if (c < gs) {
                yv = yr[c];
                g = silu(Act<Tz>::load(zr + c));
            }
            const float u = a.norm_before_gate ? yv : yv * g;
            v[k] = u;
            gate[k] = g;
            ss = fmaf(u, u, ss);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float rstd = 1.0f / sqrtf(ss / (float)gs + a.eps);

    Tout* orow = static_cast<Tout*>(a.out) + t * a.ld_out + cbase;
#pragma unroll
    for (int k = 0; k < MAXV; ++k) {
        if (k < nv) {
            const int c = k * 64 + lane;
            if (c < gs) {
                float o = v[k] * rstd * a.norm_w[cbase + c];
                if (a.norm_before_gate) o *= gate[k];
                Act<Tout>::store(orow + c, o);
            }
        }
    }
}

}  // namespace

hipError_t launch_gated_norm(const NormArgs& a, hipStream_t stream) {
    const int64_t items = a.total_tokens * a.ngroups;
    const dim3 grid((unsigned)((items + (BLOCK / 64) - 1) / (BLOCK / 64)));
    const bool zb = a.z_dtype == kBF16, ob = a.out_dtype == kBF16;
    if (zb && ob) hipLaunchKernelGGL((gated_norm_kernel<uint16_t, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
    else if (zb) hipLaunchKernelGGL((gated_norm_kernel<uint16_t, float>), grid, dim3(BLOCK), 0, stream, a);
    else if (ob) hipLaunchKernelGGL((gated_norm_kernel<float, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
    else hipLaunchKernelGGL((gated_norm_kernel<float, float>), grid, dim3(BLOCK), 0, stream, a);
    return hipGetLastError();
}

}  // namespace m2
