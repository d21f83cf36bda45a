// Grouped gated RMSNorm with the SiLU(z) gate, for gfx950.
//
// Page "Nemotron-H", section 4.1: the scan output is RMS-normalized group by
// group with the ssm_norm weight and multiplied by SiLU(z) (norm first, the
// default here); the other order (gate, then norm) is selected by a flag.  The
// NemotronH decode page names the op RmsNormGatedGroup(n_groups).
//
// HBM-bound: one wavefront per (token, group); a butterfly reduction gives the
// group's mean square and the same lanes write the result.  Group widths that
// are multiples of 8 with 16-byte aligned rows take the vector kernel (8
// channels per lane per load); others the scalar one (lanes stride by one).

#include "device_common.h"
#include "kernels.h"
#include "norm_row.h"

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
    const float rstd = __builtin_amdgcn_rsqf(ss / (float)gs + a.eps);

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

// Vector form for group widths that are multiples of 8 with 16-byte aligned
// rows: lane l handles 8-channel blocks l, l + 64, ... of its (token, group),
// each one 32-byte fp32 load of y and one 16- or 32-byte load of z
// (norm_row.h, shared with the chunk output's fused norm).
constexpr int MAXB = 4;   // 8-channel blocks per lane: group width up to 2048

template <typename Tz, typename Tout>
__global__ __launch_bounds__(BLOCK) void gated_norm_vec_kernel(NormArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * (BLOCK / 64) + (threadIdx.x >> 6);
    const int gs = a.d_inner / a.ngroups;
    if (item >= a.total_tokens * a.ngroups) return;
    const int64_t t = item / a.ngroups;
    const int j = (int)(item % a.ngroups);
    const int cbase = j * gs;
    const int nb = gs / 8;
    NormRow<MAXB, Tz> r;
    NormW<MAXB> W;
    norm_row_load_y(r, a.y + t * a.ld_y + cbase, nb, lane);
    norm_row_load_z(r, static_cast<const Tz*>(a.z) + t * a.ld_z + cbase, nb, lane);
    norm_w_load(W, a.norm_w + cbase, nb, lane);
    norm_row_store(r, W, static_cast<Tout*>(a.out) + t * a.ld_out + cbase, gs, nb, a.eps, a.norm_before_gate != 0,
                   lane);
}

}  // namespace

static bool gated_norm_vec_ok(const NormArgs& a) {
    const int gs = a.d_inner / a.ngroups;
    const int zes = a.z_dtype == kBF16 ? 2 : 4, oes = a.out_dtype == kBF16 ? 2 : 4;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    return gs % 8 == 0 && gs <= 64 * 8 * MAXB && al16(a.y) && al16(a.z) && al16(a.out) && al16(a.norm_w) &&
           (a.ld_y * 4) % 16 == 0 && (a.ld_z * zes) % 16 == 0 && (a.ld_out * oes) % 16 == 0;
}

hipError_t launch_gated_norm(const NormArgs& a, hipStream_t stream) {
    const int64_t items = a.total_tokens * a.ngroups;
    const dim3 grid((unsigned)((items + (BLOCK / 64) - 1) / (BLOCK / 64)));
    const bool zb = a.z_dtype == kBF16, ob = a.out_dtype == kBF16;
    if (gated_norm_vec_ok(a)) {
        if (zb && ob) hipLaunchKernelGGL((gated_norm_vec_kernel<uint16_t, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
        else if (zb) hipLaunchKernelGGL((gated_norm_vec_kernel<uint16_t, float>), grid, dim3(BLOCK), 0, stream, a);
        else if (ob) hipLaunchKernelGGL((gated_norm_vec_kernel<float, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
        else hipLaunchKernelGGL((gated_norm_vec_kernel<float, float>), grid, dim3(BLOCK), 0, stream, a);
        return hipGetLastError();
    }
    if (zb && ob) hipLaunchKernelGGL((gated_norm_kernel<uint16_t, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
    else if (zb) hipLaunchKernelGGL((gated_norm_kernel<uint16_t, float>), grid, dim3(BLOCK), 0, stream, a);
    else if (ob) hipLaunchKernelGGL((gated_norm_kernel<float, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
    else hipLaunchKernelGGL((gated_norm_kernel<float, float>), grid, dim3(BLOCK), 0, stream, a);
    return hipGetLastError();
}

}  // namespace m2
