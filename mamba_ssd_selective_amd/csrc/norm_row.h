// The grouped gated RMSNorm of one (row, group), on one wavefront, shared by
// the norm kernel (gated_norm.hip) and the chunk output's fused norm
// (ssd_chunked.hip), so both give the same bits.
//
// Page "Nemotron-H", section 4.1: the scan output y is RMS-normalized over each
// group of channels with the ssm_norm weight and gated by SiLU(z); with
// norm_before_gate the norm comes first (out = y rstd(y) w SiLU(z)), otherwise
// the gate (u = y SiLU(z), out = u rstd(u) w).  rstd(u) = 1 / sqrt(mean(u^2) +
// eps) over the group's gs channels.
//
// Lane l takes the 8-channel blocks l, l + 64, ... (NBL of them; blocks at or
// past nb = gs / 8 are skipped), so gs must be a multiple of 8 and at most
// 512 NBL, and the rows 16-byte aligned.  The loads are separate steps, so a
// wave can keep several rows' loads in flight and issue z (and the weights)
// before y is ready; norm_row_store reduces and writes.
#pragma once

#include "device_common.h"

namespace m2 {

template <int NBL>
struct NormW {
    float w[NBL][8];
};

template <int NBL>
__device__ __forceinline__ void norm_w_load(NormW<NBL>& W, const float* wr, int nb, int lane) {
#pragma unroll
    for (int k = 0; k < NBL; ++k)
        if (lane + 64 * k < nb) load8(wr + 8 * (lane + 64 * k), W.w[k]);
}

// z kept as loaded (bf16 bits, 8 per 16 bytes, or fp32) until the row is reduced.
template <typename Tz> struct NormZ;
template <> struct NormZ<uint16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ float at(int e) const {
        const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
        return __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};
template <> struct NormZ<float> {
    float v[8];
    __device__ __forceinline__ void load(const float* p) { load8(p, v); }
    __device__ __forceinline__ float at(int e) const { return v[e]; }
};

template <int NBL, typename Tz>
struct NormRow {
    float y[NBL][8];
    NormZ<Tz> z[NBL];
};

template <int NBL, typename Tz>
__device__ __forceinline__ void norm_row_load_z(NormRow<NBL, Tz>& r, const Tz* zr, int nb, int lane) {
#pragma unroll
    for (int k = 0; k < NBL; ++k)
        if (lane + 64 * k < nb) r.z[k].load(zr + 8 * (lane + 64 * k));
}

template <int NBL, typename Tz>
__device__ __forceinline__ void norm_row_load_y(NormRow<NBL, Tz>& r, const float* yr, int nb, int lane) {
#pragma unroll
    for (int k = 0; k < NBL; ++k)
        if (lane + 64 * k < nb) load8(yr + 8 * (lane + 64 * k), r.y[k]);
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = float4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<float4*>(p + 4) = float4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = (uint32_t)f32_to_bf16_bits(v[2 * k]) | ((uint32_t)f32_to_bf16_bits(v[2 * k + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = uint4{w[0], w[1], w[2], w[3]};
}

template <int NBL, typename Tz, typename Tout>
__device__ __forceinline__ void norm_row_store(const NormRow<NBL, Tz>& r, const NormW<NBL>& W, Tout* orow, int gs,
                                               int nb, float eps, bool norm_before_gate, int lane) {
    float v[NBL][8], gate[NBL][8];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        if (lane + 64 * k < nb) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float g = silu(r.z[k].at(e));
                const float u = norm_before_gate ? r.y[k][e] : r.y[k][e] * g;
                v[k][e] = u;
                gate[k][e] = g;
                ss = fmaf(u, u, ss);
            }
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float rstd = __builtin_amdgcn_rsqf(ss / (float)gs + eps);
#pragma unroll
    for (int k = 0; k < NBL; ++k) {
        const int b = lane + 64 * k;
        if (b < nb) {
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = v[k][e] * rstd * W.w[k][e];
                if (norm_before_gate) o[e] *= gate[k][e];
            }
            store8(orow + 8 * b, o);
        }
    }
}

}  // namespace m2
