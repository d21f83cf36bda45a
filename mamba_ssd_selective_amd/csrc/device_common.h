// Device-side helpers shared by the gfx950 kernels of the Mamba-2 prefill library:
// element loads for the two activation types, SiLU, and the matrix-core operand
// policies used by the chunked scan.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- element access

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite on every path that
// stores bf16; NaN keeps a quiet payload).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Activation element types: float (M2_F32) or raw bf16 bits (M2_BF16).
template <typename T> struct Act;
template <> struct Act<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Act<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
    __device__ __forceinline__ static void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};
template <> struct Act<double> {
    __device__ __forceinline__ static double load(const double* p) { return *p; }
    __device__ __forceinline__ static void store(double* p, double v) { *p = v; }
};

// Load 8 consecutive activations (16-byte aligned for bf16, 32-byte for fp32 callers
// use two float4) into fp32.
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __builtin_bit_cast(float, w[k] << 16);
        v[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
    }
}

// Widening copies used when fp32 / bf16 data feed an fp64 computation.
__device__ __forceinline__ void load8(const float* p, double (&v)[8]) {
    float f[8];
    load8(p, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = f[j];
}
__device__ __forceinline__ void load8(const uint16_t* p, double (&v)[8]) {
    float f[8];
    load8(p, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = f[j];
}
__device__ __forceinline__ void load8(const double* p, double (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const double2 d = *reinterpret_cast<const double2*>(p + 2 * k);
        v[2 * k] = d.x;
        v[2 * k + 1] = d.y;
    }
}

// SiLU with the hardware reciprocal (~1 ulp) instead of an IEEE division: the
// division sequence dominated the instruction count of the conv and the norm.
// Large negative v gives exp(-v) = inf and v * rcp(inf) = -0, the right limit.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }
__device__ __forceinline__ double silu(double v) { return v / (1.0 + exp(-v)); }

// ---------------------------------------------------------------- matrix-core operands
//
// Every contraction of the scan is a sum of 16x16 output tiles over K blocks of
// 32.  The output tile of a product lands as: lane l holds column l % 16 and, in
// register r, row Pol::orow(l / 16, r) -- 4q + r for the fp32-accumulating
// instructions, q + 4r for the fp64 one.  In a K block each lane supplies 8
// values: lane l serves row (or column) l % 16 of its operand and, in "slot"
// j = 0..7, the K index kslot<Pol>(l / 16, j).  Any K order is valid as long as
// both operands of a product use the same one; the scan takes the rows a pair
// of accumulator tiles already holds in lane group q (slots 0-3 from the first
// tile, 4-7 from the second), so an accumulator pair feeds the next product
// without any data exchange.

template <class Pol>
__device__ __forceinline__ int kslot(int q, int j) {
    return j < 4 ? Pol::orow(q, j) : 16 + Pol::orow(q, j - 4);
}

// Each policy fixes the value type the scan computes in (Val), the accumulator
// tile type, the largest chunk it stages in LDS, and exp of a clamped exponent.
//
// PolicyBf16x3 (bf16 inputs): bf16 matrix cores on a two-term split
// v = hi + lo with hi = bf16(v), lo = bf16(v - hi); a product is
// hi*hi + hi*lo + lo*hi (the lo*lo term, ~2^-18 relative, is dropped),
// accumulated in fp32.
struct PolicyBf16x3 {
    using Val = float;
    using Acc = f32x4_t;
    static constexpr int QMAX = 128;
    static constexpr bool kRowsContiguous = true;
    __device__ __forceinline__ static int orow(int q, int r) { return 4 * q + r; }
    struct Op { bf16x8_t hi, lo; };
    __device__ __forceinline__ static Op make(const float (&v)[8]) {
        Op o;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const __bf16 h = static_cast<__bf16>(v[j]);
            o.hi[j] = h;
            o.lo[j] = static_cast<__bf16>(v[j] - static_cast<float>(h));
        }
        return o;
    }
    __device__ __forceinline__ static void mma(Acc& acc, const Op& a, const Op& b) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    }
    __device__ __forceinline__ static float expc(double v) { return __expf(static_cast<float>(v)); }
};

// PolicyF64 (fp32 inputs): fp64 matrix cores, eight 16x16x4 products per K
// block (slot j in product j).  The output of a chunk scales with dt * (C . B)
// and with C . h, so at |dt A| ~ 1e6 an fp32 rounding of C, B or h is
// amplified far past 1e-4 of the output scale; fp64 keeps it at fp32 output
// rounding.  Chunks are staged 64 rows at a time so fp64 B and C fit in LDS.
struct PolicyF64 {
    using Val = double;
    using Acc = f64x4_t;
    static constexpr int QMAX = 64;
    static constexpr bool kRowsContiguous = false;
    __device__ __forceinline__ static int orow(int q, int r) { return q + 4 * r; }
    struct Op { double v[8]; };
    __device__ __forceinline__ static Op make(const double (&v)[8]) {
        Op o;
#pragma unroll
        for (int j = 0; j < 8; ++j) o.v[j] = v[j];
        return o;
    }
    __device__ __forceinline__ static void mma(Acc& acc, const Op& a, const Op& b) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a.v[j], b.v[j], acc, 0, 0, 0);
    }
    __device__ __forceinline__ static double expc(double v) { return exp(v); }
};

}  // namespace m2
