// Causal depthwise conv1d (width 4) + SiLU over the carried conv state and the
// new rows of a packed varlen batch, and the conv-state advance, for gfx950.
//
// Page "perf(nemotron_h): prefill single-GPU prompts in multi-token chunks",
// section Implementation: the short conv of a chunk reads the conv state carried
// from earlier rows ahead of the chunk's own rows.  Page "Nemotron-H", sections
// 3 and 4.1: the conv runs over the xBC stream and its output goes through
// SiLU; section 10: the conv state keeps (width - 1) rows per channel.
//
// The conv is HBM-bound (4 multiply-adds per element read), so the kernel is a
// streaming pass: a thread owns 8 adjacent channels (one 16-byte bf16 load, two
// for fp32) and a run of TOK consecutive packed rows, keeps the last three raw
// rows of its channels in registers as a sliding window, and refills the window
// from the slot's conv state (or zeros) whenever its run enters a new sequence.
// Weights and bias of its 8 channels stay in registers for the whole run.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace m2 {
namespace {

constexpr int TOK = 16;    // rows per thread
constexpr int CPT = 8;     // channels per thread
constexpr int BLOCK = 256;

__device__ __forceinline__ int seq_of(const int32_t* cu, int batch, int64_t t) {
    // last b with cu[b] <= t and cu[b+1] > t (skips empty sequences)
    int lo = 0, hi = batch;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

template <typename Tin>
__device__ __forceinline__ const Tin* seg_row(const ConvArgs& a, int seg, int64_t row, int cs) {
    return static_cast<const Tin*>(a.seg_ptr[seg]) + row * a.seg_ld[seg] + cs;
}

// Stores of 8 consecutive outputs (16-byte aligned rows).
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
__device__ __forceinline__ void store8(double* p, const double (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) *reinterpret_cast<double2*>(p + 2 * k) = double2{v[2 * k], v[2 * k + 1]};
}

// Computes in fp64 when the output is fp64 (the fp32-input prefill path), else fp32.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(BLOCK) void conv_rows_kernel(ConvArgs a) {
    using T = typename std::conditional<std::is_same<Tout, double>::value, double, float>::type;
    const int c0 = (blockIdx.y * BLOCK + threadIdx.x) * CPT;   // first channel of this thread
    if (c0 >= a.conv_dim) return;
    const int64_t t0 = (int64_t)blockIdx.x * TOK;
    if (t0 >= a.total_tokens) return;
    const int64_t t1 = (t0 + TOK < a.total_tokens) ? t0 + TOK : a.total_tokens;

    // segment of these channels
    int seg = 0, cs = c0;
    while (seg + 1 < a.nseg && cs >= a.seg_ch[seg]) { cs -= a.seg_ch[seg]; ++seg; }

    T w[CPT][4], bias[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const float4 wv = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)(c0 + c) * 4);
        w[c][0] = wv.x; w[c][1] = wv.y; w[c][2] = wv.z; w[c][3] = wv.w;
        bias[c] = a.conv_b ? a.conv_b[c0 + c] : 0.f;
    }

    int b = seq_of(a.cu_seqlens, a.batch, t0);
    int64_t s0 = a.cu_seqlens[b];
    int64_t s1 = a.cu_seqlens[b + 1];
    Tout* out = static_cast<Tout*>(a.out);

    if (t0 - 3 >= s0 && t1 <= s1) {
        // The run and its 3-row halo lie inside one sequence: issue every row's
        // load up front, then slide the window over registers.
        // raw 16-byte pieces: one per row for bf16, two for fp32
        constexpr int PR = (int)sizeof(Tin) / 2;
        uint4 raw[TOK + 3][PR];
#pragma unroll
        for (int k = 0; k < TOK + 3; ++k) {
            const int64_t t = t0 - 3 + k;
            if (t < t1) {
                const uint4* src = reinterpret_cast<const uint4*>(seg_row<Tin>(a, seg, t, cs));
#pragma unroll
                for (int h = 0; h < PR; ++h) raw[k][h] = src[h];
            }
        }
        auto val = [&](int k, int c) -> T {
            if constexpr (sizeof(Tin) == 2) {
                const uint32_t wd = c < 2 ? raw[k][0].x : c < 4 ? raw[k][0].y : c < 6 ? raw[k][0].z : raw[k][0].w;
                return (T)__builtin_bit_cast(float, (c & 1) ? (wd & 0xffff0000u) : (wd << 16));
            } else {
                const uint4& q4 = raw[k][c >> 2];
                const int e = c & 3;
                return (T)__builtin_bit_cast(float, e == 0 ? q4.x : e == 1 ? q4.y : e == 2 ? q4.z : q4.w);
            }
        };
#pragma unroll
        for (int k = 0; k < TOK; ++k) {
            const int64_t t = t0 + k;
            if (t < t1) {
                T o[CPT];
#pragma unroll
                for (int c = 0; c < CPT; ++c) {
                    T acc = bias[c];
                    acc = fma(w[c][0], val(k, c), acc);
                    acc = fma(w[c][1], val(k + 1, c), acc);
                    acc = fma(w[c][2], val(k + 2, c), acc);
                    acc = fma(w[c][3], val(k + 3, c), acc);
                    o[c] = a.apply_silu ? silu(acc) : acc;
                }
                store8(out + t * a.ld_out + c0, o);
            }
        }
        return;
    }

    T win[3][CPT];   // raw rows t-3, t-2, t-1

    auto fill_window = [&](int64_t t) {
        // rows t-3..t-1 of sequence b: from the stream if inside it, else from the state
        const int slot = a.state_idx ? a.state_idx[b] : b;
        const bool init = a.has_init ? (a.has_init[b] != 0) : true;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const int64_t j = (t - s0) - 3 + d;     // position of the needed row in the sequence
            T v[CPT];
            if (j >= 0) {
                load8(seg_row<Tin>(a, seg, s0 + j, cs), v);
            } else if (init) {
                load8(a.conv_state + ((int64_t)slot * 3 + (3 + j)) * a.conv_dim + c0, v);
            } else {
#pragma unroll
                for (int c = 0; c < CPT; ++c) v[c] = 0.f;
            }
#pragma unroll
            for (int c = 0; c < CPT; ++c) win[d][c] = v[c];
        }
    };
    fill_window(t0);

    for (int64_t t = t0; t < t1; ++t) {
        if (t >= s1) {   // entered a later sequence (skip empty ones)
            while (t >= a.cu_seqlens[b + 1]) ++b;
            s0 = a.cu_seqlens[b];
            s1 = a.cu_seqlens[b + 1];
            fill_window(t);
        }
        T cur[CPT];
        load8(seg_row<Tin>(a, seg, t, cs), cur);
        T o[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            T acc = bias[c];
            acc = fma(w[c][0], win[0][c], acc);
            acc = fma(w[c][1], win[1][c], acc);
            acc = fma(w[c][2], win[2][c], acc);
            acc = fma(w[c][3], cur[c], acc);
            o[c] = a.apply_silu ? silu(acc) : acc;
            win[0][c] = win[1][c];
            win[1][c] = win[2][c];
            win[2][c] = cur[c];
        }
        store8(out + t * a.ld_out + c0, o);
    }
}

// New conv state of each sequence: the last three rows of [old state ; rows].
// One thread per (sequence, channel); it reads the old values before writing.
template <typename Tin>
__global__ __launch_bounds__(BLOCK) void conv_state_kernel(ConvArgs a) {
    const int c = blockIdx.x * BLOCK + threadIdx.x;
    const int b = blockIdx.y;
    if (c >= a.conv_dim) return;
    int seg = 0, cs = c;
    while (seg + 1 < a.nseg && cs >= a.seg_ch[seg]) { cs -= a.seg_ch[seg]; ++seg; }
    const int64_t s0 = a.cu_seqlens[b];
    const int64_t L = a.cu_seqlens[b + 1] - s0;
    const int slot = a.state_idx ? a.state_idx[b] : b;
    const bool init = a.has_init ? (a.has_init[b] != 0) : true;
    float* st = a.conv_state + (int64_t)slot * 3 * a.conv_dim + c;
    float old[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) old[j] = init ? st[(int64_t)j * a.conv_dim] : 0.f;
    float nw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t k = L + j;   // index into [old(3) ; rows(L)]
        nw[j] = (k < 3) ? old[k] : Act<Tin>::load(seg_row<Tin>(a, seg, s0 + (k - 3), cs));
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) st[(int64_t)j * a.conv_dim] = nw[j];
}

}  // namespace

hipError_t launch_conv_rows(const ConvArgs& a, hipStream_t stream) {
    const int64_t tok_blocks = (a.total_tokens + TOK - 1) / TOK;
    const int ch_blocks = (a.conv_dim / CPT + BLOCK - 1) / BLOCK;
    const dim3 grid((unsigned)tok_blocks, ch_blocks);
    if (a.act_dtype == kBF16) {
        if (a.out_dtype == kBF16)
            hipLaunchKernelGGL((conv_rows_kernel<uint16_t, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
        else if (a.out_dtype == kF64)
            hipLaunchKernelGGL((conv_rows_kernel<uint16_t, double>), grid, dim3(BLOCK), 0, stream, a);
        else
            hipLaunchKernelGGL((conv_rows_kernel<uint16_t, float>), grid, dim3(BLOCK), 0, stream, a);
    } else {
        if (a.out_dtype == kBF16)
            hipLaunchKernelGGL((conv_rows_kernel<float, uint16_t>), grid, dim3(BLOCK), 0, stream, a);
        else if (a.out_dtype == kF64)
            hipLaunchKernelGGL((conv_rows_kernel<float, double>), grid, dim3(BLOCK), 0, stream, a);
        else
            hipLaunchKernelGGL((conv_rows_kernel<float, float>), grid, dim3(BLOCK), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_conv_state_update(const ConvArgs& a, hipStream_t stream) {
    const dim3 grid((a.conv_dim + BLOCK - 1) / BLOCK, a.batch);
    if (a.act_dtype == kBF16)
        hipLaunchKernelGGL((conv_state_kernel<uint16_t>), grid, dim3(BLOCK), 0, stream, a);
    else
        hipLaunchKernelGGL((conv_state_kernel<float>), grid, dim3(BLOCK), 0, stream, a);
    return hipGetLastError();
}

}  // namespace m2
