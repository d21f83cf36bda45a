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
// streaming pass: a thread owns CPT = 4 adjacent channels (an 8-byte bf16 load,
// a 16-byte fp32 one, one 16-byte store per fp32 output row) and a run of TOK
// consecutive packed rows (24; 8 when runs of 24 would leave most CUs idle, as
// for a single short prompt).  It issues the
// loads of the run's rows and 3-row halo first, then slides a window over
// registers; a run that starts a sequence or crosses into another one goes row
// by row instead, refilling the window from the slot's conv state (or zeros).
// Weights and bias of its channels stay in registers for the whole run.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace m2 {
namespace {

constexpr int TOK_LONG = 24;   // rows per thread
constexpr int TOK_SHORT = 8;   // rows per thread when the grid would be small
constexpr int CPT = 4;         // channels per thread
constexpr int BLOCK = 128;

__device__ __forceinline__ int seq_of(const int32_t* cu, int batch, int64_t t) {
    // last b with cu[b] <= t and cu[b+1] > t (skips empty sequences)
    int lo = 0, hi = batch;  // answer in [lo, hi)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}

// Column `c` of the xBC stream as (first element of that column, row stride).
// The column pointer is marked as global memory: global loads can be waited
// for one at a time, generic (flat) ones only all together.
template <typename T>
using gptr = const __attribute__((address_space(1))) T*;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef double f64x2v_t __attribute__((ext_vector_type(2)));
template <typename Tin>
struct SegCol {
    gptr<Tin> col;
    int64_t ld;
    __device__ __forceinline__ gptr<Tin> grow(int64_t t) const { return col + t * ld; }
    __device__ __forceinline__ const Tin* row(int64_t t) const { return (const Tin*)grow(t); }
};
// Per lane (channel c of the whole stream; lanes of a wave may differ).
template <typename Tin>
__device__ __forceinline__ SegCol<Tin> seg_col_lane(const ConvArgs& a, int c) {
    int seg = 0;
    while (seg + 1 < a.nseg && c >= a.seg_ch[seg]) { c -= a.seg_ch[seg]; ++seg; }
    return SegCol<Tin>{(gptr<Tin>)a.seg_ptr[seg] + c, a.seg_ld[seg]};
}

// The conv launch gives every segment its own channel blocks of BLOCK * CPT
// channels, so a block never straddles two segments and the segment is the
// same for all its lanes: its table entries are then scalar loads.  (A
// per-lane choice among the three segment pointers made the compiler copy the
// whole argument block to scratch memory.)
struct BlockSeg {
    int seg;     // segment index
    int cs0;     // first channel of the block within the segment
    int cbase;   // first channel of the segment in the whole stream
};
__device__ __forceinline__ BlockSeg block_seg(const ConvArgs& a, int y, int width) {
    BlockSeg r{0, 0, 0};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        if (r.seg != s || s + 1 >= a.nseg) break;
        const int nb = (a.seg_ch[s] + width - 1) / width;
        if (y < nb) break;
        y -= nb;
        r.cbase += a.seg_ch[s];
        r.seg = s + 1;
    }
    r.cs0 = y * width;
    return r;
}
__host__ __device__ __forceinline__ int conv_channel_blocks(const ConvArgs& a, int width) {
    int n = 0;
    for (int s = 0; s < a.nseg; ++s) n += (a.seg_ch[s] + width - 1) / width;
    return n;
}

// Global-memory vector stores of one thread's CPT outputs (CPT = 4 or 8; rows
// are 16-byte aligned and CPT-channel groups start at a multiple of CPT).
template <typename E, int L>
using vec = E __attribute__((ext_vector_type(L)));
template <typename E, int L>
using gvec = __attribute__((address_space(1))) vec<E, L>;
template <int N>
__device__ __forceinline__ void store_out(float* p, const float (&v)[N]) {
    auto* q = (gvec<float, 4>*)p;
#pragma unroll
    for (int k = 0; k < N / 4; ++k) q[k] = f32x4v_t{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
}
template <int N>
__device__ __forceinline__ void store_out(uint16_t* p, const float (&v)[N]) {
    uint32_t w[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k)
        w[k] = (uint32_t)f32_to_bf16_bits(v[2 * k]) | ((uint32_t)f32_to_bf16_bits(v[2 * k + 1]) << 16);
    if constexpr (N == 4) {
        *(gvec<uint32_t, 2>*)p = u32x2_t{w[0], w[1]};
    } else {
#pragma unroll
        for (int k = 0; k < N / 8; ++k) ((gvec<uint32_t, 4>*)p)[k] = u32x4_t{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    }
}
template <int N>
__device__ __forceinline__ void store_out(double* p, const double (&v)[N]) {
    auto* q = (gvec<double, 2>*)p;
#pragma unroll
    for (int k = 0; k < N / 2; ++k) q[k] = f64x2v_t{v[2 * k], v[2 * k + 1]};
}

// Computes in fp64 when the output is fp64 (the fp32-input prefill path), else fp32.
template <typename Tin, typename Tout, int TOK>
__global__ __launch_bounds__(BLOCK) void conv_rows_kernel(ConvArgs a) {
    using T = typename std::conditional<std::is_same<Tout, double>::value, double, float>::type;
    const BlockSeg bs = block_seg(a, blockIdx.y, BLOCK * CPT);
    const int cs = bs.cs0 + threadIdx.x * CPT;   // first channel of this thread in its segment
    if (cs >= a.seg_ch[bs.seg]) return;
    const int c0 = bs.cbase + cs;                 // ... and in the whole stream
    const int64_t t0 = (int64_t)blockIdx.x * TOK;
    if (t0 >= a.total_tokens) return;
    const int64_t t1 = (t0 + TOK < a.total_tokens) ? t0 + TOK : a.total_tokens;
    const SegCol<Tin> sc{(gptr<Tin>)a.seg_ptr[bs.seg] + cs, a.seg_ld[bs.seg]};

    // Rows t0-3 .. t0+TOK-1 are loaded before the sequence lookup below, so their
    // latency overlaps its dependent reads of cu_seqlens; row indices are clamped
    // to the stream, and runs that need other rows (a sequence starts inside the
    // window, or the stream ends) take the row-at-a-time path further down.
    // A row's CPT inputs are NW 32-bit words, loaded as NV vectors of VL words.
    constexpr int NW = CPT * (int)sizeof(Tin) / 4;
    constexpr int VL = NW < 4 ? NW : 4;
    constexpr int NV = NW / VL;
    uint32_t raw[TOK + 3][NW];
    {
        const int64_t last = a.total_tokens - 1;
#pragma unroll
        for (int k = 0; k < TOK + 3; ++k) {
            int64_t r = t0 - 3 + k;
            r = r < 0 ? 0 : r > last ? last : r;
            const auto* src = (const gvec<uint32_t, VL>*)sc.grow(r);
#pragma unroll
            for (int h = 0; h < NV; ++h) {
                const vec<uint32_t, VL> v = src[h];
#pragma unroll
                for (int e = 0; e < VL; ++e) raw[k][h * VL + e] = v[e];
            }
        }
    }

    T w[CPT][4], bias[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        const float4 wv = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)(c0 + c) * 4);
        w[c][0] = wv.x; w[c][1] = wv.y; w[c][2] = wv.z; w[c][3] = wv.w;
    }
    if (a.conv_b) {
#pragma unroll
        for (int k = 0; k < CPT / 4; ++k) {
            const float4 bv = *reinterpret_cast<const float4*>(a.conv_b + c0 + 4 * k);
            bias[4 * k] = bv.x; bias[4 * k + 1] = bv.y; bias[4 * k + 2] = bv.z; bias[4 * k + 3] = bv.w;
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) bias[c] = 0.f;
    }

    int b = seq_of(a.cu_seqlens, a.batch, t0);
    int64_t s0 = a.cu_seqlens[b];
    int64_t s1 = a.cu_seqlens[b + 1];
    // this thread's output column (its CPT channels lie in one output block)
    const int obw = a.out_bw[bs.seg];
    Tout* const ocol = static_cast<Tout*>(a.out_ptr[bs.seg]) + (int64_t)(cs / obw) * a.out_bs[bs.seg] + cs % obw;
    const int64_t old = a.out_ld[bs.seg];

    if (t0 - 3 >= s0 && t0 + TOK <= s1) {
        // A full run whose 3-row halo lies inside the same sequence: the rows
        // loaded above are exactly its window; slide it over registers.
        auto val = [&](int k, int c) -> T {
            if constexpr (sizeof(Tin) == 2) {
                const uint32_t wd = raw[k][c >> 1];
                return (T)__builtin_bit_cast(float, (c & 1) ? (wd & 0xffff0000u) : (wd << 16));
            } else {
                return (T)__builtin_bit_cast(float, raw[k][c]);
            }
        };
        Tout* dst = ocol + t0 * old;
#pragma unroll
        for (int k = 0; k < TOK; ++k) {
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
            store_out(dst + k * old, o);
        }
        return;
    }

    // Runs at a sequence start or across a sequence boundary (a few per
    // sequence): a row at a time with element loads.
    T win[3][CPT];   // raw rows t-3, t-2, t-1

    const int32_t* const state_idx = a.state_idx;
    const uint8_t* const has_init = a.has_init;
    const float* const conv_state = a.conv_state;
    const int conv_dim = a.conv_dim;
    // (captures no reference to the kernel argument block: that would make the
    // compiler copy it to scratch memory)
    auto fill_window = [&win, &sc, &s0, &b, state_idx, has_init, conv_state, conv_dim, c0](int64_t t) {
        // rows t-3..t-1 of sequence b: from the stream if inside it, else from the state
        const int slot = state_idx ? state_idx[b] : b;
        const bool init = has_init ? (has_init[b] != 0) : true;
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            const int64_t j = (t - s0) - 3 + d;     // position of the needed row in the sequence
            if (j >= 0) {
                const Tin* row = sc.row(s0 + j);
#pragma unroll
                for (int c = 0; c < CPT; ++c) win[d][c] = (T)Act<Tin>::load(row + c);
            } else if (init) {
                const float* st = conv_state + ((int64_t)slot * 3 + (3 + j)) * conv_dim + c0;
#pragma unroll
                for (int c = 0; c < CPT; ++c) win[d][c] = (T)st[c];
            } else {
#pragma unroll
                for (int c = 0; c < CPT; ++c) win[d][c] = (T)0;
            }
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
        const Tin* row = sc.row(t);
        T o[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const T cur = (T)Act<Tin>::load(row + c);
            T acc = bias[c];
            acc = fma(w[c][0], win[0][c], acc);
            acc = fma(w[c][1], win[1][c], acc);
            acc = fma(w[c][2], win[2][c], acc);
            acc = fma(w[c][3], cur, acc);
            o[c] = a.apply_silu ? silu(acc) : acc;
            win[0][c] = win[1][c];
            win[1][c] = win[2][c];
            win[2][c] = cur;
        }
        store_out(ocol + t * old, o);
    }
}

// New conv state of each sequence: the last three rows of [old state ; rows].
// One thread per (sequence, channel); it reads the old values before writing.
template <typename Tin>
__global__ __launch_bounds__(BLOCK) void conv_state_kernel(ConvArgs a) {
    const int c = blockIdx.x * BLOCK + threadIdx.x;
    const int b = blockIdx.y;
    if (c >= a.conv_dim) return;
    const SegCol<Tin> sc = seg_col_lane<Tin>(a, c);
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
        nw[j] = (k < 3) ? old[k] : Act<Tin>::load(sc.row(s0 + (k - 3)));
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) st[(int64_t)j * a.conv_dim] = nw[j];
}

}  // namespace

template <int TOK>
hipError_t launch_rows(const ConvArgs& a, hipStream_t stream) {
    const int64_t tok_blocks = (a.total_tokens + TOK - 1) / TOK;
    const dim3 grid((unsigned)tok_blocks, conv_channel_blocks(a, BLOCK * CPT));
    if (a.act_dtype == kBF16) {
        if (a.out_dtype == kBF16)
            hipLaunchKernelGGL((conv_rows_kernel<uint16_t, uint16_t, TOK>), grid, dim3(BLOCK), 0, stream, a);
        else if (a.out_dtype == kF64)
            hipLaunchKernelGGL((conv_rows_kernel<uint16_t, double, TOK>), grid, dim3(BLOCK), 0, stream, a);
        else
            hipLaunchKernelGGL((conv_rows_kernel<uint16_t, float, TOK>), grid, dim3(BLOCK), 0, stream, a);
    } else {
        if (a.out_dtype == kBF16)
            hipLaunchKernelGGL((conv_rows_kernel<float, uint16_t, TOK>), grid, dim3(BLOCK), 0, stream, a);
        else if (a.out_dtype == kF64)
            hipLaunchKernelGGL((conv_rows_kernel<float, double, TOK>), grid, dim3(BLOCK), 0, stream, a);
        else
            hipLaunchKernelGGL((conv_rows_kernel<float, float, TOK>), grid, dim3(BLOCK), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_conv_rows(const ConvArgs& a, hipStream_t stream) {
    // runs of 24 rows unless that leaves fewer workgroups than CUs
    const int64_t long_blocks = (a.total_tokens + TOK_LONG - 1) / TOK_LONG;
    if (long_blocks * conv_channel_blocks(a, BLOCK * CPT) < 256) return launch_rows<TOK_SHORT>(a, stream);
    return launch_rows<TOK_LONG>(a, stream);
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
