// Single-token decode step of the Mamba-2 mixer core, for gfx950: the causal
// conv update, the selective state update with its readout, and the grouped
// gated RMSNorm, fused in one kernel over cache slots.
//
// Page "NemotronH decodes on the single-step recurrent kernels" (PR
// description): a decode row advances the conv state and the SSM state of its
// cache slot in place, with no gather or scatter, and must agree with the
// chunk scan run over the same row at the production group count.  Page
// "Nemotron-H", sections 3 and 4.1: the conv output goes through SiLU and
// splits into x, B and C; the state follows
//   h <- e(dt A) h + dt x (outer) B,   y = C . h + D x,
// with e(v) = exp(min(v, 0)) as in the chunked form (for valid inputs the
// exponent is never positive); y is RMS-normalized per group and gated with
// SiLU(z).  A one-token sequence through the chunked prefill computes the same
// function.
//
// One workgroup per (sequence, group): the group's x, B and C channels are
// exactly what its heads read, so the conv update, every head's state update
// and the norm over the group stay in one workgroup.  The step is bound by the
// state traffic (hpg x P x N fp32 per group, read and written once).  The
// group's state is one contiguous run in the pool; thread t handles float4s
// t, t + 256, t + 512, ... of it, so each wave instruction moves 1 KiB of
// consecutive bytes, and the next batch of 8 float4s per thread is requested
// before the current one is updated.  Since 256 is a multiple of N / 4, a
// thread always holds the same four state columns (its B and C values stay in
// registers), and the N / 4 float4s of one state row sit in consecutive lanes
// of one wave.  The readout's sums over n for the 8 rows a lane touches in a
// batch are reduced together: each exchange step halves the rows a lane keeps
// (8 -> 4 -> 2 -> 1) while it sums pairs of lanes, then plain butterflies
// finish; 9 exchanges per 8 rows instead of 40, in a fixed order, so results
// are bitwise repeatable.  Every per-channel load of the conv, gate and
// weights is issued before any of them is used.  The step size comes either as
// fp32 dt or, for rows taken straight from the in-projection, as the raw value
// in the activation type, turned into softplus(raw + bias[h]) where it is read.

#include "device_common.h"
#include "kernels.h"
#include "step_size.h"

namespace m2 {
namespace {

constexpr int NT = 256;
constexpr int KB = 8;          // float4s per thread per batch of the state stream
constexpr int CU = 4;          // channels per thread per pass of the conv update
constexpr int MAXGW = 2048;    // x channels (norm width) of one group: hpg * P

using gf4 = __attribute__((address_space(1))) f32x4_t*;

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Sums over the RQ consecutive lanes of a row group for KB rows at once.  On
// entry v[k] is this lane's partial of row k; on return v[i], i < KB >> HS,
// holds the full sum of row k = i + (KB >> HS) * S with S from the lane's bits
// (returned), identical in every lane whose bits below RQ >> HS agree.
template <int RQ>
__device__ __forceinline__ int reduce_rows(float (&v)[KB], int lane) {
    constexpr int HS = ilog2(RQ) < ilog2(KB) ? ilog2(RQ) : ilog2(KB);
    int S = 0;
#pragma unroll
    for (int s = 0; s < HS; ++s) {
        const int m = RQ >> (s + 1);
        const int c = KB >> (s + 1);
        const bool hi = (lane & m) != 0;
#pragma unroll
        for (int i = 0; i < c; ++i) {
            const float send = hi ? v[i] : v[i + c];
            const float keep = hi ? v[i + c] : v[i];
            v[i] = keep + __shfl_xor(send, m, 64);
        }
        S = 2 * S + (hi ? 1 : 0);
    }
#pragma unroll
    for (int m = RQ >> (HS + 1); m >= 1; m >>= 1) {
#pragma unroll
        for (int i = 0; i < (KB >> HS); ++i) v[i] += __shfl_xor(v[i], m, 64);
    }
    return S;
}

// PART = false: the fused step, one workgroup per (sequence, group).
// PART = true (a small batch): a.split workgroups per (sequence, group), each
// taking a run of the group's heads: it convolves its heads' x channels and the
// group's B and C from the OLD conv state (which it does not write), advances
// its heads' SSM states and writes y before the norm (fp32) into y;
// decode_finish_kernel then advances the conv state and applies the norm.
template <int P, int N, typename Tin, typename Tout, bool PART>
__global__ __launch_bounds__(NT) void decode_step_kernel(DecodeArgs a) {
    constexpr int RQ = N / 4;  // float4s per state row (head j, row p)
    constexpr int HS = ilog2(RQ) < ilog2(KB) ? ilog2(RQ) : ilog2(KB);
    constexpr int CF = KB >> HS;       // row sums a lane holds after reduce_rows
    constexpr int WM = (RQ >> HS) - 1; // lanes with these bits zero write them
    static_assert(RQ <= 64 && NT % RQ == 0, "decode tile");

    const int S = PART ? a.split : 1;
    const int b = blockIdx.x / (a.ngroups * S), g = (blockIdx.x / S) % a.ngroups;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hpg = a.nheads / a.ngroups;
    const int gw = hpg * P;
    // this workgroup's heads j0 .. j0+nh-1 of the group and their x channels
    const int nh = hpg / S, j0 = (int)(blockIdx.x % S) * nh;
    const int xw = nh * P, xoff = j0 * P;
    const int ch = xw + 2 * N;
    const int d_x = a.nheads * P, d_b = a.ngroups * N;
    const int64_t conv_dim = d_x + 2 * d_b;
    const int slot = a.state_idx ? a.state_idx[b] : b;
    const bool init = a.has_init ? (a.has_init[b] != 0) : true;

    extern __shared__ float smem[];
    float* sdx = smem;            // dt * x            [xw]
    float* sxd = sdx + xw;        // D * x             [xw]
    float* sy = sxd + xw;         // y before the norm [xw]
    float* sg = sy + xw;          // SiLU(z)           [xw]
    float* sw = sg + xw;          // norm weight       [xw]
    float* sbc = sw + xw;         // post-conv B | C   [2N]
    float* sdA = sbc + 2 * N;     // e(dt A) per head  [nh]
    float* red = sdA + nh;        // [NT / 64]

    // Step size of head g*hpg + j: given in fp32, or softplus(raw + bias) of the
    // raw value in the activation type (the in-projection row's tail).
    const int64_t dto = (int64_t)b * a.ld_dt + (int64_t)g * hpg;
    auto step = [&](int j) -> float {
        if (a.dt_softplus)
            return softplus(Act<Tin>::load(static_cast<const Tin*>(a.dt) + dto + j) +
                            (a.dt_bias ? a.dt_bias[g * hpg + j] : 0.f));
        return static_cast<const float*>(a.dt)[dto + j];
    };
    const float* Ag = a.A + (int64_t)g * hpg;
    const bool has_b = a.conv_b != nullptr, has_d = a.D != nullptr;
    const float* Dg = has_d ? a.D + (int64_t)g * hpg : Ag;
    const Tin* zr = static_cast<const Tin*>(a.z) + (int64_t)b * a.ld_z + (int64_t)g * gw;
    const float* nw = a.norm_w + (int64_t)g * gw;

    // 1. Conv update of the group's ch = gw + 2N channels, out = SiLU(bias + w . [state ; x])
    //    with the state keeping its last three rows (oldest first); with it the
    //    per-channel factors of the state update and of the norm.
    for (int k0 = 0; k0 < ch; k0 += NT * CU) {
        float xin[CU], s0[CU], s1[CU], s2[CU], cb[CU], dtv[CU], dv[CU], zv[CU], wv[CU];
        f32x4_t w[CU];
        float* stp[CU];
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int k = min(k0 + tid + NT * u, ch - 1);
            int64_t cg;
            const Tin* src;
            if (k < xw) {
                cg = (int64_t)g * gw + xoff + k;
                src = static_cast<const Tin*>(a.x) + (int64_t)b * a.ld_x + cg;
            } else if (k < xw + N) {
                const int64_t n = (int64_t)g * N + (k - xw);
                cg = d_x + n;
                src = static_cast<const Tin*>(a.B) + (int64_t)b * a.ld_B + n;
            } else {
                const int64_t n = (int64_t)g * N + (k - xw - N);
                cg = d_x + d_b + n;
                src = static_cast<const Tin*>(a.C) + (int64_t)b * a.ld_C + n;
            }
            stp[u] = a.conv_state + (int64_t)slot * 3 * conv_dim + cg;
            s0[u] = stp[u][0];
            s1[u] = stp[u][conv_dim];
            s2[u] = stp[u][2 * conv_dim];
            xin[u] = Act<Tin>::load(src);
            w[u] = *reinterpret_cast<const f32x4_t*>(a.conv_w + cg * 4);
            cb[u] = (has_b ? a.conv_b : a.conv_w)[cg];
            const int kx = min(k, xw - 1);
            dtv[u] = step(j0 + kx / P);
            dv[u] = Dg[j0 + kx / P];
            if constexpr (!PART) {
                zv[u] = Act<Tin>::load(zr + kx);
                wv[u] = nw[kx];
            }
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
            const int k = k0 + tid + NT * u;
            const float t0 = init ? s0[u] : 0.f, t1 = init ? s1[u] : 0.f, t2 = init ? s2[u] : 0.f;
            float acc = has_b ? cb[u] : 0.f;
            acc = fmaf(w[u][0], t0, acc);
            acc = fmaf(w[u][1], t1, acc);
            acc = fmaf(w[u][2], t2, acc);
            acc = fmaf(w[u][3], xin[u], acc);
            const float v = silu(acc);
            if (k < xw) {
                sdx[k] = dtv[u] * v;
                sxd[k] = has_d ? dv[u] * v : 0.f;
                if constexpr (!PART) {
                    sg[k] = silu(zv[u]);
                    sw[k] = wv[u];
                }
            } else if (k < ch) {
                sbc[k - xw] = v;
            }
            if constexpr (!PART) {
                if (k < ch) {
                    stp[u][0] = t1;
                    stp[u][conv_dim] = t2;
                    stp[u][2 * conv_dim] = xin[u];
                }
            }
        }
    }
    for (int j = tid; j < nh; j += NT) sdA[j] = expf(fminf(step(j0 + j) * Ag[j0 + j], 0.f));
    __syncthreads();

    // 2. State update and readout over the group's state, a contiguous run of
    //    F float4s; thread t takes float4s base + t + NT k, k < KB, per batch.
    const int F = nh * P * RQ;
    gf4 sp = (gf4)(a.ssm_state + ((int64_t)slot * a.nheads + (int64_t)g * hpg + j0) * (P * N));
    const int n0 = (tid % RQ) * 4;
    const f32x4_t Bq = *reinterpret_cast<const f32x4_t*>(sbc + n0);
    const f32x4_t Cq = *reinterpret_cast<const f32x4_t*>(sbc + N + n0);
    f32x4_t buf0[KB], buf1[KB];
    auto load_batch = [&](f32x4_t (&v)[KB], int base) {
#pragma unroll
        for (int k = 0; k < KB; ++k) v[k] = sp[min(base + tid + NT * k, F - 1)];
    };
    // Update, store and read out one batch; float4s at or past F are skipped.
    auto update_batch = [&](const f32x4_t (&v)[KB], int base) {
        float part[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int f = base + tid + NT * k;
            const int row = min(f / RQ, xw - 1);  // j * P + p of this workgroup's heads
            const float dA = sdA[row / P];
            const float dx = sdx[row];
            f32x4_t h = init ? v[k] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = fmaf(dA, h[e], dx * Bq[e]);
            if (f < F) sp[f] = h;
            float acc = Cq[0] * h[0];
#pragma unroll
            for (int e = 1; e < 4; ++e) acc = fmaf(Cq[e], h[e], acc);
            part[k] = acc;
        }
        const int S = reduce_rows<RQ>(part, lane);
        if ((lane & WM) == 0) {
#pragma unroll
            for (int i = 0; i < CF; ++i) {
                const int row = (base + NT * (i + CF * S)) / RQ + tid / RQ;
                if (row < xw) sy[row] = part[i] + sxd[row];
            }
        }
    };
    // Two buffers in turn: the next batch is in flight while one is updated.
    // The loads are unconditional: past the end every lane reads float4 F - 1
    // (one cache line); a branch around them would make the compiler wait for
    // them before the update that they should overlap.
    load_batch(buf0, 0);
    for (int base = 0; base < F; base += 2 * NT * KB) {
        load_batch(buf1, base + NT * KB);
        update_batch(buf0, base);
        load_batch(buf0, base + 2 * NT * KB);
        update_batch(buf1, base + NT * KB);
    }
    __syncthreads();
    if constexpr (PART) {
        float* yo = static_cast<float*>(a.y) + (int64_t)b * a.ld_y + (int64_t)g * gw + xoff;
        for (int c = tid; c < xw; c += NT) yo[c] = sy[c];
        return;
    }

    // 3. Grouped gated RMSNorm over the group's gw channels.
    float ss = 0.f;
    for (int c = tid; c < gw; c += NT) {
        const float v = a.norm_before_gate ? sy[c] : sy[c] * sg[c];
        ss = fmaf(v, v, ss);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) tot += red[k];
    const float rstd = __builtin_amdgcn_rsqf(tot / (float)gw + a.eps);
    Tout* yo = static_cast<Tout*>(a.y) + (int64_t)b * a.ld_y + (int64_t)g * gw;
    for (int c = tid; c < gw; c += NT) {
        const float v = a.norm_before_gate ? sy[c] * rstd * sw[c] * sg[c] : sy[c] * sg[c] * rstd * sw[c];
        Act<Tout>::store(yo + c, v);
    }
}

// After the PART kernel: one workgroup per (sequence, group) advances the conv
// state of the group's channels (the rows were read by every PART workgroup
// before this launch) and applies the grouped gated RMSNorm to y in place.
template <int P, int N, typename Tin>
__global__ __launch_bounds__(NT) void decode_finish_kernel(DecodeArgs a) {
    __shared__ float red[NT / 64];
    const int b = blockIdx.x / a.ngroups, g = blockIdx.x % a.ngroups;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hpg = a.nheads / a.ngroups;
    const int gw = hpg * P;
    const int d_x = a.nheads * P, d_b = a.ngroups * N;
    const int64_t conv_dim = d_x + 2 * d_b;
    const int slot = a.state_idx ? a.state_idx[b] : b;
    const bool init = a.has_init ? (a.has_init[b] != 0) : true;
    for (int k = tid; k < gw + 2 * N; k += NT) {
        int64_t cg;
        const Tin* src;
        if (k < gw) {
            cg = (int64_t)g * gw + k;
            src = static_cast<const Tin*>(a.x) + (int64_t)b * a.ld_x + cg;
        } else if (k < gw + N) {
            const int64_t n = (int64_t)g * N + (k - gw);
            cg = d_x + n;
            src = static_cast<const Tin*>(a.B) + (int64_t)b * a.ld_B + n;
        } else {
            const int64_t n = (int64_t)g * N + (k - gw - N);
            cg = d_x + d_b + n;
            src = static_cast<const Tin*>(a.C) + (int64_t)b * a.ld_C + n;
        }
        float* st = a.conv_state + (int64_t)slot * 3 * conv_dim + cg;
        const float t1 = init ? st[conv_dim] : 0.f, t2 = init ? st[2 * conv_dim] : 0.f;
        const float xin = Act<Tin>::load(src);
        st[0] = t1;
        st[conv_dim] = t2;
        st[2 * conv_dim] = xin;
    }
    float* yo = static_cast<float*>(a.y) + (int64_t)b * a.ld_y + (int64_t)g * gw;
    const Tin* zr = static_cast<const Tin*>(a.z) + (int64_t)b * a.ld_z + (int64_t)g * gw;
    const float* nw = a.norm_w + (int64_t)g * gw;
    constexpr int MAXC = MAXGW / NT;   // channels per thread
    float yv[MAXC], gv[MAXC];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + NT * i;
        yv[i] = c < gw ? yo[c] : 0.f;
        gv[i] = c < gw ? silu(Act<Tin>::load(zr + c)) : 0.f;
        const float v = a.norm_before_gate ? yv[i] : yv[i] * gv[i];
        ss = fmaf(v, v, ss);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) tot += red[k];
    const float rstd = __builtin_amdgcn_rsqf(tot / (float)gw + a.eps);
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = tid + NT * i;
        if (c < gw)
            yo[c] = a.norm_before_gate ? yv[i] * rstd * nw[c] * gv[i] : yv[i] * gv[i] * rstd * nw[c];
    }
}

size_t lds_bytes(int gw, int hpg, int N) { return sizeof(float) * (5 * (size_t)gw + 2 * N + hpg + NT / 64); }

// Workgroups per (sequence, group) for a small batch with an fp32 output: the
// largest power of two dividing the heads per group that keeps the grid within
// one workgroup per CU; 1 = the fused kernel.
int decode_split(const DecodeArgs& a) {
    if (a.y_dtype != kF32) return 1;
    const int hpg = a.nheads / a.ngroups;
    const int64_t wgs = (int64_t)a.batch * a.ngroups;
    int s = 1;
    while (hpg % (2 * s) == 0 && wgs * 2 * s <= 256) s *= 2;
    return s;
}

template <int P, int N, typename Tin>
hipError_t launch_pn(const DecodeArgs& a0, hipStream_t stream) {
    DecodeArgs a = a0;
    a.split = decode_split(a0);
    const int hpg = a.nheads / a.ngroups;
    if (a.split > 1) {
        const int nh = hpg / a.split;
        hipLaunchKernelGGL((decode_step_kernel<P, N, Tin, float, true>), dim3((unsigned)(a.batch * a.ngroups * a.split)),
                           dim3(NT), lds_bytes(nh * P, nh, N), stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((decode_finish_kernel<P, N, Tin>), dim3((unsigned)(a.batch * a.ngroups)), dim3(NT), 0,
                           stream, a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(a.batch * a.ngroups));
    const size_t lds = lds_bytes(hpg * P, hpg, N);
    if (a.y_dtype == kBF16)
        hipLaunchKernelGGL((decode_step_kernel<P, N, Tin, uint16_t, false>), grid, dim3(NT), lds, stream, a);
    else
        hipLaunchKernelGGL((decode_step_kernel<P, N, Tin, float, false>), grid, dim3(NT), lds, stream, a);
    return hipGetLastError();
}

template <typename Tin>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    if (a.headdim == 16 && a.dstate == 16) return launch_pn<16, 16, Tin>(a, stream);
    if (a.headdim == 32 && a.dstate == 64) return launch_pn<32, 64, Tin>(a, stream);
    if (a.headdim == 64 && a.dstate == 64) return launch_pn<64, 64, Tin>(a, stream);
    return launch_pn<64, 128, Tin>(a, stream);
}

}  // namespace

bool decode_supported(int nheads, int ngroups, int headdim, int dstate) {
    const bool shape = (headdim == 16 && dstate == 16) || (headdim == 32 && dstate == 64) ||
                       (headdim == 64 && dstate == 64) || (headdim == 64 && dstate == 128);
    if (!shape || ngroups <= 0 || nheads <= 0 || nheads % ngroups) return false;
    return (nheads / ngroups) * headdim <= MAXGW;
}

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream) {
    if (a.batch <= 0) return hipSuccess;
    return a.act_dtype == kBF16 ? launch_t<uint16_t>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace m2
