// Chunked selective scan (Mamba-2 SSD) for gfx950.
//
// Method (page "perf(nemotron_h): prefill single-GPU prompts in multi-token
// chunks", section Implementation): inside a chunk of S rows there is no
// sequential step.  With a_t = dt_t * A and gamma the inclusive cumulative sum
// of a over the chunk, the chunk total gamma_S is read from the last element of
// that sum and every exponent is clamped at 0.  The chunk's outputs and the
// state it hands on are (e(v) = exp(min(v, 0))):
//   y_t   = e(gamma_t) C_t . h_in + sum_{i<=t} e(gamma_t - gamma_i) (C_t . B_i) dt_i x_i + D x_t
//   h_out = e(gamma_S) h_in + sum_i e(gamma_S - gamma_i) dt_i x_i (outer) B_i
// which is the token recurrence of page "Nemotron-H", section 4.1, unrolled
// over the chunk.
//
// One workgroup owns one (sequence, head) and walks the sequence's chunks in
// order, keeping the head's state h [P x N] in fp32 accumulator registers the
// whole time (the state never round-trips through HBM between chunks).  Wave w
// of the P/16 waves owns headdim columns p in [16w, 16w + 16).  Per chunk:
//   1. B and C rows of the head's group are staged in LDS as fp32; dt in LDS.
//   2. wave 0 forms a_i = dt_i * A in fp64 (exact product of two fp32 values)
//      and its inclusive prefix sum gamma with a wavefront shuffle scan; all
//      exponent differences are taken in fp64, clamped at 0, then exp'd in fp32.
//   3. G^T = B C^T over the causal 16x16 tiles (split over waves), turned in
//      registers into M^T[i, t] = G^T[i, t] dt_i e(gamma_t - gamma_i) for i <= t,
//      with D added on the diagonal (so the skip term rides in the same product).
//   4. y^T += h_in C^T scaled by e(gamma_t)   (h_in taken straight from the
//      state accumulators: their register layout is the operand layout);
//      h <- e(gamma_S) h + B^T (x dt e(gamma_S - gamma_i)).
//   5. M^T tiles go through LDS (reusing the B buffer) and y^T += X^T M^T.
//   6. y rows of the chunk are stored; after the last chunk the state is stored.
// Matrix products use PolicyBf16x3 (bf16 inputs; fp32 values, 128-row chunks)
// or PolicyF64 (fp32 inputs; fp64 values, chunks evaluated 64 rows at a time,
// which is the same function of the inputs).

#include "device_common.h"
#include "kernels.h"

namespace m2 {
namespace {

__device__ __forceinline__ void tile_of(int k, int& it, int& tt) {
    // causal tile k = tt*(tt+1)/2 + it, 0 <= it <= tt
    int t = 0;
    while ((t + 1) * (t + 2) / 2 <= k) ++t;
    tt = t;
    it = k - t * (t + 1) / 2;
}

template <int P, int N, class Pol, typename Tin>
__global__ __launch_bounds__(64 * (P / 16)) void ssd_scan_kernel(ScanArgs a) {
    using V = typename Pol::Val;
    using Acc = typename Pol::Acc;
    using Op = typename Pol::Op;
    constexpr int QMAX = Pol::QMAX;      // rows staged per step
    constexpr int NTQ = QMAX / 16;       // row tiles per step
    constexpr int NKBQ = QMAX / 32;      // K blocks over rows
    constexpr int W = P / 16;
    constexpr int NTN = N / 16;          // 16-wide n tiles of the state
    constexpr int NKBN = (N + 31) / 32;  // K blocks over n
    constexpr int LDS_ROW = N + 16 / (int)sizeof(V);   // padded row of the staged B / C
    constexpr int MAXT = NTQ * (NTQ + 1) / 2;           // causal 16x16 tiles of a full step
    constexpr int BS_SIZE = (QMAX * LDS_ROW > MAXT * 64 * 4) ? QMAX * LDS_ROW : MAXT * 64 * 4;

    __shared__ __align__(16) V Bs[BS_SIZE];      // B rows; later the M^T tiles
    __shared__ __align__(16) V Cs[QMAX * LDS_ROW];
    __shared__ __align__(16) double gam[QMAX];
    __shared__ __align__(16) V dts[QMAX];
    __shared__ __align__(16) V wout[QMAX];       // dt_i * e(gamma_S - gamma_i)
    __shared__ __align__(16) V din[QMAX];        // e(gamma_t)

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int q = lane >> 4;
    const int l16 = lane & 15;

    // Work item: heads of one group share B/C, so consecutive items on one XCD
    // (workgroups are dealt round-robin over 8 XCDs) take consecutive heads.
    const int total = a.nheads * a.batch;
    const int lin = blockIdx.x;
    const int item = (total % 8 == 0) ? (lin % 8) * (total / 8) + lin / 8 : lin;
    const int seq = item / a.nheads;
    const int head = item % a.nheads;
    const int hpg = a.nheads / a.ngroups;
    const int grp = head / hpg;

    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    const int slot = a.state_idx ? a.state_idx[seq] : seq;
    const bool init = a.has_init ? (a.has_init[seq] != 0) : true;
    const int chunk = a.chunk < QMAX ? a.chunk : QMAX;

    const Tin* X = static_cast<const Tin*>(a.x);
    const Tin* Bg = static_cast<const Tin*>(a.B);
    const Tin* Cg = static_cast<const Tin*>(a.C);
    const V Ah = a.A[head];
    const V Dh = a.D ? a.D[head] : 0.0f;
    const int p = wave * 16 + l16;     // this lane's headdim column

    float* st = a.ssm_state + ((int64_t)slot * a.nheads + head) * (int64_t)(P * N);

    // State accumulators: hacc[nt][r] = h[p][16 nt + orow(q, r)].
    Acc hacc[NTN];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            hacc[nt][r] = (init && L > 0) ? (V)st[p * N + 16 * nt + Pol::orow(q, r)] : (V)0;
    }
    if (L <= 0) {
        // Empty sequence: a fresh slot is still reset, a carried one is untouched.
        if (!init) {
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[p * N + 16 * nt + Pol::orow(q, r)] = 0.f;
        }
        return;
    }

    for (int64_t c0 = 0; c0 < L; c0 += chunk) {
        const int S = (int)((L - c0) < chunk ? (L - c0) : chunk);
        const int nT = (S + 15) >> 4;            // row tiles in this chunk
        const int nkbi = (nT + 1) >> 1;          // K blocks over rows
        const int rows = nkbi * 32;              // staged rows: whole K blocks
        const int64_t r0 = s0 + c0;              // first packed row of the chunk

        __syncthreads();  // previous chunk finished with the LDS buffers

        // 1. stage B, C and dt; rows >= S are zero
        {
            constexpr int PER_ROW = N / 8;
            for (int e = tid; e < rows * PER_ROW; e += 64 * W) {
                const int i = e / PER_ROW;
                const int n0 = (e % PER_ROW) * 8;
                V vb[8], vc[8];
                if (i < S) {
                    load8(Bg + (r0 + i) * a.ld_B + grp * a.gs_B + n0, vb);
                    load8(Cg + (r0 + i) * a.ld_C + grp * a.gs_C + n0, vc);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) { vb[j] = 0; vc[j] = 0; }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    Bs[i * LDS_ROW + n0 + j] = vb[j];
                    Cs[i * LDS_ROW + n0 + j] = vc[j];
                }
            }
            for (int i = tid; i < QMAX; i += 64 * W)
                dts[i] = (i < S) ? (V)a.dt[(r0 + i) * a.ld_dt + head] : (V)0;
        }

        // X operand values for this lane: xr[kb][j] = x[i][p], i = 32 kb + kslot<Pol>(q, j).
        V xr[NKBQ][8];
#pragma unroll
        for (int kb = 0; kb < NKBQ; ++kb) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = 32 * kb + kslot<Pol>(q, j);
                xr[kb][j] = (i < S) ? (V)Act<Tin>::load(X + (r0 + i) * a.ld_x + head * a.hs_x + p) : (V)0;
            }
        }
        __syncthreads();

        // 2. gamma: inclusive prefix sum of a = dt * A in fp64 on wave 0, each
        //    lane summing RPL consecutive rows before the wavefront scan.
        if (wave == 0) {
            constexpr int RPL = QMAX / 64;
            double av[RPL];
            double v = 0.0;
#pragma unroll
            for (int k = 0; k < RPL; ++k) {
                av[k] = (double)dts[RPL * lane + k] * (double)Ah;
                v += av[k];
            }
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const double t = __shfl_up(v, d, 64);
                if (lane >= d) v += t;
            }
            double run = __shfl_up(v, 1, 64);
            if (lane == 0) run = 0.0;
#pragma unroll
            for (int k = 0; k < RPL; ++k) {
                run += av[k];
                gam[RPL * lane + k] = run;
            }
        }
        __syncthreads();
        const double gS = gam[S - 1];
        for (int i = tid; i < QMAX; i += 64 * W) {
            const double gi = gam[i];
            din[i] = Pol::expc(fmin(gi, 0.0));
            wout[i] = dts[i] * Pol::expc(fmin(gS - gi, 0.0));
        }
        const V chunk_decay = Pol::expc(fmin(gS, 0.0));
        __syncthreads();

        // 3. M^T tiles (causal), computed by wave (k mod W)
        constexpr int MYT = (MAXT + W - 1) / W;
        const int ntiles = nT * (nT + 1) / 2;
        Acc mt[MYT];
#pragma unroll
        for (int s = 0; s < MYT; ++s) {
            const int k = wave + s * W;
            mt[s] = Acc{0, 0, 0, 0};
            if (k < ntiles) {
                int it, tt;
                tile_of(k, it, tt);
                const int ia = 16 * it + l16;    // A row (B row i)
                const int tb = 16 * tt + l16;    // B column (C row t)
#pragma unroll
                for (int kb = 0; kb < NKBN; ++kb) {
                    V va[8], vb[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int n = 32 * kb + kslot<Pol>(q, j);
                        va[j] = (n < N) ? Bs[ia * LDS_ROW + n] : (V)0;
                        vb[j] = (n < N) ? Cs[tb * LDS_ROW + n] : (V)0;
                    }
                    Pol::mma(mt[s], Pol::make(va), Pol::make(vb));
                }
                // mask / decay / dt / skip
                const int t = 16 * tt + l16;
                const double gt = gam[t];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * it + Pol::orow(q, r);
                    V v = 0;
                    if (i <= t) {
                        v = mt[s][r] * dts[i] * Pol::expc(fmin(gt - gam[i], 0.0));
                        if (i == t) v += Dh;
                    }
                    mt[s][r] = v;
                }
            }
        }

        // 4a. y^T[p, t] = sum_n h_in[p, n] C[t, n] e(gamma_t)
        Acc yacc[NTQ];
#pragma unroll
        for (int tt = 0; tt < NTQ; ++tt) yacc[tt] = Acc{0, 0, 0, 0};
#pragma unroll
        for (int kb = 0; kb < NKBN; ++kb) {
            V va[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int nt = 2 * kb + (j >> 2);
                va[j] = (nt < NTN) ? (V)hacc[nt < NTN ? nt : 0][j & 3] : (V)0;
            }
            const Op ha = Pol::make(va);
#pragma unroll
            for (int tt = 0; tt < NTQ; ++tt) {
                if (tt < nT) {
                    const int t = 16 * tt + l16;
                    const V dt_in = din[t];
                    V vb[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int n = 32 * kb + kslot<Pol>(q, j);
                        vb[j] = (n < N) ? Cs[t * LDS_ROW + n] * dt_in : (V)0;
                    }
                    Pol::mma(yacc[tt], ha, Pol::make(vb));
                }
            }
        }

        // 4b. h <- e(gamma_S) h + B^T (x dt e(gamma_S - gamma_i))
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) hacc[nt] *= chunk_decay;
#pragma unroll
        for (int kb = 0; kb < NKBQ; ++kb) {
            if (kb < nkbi) {
                V vb[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) vb[j] = xr[kb][j] * wout[32 * kb + kslot<Pol>(q, j)];
                const Op xb = Pol::make(vb);
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) {
                    const int n = 16 * nt + l16;
                    V va[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) va[j] = Bs[(32 * kb + kslot<Pol>(q, j)) * LDS_ROW + n];
                    Pol::mma(hacc[nt], Pol::make(va), xb);
                }
            }
        }
        __syncthreads();  // every wave is done reading Bs / Cs

        // 5. M^T tiles to LDS in accumulator layout, then y^T += X^T M^T
        V* Ms = Bs;
#pragma unroll
        for (int s = 0; s < MYT; ++s) {
            const int k = wave + s * W;
            if (k < ntiles) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Ms[(k * 64 + lane) * 4 + r] = mt[s][r];
            }
        }
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < NKBQ; ++kb) {
            if (kb < nkbi) {
                const Op xa = Pol::make(xr[kb]);
#pragma unroll
                for (int tt = 0; tt < NTQ; ++tt) {
                    if (tt < nT && 2 * kb <= tt) {
                        V vb[8];
                        const V* lo4 = Ms + ((tt * (tt + 1) / 2 + 2 * kb) * 64 + lane) * 4;
#pragma unroll
                        for (int r = 0; r < 4; ++r) vb[r] = lo4[r];
                        if (2 * kb + 1 <= tt) {
                            const V* hi4 = Ms + ((tt * (tt + 1) / 2 + 2 * kb + 1) * 64 + lane) * 4;
#pragma unroll
                            for (int r = 0; r < 4; ++r) vb[4 + r] = hi4[r];
                        } else {
                            vb[4] = vb[5] = vb[6] = vb[7] = 0;
                        }
                        Pol::mma(yacc[tt], xa, Pol::make(vb));
                    }
                }
            }
        }

        // 6. store y rows of the chunk: lane holds y[t = 16 tt + l16][16 w + orow(q, r)]
#pragma unroll
        for (int tt = 0; tt < NTQ; ++tt) {
            const int t = 16 * tt + l16;
            if (tt < nT && t < S) {
                float* dst = a.y + (r0 + t) * a.ld_y + (int64_t)head * P + 16 * wave;
                if constexpr (Pol::kRowsContiguous) {
                    *reinterpret_cast<float4*>(dst + 4 * q) =
                        float4{(float)yacc[tt][0], (float)yacc[tt][1], (float)yacc[tt][2], (float)yacc[tt][3]};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[Pol::orow(q, r)] = (float)yacc[tt][r];
                }
            }
        }
    }

#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[p * N + 16 * nt + Pol::orow(q, r)] = (float)hacc[nt][r];
}

template <int P, int N>
hipError_t launch_pn(const ScanArgs& a, hipStream_t stream) {
    const dim3 grid(a.nheads * a.batch);
    const dim3 block(64 * (P / 16));
    if (a.policy == kPolicyBf16x3) {
        if (a.act_dtype == kBF16)
            hipLaunchKernelGGL((ssd_scan_kernel<P, N, PolicyBf16x3, uint16_t>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((ssd_scan_kernel<P, N, PolicyBf16x3, float>), grid, block, 0, stream, a);
    } else {
        if (a.act_dtype == kF64)
            hipLaunchKernelGGL((ssd_scan_kernel<P, N, PolicyF64, double>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((ssd_scan_kernel<P, N, PolicyF64, float>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace

bool scan_supported(int headdim, int dstate) {
    return (headdim == 16 && dstate == 16) || (headdim == 32 && dstate == 64) ||
           (headdim == 64 && dstate == 64) || (headdim == 64 && dstate == 128);
}

hipError_t launch_ssd_scan(const ScanArgs& a, hipStream_t stream) {
    if (a.headdim == 16 && a.dstate == 16) return launch_pn<16, 16>(a, stream);
    if (a.headdim == 32 && a.dstate == 64) return launch_pn<32, 64>(a, stream);
    if (a.headdim == 64 && a.dstate == 64) return launch_pn<64, 64>(a, stream);
    if (a.headdim == 64 && a.dstate == 128) return launch_pn<64, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace m2
