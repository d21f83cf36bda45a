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
// which is the same function of the inputs).  On the fp64 path, few long
// sequences are split into segments walked by separate workgroups and joined
// afterwards (see the segment kernels below).

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
    const int lin = (int)(blockIdx.x % (unsigned)total);
    const int seg_k = (int)(blockIdx.x / (unsigned)total);   // segment (0 unless split)
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
    // rows [c_begin, c_end) of the sequence: all of them, or segment seg_k's
    // (a.seg steps of `chunk` rows; a later segment starts from a zero state)
    const int64_t seg_rows = a.seg > 0 ? (int64_t)a.seg * chunk : 0;
    const int64_t c_begin = seg_rows * seg_k;
    if (seg_k > 0 && c_begin >= L) return;
    const int64_t c_end = (seg_rows > 0 && c_begin + seg_rows < L) ? c_begin + seg_rows : L;

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
            hacc[nt][r] = (init && L > 0 && seg_k == 0) ? (V)st[p * N + 16 * nt + Pol::orow(q, r)] : (V)0;
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

    double lrun = 0.0;   // log decay over the rows done so far
    for (int64_t c0 = c_begin; c0 < c_end; c0 += chunk) {
        const int S = (int)((c_end - c0) < chunk ? (c_end - c0) : chunk);
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
        lrun += gS;
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

    if (seg_k == 0 && c_end >= L) {
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[p * N + 16 * nt + Pol::orow(q, r)] = (float)hacc[nt][r];
    } else {
        // a split sequence: the segment's local end state and total log decay,
        // for the carry kernel
        const int64_t k = ((int64_t)seg_k * a.batch + seq) * a.nheads + head;
        double* E = a.seg_state + k * (int64_t)(P * N);
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) E[p * N + 16 * nt + Pol::orow(q, r)] = (double)hacc[nt][r];
        if (tid == 0) a.lam[k] = lrun;
    }
}

// ------------------------------------------------------------------ segments
//
// Few long sequences leave most CUs idle when each (sequence, head) walks all
// its rows alone, so the fp64 path can split them into segments of a.seg steps
// that run in parallel, each later segment from a zero state.  With E_k the
// local end state of segment k (E_0 from the true initial state) and lam_k its
// total log decay, the true end states are T_0 = E_0, T_k = e(lam_k) T_{k-1}
// + E_k (the recurrence is linear in its state).  A row t of segment k >= 1
// then lacks only the readout of the carried-in state: e(Gamma_t) C_t . T_{k-1},
// Gamma_t the log decay from the segment's start to t inclusive.

// One workgroup per (sequence, head): walks the segment boundaries, leaves
// T_{k-1} in segment k-1's slot (segment k's entry state) and writes the final
// state to the cache slot.
template <int P, int N>
__global__ __launch_bounds__(256) void seg_carry_f64_kernel(ScanArgs a) {
    constexpr int PT = P * N / 256;   // elements per thread
    const int seq = (int)blockIdx.x / a.nheads, head = (int)blockIdx.x % a.nheads;
    const int tid = threadIdx.x;
    const int64_t L = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    const int chunk = a.chunk < PolicyF64::QMAX ? a.chunk : PolicyF64::QMAX;
    const int64_t seg_rows = (int64_t)a.seg * chunk;
    int nseg = (int)((L + seg_rows - 1) / seg_rows);
    if (nseg <= 1) return;   // one segment: it wrote the final state itself
    if (nseg > a.seg_levels) nseg = a.seg_levels;   // (a sequence longer than max_seqlen)
    auto slot_of = [&](int k) { return ((int64_t)k * a.batch + seq) * a.nheads + head; };
    double T[PT];
    const double* E0 = a.seg_state + slot_of(0) * (int64_t)(P * N);
#pragma unroll
    for (int j = 0; j < PT; ++j) T[j] = E0[tid + 256 * j];
    for (int k = 1; k < nseg; ++k) {
        double* Ep = a.seg_state + slot_of(k - 1) * (int64_t)(P * N);
        const double* Ek = a.seg_state + slot_of(k) * (int64_t)(P * N);
        const double dk = PolicyF64::expc(fmin(a.lam[slot_of(k)], 0.0));
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            Ep[tid + 256 * j] = T[j];
            T[j] = fma(dk, T[j], Ek[tid + 256 * j]);
        }
    }
    const int slot = a.state_idx ? a.state_idx[seq] : seq;
    float* st = a.ssm_state + ((int64_t)slot * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
    for (int j = 0; j < PT; ++j) st[tid + 256 * j] = (float)T[j];
}

// One workgroup per (sequence, head, step of a later segment): adds
// e(Gamma_t) C_t . T_{k-1} to the step's y rows, the matrix product laid out as
// in the scan kernel's inter-chunk term (wave w owns headdim columns 16w ..).
template <int P, int N, typename Tin>
__global__ __launch_bounds__(64 * (P / 16)) void seg_fix_f64_kernel(ScanArgs a) {
    using Pol = PolicyF64;
    using V = double;
    using Acc = typename Pol::Acc;
    constexpr int QMAX = Pol::QMAX;
    constexpr int NTQ = QMAX / 16;
    constexpr int W = P / 16;
    constexpr int NTN = N / 16;
    constexpr int NKBN = (N + 31) / 32;
    constexpr int NTH = 64 * W;
    constexpr int LDS_ROW = N + 2;
    constexpr int T_ROW = N + 1;       // padded row of the staged T (lanes read 16 rows at once)
    __shared__ __align__(16) V Cs[QMAX * LDS_ROW];
    __shared__ __align__(16) V Ts[P * T_ROW];
    __shared__ __align__(16) V din[QMAX];
    __shared__ double part[W];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, q = lane >> 4, l16 = lane & 15;
    const int seq = (int)blockIdx.x / a.nheads, head = (int)blockIdx.x % a.nheads;
    const int hpg = a.nheads / a.ngroups;
    const int grp = head / hpg;
    const int chunk = a.chunk < QMAX ? a.chunk : QMAX;
    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    const int64_t c0 = (int64_t)(blockIdx.y + a.seg) * chunk;   // steps of segment 0 need no fix
    if (c0 >= L) return;
    const int64_t seg_rows = (int64_t)a.seg * chunk;
    const int k = (int)(c0 / seg_rows);
    const int64_t g0 = (int64_t)k * seg_rows;                   // the segment's first row
    const int S = (int)((L - c0) < chunk ? (L - c0) : chunk);
    const int64_t r0 = s0 + c0;
    const double Ah = (double)a.A[head];
    const Tin* Cg = static_cast<const Tin*>(a.C);
    const int p = wave * 16 + l16;

    // T_{k-1} and the step's C rows (rows >= S zero), two consecutive elements
    // per piece; every load is issued before the first LDS store
    const double* Tk = a.seg_state + (((int64_t)(k - 1) * a.batch + seq) * a.nheads + head) * (int64_t)(P * N);
    {
        constexpr int TE = P * N / 2 / NTH;      // pieces of T per thread
        constexpr int CE = QMAX * N / 2 / NTH;   // pieces of C per thread
        static_assert(TE * 2 * NTH == P * N && CE * 2 * NTH == QMAX * N, "staging pieces");
        V tv[TE][2], cv[CE][2];
#pragma unroll
        for (int j = 0; j < TE; ++j) {
            const int e = 2 * (tid + NTH * j);
            tv[j][0] = Tk[e];
            tv[j][1] = Tk[e + 1];
        }
#pragma unroll
        for (int j = 0; j < CE; ++j) {
            const int e = 2 * (tid + NTH * j);
            const int i = e / N, n = e % N;
            const Tin* src = Cg + (r0 + (i < S ? i : S - 1)) * a.ld_C + grp * a.gs_C + n;
            cv[j][0] = (V)Act<Tin>::load(src);
            cv[j][1] = (V)Act<Tin>::load(src + 1);
        }
#pragma unroll
        for (int j = 0; j < TE; ++j) {
            const int e = 2 * (tid + NTH * j);
            Ts[(e / N) * T_ROW + e % N] = tv[j][0];
            Ts[(e / N) * T_ROW + e % N + 1] = tv[j][1];
        }
#pragma unroll
        for (int j = 0; j < CE; ++j) {
            const int e = 2 * (tid + NTH * j);
            const int i = e / N, n = e % N;
            Cs[i * LDS_ROW + n] = i < S ? cv[j][0] : (V)0;
            Cs[i * LDS_ROW + n + 1] = i < S ? cv[j][1] : (V)0;
        }
    }
    // Gamma: the log decay of rows g0 .. c0-1 (every thread sums a strided
    // share, four independent loads at a time), then the step's inclusive
    // prefix sum on wave 0
    {
        double v0 = 0.0, v1 = 0.0, v2 = 0.0, v3 = 0.0;
        int64_t i = g0 + tid;
        for (; i + 3 * NTH < c0; i += 4 * NTH) {
            v0 += (double)a.dt[(s0 + i) * a.ld_dt + head];
            v1 += (double)a.dt[(s0 + i + NTH) * a.ld_dt + head];
            v2 += (double)a.dt[(s0 + i + 2 * NTH) * a.ld_dt + head];
            v3 += (double)a.dt[(s0 + i + 3 * NTH) * a.ld_dt + head];
        }
        for (; i < c0; i += NTH) v0 += (double)a.dt[(s0 + i) * a.ld_dt + head];
        double v = (v0 + v1) + (v2 + v3);
#pragma unroll
        for (int d = 32; d > 0; d >>= 1) v += __shfl_xor(v, d, 64);
        if (lane == 0) part[wave] = v;
    }
    __syncthreads();
    Acc hacc[NTN];
#pragma unroll
    for (int nt = 0; nt < NTN; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) hacc[nt][r] = Ts[p * T_ROW + 16 * nt + Pol::orow(q, r)];
    if (wave == 0) {
        double sdt = 0.0;
#pragma unroll
        for (int w = 0; w < W; ++w) sdt += part[w];
        const double base = sdt * Ah;
        const double ai = lane < S ? (double)a.dt[(r0 + lane) * a.ld_dt + head] * Ah : 0.0;
        double w = ai;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double t = __shfl_up(w, d, 64);
            if (lane >= d) w += t;
        }
        din[lane] = lane < S ? Pol::expc(fmin(base + w, 0.0)) : 0.0;
    }
    __syncthreads();

    // y^T[p, t] += sum_n T[p, n] C[t, n] e(Gamma_t)
    Acc yacc[NTQ];
#pragma unroll
    for (int tt = 0; tt < NTQ; ++tt) yacc[tt] = Acc{0, 0, 0, 0};
    const int nT = (S + 15) >> 4;
#pragma unroll
    for (int kb = 0; kb < NKBN; ++kb) {
        V va[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int nt = 2 * kb + (j >> 2);
            va[j] = (nt < NTN) ? (V)hacc[nt < NTN ? nt : 0][j & 3] : (V)0;
        }
        const typename Pol::Op ha = Pol::make(va);
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
#pragma unroll
    for (int tt = 0; tt < NTQ; ++tt) {
        const int t = 16 * tt + l16;
        if (tt < nT && t < S) {
            float* dst = a.y + (r0 + t) * a.ld_y + (int64_t)head * P + 16 * wave;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[Pol::orow(q, r)] += (float)yacc[tt][r];
        }
    }
}

template <int P, int N>
hipError_t launch_pn(const ScanArgs& a, hipStream_t stream) {
    const dim3 grid(a.nheads * a.batch * (a.seg > 0 ? a.seg_levels : 1));
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
        if (a.seg > 0) {
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((seg_carry_f64_kernel<P, N>), dim3(a.nheads * a.batch), dim3(256), 0, stream, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            const dim3 fgrid(a.nheads * a.batch, (unsigned)((a.seg_levels - 1) * a.seg));
            if (a.act_dtype == kF64)
                hipLaunchKernelGGL((seg_fix_f64_kernel<P, N, double>), fgrid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((seg_fix_f64_kernel<P, N, float>), fgrid, block, 0, stream, a);
        }
    }
    return hipGetLastError();
}

}  // namespace

bool scan_supported(int headdim, int dstate) {
    return (headdim == 16 && dstate == 16) || (headdim == 32 && dstate == 64) ||
           (headdim == 64 && dstate == 64) || (headdim == 64 && dstate == 128);
}

// Segments of the fp64 path: when fewer than SEG1_TARGET (sequence, head)
// items would run, sequences are split into up to SEG1_TARGET / items
// segments of at least SEG1_MIN steps each.
constexpr int SEG1_TARGET = 256;
constexpr int SEG1_MIN = 4;

static size_t r256(size_t v) { return (v + 255) / 256 * 256; }

size_t one_pass_seg_bytes(int batch, int nheads, int headdim, int dstate, int policy) {
    const int64_t level = (int64_t)batch * nheads;
    if (policy != kPolicyF64 || level <= 0 || level >= SEG1_TARGET) return 0;
    const int64_t nseg = (SEG1_TARGET + level - 1) / level;
    return r256((size_t)(nseg * level) * (size_t)headdim * (size_t)dstate * sizeof(double)) +
           r256((size_t)(nseg * level) * sizeof(double));
}

void one_pass_plan(ScanArgs& a, int max_seqlen, void* ws) {
    a.seg = 0;
    a.seg_levels = 1;
    a.seg_state = nullptr;
    const int64_t level = (int64_t)a.batch * a.nheads;
    if (!ws || a.policy != kPolicyF64 || level >= SEG1_TARGET) return;
    const int chunk = a.chunk < PolicyF64::QMAX ? a.chunk : PolicyF64::QMAX;
    const int nsteps = (int)(((int64_t)max_seqlen + chunk - 1) / chunk);
    int nseg = (int)((SEG1_TARGET + level - 1) / level);
    if (nseg > nsteps / SEG1_MIN) nseg = nsteps / SEG1_MIN;
    if (nseg < 2) return;
    a.seg = (nsteps + nseg - 1) / nseg;
    a.seg_levels = (nsteps + a.seg - 1) / a.seg;
    const size_t cap = (size_t)((SEG1_TARGET + level - 1) / level) * (size_t)level;
    a.seg_state = static_cast<double*>(ws);
    a.lam = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                      r256(cap * (size_t)a.headdim * (size_t)a.dstate * sizeof(double)));
}

hipError_t launch_ssd_scan(const ScanArgs& a, hipStream_t stream) {
    if (a.headdim == 16 && a.dstate == 16) return launch_pn<16, 16>(a, stream);
    if (a.headdim == 32 && a.dstate == 64) return launch_pn<32, 64>(a, stream);
    if (a.headdim == 64 && a.dstate == 64) return launch_pn<64, 64>(a, stream);
    if (a.headdim == 64 && a.dstate == 128) return launch_pn<64, 128>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace m2
