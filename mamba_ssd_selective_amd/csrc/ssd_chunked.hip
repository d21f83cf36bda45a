// Chunk-parallel selective scan (Mamba-2 SSD) for bf16 activations on gfx950:
// headdim 64, dstate 64 or 128, chunks of 128 rows.
//
// The chunk formulas are those of page "perf(nemotron_h): prefill single-GPU
// prompts in multi-token chunks", section Implementation: a_t = dt_t * A,
// gamma the inclusive cumulative sum of a over the chunk, gamma_S its last
// element, every exponent clamped at 0 (e(v) = exp(min(v, 0))):
//   y_t   = e(gamma_t) C_t . h_in + sum_{i<=t} e(gamma_t - gamma_i) (C_t . B_i) dt_i x_i + D x_t
//   h_out = e(gamma_S) h_in + sum_i e(gamma_S - gamma_i) dt_i x_i (outer) B_i
// The only sequential dependence between chunks is h_in, so the work splits in
// two kernels:
//
//  state pass  walks the chunks of a (sequence, head) in order and keeps h^T
//              [N x P] in matrix-core accumulators (two heads of one group per
//              workgroup when they can share the staged B tile).  Per chunk it
//              writes h_in to the entry-state buffer (fp32; 16-bit rows with a
//              scale each for the raw-row kernels at dstate 128 when no sequence
//              is split, see store_entry_q16), scales the accumulators by
//              e(gamma_S) and adds B^T (dt e(gamma_S - gamma_i) x) with the
//              accumulators as the running sum.  Only B, x and dt are read.
//  chunk out   one workgroup per (chunk, group), all chunks at once.  It forms
//              G^T = B C^T once for the group's heads, then for each head
//              y^T = e(gamma_t) (h_in C^T) + X^T M^T with
//              M^T[i, t] = G^T[i, t] dt_i e(gamma_t - gamma_i) (i <= t) and D on
//              the diagonal, and stores y.
//
// Three choices depend on the batch's shape.  The state pass deals its
// (sequence, group) pairs longest sequence first (seq_order_kernel ranks them),
// so that long chunk walks never start last.  When the walks would fill fewer
// workgroups than CUs, long sequences are split into segments: a segment after
// the first starts from a zero state, segment_carry_kernel joins the segments
// (T_k = e(lambda_k) T_{k-1} + E_k), and the chunk output adds
// e(log decay since the segment's start) T_{k-1} to the local entry states of
// the segment's later chunks.  And a chunk-output grid smaller than the CU
// count splits each group's heads over several workgroups.
//
// Operands: x, B and C come as fp32 (the prefill's post-conv activations) or
// as bf16 (given to the scan directly, then exact in bf16).  Every fp32 operand,
// input or computed (dt-weighted x, M^T, h_in), is split as v = hi + lo (hi =
// bf16(v), lo = bf16(v - hi)); a product takes hi*hi + hi*lo + lo*hi (lo*lo,
// ~2^-18 relative, is dropped) with fp32 accumulation, and a bf16 operand skips
// its lo products.  Cumulative sums of a are fp64, exponent differences fp64,
// clamped, then exp'd in fp32.
//
// Matrix-core tile layouts.  16x16x32 bf16 (chunk out): an A operand lane l
// holds row l%16 and K slots 8(l/16)..8(l/16)+7; a B operand lane holds column
// l%16 and the same K slots; the 16x16 fp32 result lands with lane l holding
// column l%16 and rows 4(l/16)+r in register r.  32x32x16 bf16 (state pass): an
// operand lane holds row (or column) l%32 and K slots 8(l/32)..+7; result
// register r of lane l is column l%32, row 8(r/4) + 4(l/32) + r%4.

#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "norm_row.h"

namespace m2 {
namespace {

constexpr int Q = 128;     // chunk rows
constexpr int P = 64;      // headdim
constexpr int MAXHPG = 256;  // heads per group the chunk-parallel path takes
constexpr int RS = Q + 8;  // LDS row stride (bf16 elements) of token-indexed rows: 272 bytes

typedef uint16_t u16;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint4 lds128(const u16* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ f32x4_t mfma(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Half e (0 = low) of the bf16 pair packed in w.
__device__ __forceinline__ uint32_t half_of(uint32_t w, int e) { return e ? (w >> 16) : (w & 0xffffu); }
__device__ __forceinline__ uint32_t word_of(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}


// A double moved between lanes by one DPP control (applied to both halves);
// lanes with no source lane (or outside the row mask) get 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Inclusive prefix sum of a = dt * A over the 128 rows of a chunk on one wave:
// lane l holds rows 2l and 2l+1 (dt already 0 beyond the chunk's rows).  The
// lane moves are DPP: row shifts give the scan within each row of 16 lanes,
// the two row broadcasts carry it across rows, a wave shift makes it exclusive.
__device__ __forceinline__ void gamma_scan(float d0, float d1, float Ah, double& g0, double& g1) {
    const double a0 = (double)d0 * (double)Ah;
    const double a1 = (double)d1 * (double)Ah;
    double v = a0 + a1;
    v += dpp_f64<0x111, 0xf>(v);   // row_shr:1
    v += dpp_f64<0x112, 0xf>(v);   // row_shr:2
    v += dpp_f64<0x114, 0xf>(v);   // row_shr:4
    v += dpp_f64<0x118, 0xf>(v);   // row_shr:8
    v += dpp_f64<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f64<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    const double run = dpp_f64<0x138, 0xf>(v);   // wave_shr:1
    g0 = run + a0;
    g1 = g0 + a1;
}

// The value of v in lane l (l uniform), as a uniform double.
__device__ __forceinline__ double readlane_f64(double v, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float expc(double v) { return __expf(static_cast<float>(fmin(v, 0.0))); }

// State-pass workgroup -> (sequence, head).  A (sequence, group) pair takes
// wpp = hpg / ipw consecutive workgroups on one XCD (workgroups are dealt
// round-robin over the 8 XCDs, lin % 8), so the group's B rows are shared
// through that XCD's L2.  Pairs are dealt in the order of `order` -- the
// sequences by length, longest first -- round-robin over the XCDs: a
// workgroup walks its sequence's chunks one after another, so dispatching the
// longest walks first keeps the short ones for the end, where they fill the
// CUs the long ones leave idle, instead of leaving a long walk as the tail.
__device__ __forceinline__ void state_item(int lin, const ScanArgs& a, int ipw, int sub, int& seq,
                                           int& head) {
    const int hpg = a.nheads / a.ngroups;
    const int wpp = hpg / ipw;
    int r, w;
    if ((a.batch * a.ngroups) % 8 == 0) {
        const int pos = lin >> 3;
        r = 8 * (pos / wpp) + (lin & 7);
        w = pos % wpp;
    } else {
        r = lin / wpp;
        w = lin % wpp;
    }
    seq = a.order ? a.order[r / a.ngroups] : r / a.ngroups;
    head = (r % a.ngroups) * hpg + ipw * w + sub;
}

// order[k] = the sequence of rank k by length, longest first (ties by index),
// so the result is a permutation of 0 .. batch-1 whatever cu_seqlens holds.
// Thread b ranks sequence b against every length, staged through LDS.
constexpr int ORD_NT = 256;
constexpr int ORD_TILE = 1024;
__global__ __launch_bounds__(ORD_NT) void seq_order_kernel(const int32_t* cu, int batch, int32_t* order) {
    __shared__ int32_t len[ORD_TILE];
    const int b = blockIdx.x * ORD_NT + threadIdx.x;
    const int Lb = b < batch ? cu[b + 1] - cu[b] : 0;
    int rank = 0;
    for (int j0 = 0; j0 < batch; j0 += ORD_TILE) {
        const int n = min(ORD_TILE, batch - j0);
        __syncthreads();
        for (int j = threadIdx.x; j < n; j += ORD_NT) len[j] = cu[j0 + j + 1] - cu[j0 + j];
        __syncthreads();
        for (int j = 0; j < n; ++j) {
            const int Lj = len[j];
            rank += (Lj > Lb || (Lj == Lb && j0 + j < b)) ? 1 : 0;
        }
    }
    if (b < batch) order[rank] = b;
}

// Inputs come as bf16 (8 channels per 16-byte load, exact in bf16) or fp32 (4
// channels per load, entering the products as a (hi, lo) pair).
template <typename Tin>
struct In {
    static constexpr bool kSplit = sizeof(Tin) == 4;
    static constexpr int CPL = 16 / (int)sizeof(Tin);
    __device__ __forceinline__ static float val(const uint4& v, int j) {
        if constexpr (kSplit) return __builtin_bit_cast(float, word_of(v, j));
        else return bf16_bits_to_f32((u16)half_of(word_of(v, j >> 1), j & 1));
    }
};

// Raw input: the pre-conv bf16 xBC rows.  A kernel reading them convolves on
// the fly (width 4, bias, SiLU in fp32, the same operations in the same order as
// the conv kernel, so the post-conv values are those the conv kernel writes)
// and takes every post-conv value as an fp32 (hi, lo) operand.
struct RawBf16 {};
template <>
struct In<RawBf16> {
    static constexpr bool kSplit = true;
    static constexpr int CPL = 8;
};
template <typename Tin>
constexpr bool is_raw() { return std::is_same<Tin, RawBf16>::value; }

// A raw piece: RR consecutive rows of 8 channels, read as the RR + 3 raw rows
// that start 3 rows earlier (the conv's halo).
constexpr int RR = 4;
constexpr int RW = RR + 3;

__device__ __forceinline__ float bf16_lane(const uint4& v, int k) {
    const uint32_t w = word_of(v, k >> 1);
    return __builtin_bit_cast(float, (k & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Conv-weight tables in LDS hold channel 8 cg + k of each 64-channel block at
// slot 8 k + cg: the 8 channel groups of a wave then read 8 consecutive
// entries for one k (in channel order the same reads were 128 bytes apart and
// fell into 2 of the 64 banks).  Bias tables stay in channel order, read as
// two 16-byte runs per channel group.
__device__ __forceinline__ int wsw(int e) { return (e & ~63) | ((e & 7) << 3) | ((e >> 3) & 7); }

// The conv biases of channel group base .. base + 7 from LDS (the weights are
// read one channel at a time where they are used: held for all 8 channels at
// once they made the chunk output spill).
struct ConvW {
    const float4* wt;
    int base;
    float b[8];
    __device__ __forceinline__ float4 w(int k) const { return wt[wsw(base + k)]; }
};
__device__ __forceinline__ ConvW read_convw(const float4* wt, const float* bt, int base) {
    ConvW c;
    c.wt = wt;
    c.base = base;
    const float4 b0 = *reinterpret_cast<const float4*>(bt + base);
    const float4 b1 = *reinterpret_cast<const float4*>(bt + base + 4);
    c.b[0] = b0.x; c.b[1] = b0.y; c.b[2] = b0.z; c.b[3] = b0.w;
    c.b[4] = b1.x; c.b[5] = b1.y; c.b[6] = b1.z; c.b[7] = b1.w;
    return c;
}

// Raw rows row0 - 3 .. row0 + RR - 1 of a chunk, rows clamped into the
// sequence [lo, hi] (chunk-relative: lo = -(chunk's first row in the
// sequence), hi = lo + L - 1); the conv of a piece that starts the sequence
// takes its first 3 rows from the conv state instead (conv_piece_start).  col
// points at the piece's first channel in the chunk's first row; row offsets
// are 32-bit (a chunk's rows lie within 2^31 elements of its first row).
//
// Lanes 8m .. 8m + 7 hold consecutive row groups of one channel group, so the
// 3 halo rows of a piece are rows 1..3 of the previous lane's piece (raw_halo,
// a row shift between lanes); only lanes 8m (own_halo) read theirs.
__device__ __forceinline__ void load_raw_piece(const uint16_t* col, int ld, int row0, int lo, int hi,
                                               bool own_halo, uint4 (&r)[RW]) {
    // The row offsets are recomputed at every call: kept across a loop instead
    // (they do not change from head to head) they made the chunk output spill.
    asm volatile("" : "+v"(ld));
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        int rr = row0 - 3 + j;
        rr = rr < lo ? lo : rr > hi ? hi : rr;
        if (j >= 3 || own_halo) r[j] = *reinterpret_cast<const uint4*>(col + rr * ld);
    }
}

// Rows 0..2 of every piece whose lane did not read them, from lane - 1 (DPP
// row_shr:1; the lanes 8m keep what they read).
__device__ __forceinline__ int dpp_prev(int v) { return __builtin_amdgcn_update_dpp(v, v, 0x111, 0xf, 0xf, false); }
__device__ __forceinline__ void raw_halo(uint4 (&r)[RW], int lane) {
    const bool own = (lane & 7) == 0;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const uint4 v = r[4 + j];
        const uint4 u = uint4{(uint32_t)dpp_prev((int)v.x), (uint32_t)dpp_prev((int)v.y),
                              (uint32_t)dpp_prev((int)v.z), (uint32_t)dpp_prev((int)v.w)};
        if (!own) r[j] = u;
    }
}

// The 3 rows before a sequence's first row for the 8 channels at conv-state
// column ch: the slot's carried state (oldest first) or zeros.
__device__ __forceinline__ void load_halo(const float* conv_state, int conv_dim, int slot, bool init, int ch,
                                          float (&hv)[3][8]) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        float4 v0 = float4{0.f, 0.f, 0.f, 0.f}, v1 = v0;
        if (init) {
            const float* p = conv_state + ((int64_t)slot * 3 + j) * conv_dim + ch;
            v0 = *reinterpret_cast<const float4*>(p);
            v1 = *reinterpret_cast<const float4*>(p + 4);
        }
        hv[j][0] = v0.x; hv[j][1] = v0.y; hv[j][2] = v0.z; hv[j][3] = v0.w;
        hv[j][4] = v1.x; hv[j][5] = v1.y; hv[j][6] = v1.z; hv[j][7] = v1.w;
    }
}

// SiLU(b + w0 v[t] + w1 v[t+1] + w2 v[t+2] + w3 v[t+3]) for the RR rows t of
// channel k of a piece; with `start` the first 3 window rows are hv[.][k].
__device__ __forceinline__ void conv_piece(const uint4 (&r)[RW], int k, bool start, const float (&hv)[3][8],
                                           float4 w, float b, float (&u)[RR]) {
    float v[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) v[j] = bf16_lane(r[j], k);
    if (start) {
        v[0] = hv[0][k];
        v[1] = hv[1][k];
        v[2] = hv[2][k];
    }
#pragma unroll
    for (int t = 0; t < RR; ++t) {
        float acc = b;
        acc = fmaf(w.x, v[t], acc);
        acc = fmaf(w.y, v[t + 1], acc);
        acc = fmaf(w.z, v[t + 2], acc);
        acc = fmaf(w.w, v[t + 3], acc);
        u[t] = silu(acc);
    }
}

// conv_piece for a piece that starts its sequence, reading channel k's 3 carried
// rows from the conv state (zeros when init is 0) as it goes.
__device__ __forceinline__ void conv_piece_start(const uint4 (&r)[RW], int k, const float* conv_state, int conv_dim,
                                                 int slot, bool init, int ch, float4 w, float b, float (&u)[RR]) {
    float v[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) v[j] = bf16_lane(r[j], k);
#pragma unroll
    for (int j = 0; j < 3; ++j) v[j] = init ? conv_state[((int64_t)slot * 3 + j) * conv_dim + ch + k] : 0.f;
#pragma unroll
    for (int t = 0; t < RR; ++t) {
        float acc = b;
        acc = fmaf(w.x, v[t], acc);
        acc = fmaf(w.y, v[t + 1], acc);
        acc = fmaf(w.z, v[t + 2], acc);
        acc = fmaf(w.w, v[t + 3], acc);
        u[t] = silu(acc);
    }
}

// conv + SiLU of a whole piece, all 8 channels x RR rows at once (the same
// operations in the same order per output as conv_piece, laid out breadth
// first so that a single wave has 32 independent chains to interleave):
// u[k][t] = SiLU(b_k + w_k0 v[t] + w_k1 v[t+1] + w_k2 v[t+2] + w_k3 v[t+3]).
__device__ __forceinline__ void conv_piece8(const uint4 (&r)[RW], bool start, const float (&hv)[3][8],
                                            const float4 (&w)[8], const float (&b)[8], float (&u)[8][RR]) {
    float acc[8][RR];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int t = 0; t < RR; ++t) acc[k][t] = b[k];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int t = 0; t < RR; ++t) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float v = bf16_lane(r[t + j], k);
                if (start && t + j < 3) v = hv[t + j][k];
                const float wj = j == 0 ? w[k].x : j == 1 ? w[k].y : j == 2 ? w[k].z : w[k].w;
                acc[k][t] = fmaf(wj, v, acc[k][t]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int t = 0; t < RR; ++t) u[k][t] = silu(acc[k][t]);
}

// acc += a b over (hi, lo) operands: the lo x lo term (~2^-18 relative) is dropped,
// and a lo part that is known to be zero (SA / SB false) is skipped.
template <bool SA, bool SB>
__device__ __forceinline__ void mma2(f32x4_t& acc, bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl) {
    if constexpr (SA) acc = mfma(al, bh, acc);
    if constexpr (SB) acc = mfma(ah, bl, acc);
    acc = mfma(ah, bh, acc);
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 32x32x16 counterpart of mma2.
template <bool SA, bool SB>
__device__ __forceinline__ void mma32(f32x16_t& acc, bf16x8_t ah, bf16x8_t al, bf16x8_t bh, bf16x8_t bl) {
    if constexpr (SA) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
    if constexpr (SB) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// High and low parts of the pair (a, b) as packed bf16 (a in the low half):
// one two-source conversion per part, so the pair is already packed.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
    const float ha = __builtin_bit_cast(float, h << 16);
    const float hb = __builtin_bit_cast(float, h & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a - ha, b - hb}, bf16x2_t));
    hi = h;
}

// 8 values -> packed bf16 high parts and low parts.
__device__ __forceinline__ void split8(const float (&v)[8], uint4& hi, uint4& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) split2(v[2 * m], v[2 * m + 1], h[m], l[m]);
    hi = uint4{h[0], h[1], h[2], h[3]};
    lo = uint4{l[0], l[1], l[2], l[3]};
}

// Entry-state layout.  Within a (chunk slot, head) block the P x N fp32 state
// is stored in the state pass's accumulator order: float4 f = ((tile * 4 + m)
// * 64 + lane) holds p = 32 (tile & 1) + lane % 32 and n = 32 (tile >> 1) + 8 m
// + 4 (lane / 32) .. + 3.
__device__ __forceinline__ void state_pn(int f, int& p, int& n) {
    const int lane = f & 63, m = (f >> 6) & 3, tile = f >> 8;
    p = 32 * (tile & 1) + (lane & 31);
    n = 32 * (tile >> 1) + 8 * m + 4 * (lane >> 5);
}

// 16-bit entry states (the raw-row kernels at dstate 128 when no sequence is
// split): the state's values enter the chunk output only through its read-out
// C h_in, so each row of 32 values (one p, one n tile) is stored as 16-bit
// fixed point on its own scale s = max |v| of the row: q = round-half-even(v /
// s * 32767) (the hardware's pack to signed normalized 16-bit), read back as q
// * s / 32767.  The absolute error is at most s / 65534 per value.  A block
// then moves 17 KB instead of 32 KB, in 5 store instructions per consumer lane
// and head instead of 8.  Within a (chunk slot, head) block (the fp32 block's
// place, P * N floats):
//   uint4 u = ((tile * 2 + m2) * 64 + lane) holds the 16-bit values of float4s
//     f = (tile * 4 + 2 m2) * 64 + lane and f + 64 (in the fp32 order above),
//     four each;
//   float P * N / 2 + r * NTQ + tile, r = p % 32, holds s / 32767 of row
//     (p = 32 (tile & 1) + r, n tile tile >> 1).
constexpr int NTQ = (P / 32) * (128 / 32);   // 32 x 32 tiles of a dstate-128 state

// Store one head's entry state, held by a consumer of the raw state pass as the
// two 32 x 32 accumulator tiles 2 cw and 2 cw + 1 (lane l: p = 32 pt + l % 32,
// n = 32 cw + 8 m + 4 (l / 32) + e in register 4 m + e).
__device__ __forceinline__ void store_entry_q16(float* he, const f32x16_t (&h)[2], int cw, int lane) {
    uint4* dq = reinterpret_cast<uint4*>(he);
    float dec[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(h[pt][e]));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));   // lanes l and l ^ 32 share the row
        const float enc = mx > 0.f ? __builtin_amdgcn_rcpf(mx) : 0.f;
        dec[pt] = mx * (1.f / 32767.f);
        const int tile = 2 * cw + pt;
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(h[pt][8 * m2 + 2 * j] * enc,
                                                                                   h[pt][8 * m2 + 2 * j + 1] * enc));
            dq[(tile * 2 + m2) * 64 + lane] = uint4{w[0], w[1], w[2], w[3]};
        }
    }
    if (lane < 32)
        *reinterpret_cast<float2*>(he + P * 128 / 2 + lane * NTQ + 2 * cw) = float2{dec[0], dec[1]};
}

// The two float4s of a 16-bit uint4, scaled: lo = values of float4 f, hi of f + 64.
__device__ __forceinline__ void q16_values(uint4 u, float d, float4& lo, float4& hi) {
    auto v = [&](uint32_t w, int half) {
        return (float)(int16_t)(uint16_t)(half ? (w >> 16) : (w & 0xffffu)) * d;
    };
    lo = float4{v(u.x, 0), v(u.x, 1), v(u.y, 0), v(u.y, 1)};
    hi = float4{v(u.z, 0), v(u.z, 1), v(u.w, 0), v(u.w, 1)};
}

// ------------------------------------------------------------------ state pass
//
// 4 waves.  h^T [N x P] lives in matrix-core accumulators (32x32 tiles spread
// over the waves).  Each chunk is staged and
// multiplied in two halves of 64 rows, so the LDS tiles are small enough for
// two workgroups per CU (one stages while the other multiplies).  The loads of
// the next half are in flight while the current half is multiplied; they are
// branch-free (rows clamped into the chunk and zeroed after the load), so the
// compiler's wait counts stay exact.

constexpr int QH = Q / 2;        // rows per staged half
constexpr int RH = QH + 8;       // LDS row stride (bf16) of token-indexed half rows: 144 bytes

template <typename Tin, int TB, int TX>
struct HalfBuf {
    uint4 br[TB];      // B piece: TB tokens x CPL channels
    uint4 xr[TX];      // x piece: TX tokens x CPL columns
};
// Raw input: one piece per thread, of x or of B (see the state pass).
struct RawBuf {
    uint4 r[RW];
};

template <int K, typename Tin>
__device__ __forceinline__ void load_rows_clamped(const Tin* base, int64_t ld, int valid, uint4 (&r)[K]) {
    const int last = valid < 1 ? 0 : valid - 1;
#pragma unroll
    for (int k = 0; k < K; ++k) r[k] = *reinterpret_cast<const uint4*>(base + (k < last ? k : last) * ld);
}

// Stores the packed bf16 words of TB tokens of one channel of a staged piece.
template <int TB>
__device__ __forceinline__ void store_tokens(u16* dst, const uint32_t (&w)[(TB + 1) / 2]) {
    if constexpr (TB == 8) *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
    else if constexpr (TB == 4) *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
    else *reinterpret_cast<uint32_t*>(dst) = w[0];
}

// IPW = 2: one workgroup of 8 waves takes heads 2k and 2k + 1 of one sequence
// (one group): waves 0-3 the first, 4-7 the second.  The two heads read and
// stage the group's B tile once, into one shared LDS tile, which halves the B
// loads, the largest part of the per-CU load instructions (the vector memory
// units of a CU were busy 80-90% of the kernel).  Both items share their
// sequence, so they have the same chunk count and take every barrier together.
//
// Raw input (pre-conv bf16 rows, N = 64 * IPW): each thread convolves one piece
// of RR rows x 8 channels per half.  Threads 0-127 of an item take its head's x
// (8 channel groups x 16 row groups), threads 128-255 its share of B (8 channel
// groups x 16 row groups: all of B for N = 64, half of it per item for N = 128);
// the conv weights of the workgroup's channels are staged in LDS once.
template <int N, int IPW, typename Tin>
__global__ __launch_bounds__(256 * IPW, IPW == 1 ? 2 : 1) void ssd_state_pass_kernel(ScanArgs a) {
    constexpr bool RAW = is_raw<Tin>();
    constexpr bool SP = In<Tin>::kSplit;
    constexpr int CPL = In<Tin>::CPL;
    constexpr int NT = 256;                            // threads per item
    constexpr int NTB = NT * IPW;                      // threads that stage B
    constexpr int TPW = N / 64;                        // 32x32 state tiles per wave
    constexpr int TB = RAW ? 2 : QH * N / (CPL * NTB); // tokens per B piece (one piece per thread)
    constexpr int TX = RAW ? 2 : QH * P / (CPL * NT);  // tokens per x piece
    constexpr int BG = QH / TB, XG = QH / TX;          // token groups
    constexpr int BC = N / CPL;                        // B channel groups
    static_assert(TB >= 2 && TX >= 2, "staging pieces");
    static_assert(!RAW || N == 64 * IPW, "raw pieces: 8 B channel groups per item");
    constexpr int NCW = RAW ? IPW * P + N : 1;         // conv channels of the workgroup (raw input)
    __shared__ float4 sCW[NCW];                        // their conv weights (slots wsw)
    __shared__ __align__(16) float sCB[NCW];           // and biases (channel order)
    // Two items per workgroup (one per CU anyway) keep a tile set per half,
    // so one barrier per half suffices; one item keeps one set (two
    // workgroups then share a CU).
    constexpr int NB = IPW == 2 ? 2 : 1;
    __shared__ __align__(16) u16 sBTh[NB][N * RH];           // B^T [n][token of the half], high parts
    __shared__ __align__(16) u16 sBTl[NB][SP ? N * RH : 8];  // low parts (fp32 inputs)
    __shared__ __align__(16) u16 sXH[NB][IPW][P * RH];       // (w x)^T [p][token] per item, high parts
    __shared__ __align__(16) u16 sXL[NB][IPW][P * RH];       // low parts
    __shared__ __align__(16) float sW[4 * IPW][Q];           // per wave: the chunk's weights w_i

    const int sub = IPW > 1 ? (int)(threadIdx.x >> 8) : 0;   // item within the workgroup
    const int tid = threadIdx.x & (NT - 1);
    const int wave = tid >> 6, lane = tid & 63;
    const int gwave = (int)(threadIdx.x >> 6);                // wave within the workgroup
    // grid: one level of batch * nheads / IPW workgroups per segment index
    const int level = a.nheads * a.batch / IPW;
    const int seg_k = (int)blockIdx.x / level;
    int seq, head;
    state_item((int)blockIdx.x % level, a, IPW, sub, seq, head);
    const int grp = head / (a.nheads / a.ngroups);
    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    // segment seg_k of this sequence has no chunk (uniform over the workgroup: both
    // items share the sequence)
    if (seg_k > 0 && (int64_t)seg_k * a.seg * Q >= L) return;
    const int slot = a.state_idx ? a.state_idx[seq] : seq;
    const bool init = a.has_init ? (a.has_init[seq] != 0) : true;
    const float Ah = a.A[head];
    float* st = a.ssm_state + ((int64_t)slot * a.nheads + head) * (int64_t)(P * N);

    // h^T [N x P] in 32x32 tiles (the 32x32x16 instruction does twice the work of
    // the 16x16x32 one in about the same time): N/32 n tiles x 2 p tiles over the
    // 4 waves, TPW tiles each.  acc[i] is tile wave * TPW + i = (n tile mt, p tile
    // pt); lane l has p = 32 pt + l % 32 and, in registers 4m .. 4m + 3, the four
    // consecutive n = 32 mt + 8m + 4 (l / 32) + 0..3.
    const int l32 = lane & 31, g32 = lane >> 5;
    auto tile_mt = [&](int i) { return (wave * TPW + i) >> 1; };
    auto tile_pt = [&](int i) { return (wave * TPW + i) & 1; };
    auto soff = [&](int i, int m) { return (32 * tile_pt(i) + l32) * N + 32 * tile_mt(i) + 8 * m + 4 * g32; };
    // Entry states are stored in accumulator order (float4 index ((tile * 4 + m) * 64
    // + lane)), so each store instruction writes 1 KB in one piece; the chunk
    // output pass decodes the same order (see state_pn).
    auto eoff = [&](int i, int m) { return 4 * (((wave * TPW + i) * 4 + m) * 64 + lane); };
    f32x16_t acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            float4 v = float4{0.f, 0.f, 0.f, 0.f};
            if (init && L > 0 && seg_k == 0) v = *reinterpret_cast<const float4*>(st + soff(i, m));
            acc[i][4 * m + 0] = v.x; acc[i][4 * m + 1] = v.y; acc[i][4 * m + 2] = v.z; acc[i][4 * m + 3] = v.w;
        }
    if (L <= 0) {
        // Empty sequence: a fresh slot is still reset, a carried one is untouched.
        if (!init) {
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int m = 0; m < 4; ++m) *reinterpret_cast<float4*>(st + soff(i, m)) = float4{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }

    // raw input: this thread's piece (x of the item's head, or a share of B),
    // and the conv weights of the workgroup's channels into LDS
    const bool rx = tid < 128;                                   // wave-uniform
    const int r_rg = (lane & 7) + 8 * (wave & 1);                // row group: rows 4 r_rg .. + 3 of a half
    const int r_cg = (rx ? 0 : (IPW == 2 ? 8 * sub : 0)) + (lane >> 3);  // channel group of x or of B
    const int d_inner = a.nheads * P;
    const int r_ch = rx ? head * P + 8 * r_cg : d_inner + grp * N + 8 * r_cg;   // first xBC channel
    const int r_lch = rx ? sub * P + 8 * r_cg : IPW * P + 8 * r_cg;             // its weights in LDS
    if constexpr (RAW) {
        const int head0 = head - sub;
        for (int e = (int)threadIdx.x; e < NCW; e += NT * IPW) {
            const int ch = e < IPW * P ? (head0 + e / P) * P + e % P : d_inner + grp * N + (e - IPW * P);
            sCW[wsw(e)] = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)ch * 4);
            sCB[e] = a.conv_b ? a.conv_b[ch] : 0.f;
        }
        __syncthreads();
    }

    const int nch = (int)((L + Q - 1) / Q);
    const int64_t cbase = s0 / Q + seq;   // entry-state slot of the sequence's first chunk
    // this workgroup's chunks: all of them, or segment seg_k's (a later segment
    // starts from zero; its first entry slot belongs to the segment before)
    // (the last level runs to the sequence's end, so a sequence longer than the
    // max_seqlen the plan was made for still gets every chunk)
    const int cfirst = seg_k * a.seg;
    const int cend = a.seg > 0 && seg_k < a.seg_levels - 1 ? (cfirst + a.seg < nch ? cfirst + a.seg : nch) : nch;
    const Tin* Xg = static_cast<const Tin*>(a.x);
    const Tin* Bg = static_cast<const Tin*>(a.B);

    // B piece: tokens TB b_tg .., channels CPL b_cg .. (a wave reads 8 whole
    // 128-byte row segments per load for fp32 B).  x piece: for fp32 x a wave
    // takes 8 token groups x 8 channel groups, so each load also reads whole
    // 128-byte segments (and 32 lanes' LDS writes cover the 64 banks once).
    // (B: each wave takes 8 token groups x 8 channel groups when the shape allows)
    constexpr bool B88 = BC % 8 == 0 && BG % 8 == 0 && (BC / 8) * (BG / 8) == NTB / 64;
    const int b_tg = B88 ? (lane & 7) + 8 * (gwave / (BC / 8)) : (int)threadIdx.x % BG;
    const int b_cg = B88 ? (lane >> 3) + 8 * (gwave % (BC / 8)) : (int)threadIdx.x / BG;
    const int x_tg = SP ? (lane & 7) + 8 * (wave & 1) : tid % XG;
    const int x_cg = SP ? (lane >> 3) + 8 * (wave >> 1) : tid / XG;
    static_assert(RAW || !SP || (XG == 16 && P / CPL == 16), "fp32 x piece mapping");

    // Loads of half h (0, 1) of chunk c, clamped to the last chunk so the call is
    // unconditional; rows beyond the chunk re-read its last row (zeroed later).
    using Buf = typename std::conditional<RAW, RawBuf, HalfBuf<Tin, TB, TX>>::type;
    auto load_half = [&](Buf& b, int c, int h) __attribute__((always_inline)) {
        c = c < cend ? c : cend - 1;
        if constexpr (RAW) {
            const int64_t ld = rx ? a.ld_x : a.ld_B;
            const uint16_t* col = rx ? static_cast<const uint16_t*>(a.x) + head * a.hs_x + 8 * r_cg
                                     : static_cast<const uint16_t*>(a.B) + grp * a.gs_B + 8 * r_cg;
            load_raw_piece(col + (s0 + (int64_t)c * Q) * ld, (int)ld, h * QH + 4 * r_rg, -c * Q,
                           (int)(L - 1 - (int64_t)c * Q), (lane & 7) == 0, b.r);
            return;
        } else {
        const int64_t left = L - (int64_t)c * Q - h * QH;     // rows of the sequence from this half on
        const int S = (int)(left < QH ? left : QH);
        // an empty half (the chunk ends in its first half) reads the chunk's first row
        const int64_t r0 = s0 + (int64_t)c * Q + (S > 0 ? h * QH : 0);
        const int rb = TB * b_tg < S ? TB * b_tg : 0;
        load_rows_clamped<TB>(Bg + (r0 + rb) * a.ld_B + grp * a.gs_B + b_cg * CPL, a.ld_B, S - rb, b.br);
        const int rxo = TX * x_tg < S ? TX * x_tg : 0;
        load_rows_clamped<TX>(Xg + (r0 + rxo) * a.ld_x + head * a.hs_x + x_cg * CPL, a.ld_x, S - rxo, b.xr);
        }
    };
    auto load_dt = [&](int c, float& d0, float& d1) __attribute__((always_inline)) {
        c = c < cend ? c : cend - 1;
        const int64_t r0 = s0 + (int64_t)c * Q;
        const int S = (int)((L - (int64_t)c * Q) < Q ? (L - (int64_t)c * Q) : Q);
        d0 = a.dt[(r0 + (2 * lane < S ? 2 * lane : S - 1)) * a.ld_dt + head];
        d1 = a.dt[(r0 + (2 * lane + 1 < S ? 2 * lane + 1 : S - 1)) * a.ld_dt + head];
    };

    // Stage half h of chunk c from b, with the weights of this wave's table.
    // Rows past the sequence's end hold re-read (finite) rows and have weight 0
    // (dt is zeroed there), so their (w x) is 0 and they add nothing; no mask.
    auto stage = [&](Buf& b, int c, int h) __attribute__((always_inline)) {
        u16* const BTh = sBTh[h % NB];
        u16* const BTl = sBTl[h % NB];
        u16* const XH = sXH[h % NB][sub];
        u16* const XL = sXL[h % NB][sub];
        if constexpr (RAW) {
            // conv + SiLU of the piece; x rows are then weighted by w
            const int row0 = QH * h + 4 * r_rg;               // first row of the piece in the chunk
            const bool start = c == 0 && row0 == 0;           // the piece starts the sequence
            raw_halo(b.r, lane);
            float hv[3][8];
            if (start) load_halo(a.conv_state, a.conv_dim, slot, init, r_ch, hv);
            const float4 w4 = *reinterpret_cast<const float4*>(&sW[gwave][row0]);
            const float wx[RR] = {w4.x, w4.y, w4.z, w4.w};
            const ConvW cw = read_convw(sCW, sCB, r_lch);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float u[RR];
                conv_piece(b.r, k, start, hv, cw.w(k), cw.b[k], u);
                uint32_t wh[RR / 2], wl[RR / 2];
                if (rx) {
#pragma unroll
                    for (int m = 0; m < RR / 2; ++m) split2(u[2 * m] * wx[2 * m], u[2 * m + 1] * wx[2 * m + 1], wh[m], wl[m]);
                    store_tokens<RR>(XH + (8 * r_cg + k) * RH + 4 * r_rg, wh);
                    store_tokens<RR>(XL + (8 * r_cg + k) * RH + 4 * r_rg, wl);
                } else {
#pragma unroll
                    for (int m = 0; m < RR / 2; ++m) split2(u[2 * m], u[2 * m + 1], wh[m], wl[m]);
                    store_tokens<RR>(BTh + (8 * r_cg + k) * RH + 4 * r_rg, wh);
                    store_tokens<RR>(BTl + (8 * r_cg + k) * RH + 4 * r_rg, wl);
                }
            }
            return;
        } else {
        // B^T: channel CPL b_cg + j, tokens TB b_tg ..
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            uint32_t wh[TB / 2], wl[TB / 2];
#pragma unroll
            for (int m = 0; m < TB / 2; ++m) {
                if constexpr (SP) {
                    split2(In<Tin>::val(b.br[2 * m], j), In<Tin>::val(b.br[2 * m + 1], j), wh[m], wl[m]);
                } else {
                    wh[m] = half_of(word_of(b.br[2 * m], j >> 1), j & 1) |
                            (half_of(word_of(b.br[2 * m + 1], j >> 1), j & 1) << 16);
                }
            }
            store_tokens<TB>(BTh + (b_cg * CPL + j) * RH + TB * b_tg, wh);
            if constexpr (SP) store_tokens<TB>(BTl + (b_cg * CPL + j) * RH + TB * b_tg, wl);
        }
        // (w x)^T: weights of rows 64 h + TX x_tg + k, held by lane (64 h + TX x_tg + k) / 2
        float wx[TX];
#pragma unroll
        for (int k = 0; k < TX; ++k) wx[k] = sW[gwave][QH * h + TX * x_tg + k];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            uint32_t wh[TX / 2], wl[TX / 2];
#pragma unroll
            for (int m = 0; m < TX / 2; ++m)
                split2(In<Tin>::val(b.xr[2 * m], j) * wx[2 * m], In<Tin>::val(b.xr[2 * m + 1], j) * wx[2 * m + 1],
                       wh[m], wl[m]);
            store_tokens<TX>(XH + (x_cg * CPL + j) * RH + TX * x_tg, wh);
            store_tokens<TX>(XL + (x_cg * CPL + j) * RH + TX * x_tg, wl);
        }
        }
    };

    // h^T += B^T (w x) over the 16-row K blocks of a staged half (32x32x16: an
    // operand lane supplies row (or column) l % 32 and K slots 8 (l / 32) .. + 7)
    auto multiply = [&](int nkb, int h) __attribute__((always_inline)) {
        const u16* const BTh = sBTh[h % NB];
        const u16* const BTl = sBTl[h % NB];
        const u16* const XH = sXH[h % NB][sub];
        const u16* const XL = sXL[h % NB][sub];
#pragma unroll
        for (int k = 0; k < QH / 16; ++k) {
            if (k < nkb) {
#pragma unroll
                for (int i = 0; i < TPW; ++i) {
                    const int xo = (32 * tile_pt(i) + l32) * RH + 16 * k + 8 * g32;
                    const int bo = (32 * tile_mt(i) + l32) * RH + 16 * k + 8 * g32;
                    const bf16x8_t xh = as_bf16x8(lds128(XH + xo));
                    const bf16x8_t xl = as_bf16x8(lds128(XL + xo));
                    const bf16x8_t bh = as_bf16x8(lds128(BTh + bo));
                    const bf16x8_t bl = SP ? as_bf16x8(lds128(BTl + (SP ? bo : 0))) : bh;
                    mma32<SP, true>(acc[i], bh, bl, xh, xl);
                }
            }
        }
    };

    // One register buffer per half, each refilled a whole chunk ahead; dt of the
    // next chunk is requested right after the gamma scan consumed the current one.
    // Every wait therefore covers loads issued about a chunk earlier, while the
    // newer ones stay in flight.  The first loads go out in the loop's own order
    // (dt, first half, second half): the compiler's wait counts at the loop head
    // take the later position of each register over both ways in, so a different
    // order here would make every chunk wait for both halves at once.
    Buf buf0, buf1;
    float d0, d1;
    load_dt(cfirst, d0, d1);
    __builtin_amdgcn_sched_barrier(0);
    load_half(buf0, cfirst, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_half(buf1, cfirst, 1);
    __builtin_amdgcn_sched_barrier(0);
    double lrun = 0.0;   // log decay from the segment's start to the current chunk
    for (int c = cfirst; c < cend; ++c) {
        const int S = (int)((L - (int64_t)c * Q) < Q ? (L - (int64_t)c * Q) : Q);
        if (2 * lane >= S) d0 = 0.f;
        if (2 * lane + 1 >= S) d1 = 0.f;
        // gamma over the chunk (every wave), weights w_i = dt_i e(gamma_S - gamma_i)
        double g0, g1;
        gamma_scan(d0, d1, Ah, g0, g1);
        const double gS = ((S - 1) & 1) ? readlane_f64(g1, (S - 1) >> 1) : readlane_f64(g0, (S - 1) >> 1);
        const float w0 = d0 * expc(gS - g0);
        const float w1 = d1 * expc(gS - g1);
        // this wave's table of the weights (read back by the same wave's lanes:
        // its LDS operations complete in order)
        *reinterpret_cast<float2*>(&sW[gwave][2 * lane]) = float2{w0, w1};
        const float decay = expc(gS);
        // entry state of this chunk, then h <- e(gamma_S) h (the stores go out first,
        // so they are the oldest memory operations whenever a later load is awaited)
        float* he = a.states + ((cbase + c) * a.nheads + head) * (int64_t)(P * N);
        const bool store = seg_k == 0 || c > cfirst;
        if (seg_k > 0 && c > cfirst && tid == 0) a.cum[(cbase + c) * a.nheads + head] = lrun;
        lrun += gS;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            if (store) {
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    *reinterpret_cast<float4*>(he + eoff(i, m)) =
                        float4{acc[i][4 * m], acc[i][4 * m + 1], acc[i][4 * m + 2], acc[i][4 * m + 3]};
            }
            acc[i] *= decay;
        }
        load_dt(c + 1, d0, d1);

        // first half.  The scheduling barriers keep each half's staging arithmetic
        // in its phase: hoisted above the barriers it would make the compiler wait
        // for that half's loads early and undo the prefetch distance.
        // With one tile set, a barrier first waits for the previous half's
        // products; with a set per half, the barrier after the previous half's
        // staging already did (every wave multiplied this set before it).
        const int S0 = S < QH ? S : QH;
        if (NB == 1) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        stage(buf0, c, 0);
        load_half(buf0, c + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        multiply((S0 + 15) >> 4, 0);

        // second half
        const int S1 = S - QH;
        if (NB == 1) __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        stage(buf1, c, 1);
        load_half(buf1, c + 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        multiply(S1 > 0 ? (S1 + 15) >> 4 : 0, 1);
    }

    // The end state: the sequence's final state when this is its only segment;
    // otherwise a local end state, left in the next segment's first entry slot
    // (for segment 0 that is already the true entry state there) or, for the
    // last segment, in seg_end, for the carry kernel to complete.
    if (cend == nch && seg_k == 0) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<float4*>(st + soff(i, m)) =
                    float4{acc[i][4 * m], acc[i][4 * m + 1], acc[i][4 * m + 2], acc[i][4 * m + 3]};
    } else {
        float* he = cend < nch ? a.states + ((cbase + cend) * a.nheads + head) * (int64_t)(P * N)
                               : a.seg_end + ((int64_t)seq * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int m = 0; m < 4; ++m)
                *reinterpret_cast<float4*>(he + eoff(i, m)) =
                    float4{acc[i][4 * m], acc[i][4 * m + 1], acc[i][4 * m + 2], acc[i][4 * m + 3]};
        if (seg_k > 0 && tid == 0) a.lam[(cbase + cfirst) * a.nheads + head] = lrun;
    }
}

// ------------------------------------------------------------------ segment carry
//
// For a sequence split into segments, one workgroup per (sequence, head) runs
// the recurrence over segment boundaries: with E_k segment k's end state from a
// zero start (E_0 from the true initial state) and lam_k its total log decay,
// the true end states are T_0 = E_0, T_k = e(lam_k) T_{k-1} + E_k.  T_{k-1} is
// the entry state of segment k's first chunk, written over E_{k-1} there; the
// last T is the sequence's final state.  Elementwise over the P x N state, in
// the accumulator order of the entry slots.
template <int N>
__global__ __launch_bounds__(256) void segment_carry_kernel(ScanArgs a) {
    constexpr int F = P * N / 4;      // float4 per state
    constexpr int PT = F / 256;       // float4 per thread
    const int seq = (int)blockIdx.x / a.nheads, head = (int)blockIdx.x % a.nheads;
    const int tid = threadIdx.x;
    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    if (L <= 0) return;
    const int nch = (int)((L + Q - 1) / Q);
    int nseg = (nch + a.seg - 1) / a.seg;
    if (nseg > a.seg_levels) nseg = a.seg_levels;   // the last level takes the rest
    if (nseg <= 1) return;
    const int64_t cbase = s0 / Q + seq;
    auto entry = [&](int c) {
        return reinterpret_cast<float4*>(a.states + ((cbase + c) * a.nheads + head) * (int64_t)(P * N));
    };
    float4 T[PT];
    const float4* e1 = entry(a.seg);
#pragma unroll
    for (int j = 0; j < PT; ++j) T[j] = e1[tid + 256 * j];
    for (int k = 1; k < nseg; ++k) {
        const float d = expc(a.lam[(cbase + (int64_t)k * a.seg) * a.nheads + head]);
        const bool last = k == nseg - 1;
        float4* E = last ? reinterpret_cast<float4*>(a.seg_end + ((int64_t)seq * a.nheads + head) * (int64_t)(P * N))
                         : entry((k + 1) * a.seg);
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const float4 e = E[tid + 256 * j];
            T[j] = float4{fmaf(d, T[j].x, e.x), fmaf(d, T[j].y, e.y), fmaf(d, T[j].z, e.z), fmaf(d, T[j].w, e.w)};
        }
        if (!last) {
#pragma unroll
            for (int j = 0; j < PT; ++j) E[tid + 256 * j] = T[j];
        }
    }
    const int slot = a.state_idx ? a.state_idx[seq] : seq;
    float* st = a.ssm_state + ((int64_t)slot * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        int p, n;
        state_pn(tid + 256 * j, p, n);
        *reinterpret_cast<float4*>(st + p * N + n) = T[j];
    }
}

// ------------------------------------------------------------------ chunk out
//
// 8 waves; wave w owns t tile T = w (w < 4) or 11 - w, so the two waves that
// share a SIMD (w and w + 4) hold tiles T and 7 - T: 9 causal (i, t) tiles per
// SIMD.  The decay e(gamma_t - gamma_i) of an off-diagonal tile is the product
// of a row factor dt_i e(gamma_r - gamma_i) and a column factor
// e(gamma_t - gamma_r), r the last row of i's tile (both exponents <= 0, so
// neither factor overflows); diagonal tiles take the exponential per element.

//
// Raw input (pre-conv bf16 rows): the G phase convolves B and C in pieces of
// RR rows x 8 channels (threads 0-255 B, 256-511 C, one piece per 64-n slice),
// with their conv weights staged over head buffer 0; each head's x is
// convolved by threads 0-255 in the same pieces, with the head's conv weights
// staged into LDS one head ahead by threads 256 .. 256 + 5P/4 - 1.
template <int N, typename Tin>
__global__ __launch_bounds__(512) void ssd_chunk_out_kernel(ScanArgs a) {
    constexpr bool RAW = is_raw<Tin>();
    constexpr bool SP = In<Tin>::kSplit;
    constexpr int CPL = In<Tin>::CPL;
    constexpr int NT = 512;
    constexpr int NKB = N / 32;        // K blocks over n
    constexpr int NPASS = N / 64;      // B, C staged 64 n at a time
    constexpr int HR = 64 + 8;         // LDS row stride of a staged 64-n slice
    constexpr int NRS = N + 8;         // LDS row stride of the h_in planes
    constexpr int STAGE = (SP ? 4 : 2) * Q * HR;
    constexpr int HX = (SP ? 2 : 1) * P * RS;   // x^T planes of one head
    constexpr int HBUF = HX + 2 * P * NRS;      // + h_in planes: one head buffer
    constexpr int SMEM = HBUF + STAGE > 2 * HBUF ? HBUF + STAGE : 2 * HBUF;
    constexpr int NXP = 16 * P / CPL;  // x pieces: 8 tokens x CPL columns
    constexpr int NHV = (P * N / 4) / NT;   // float4 of h_in per thread
    // Two head buffers: head j + 1 is staged into one while head j is multiplied
    // out of the other.  The B / C slices of the G phase lie past head buffer 0
    // (over buffer 1), so the first head is staged while other waves still
    // multiply the last slice.
    __shared__ __align__(16) u16 smem[SMEM];
    __shared__ __align__(16) float rowf[2][Q];      // dt_i e(gamma_r(i) - gamma_i)
    __shared__ __align__(16) float colf[2][Q * 8];  // [t][it]: e(gamma_t - gamma_r(it)), it below t's tile
    __shared__ __align__(16) double gam[2][Q];
    __shared__ __align__(16) float dts[2][Q];
    __shared__ __align__(16) float din[2][Q];       // e(gamma_t)
    __shared__ float sA[MAXHPG], sD[MAXHPG];        // A and D of the group's heads
    __shared__ float4 sXW[2][RAW ? P : 1];          // raw input: conv weights of a head's x, per head buffer
    __shared__ __align__(16) float sXB[2][RAW ? P : 1];   // and biases (channel order)
    static_assert(!RAW || 2 * N * 5 * 4 <= 2 * HBUF, "G-phase conv weights fit over head buffer 0");
    u16* Bh = smem + HBUF;
    u16* Ch = Bh + Q * HR;
    u16* Bl = Bh + 2 * Q * HR;
    u16* Cl = Bh + 3 * Q * HR;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, q = lane >> 4, l16 = lane & 15;
    const int G = a.ngroups;
    const int hpg = a.nheads / G;
    // a small grid splits each group's heads over out_split workgroups (each
    // forms G^T itself): heads j0 .. j1-1 of the group
    const int split = a.out_split > 1 ? a.out_split : 1;
    const int cg = (int)blockIdx.x / split;
    const int j0 = ((int)blockIdx.x % split) * (hpg / split), j1 = j0 + hpg / split;
    const int cslot = cg / G;
    const int grp = cg % G;

    // chunk slot -> (sequence, chunk): sequence b owns slots cu[b]/Q + b + c
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu_seqlens[mid] / Q + mid <= cslot) lo = mid; else hi = mid;
    }
    const int seq = lo;
    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    const int64_t c = cslot - (s0 / Q + seq);
    if (c * Q >= L) return;
    const int S = (int)((L - c * Q) < Q ? (L - c * Q) : Q);
    const int64_t r0 = s0 + c * Q;

    const Tin* Xg = static_cast<const Tin*>(a.x);
    const Tin* Bg = static_cast<const Tin*>(a.B);
    const Tin* Cg = static_cast<const Tin*>(a.C);
    // raw input: the conv state's slot of this sequence (for the chunk's first rows)
    const int slot = a.state_idx ? a.state_idx[seq] : seq;
    const bool init = a.has_init ? (a.has_init[seq] != 0) : true;
    const int d_inner = a.nheads * P;
    // raw input: this thread's x piece (threads 0-255): 8 channels x RR rows
    const int x_cg = lane >> 3, x_rg = (lane & 7) + 8 * (wave & 3);
    // (threads 256 .. hold the conv weights of the workgroup's next head in xraw[0])
    uint4 xraw[RAW ? RW : 1];

    // per-head staging registers: x piece (8 tokens x CPL columns), h_in, dt
    const int tg = tid % 16;
    uint4 xr[8];
    float4 hr[NHV];
    // In a split sequence, a chunk after the first of a later segment holds a
    // local entry state: the true one adds e(log decay since the segment's start)
    // times the segment's true entry state (its first chunk's slot).
    // (the last segment takes every chunk from its start on)
    const int kseg = a.seg > 0 ? min((int)(c / a.seg), a.seg_levels - 1) : 0;
    const bool fix = kseg >= 1 && c != (int64_t)kseg * a.seg;
    const int64_t cslot0 = cslot - (fix ? c - (int64_t)kseg * a.seg : 0);
    float4 hs[NHV];
    float fcum = 0.f;
    float dr0 = 0.f, dr1 = 0.f;
    // x piece tg holds the chunk rows the intra products take as one K slot
    // group: rows 32 kb + 4 q + r (slots 0-3) and 32 kb + 16 + 4 q + r (slots
    // 4-7), kb = tg / 4, q = tg % 4, so it is staged as one contiguous 16-byte
    // run per column and read back with one 16-byte LDS read.
    const int xrow0 = 32 * (tg >> 2) + 4 * (tg & 3);
    auto prefetch = [&](int head) {
        if constexpr (RAW) {
            if (tid < 256) {
                load_raw_piece(static_cast<const uint16_t*>(a.x) + r0 * a.ld_x + head * a.hs_x + 8 * x_cg,
                               (int)a.ld_x, 4 * x_rg, (int)(-c * Q), (int)(L - 1 - c * Q), (lane & 7) == 0, xraw);
            } else if (tid < 256 + P + P / 4) {
                // conv weights of the workgroup's next head (or this one again at the end)
                const int hn = head + 1 < grp * hpg + j1 ? head + 1 : head;
                const int e = tid - 256;
                xraw[0] = uint4{0u, 0u, 0u, 0u};
                if (e < P) xraw[0] = *reinterpret_cast<const uint4*>(a.conv_w + ((int64_t)hn * P + e) * 4);
                else if (a.conv_b) xraw[0] = *reinterpret_cast<const uint4*>(a.conv_b + hn * P + 4 * (e - P));
            }
        } else if (tid < NXP) {
            const Tin* xb = Xg + r0 * a.ld_x + head * a.hs_x + (tid / 16) * CPL;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int row = xrow0 + (k & 3) + 16 * (k >> 2);
                xr[k] = row < S ? *reinterpret_cast<const uint4*>(xb + row * a.ld_x) : uint4{0u, 0u, 0u, 0u};
            }
        }
        const float* he = a.states + ((s0 / Q + seq + c) * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
        for (int k = 0; k < NHV; ++k) hr[k] = *reinterpret_cast<const float4*>(he + 4 * (tid + NT * k));
        if (fix && !RAW) {
            const float* hf = a.states + (cslot0 * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
            for (int k = 0; k < NHV; ++k) hs[k] = *reinterpret_cast<const float4*>(hf + 4 * (tid + NT * k));
            fcum = expc(a.cum[(int64_t)cslot * a.nheads + head]);
        }
        if (wave == 0) {
            dr0 = (2 * lane < S) ? a.dt[(r0 + 2 * lane) * a.ld_dt + head] : 0.f;
            dr1 = (2 * lane + 1 < S) ? a.dt[(r0 + 2 * lane + 1) * a.ld_dt + head] : 0.f;
        }
    };
    prefetch(grp * hpg + j0);
    // A and D of the group's heads, read once (a per-head load issued after the
    // next head's prefetch would make the compiler wait for that prefetch too)
    for (int e = tid; e < hpg; e += NT) {
        sA[e] = a.A[grp * hpg + e];
        sD[e] = a.D ? a.D[grp * hpg + e] : 0.f;
    }

    const int T = wave < 4 ? wave : 11 - wave;
    const bool act = 16 * T < S;
    const int t = 16 * T + l16;          // this lane's output row
    // C operands of tile T (column t, K = n), kept for every head
    bf16x8_t ch[NKB], cl[NKB];
    // G^T[i, t] = B_i . C_t for i tiles it <= T
    f32x4_t g[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) g[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Every slice's B and C pieces are requested up front, branch-free (rows
    // clamped into the chunk): with a load and its use in the same iteration the
    // slices cost one memory round trip per piece.  Rows past the chunk's end
    // only reach G entries that the causal mask or a zero dt leaves unused.
    constexpr int PPR = 64 / CPL;            // pieces per 64-n row slice
    constexpr int GIT = RAW ? 1 : Q * PPR / NT;   // pieces per thread per slice
    uint4 gbv[NPASS][GIT], gcv[NPASS][GIT];
    // raw input: one piece per slice, of B (threads 0-255) or C (256-511)
    const bool gB = tid < 256;
    const int g_cg = lane >> 3, g_rg = (lane & 7) + 8 * (wave & 3);
    uint4 graw[RAW ? NPASS : 1][RAW ? RW : 1];
    float4* gW = reinterpret_cast<float4*>(smem);          // G-phase conv weights, over head buffer 0:
    float* gBias = reinterpret_cast<float*>(smem + 16 * N);  // [B channels ; C channels]
    if constexpr (RAW) {
        const int64_t gld = gB ? a.ld_B : a.ld_C;
        const uint16_t* gcol = gB ? static_cast<const uint16_t*>(a.B) + r0 * a.ld_B + grp * a.gs_B
                                  : static_cast<const uint16_t*>(a.C) + r0 * a.ld_C + grp * a.gs_C;
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps)
            load_raw_piece(gcol + 64 * ps + 8 * g_cg, (int)gld, 4 * g_rg, (int)(-c * Q), (int)(L - 1 - c * Q),
                           (lane & 7) == 0, graw[ps]);
        for (int e = tid; e < 2 * N; e += NT) {
            const int ch = d_inner + (e < N ? grp * N + e : G * N + grp * N + (e - N));
            gW[wsw(e)] = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)ch * 4);
            gBias[e] = a.conv_b ? a.conv_b[ch] : 0.f;
        }
        // the first head's x conv weights
        for (int e = tid; e < P; e += NT) {
            const int ch = (grp * hpg + j0) * P + e;
            sXW[0][wsw(e)] = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)ch * 4);
            sXB[0][e] = a.conv_b ? a.conv_b[ch] : 0.f;
        }
        __syncthreads();
    } else {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps)
#pragma unroll
        for (int k = 0; k < GIT; ++k) {
            const int e = tid + NT * k;
            const int i = e / PPR, o = e % PPR;
            const int64_t row = r0 + (i < S ? i : S - 1);
            const int col = 64 * ps + o * CPL;
            gbv[ps][k] = *reinterpret_cast<const uint4*>(Bg + row * a.ld_B + grp * a.gs_B + col);
            gcv[ps][k] = *reinterpret_cast<const uint4*>(Cg + row * a.ld_C + grp * a.gs_C + col);
        }
    }
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        if (ps > 0) __syncthreads();   // the previous slice's products are done
        if constexpr (RAW) {
            // conv + SiLU of this thread's piece of the slice, rows 4 g_rg .. + 3
            raw_halo(graw[ps], lane);
            const int row0 = 4 * g_rg;
            const bool start = c == 0 && row0 == 0;
            const int wi = (gB ? 0 : N) + 64 * ps + 8 * g_cg;
            const int ch0 = d_inner + (gB ? 0 : G * N) + grp * N + 64 * ps + 8 * g_cg;
            u16* const dh = gB ? Bh : Ch;
            u16* const dl = gB ? Bl : Cl;
            const ConvW cw = read_convw(gW, gBias, wi);
            // one output row (8 channels) at a time; window row j of output row tt
            // is raw row tt + j, or for a piece that starts the sequence and
            // tt + j < 3, carried row tt + j of the conv state
#pragma unroll
            for (int tt = 0; tt < RR; ++tt) {
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 w4 = cw.w(k);
                    const float wk[4] = {w4.x, w4.y, w4.z, w4.w};
                    float acc = cw.b[k];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float xv = bf16_lane(graw[ps][tt + j], k);
                        if (tt + j < 3 && start)
                            xv = init ? a.conv_state[((int64_t)slot * 3 + tt + j) * a.conv_dim + ch0 + k] : 0.f;
                        acc = fmaf(wk[j], xv, acc);
                    }
                    v[k] = silu(acc);
                }
                uint4 h4, l4;
                split8(v, h4, l4);
                const int off = (row0 + tt) * HR + 8 * g_cg;
                *reinterpret_cast<uint4*>(dh + off) = h4;
                *reinterpret_cast<uint4*>(dl + off) = l4;
            }
        } else {
#pragma unroll
        for (int k = 0; k < GIT; ++k) {
            const int e = tid + NT * k;
            const int i = e / PPR, o = e % PPR;
            const uint4 vb = gbv[ps][k], vc = gcv[ps][k];
            const int off = i * HR + o * CPL;
            if constexpr (SP) {
                uint32_t bh2[2], bl2[2], ch2[2], cl2[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    split2(In<Tin>::val(vb, 2 * m), In<Tin>::val(vb, 2 * m + 1), bh2[m], bl2[m]);
                    split2(In<Tin>::val(vc, 2 * m), In<Tin>::val(vc, 2 * m + 1), ch2[m], cl2[m]);
                }
                *reinterpret_cast<uint2*>(Bh + off) = uint2{bh2[0], bh2[1]};
                *reinterpret_cast<uint2*>(Bl + off) = uint2{bl2[0], bl2[1]};
                *reinterpret_cast<uint2*>(Ch + off) = uint2{ch2[0], ch2[1]};
                *reinterpret_cast<uint2*>(Cl + off) = uint2{cl2[0], cl2[1]};
            } else {
                *reinterpret_cast<uint4*>(Bh + off) = vb;
                *reinterpret_cast<uint4*>(Ch + off) = vc;
            }
        }
        }
        __syncthreads();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const int k = 2 * ps + k2;
            ch[k] = as_bf16x8(lds128(Ch + t * HR + 32 * k2 + 8 * q));
            cl[k] = SP ? as_bf16x8(lds128(Cl + (SP ? t * HR + 32 * k2 + 8 * q : 0))) : ch[k];
            if (act) {
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    if (it <= T && 16 * it < S) {
                        const int row = (16 * it + l16) * HR + 32 * k2 + 8 * q;
                        const bf16x8_t bh = as_bf16x8(lds128(Bh + row));
                        const bf16x8_t bl = SP ? as_bf16x8(lds128(Bl + (SP ? row : 0))) : bh;
                        mma2<SP, SP>(g[it], bh, bl, ch[k], cl[k]);
                    }
                }
            }
        }
    }

    // Stage head j (whose loads are in xr / hr / dr) into head buffer bf.
    auto stage_head = [&](int bf, int j) __attribute__((always_inline)) {
        u16* Xh = smem + bf * HBUF;
        u16* Xl = Xh + P * RS;
        u16* HH = Xh + HX;
        u16* HL = HH + P * NRS;
        // wave 0: gamma and the decay factors of this head, from the prefetched dt
        double ga0 = 0.0, ga1 = 0.0;
        float rf0 = 0.f, rf1 = 0.f, cf0[8], cf1[8];
        if (wave == 0) {
            gamma_scan(dr0, dr1, sA[j], ga0, ga1);
            // rows 2 lane, 2 lane + 1 lie in tile lane / 8, whose last row 16 (lane / 8) + 15
            // is held (as ga1) by lane 8 (lane / 8) + 7
            double gri[8];
#pragma unroll
            for (int it = 0; it < 8; ++it) gri[it] = readlane_f64(ga1, 8 * it + 7);
            double gr = gri[0];
#pragma unroll
            for (int it = 1; it < 8; ++it) gr = (lane >> 3) == it ? gri[it] : gr;
            rf0 = dr0 * expc(gr - ga0);
            rf1 = dr1 * expc(gr - ga1);
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                cf0[it] = (it < (lane >> 3)) ? expc(ga0 - gri[it]) : 0.f;
                cf1[it] = (it < (lane >> 3)) ? expc(ga1 - gri[it]) : 0.f;
            }
        }

        if constexpr (RAW) {
            // the next head's conv weights into the other buffer (read one phase later)
            if (tid >= 256 && tid < 256 + P) {
                sXW[bf ^ 1][wsw(tid - 256)] = __builtin_bit_cast(float4, xraw[0]);
            } else if (tid >= 256 + P && tid < 256 + P + P / 4) {
                *reinterpret_cast<float4*>(&sXB[bf ^ 1][4 * (tid - 256 - P)]) = __builtin_bit_cast(float4, xraw[0]);
            }
            // a later segment's local entry state: its true part is added here (the
            // loads wait in place; only split sequences take this path)
            if (fix) {
                const int head = grp * hpg + j;
                const float* hf = a.states + (cslot0 * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
                for (int k = 0; k < NHV; ++k) hs[k] = *reinterpret_cast<const float4*>(hf + 4 * (tid + NT * k));
                fcum = expc(a.cum[(int64_t)cslot * a.nheads + head]);
            }
            // conv + SiLU of the x piece: rows 4 x_rg .. + 3 of the chunk, placed at
            // their positions in the K-slot order of the x^T planes (row i sits at
            // 8 (4 (i / 32) + (i / 4) % 4) + 4 ((i / 16) % 2) + i % 4)
            if (tid < 256) {
                raw_halo(xraw, lane);
                const int head = grp * hpg + j;
                const int row0 = 4 * x_rg;
                const bool start = c == 0 && row0 == 0;
                const int pos = 8 * (4 * (row0 >> 5) + ((row0 >> 2) & 3)) + 4 * ((row0 >> 4) & 1);
                auto put = [&](int k, float (&u)[RR]) __attribute__((always_inline)) {
#pragma unroll
                    for (int tt = 0; tt < RR; ++tt)
                        if (row0 + tt >= S) u[tt] = 0.f;
                    uint32_t hb[2], lb[2];
                    split2(u[0], u[1], hb[0], lb[0]);
                    split2(u[2], u[3], hb[1], lb[1]);
                    const int off = (8 * x_cg + k) * RS + pos;
                    *reinterpret_cast<uint2*>(Xh + off) = uint2{hb[0], hb[1]};
                    *reinterpret_cast<uint2*>(Xl + off) = uint2{lb[0], lb[1]};
                };
                const ConvW cw = read_convw(sXW[bf], sXB[bf], 8 * x_cg);
                if (start) {
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        float u[RR];
                        conv_piece_start(xraw, k, a.conv_state, a.conv_dim, slot, init, head * P + 8 * x_cg,
                                         cw.w(k), cw.b[k], u);
                        put(k, u);
                    }
                } else {
                    const float hv[3][8] = {};
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        float u[RR];
                        conv_piece(xraw, k, false, hv, cw.w(k), cw.b[k], u);
                        put(k, u);
                    }
                }
            }
        } else
        // x^T planes: column (tid / 16) * CPL + jj, positions 8 tg .. +7 (the rows above)
        if (tid < NXP) {
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                const int off = ((tid / 16) * CPL + jj) * RS + 8 * tg;
                if constexpr (SP) {
                    float v[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) v[k] = In<Tin>::val(xr[k], jj);
                    uint4 hi4, lo4;
                    split8(v, hi4, lo4);
                    *reinterpret_cast<uint4*>(Xh + off) = hi4;
                    *reinterpret_cast<uint4*>(Xl + off) = lo4;
                } else {
                    uint32_t hb[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) hb[k] = half_of(word_of(xr[k], jj >> 1), jj & 1);
                    *reinterpret_cast<uint4*>(Xh + off) =
                        uint4{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16), hb[4] | (hb[5] << 16), hb[6] | (hb[7] << 16)};
                }
            }
        }
        // h_in split planes: float4 k of the entry state covers (p, n .. n + 3)
        if (fix) {
#pragma unroll
            for (int k = 0; k < NHV; ++k)
                hr[k] = float4{fmaf(fcum, hs[k].x, hr[k].x), fmaf(fcum, hs[k].y, hr[k].y),
                               fmaf(fcum, hs[k].z, hr[k].z), fmaf(fcum, hs[k].w, hr[k].w)};
        }
#pragma unroll
        for (int k = 0; k < NHV; ++k) {
            int p, n;
            state_pn(tid + NT * k, p, n);
            uint32_t hb[2], lb[2];
            split2(hr[k].x, hr[k].y, hb[0], lb[0]);
            split2(hr[k].z, hr[k].w, hb[1], lb[1]);
            *reinterpret_cast<uint2*>(HH + p * NRS + n) = uint2{hb[0], hb[1]};
            *reinterpret_cast<uint2*>(HL + p * NRS + n) = uint2{lb[0], lb[1]};
        }
        if (wave == 0) {
            gam[bf][2 * lane] = ga0;
            gam[bf][2 * lane + 1] = ga1;
            dts[bf][2 * lane] = dr0;
            dts[bf][2 * lane + 1] = dr1;
            din[bf][2 * lane] = expc(ga0);
            din[bf][2 * lane + 1] = expc(ga1);
            rowf[bf][2 * lane] = rf0;
            rowf[bf][2 * lane + 1] = rf1;
            *reinterpret_cast<float4*>(colf[bf] + 16 * lane) = float4{cf0[0], cf0[1], cf0[2], cf0[3]};
            *reinterpret_cast<float4*>(colf[bf] + 16 * lane + 4) = float4{cf0[4], cf0[5], cf0[6], cf0[7]};
            *reinterpret_cast<float4*>(colf[bf] + 16 * lane + 8) = float4{cf1[0], cf1[1], cf1[2], cf1[3]};
            *reinterpret_cast<float4*>(colf[bf] + 16 * lane + 12) = float4{cf1[4], cf1[5], cf1[6], cf1[7]};
        }
    };
    // Multiply head j out of head buffer bf and store its y rows.
    auto compute_head = [&](int bf, int j) __attribute__((always_inline)) {
        const int head = grp * hpg + j;
        const float Dh = sD[j];
        const u16* Xh = smem + bf * HBUF;
        const u16* Xl = Xh + P * RS;
        const u16* HH = Xh + HX;
        const u16* HL = HH + P * NRS;
        const float* rowfb = rowf[bf];
        const float* dtsb = dts[bf];
        const double* gamb = gam[bf];
        if (act) {
            // y^T[p, t] tiles: yacc[pt], lane has t, p = 16 pt + 4q + r
            f32x4_t yacc[4];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) yacc[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

            // inter-chunk term: h_in C^T (A = h_in rows p, B = C columns t, K = n)
#pragma unroll
            for (int k = 0; k < NKB; ++k) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const bf16x8_t ah = as_bf16x8(lds128(HH + (16 * pt + l16) * NRS + 32 * k + 8 * q));
                    const bf16x8_t al = as_bf16x8(lds128(HL + (16 * pt + l16) * NRS + 32 * k + 8 * q));
                    mma2<true, SP>(yacc[pt], ah, al, ch[k], cl[k]);
                }
            }
            const float sc = din[bf][t];
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) yacc[pt] *= sc;

            // intra-chunk term: X^T M^T over i tile pairs (2kb, 2kb+1); the M^T
            // operand slot j < 4 is row 4q + j of tile 2kb, j >= 4 row 4q + j - 4
            // of tile 2kb + 1 (the rows this lane's accumulators hold); the x^T
            // planes hold the rows in that order (8 per (kb, q) group).
            const float4* cft = reinterpret_cast<const float4*>(colf[bf] + 8 * t);
            const float4 cfa = cft[0], cfb = cft[1];
            const float cfv[8] = {cfa.x, cfa.y, cfa.z, cfa.w, cfb.x, cfb.y, cfb.z, cfb.w};
            // the tile index is a compile-time constant inside (one instance per tile)
            auto intra = [&](auto Tc) __attribute__((always_inline)) {
                constexpr int TT = decltype(Tc)::value;
#pragma unroll
                for (int kb = 0; kb <= TT / 2; ++kb) {
                    float m[8];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int it = 2 * kb + h2;
                        const int i0 = 16 * it + 4 * q;
                        if (it < TT) {
                            const float4 rf = *reinterpret_cast<const float4*>(rowfb + i0);
                            const float cv = cfv[it];
                            m[4 * h2 + 0] = g[it][0] * rf.x * cv;
                            m[4 * h2 + 1] = g[it][1] * rf.y * cv;
                            m[4 * h2 + 2] = g[it][2] * rf.z * cv;
                            m[4 * h2 + 3] = g[it][3] * rf.w * cv;
                        } else if (it == TT) {
                            const double gt = gamb[t];
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int i = i0 + r;
                                float v = 0.f;
                                if (i <= t) {
                                    v = g[it][r] * dtsb[i] * expc(gt - gamb[i]);
                                    if (i == t) v += Dh;
                                }
                                m[4 * h2 + r] = v;
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r) m[4 * h2 + r] = 0.f;
                        }
                    }
                    uint4 mh4, ml4;
                    split8(m, mh4, ml4);
                    const bf16x8_t mh = as_bf16x8(mh4), ml = as_bf16x8(ml4);
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        const int xo = (16 * pt + l16) * RS + 32 * kb + 8 * q;
                        const bf16x8_t xh = as_bf16x8(lds128(Xh + xo));
                        const bf16x8_t xl = SP ? as_bf16x8(lds128(Xl + (SP ? xo : 0))) : xh;
                        mma2<SP, true>(yacc[pt], xh, xl, mh, ml);
                    }
                }
            };
            switch (T) {
                case 0: intra(std::integral_constant<int, 0>{}); break;
                case 1: intra(std::integral_constant<int, 1>{}); break;
                case 2: intra(std::integral_constant<int, 2>{}); break;
                case 3: intra(std::integral_constant<int, 3>{}); break;
                case 4: intra(std::integral_constant<int, 4>{}); break;
                case 5: intra(std::integral_constant<int, 5>{}); break;
                case 6: intra(std::integral_constant<int, 6>{}); break;
                default: intra(std::integral_constant<int, 7>{}); break;
            }

            // store y row t of the chunk: lane has y[t][16 pt + 4q .. +3]
            if (t < S) {
                float* dst = a.y + (r0 + t) * a.ld_y + (int64_t)head * P + 4 * q;
#pragma unroll
                for (int pt = 0; pt < 4; ++pt)
                    *reinterpret_cast<float4*>(dst + 16 * pt) =
                        float4{yacc[pt][0], yacc[pt][1], yacc[pt][2], yacc[pt][3]};
            }
        }
    };

    stage_head(0, j0);   // (buffer 0: no G slice there)
    prefetch(j0 + 1 < j1 ? grp * hpg + j0 + 1 : grp * hpg + j0);
    __syncthreads();
    for (int j = j0; j < j1; ++j) {
        if (j + 1 < j1) {
            stage_head((j - j0 + 1) & 1, j + 1);
            if (j + 2 < j1) prefetch(grp * hpg + j + 2);
        }
        compute_head((j - j0) & 1, j);
        __syncthreads();
    }
}


// x^T plane layout of the raw chunk output: the 32-row block kb of plane row p
// sits at block kb ^ ((p / 16) % 4).  A consumer's operand read (16 plane rows
// of one 16-row group, one block) moves as a whole; a producer's store (8 plane
// rows 8 apart, one block) then spreads over 4 bank windows instead of 2.
__device__ __forceinline__ int xsw(int kb, int p) { return kb ^ ((p >> 4) & 3); }


// The fused norm of a chunk's rows i0, i0 + 8, ... (one wave per row, NR rows'
// loads in flight at once, NBL 8-channel blocks per lane): see norm_row.h.  The
// first rows' z and the weights are loaded before the barrier that makes y
// visible (they do not depend on it), y after it.
template <typename Tout, int NBL, int NR>
__device__ __forceinline__ void chunk_norm_rows(const ScanArgs& a, int64_t r0, int S, int cbase, int gs, int i0,
                                                int lane) {
    const int nb = gs / 8;
    const uint16_t* zb = static_cast<const uint16_t*>(a.z);
    Tout* ob = static_cast<Tout*>(a.norm_out);
    NormRow<NBL, uint16_t> r[NR];
    NormW<NBL> W;
    auto load_z = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int row = i + 8 * k < S ? i + 8 * k : (i < S ? i : 0);
            norm_row_load_z(r[k], zb + (r0 + row) * a.ld_z + cbase, nb, lane);
        }
    };
    load_z(i0);
    norm_w_load(W, a.norm_w + cbase, nb, lane);
    __syncthreads();   // every wave's y stores are visible
    for (int i = i0; i < S; i += 8 * NR) {
        if (i != i0) load_z(i);
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            const int row = i + 8 * k < S ? i + 8 * k : i;
            norm_row_load_y(r[k], a.y + (r0 + row) * a.ld_y + cbase, nb, lane);
        }
#pragma unroll
        for (int k = 0; k < NR; ++k) {
            if (i + 8 * k < S)
                norm_row_store(r[k], W, ob + (r0 + i + 8 * k) * a.ld_out + cbase, gs, nb, a.eps,
                               a.norm_before_gate != 0, lane);
        }
    }
}

// ------------------------------------------------------------------ chunk output, raw rows
//
// The chunk output for raw bf16 rows, with the waves split by role.  Waves 0-3
// (producers) convolve and stage the next head into one head buffer: its x
// rows (conv + SiLU of the raw rows, as hi / lo planes), its entry state h_in
// (hi / lo planes; Q16: read as 16-bit rows and their scales, the format
// store_entry_q16 writes) and its decay factors.  Waves 4-7 (consumers) multiply the
// current head out of the other buffer.  A producer and a consumer share each
// SIMD, so the conv's vector work runs beside the matrix products instead of
// before them, and each role keeps only its own registers (the two roles run
// separate loops with the same barriers).  Consumer w owns the 16-row tiles
// T = w and 7 - w of the chunk: every consumer then issues the same number of
// causal products, and each h_in or x operand read from LDS serves both tiles.
// All 8 waves convolve the group's B and C for G^T at the start.
template <int N, bool Q16>
__global__ __launch_bounds__(512) void ssd_chunk_out_raw_kernel(ScanArgs a) {
    static_assert(!Q16 || N == 128, "16-bit entry states at dstate 128");
    constexpr int NT = 512;
    constexpr int NKB = N / 32;        // K blocks over n
    constexpr int NPASS = N / 64;      // B, C staged 64 n at a time
    constexpr int HR = 64 + 8;         // LDS row stride of a staged 64-n slice
    constexpr int NRS = N + 8;         // LDS row stride of the h_in planes
    constexpr int STAGE = 4 * Q * HR;
    constexpr int HX = 2 * P * RS;     // x^T planes of one head
    constexpr int HBUF = HX + 2 * P * NRS;
    constexpr int SMEM = HBUF + STAGE > 2 * HBUF ? HBUF + STAGE : 2 * HBUF;
    constexpr int NHP = (P * N / 4) / 256;   // float4 of h_in per producer thread
    // Two head buffers: the producers stage head j + 1 into one while the
    // consumers multiply head j out of the other.  The B / C slices of the G
    // phase lie past head buffer 0 (over buffer 1), so the producers stage the
    // first head while the consumers still multiply the last slice.
    __shared__ __align__(16) u16 smem[SMEM];
    __shared__ __align__(16) float rowf[2][Q];      // dt_i e(gamma_r(i) - gamma_i)
    __shared__ __align__(16) float colf[2][Q * 8];  // [t][it]: e(gamma_t - gamma_r(it)), it below t's tile
    __shared__ __align__(16) double gam[2][Q];
    __shared__ __align__(16) float dts[2][Q];
    __shared__ __align__(16) float din[2][Q];       // e(gamma_t)
    __shared__ float sA[MAXHPG], sD[MAXHPG];        // A and D of the group's heads
    __shared__ float4 sXW[2][P];                    // conv weights of a head's x, per head buffer
    __shared__ __align__(16) float sXB[2][P];       // and biases (channel order)
    static_assert(2 * N * 5 * 4 <= 2 * HBUF, "G-phase conv weights fit over head buffer 0");
    u16* Bh = smem + HBUF;
    u16* Ch = Bh + Q * HR;
    u16* Bl = Bh + 2 * Q * HR;
    u16* Cl = Bh + 3 * Q * HR;
    float4* gW = reinterpret_cast<float4*>(smem);          // G-phase conv weights, over head buffer 0:
    float* gBias = reinterpret_cast<float*>(smem + 16 * N);  // [B channels ; C channels]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, q = lane >> 4, l16 = lane & 15;
    const int G = a.ngroups;
    const int hpg = a.nheads / G;
    // a small grid splits each group's heads over out_split workgroups (each
    // forms G^T itself): heads j0 .. j1-1 of the group
    const int split = a.out_split > 1 ? a.out_split : 1;
    const int cg = (int)blockIdx.x / split;
    const int j0 = ((int)blockIdx.x % split) * (hpg / split), j1 = j0 + hpg / split;
    const int cslot = cg / G;
    const int grp = cg % G;

    // chunk slot -> (sequence, chunk): sequence b owns slots cu[b]/Q + b + c
    int lo = 0, hi = a.batch;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu_seqlens[mid] / Q + mid <= cslot) lo = mid; else hi = mid;
    }
    const int seq = lo;
    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    const int64_t c = cslot - (s0 / Q + seq);
    if (c * Q >= L) return;
    const int S_ = (int)((L - c * Q) < Q ? (L - c * Q) : Q);
    // At dstate 128 the rest of the kernel is compiled twice: for a full chunk
    // that is not its sequence's first (every chunk but a sequence's first and
    // last), with its row count a constant and no rows from the carried conv
    // state, so every row test, bound and start-of-sequence path folds away,
    // and for any chunk.  The LDS arrays above serve both.
    auto body = [&](auto sqc) __attribute__((always_inline)) {
        constexpr int SQ = decltype(sqc)::value;
        const int S = SQ ? SQ : S_;
        const bool c0 = !SQ && c == 0;   // the sequence's first chunk
        const int64_t r0 = s0 + c * Q;
        const int slot = a.state_idx ? a.state_idx[seq] : seq;
        const bool init = a.has_init ? (a.has_init[seq] != 0) : true;
        const int d_inner = a.nheads * P;
        // In a split sequence, a chunk after the first of a later segment holds a
        // local entry state: the true one adds e(log decay since the segment's start)
        // times the segment's true entry state (its first chunk's slot).
        // (the last segment takes every chunk from its start on)
        const int kseg = a.seg > 0 ? min((int)(c / a.seg), a.seg_levels - 1) : 0;
        const bool fix = kseg >= 1 && c != (int64_t)kseg * a.seg;
        const int64_t cslot0 = cslot - (fix ? c - (int64_t)kseg * a.seg : 0);

        // LDS tables: A and D of the group's heads, the G-phase conv weights (B
        // channels, then C channels), the first head's x conv weights
        for (int e = tid; e < hpg; e += NT) {
            sA[e] = a.A[grp * hpg + e];
            sD[e] = a.D ? a.D[grp * hpg + e] : 0.f;
        }
        for (int e = tid; e < 2 * N; e += NT) {
            const int ch = d_inner + (e < N ? grp * N + e : G * N + grp * N + (e - N));
            gW[wsw(e)] = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)ch * 4);
            gBias[e] = a.conv_b ? a.conv_b[ch] : 0.f;
        }
        for (int e = tid; e < P; e += NT) {
            const int ch = (grp * hpg + j0) * P + e;
            sXW[0][wsw(e)] = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)ch * 4);
            sXB[0][e] = a.conv_b ? a.conv_b[ch] : 0.f;
        }

        // G phase: each thread convolves one piece (RR rows x 8 channels) of each
        // 64-n slice, of B (producers) or C (consumers), into the slice planes.
        const bool gIsB = wave < 4;
        const int g_cg = lane >> 3, g_rg = (lane & 7) + 8 * (wave & 3);
        auto g_load = [&](uint4 (&graw)[NPASS][RW]) __attribute__((always_inline)) {
            const int64_t gld = gIsB ? a.ld_B : a.ld_C;
            const uint16_t* gcol = gIsB ? static_cast<const uint16_t*>(a.B) + r0 * a.ld_B + grp * a.gs_B
                                      : static_cast<const uint16_t*>(a.C) + r0 * a.ld_C + grp * a.gs_C;
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps)
                load_raw_piece(gcol + 64 * ps + 8 * g_cg, (int)gld, 4 * g_rg, (int)(-c * Q), (int)(L - 1 - c * Q),
                               (lane & 7) == 0, graw[ps]);
        };
        auto g_conv = [&](int ps, uint4 (&gr)[RW]) __attribute__((always_inline)) {
            raw_halo(gr, lane);
            const int row0 = 4 * g_rg;
            const bool start = c0 && row0 == 0;
            const int wi = (gIsB ? 0 : N) + 64 * ps + 8 * g_cg;
            const int ch0 = d_inner + (gIsB ? 0 : G * N) + grp * N + 64 * ps + 8 * g_cg;
            u16* const dh = gIsB ? Bh : Ch;
            u16* const dl = gIsB ? Bl : Cl;
            const ConvW cw = read_convw(gW, gBias, wi);
            // one output row (8 channels) at a time; window row j of output row tt
            // is raw row tt + j, or for a piece that starts the sequence and
            // tt + j < 3, carried row tt + j of the conv state
#pragma unroll
            for (int tt = 0; tt < RR; ++tt) {
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 w4 = cw.w(k);
                    const float wk[4] = {w4.x, w4.y, w4.z, w4.w};
                    float acc = cw.b[k];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float xv = bf16_lane(gr[tt + j], k);
                        if (tt + j < 3 && start)
                            xv = init ? a.conv_state[((int64_t)slot * 3 + tt + j) * a.conv_dim + ch0 + k] : 0.f;
                        acc = fmaf(wk[j], xv, acc);
                    }
                    v[k] = silu(acc);
                }
                uint4 h4, l4;
                split8(v, h4, l4);
                const int off = (row0 + tt) * HR + 8 * g_cg;
                *reinterpret_cast<uint4*>(dh + off) = h4;
                *reinterpret_cast<uint4*>(dl + off) = l4;
            }
        };

        if (wave < 4) {
            // ---------------------------------------------------------- producers
            const int x_cg = lane >> 3, x_rg = (lane & 7) + 8 * wave;
            uint4 xraw[RW];           // the x piece of the head being prefetched: 8 channels x RR rows
            float4 hr[Q16 ? 1 : NHP]; // its h_in (fp32 entry states)
            uint4 hq[Q16 ? NHP / 2 : 1];   // or its 16-bit values
            float4 hd0, hd1;               // and their row scales (tiles 0-3, 4-7 of row tid % 32)
            uint4 wreg = uint4{0u, 0u, 0u, 0u};   // the conv weights (threads < P) or biases of the head after it
            float dr0 = 0.f, dr1 = 0.f;           // wave 0: its dt of rows 2 lane, 2 lane + 1
            auto prefetch = [&](int head) __attribute__((always_inline)) {
                load_raw_piece(static_cast<const uint16_t*>(a.x) + r0 * a.ld_x + head * a.hs_x + 8 * x_cg, (int)a.ld_x,
                               4 * x_rg, (int)(-c * Q), (int)(L - 1 - c * Q), (lane & 7) == 0, xraw);
                if (tid < P + P / 4) {
                    const int hn = head + 1 < grp * hpg + j1 ? head + 1 : head;
                    wreg = uint4{0u, 0u, 0u, 0u};
                    if (tid < P) wreg = *reinterpret_cast<const uint4*>(a.conv_w + ((int64_t)hn * P + tid) * 4);
                    else if (a.conv_b) wreg = *reinterpret_cast<const uint4*>(a.conv_b + hn * P + 4 * (tid - P));
                }
                const float* he = a.states + ((s0 / Q + seq + c) * a.nheads + head) * (int64_t)(P * N);
                if constexpr (Q16) {
#pragma unroll
                    for (int k = 0; k < NHP / 2; ++k) hq[k] = reinterpret_cast<const uint4*>(he)[tid + 256 * k];
                    const float4* hs = reinterpret_cast<const float4*>(he + P * N / 2 + (tid & 31) * NTQ);
                    hd0 = hs[0];
                    hd1 = hs[1];
                } else {
#pragma unroll
                    for (int k = 0; k < NHP; ++k) hr[k] = *reinterpret_cast<const float4*>(he + 4 * (tid + 256 * k));
                }
                if (wave == 0) {
                    dr0 = (2 * lane < S) ? a.dt[(r0 + 2 * lane) * a.ld_dt + head] : 0.f;
                    dr1 = (2 * lane + 1 < S) ? a.dt[(r0 + 2 * lane + 1) * a.ld_dt + head] : 0.f;
                }
            };
            // Stage head j (whose loads are in xraw / hr / dr / wreg) into head buffer bf.
            auto stage = [&](int bf, int j) __attribute__((always_inline)) {
                u16* Xh = smem + bf * HBUF;
                u16* Xl = Xh + P * RS;
                u16* HH = Xh + HX;
                u16* HL = HH + P * NRS;
                const int head = grp * hpg + j;
                // wave 0: gamma and the decay factors of this head, from the prefetched dt
                double ga0 = 0.0, ga1 = 0.0;
                float rf0 = 0.f, rf1 = 0.f, cf0[8], cf1[8];
                if (wave == 0) {
                    gamma_scan(dr0, dr1, sA[j], ga0, ga1);
                    // rows 2 lane, 2 lane + 1 lie in tile lane / 8, whose last row 16 (lane / 8) + 15
                    // is held (as ga1) by lane 8 (lane / 8) + 7
                    double gri[8];
#pragma unroll
                    for (int it = 0; it < 8; ++it) gri[it] = readlane_f64(ga1, 8 * it + 7);
                    double gr = gri[0];
#pragma unroll
                    for (int it = 1; it < 8; ++it) gr = (lane >> 3) == it ? gri[it] : gr;
                    rf0 = dr0 * expc(gr - ga0);
                    rf1 = dr1 * expc(gr - ga1);
#pragma unroll
                    for (int it = 0; it < 8; ++it) {
                        cf0[it] = (it < (lane >> 3)) ? expc(ga0 - gri[it]) : 0.f;
                        cf1[it] = (it < (lane >> 3)) ? expc(ga1 - gri[it]) : 0.f;
                    }
                }
                // the next head's conv weights into the other buffer (read one phase later)
                if (tid < P) {
                    sXW[bf ^ 1][wsw(tid)] = __builtin_bit_cast(float4, wreg);
                } else if (tid < P + P / 4) {
                    *reinterpret_cast<float4*>(&sXB[bf ^ 1][4 * (tid - P)]) = __builtin_bit_cast(float4, wreg);
                }
                // conv + SiLU of the x piece: rows 4 x_rg .. + 3 of the chunk, placed at
                // their positions in the K-slot order of the x^T planes (row i sits at
                // 8 (4 (i / 32) + (i / 4) % 4) + 4 ((i / 16) % 2) + i % 4), the 32-row
                // block i / 32 swizzled by plane row (xsw)
                {
                    raw_halo(xraw, lane);
                    const int row0 = 4 * x_rg;
                    const bool start = c0 && row0 == 0;
                    const int pos = 8 * ((row0 >> 2) & 3) + 4 * ((row0 >> 4) & 1);
                    auto put = [&](int k, float (&u)[RR]) __attribute__((always_inline)) {
                        if (S < Q) {
#pragma unroll
                            for (int tt = 0; tt < RR; ++tt)
                                if (row0 + tt >= S) u[tt] = 0.f;
                        }
                        uint32_t hb[2], lb[2];
                        split2(u[0], u[1], hb[0], lb[0]);
                        split2(u[2], u[3], hb[1], lb[1]);
                        const int off = (8 * x_cg + k) * RS + 32 * xsw(row0 >> 5, 8 * x_cg + k) + pos;
                        *reinterpret_cast<uint2*>(Xh + off) = uint2{hb[0], hb[1]};
                        *reinterpret_cast<uint2*>(Xl + off) = uint2{lb[0], lb[1]};
                    };
                    // (the producers have the registers to hold all 8 channels' weights)
                    const ConvW cw = read_convw(sXW[bf], sXB[bf], 8 * x_cg);
                    float4 wv[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) wv[k] = cw.w(k);
                    if (start) {
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            float u[RR];
                            conv_piece_start(xraw, k, a.conv_state, a.conv_dim, slot, init, head * P + 8 * x_cg,
                                             wv[k], cw.b[k], u);
                            put(k, u);
                        }
                    } else {
                        const float hv[3][8] = {};
#pragma unroll
                        for (int k = 0; k < 8; ++k) {
                            float u[RR];
                            conv_piece(xraw, k, false, hv, wv[k], cw.b[k], u);
                            put(k, u);
                        }
                    }
                }
                // a later segment's local entry state: its true part is added here (the
                // loads wait in place; only split sequences take this path, and they
                // keep fp32 entry states)
                if constexpr (!Q16) if (fix) {
                    const float* hf = a.states + (cslot0 * a.nheads + head) * (int64_t)(P * N);
                    const float fcum = expc(a.cum[(int64_t)cslot * a.nheads + head]);
#pragma unroll
                    for (int k = 0; k < NHP; ++k) {
                        const float4 hs = *reinterpret_cast<const float4*>(hf + 4 * (tid + 256 * k));
                        hr[k] = float4{fmaf(fcum, hs.x, hr[k].x), fmaf(fcum, hs.y, hr[k].y),
                                       fmaf(fcum, hs.z, hr[k].z), fmaf(fcum, hs.w, hr[k].w)};
                    }
                }
                // h_in split planes: float4 f of the entry state covers (p, n .. n + 3)
                auto put_h = [&](int f, float4 v) __attribute__((always_inline)) {
                    int p, n;
                    state_pn(f, p, n);
                    uint32_t hb[2], lb[2];
                    split2(v.x, v.y, hb[0], lb[0]);
                    split2(v.z, v.w, hb[1], lb[1]);
                    *reinterpret_cast<uint2*>(HH + p * NRS + n) = uint2{hb[0], hb[1]};
                    *reinterpret_cast<uint2*>(HL + p * NRS + n) = uint2{lb[0], lb[1]};
                };
                if constexpr (Q16) {
                    // uint4 tid + 256 k: tile 2 k + tid / 128, float4s f and f + 64 with
                    // f = (tile * 4 + 2 ((tid / 64) % 2)) * 64 + tid % 64
                    const bool hb2 = tid >= 128;
                    const float dk[4] = {hb2 ? hd0.y : hd0.x, hb2 ? hd0.w : hd0.z, hb2 ? hd1.y : hd1.x,
                                         hb2 ? hd1.w : hd1.z};
#pragma unroll
                    for (int k = 0; k < NHP / 2; ++k) {
                        const int f = ((2 * k + (tid >> 7)) * 4 + 2 * ((tid >> 6) & 1)) * 64 + (tid & 63);
                        float4 lo, hi;
                        q16_values(hq[k], dk[k], lo, hi);
                        put_h(f, lo);
                        put_h(f + 64, hi);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < NHP; ++k) put_h(tid + 256 * k, hr[k]);
                }
                if (wave == 0) {
                    gam[bf][2 * lane] = ga0;
                    gam[bf][2 * lane + 1] = ga1;
                    dts[bf][2 * lane] = dr0;
                    dts[bf][2 * lane + 1] = dr1;
                    din[bf][2 * lane] = expc(ga0);
                    din[bf][2 * lane + 1] = expc(ga1);
                    rowf[bf][2 * lane] = rf0;
                    rowf[bf][2 * lane + 1] = rf1;
                    *reinterpret_cast<float4*>(colf[bf] + 16 * lane) = float4{cf0[0], cf0[1], cf0[2], cf0[3]};
                    *reinterpret_cast<float4*>(colf[bf] + 16 * lane + 4) = float4{cf0[4], cf0[5], cf0[6], cf0[7]};
                    *reinterpret_cast<float4*>(colf[bf] + 16 * lane + 8) = float4{cf1[0], cf1[1], cf1[2], cf1[3]};
                    *reinterpret_cast<float4*>(colf[bf] + 16 * lane + 12) = float4{cf1[4], cf1[5], cf1[6], cf1[7]};
                }
            };

            uint4 graw[NPASS][RW];
            g_load(graw);
            prefetch(grp * hpg + j0);
            __syncthreads();   // LDS tables
#pragma unroll
            for (int ps = 0; ps < NPASS; ++ps) {
                if (ps > 0) __syncthreads();   // the previous slice's products are done
                g_conv(ps, graw[ps]);
                __syncthreads();
            }
            stage(0, j0);   // (buffer 0: no G slice there, and the G-phase weights are read)
            if (j0 + 1 < j1) prefetch(grp * hpg + j0 + 1);
            __syncthreads();
            for (int j = j0; j < j1; ++j) {
                if (j + 1 < j1) {
                    stage((j - j0 + 1) & 1, j + 1);
                    if (j + 2 < j1) prefetch(grp * hpg + j + 2);
                }
                __syncthreads();
            }
        } else {
            // ---------------------------------------------------------- consumers
            auto consumer = [&](auto TAc) __attribute__((always_inline)) {
                constexpr int TA = decltype(TAc)::value;
                constexpr int TB = 7 - TA;
                // this lane's output rows.  Tiles past a short chunk's end are
                // multiplied all the same (their rows are finite: B and C rows are
                // clamped into the sequence, x rows and dt are 0 there) and not
                // stored: the products stay free of branches.
                const int tA = 16 * TA + l16, tB = 16 * TB + l16;
                // C operands of the two tiles (column t, K = n), kept for every head
                bf16x8_t chA[NKB], clA[NKB], chB[NKB], clB[NKB];
                // G^T[i, t] = B_i . C_t for the i tiles it <= T of each tile
                f32x4_t gtA[TA + 1], gtB[TB + 1];
#pragma unroll
                for (int it = 0; it <= TA; ++it) gtA[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int it = 0; it <= TB; ++it) gtB[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};

                {
                    uint4 graw[NPASS][RW];
                    g_load(graw);
                    __syncthreads();   // LDS tables
#pragma unroll
                    for (int ps = 0; ps < NPASS; ++ps) {
                        if (ps > 0) __syncthreads();
                        g_conv(ps, graw[ps]);
                        __syncthreads();
#pragma unroll
                        for (int k2 = 0; k2 < 2; ++k2) {
                            const int k = 2 * ps + k2;
                            chA[k] = as_bf16x8(lds128(Ch + tA * HR + 32 * k2 + 8 * q));
                            clA[k] = as_bf16x8(lds128(Cl + tA * HR + 32 * k2 + 8 * q));
                            chB[k] = as_bf16x8(lds128(Ch + tB * HR + 32 * k2 + 8 * q));
                            clB[k] = as_bf16x8(lds128(Cl + tB * HR + 32 * k2 + 8 * q));
#pragma unroll
                            for (int it = 0; it <= TB; ++it) {
                                const int row = (16 * it + l16) * HR + 32 * k2 + 8 * q;
                                const bf16x8_t bh = as_bf16x8(lds128(Bh + row));
                                const bf16x8_t bl = as_bf16x8(lds128(Bl + row));
                                mma2<true, true>(gtB[it], bh, bl, chB[k], clB[k]);
                                if (it <= TA) mma2<true, true>(gtA[it], bh, bl, chA[k], clA[k]);
                            }
                        }
                    }
                }
                __syncthreads();   // the first head is staged

                for (int j = j0; j < j1; ++j) {
                    const int bf = (j - j0) & 1;
                    const int head = grp * hpg + j;
                    const float Dh = sD[j];
                    const u16* Xh = smem + bf * HBUF;
                    const u16* Xl = Xh + P * RS;
                    const u16* HH = Xh + HX;
                    const u16* HL = HH + P * NRS;
                    const float* rowfb = rowf[bf];
                    const float* dtsb = dts[bf];
                    const double* gamb = gam[bf];
                    // y^T[p, t] tiles: lane has t, p = 16 pt + 4q + r
                    f32x4_t yA[4], yB[4];
#pragma unroll
                    for (int pt = 0; pt < 4; ++pt) {
                        yA[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                        yB[pt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    }
                    // inter-chunk term: h_in C^T (A = h_in rows p, B = C columns t, K = n)
#pragma unroll
                    for (int k = 0; k < NKB; ++k) {
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt) {
                            const bf16x8_t ah = as_bf16x8(lds128(HH + (16 * pt + l16) * NRS + 32 * k + 8 * q));
                            const bf16x8_t al = as_bf16x8(lds128(HL + (16 * pt + l16) * NRS + 32 * k + 8 * q));
                            mma2<true, true>(yA[pt], ah, al, chA[k], clA[k]);
                            mma2<true, true>(yB[pt], ah, al, chB[k], clB[k]);
                        }
                    }
                    {
                        const float sa = din[bf][tA], sb = din[bf][tB];
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt) {
                            yA[pt] *= sa;
                            yB[pt] *= sb;
                        }
                    }
                    // intra-chunk term: X^T M^T over i tile pairs (2kb, 2kb+1); the M^T
                    // operand slot s < 4 is row 4q + s of tile 2kb, s >= 4 row 4q + s - 4
                    // of tile 2kb + 1 (the rows this lane's accumulators hold); the x^T
                    // planes hold the rows in that order (8 per (kb, q) group).
                    float cfA[8], cfB[8];
                    {
                        const float4* ca = reinterpret_cast<const float4*>(colf[bf] + 8 * tA);
                        const float4* cb = reinterpret_cast<const float4*>(colf[bf] + 8 * tB);
                        const float4 a0 = ca[0], a1 = ca[1], b0 = cb[0], b1 = cb[1];
                        cfA[0] = a0.x; cfA[1] = a0.y; cfA[2] = a0.z; cfA[3] = a0.w;
                        cfA[4] = a1.x; cfA[5] = a1.y; cfA[6] = a1.z; cfA[7] = a1.w;
                        cfB[0] = b0.x; cfB[1] = b0.y; cfB[2] = b0.z; cfB[3] = b0.w;
                        cfB[4] = b1.x; cfB[5] = b1.y; cfB[6] = b1.z; cfB[7] = b1.w;
                    }
                    // M^T slots of tile TT (column t) for i tiles 2kb, 2kb + 1
                    auto mslots = [&](auto TTc, int kb, const f32x4_t* gT, const float (&cfv)[8], int t,
                                      bf16x8_t& mh, bf16x8_t& ml) __attribute__((always_inline)) {
                        constexpr int TT = decltype(TTc)::value;
                        float m[8];
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const int it = 2 * kb + h2;
                            const int i0 = 16 * it + 4 * q;
                            if (it < TT) {
                                const float4 rf = *reinterpret_cast<const float4*>(rowfb + i0);
                                const float cv = cfv[it];
                                m[4 * h2 + 0] = gT[it][0] * rf.x * cv;
                                m[4 * h2 + 1] = gT[it][1] * rf.y * cv;
                                m[4 * h2 + 2] = gT[it][2] * rf.z * cv;
                                m[4 * h2 + 3] = gT[it][3] * rf.w * cv;
                            } else if (it == TT) {
                                // the diagonal tile, branch-free: for i > t the clamped
                                // exponent gives a finite factor that the select drops
                                const double gt = gamb[t];
                                const float4 d4 = *reinterpret_cast<const float4*>(dtsb + i0);
                                const double2 ga = *reinterpret_cast<const double2*>(gamb + i0);
                                const double2 gb = *reinterpret_cast<const double2*>(gamb + i0 + 2);
                                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
                                const double gv[4] = {ga.x, ga.y, gb.x, gb.y};
#pragma unroll
                                for (int r = 0; r < 4; ++r) {
                                    const int i = i0 + r;
                                    float v = gT[it][r] * dv[r] * expc(gt - gv[r]);
                                    v = (i == t) ? v + Dh : v;
                                    m[4 * h2 + r] = (i <= t) ? v : 0.f;
                                }
                            } else {
#pragma unroll
                                for (int r = 0; r < 4; ++r) m[4 * h2 + r] = 0.f;
                            }
                        }
                        uint4 mh4, ml4;
                        split8(m, mh4, ml4);
                        mh = as_bf16x8(mh4);
                        ml = as_bf16x8(ml4);
                    };
#pragma unroll
                    for (int kb = 0; kb <= TB / 2; ++kb) {
                        bf16x8_t mhB, mlB, mhA, mlA;
                        mslots(std::integral_constant<int, TB>{}, kb, gtB, cfB, tB, mhB, mlB);
                        if (kb <= TA / 2) mslots(std::integral_constant<int, TA>{}, kb, gtA, cfA, tA, mhA, mlA);
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt) {
                            const int xo = (16 * pt + l16) * RS + 32 * xsw(kb, 16 * pt) + 8 * q;
                            const bf16x8_t xh = as_bf16x8(lds128(Xh + xo));
                            const bf16x8_t xl = as_bf16x8(lds128(Xl + xo));
                            mma2<true, true>(yB[pt], xh, xl, mhB, mlB);
                            if (kb <= TA / 2) mma2<true, true>(yA[pt], xh, xl, mhA, mlA);
                        }
                    }
                    // store y rows tA, tB of the chunk: lane has y[t][16 pt + 4q .. +3]
                    if (tA < S) {
                        float* dst = a.y + (r0 + tA) * a.ld_y + (int64_t)head * P + 4 * q;
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt)
                            *reinterpret_cast<float4*>(dst + 16 * pt) =
                                float4{yA[pt][0], yA[pt][1], yA[pt][2], yA[pt][3]};
                    }
                    if (tB < S) {
                        float* dst = a.y + (r0 + tB) * a.ld_y + (int64_t)head * P + 4 * q;
#pragma unroll
                        for (int pt = 0; pt < 4; ++pt)
                            *reinterpret_cast<float4*>(dst + 16 * pt) =
                                float4{yB[pt][0], yB[pt][1], yB[pt][2], yB[pt][3]};
                    }
                    __syncthreads();
                }
            };
            switch (wave) {
                case 4: consumer(std::integral_constant<int, 0>{}); break;
                case 5: consumer(std::integral_constant<int, 1>{}); break;
                case 6: consumer(std::integral_constant<int, 2>{}); break;
                default: consumer(std::integral_constant<int, 3>{}); break;
            }
        }

        if (a.fuse_norm) {
            // The grouped gated RMSNorm of this chunk's rows over this group's
            // channels, wave w the rows w, w + 8, ..., read back while they are
            // still in cache.  (The norm's barrier sits inside chunk_norm_rows.)
            const int gs = hpg * P;
            const int nbl = (gs / 8 + 63) / 64;
            // (one block per lane: 16 rows per wave in flight, a chunk's 128 rows in
            // one batch, as the norm is bound by the rows it has in flight; wider
            // groups keep fewer rows for their registers: 6 rows at two blocks ran
            // slower than 4)
            if (a.out_dtype == kBF16) {
                if (nbl == 1) chunk_norm_rows<uint16_t, 1, 16>(a, r0, S, grp * gs, gs, wave, lane);
                else if (nbl == 2) chunk_norm_rows<uint16_t, 2, 4>(a, r0, S, grp * gs, gs, wave, lane);
                else chunk_norm_rows<uint16_t, 4, 2>(a, r0, S, grp * gs, gs, wave, lane);
            } else {
                if (nbl == 1) chunk_norm_rows<float, 1, 16>(a, r0, S, grp * gs, gs, wave, lane);
                else if (nbl == 2) chunk_norm_rows<float, 2, 4>(a, r0, S, grp * gs, gs, wave, lane);
                else chunk_norm_rows<float, 4, 2>(a, r0, S, grp * gs, gs, wave, lane);
            }
        }
    };
    if constexpr (N == 128) {
        if (S_ == Q && c > 0) body(std::integral_constant<int, Q>{});
        else body(std::integral_constant<int, 0>{});
    } else {
        body(std::integral_constant<int, 0>{});   // (at dstate 64 the second copy spilled)
    }
}

// ------------------------------------------------------------------ state pass, raw rows
//
// The state pass for raw bf16 rows at dstate 128, two heads of one group per
// workgroup, with the waves split by role.  The walk goes in units of half a
// chunk (64 rows).  Waves 0-3 (producers) convolve the next unit's x: waves 0-1
// the first head's, 2-3 the second's, each thread a piece of 4 rows x 8
// channels, weighted by the rows' w_i; at a chunk's first unit they also run
// the gamma scan of their head, the weights and the decay.  Waves 4-7
// (consumers) hold h^T of both heads in matrix-core accumulators, consumer w
// the n tile w of each head (both p tiles), so each B operand read serves four
// tiles; they convolve the next unit's B (16 row groups x 16 channel groups
// over their 256 threads) in the same stretch of code as the current unit's
// products, so the conv's vector work fills the gaps between matrix
// instructions, and at a chunk's start they store the entry state (Q16: as
// 16-bit rows, store_entry_q16; for split sequences fp32, which the segment
// carry reads) and scale by the decay.  Every SIMD then holds one producer and
// one consumer, both convolving.
template <int N, bool Q16>
__global__ __launch_bounds__(512) void ssd_state_pass_raw_kernel(ScanArgs a) {
    static_assert(N == 128, "two heads of 64 B channels each");
    constexpr int IPW = 2;
    constexpr int NCW = IPW * P + N;                   // conv channels of the workgroup
    __shared__ float4 sCW[NCW];                        // their conv weights (slots wsw)
    __shared__ __align__(16) float sCB[NCW];           // and biases (channel order)
    __shared__ __align__(16) u16 sBTh[2][N * RH];      // per unit buffer: B^T [n][row of the half], high parts
    __shared__ __align__(16) u16 sBTl[2][N * RH];      // low parts
    __shared__ __align__(16) u16 sXH[2][IPW][P * RH];  // (w x)^T [p][row] per head, high parts
    __shared__ __align__(16) u16 sXL[2][IPW][P * RH];  // low parts
    __shared__ __align__(16) float sW[4][Q];           // per producer wave: its head's weights w_i of the chunk
    __shared__ float sDecay[IPW];                      // e(gamma_S) of the chunk being started, per head

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int l32 = lane & 31, g32 = lane >> 5;
    // grid: one level of batch * nheads / 2 workgroups per segment index
    const int level = a.nheads * a.batch / IPW;
    const int seg_k = (int)blockIdx.x / level;
    int seq, head0;
    state_item((int)blockIdx.x % level, a, IPW, 0, seq, head0);
    const int hpg = a.nheads / a.ngroups;
    const int grp = head0 / hpg;
    const int64_t s0 = a.cu_seqlens[seq];
    const int64_t L = a.cu_seqlens[seq + 1] - s0;
    // segment seg_k of this sequence has no chunk
    if (seg_k > 0 && (int64_t)seg_k * a.seg * Q >= L) return;
    const int slot = a.state_idx ? a.state_idx[seq] : seq;
    const bool init = a.has_init ? (a.has_init[seq] != 0) : true;
    if (L <= 0) {
        // Empty sequence: a fresh slot is still reset, a carried one is untouched.
        if (!init) {
            for (int e = tid; e < IPW * P * N / 4; e += 512) {
                float* st = a.ssm_state + ((int64_t)slot * a.nheads + head0 + e / (P * N / 4)) * (int64_t)(P * N);
                *reinterpret_cast<float4*>(st + 4 * (e % (P * N / 4))) = float4{0.f, 0.f, 0.f, 0.f};
            }
        }
        return;
    }
    const int d_inner = a.nheads * P;
    for (int e = tid; e < NCW; e += 512) {
        const int ch = e < IPW * P ? (head0 + e / P) * P + e % P : d_inner + grp * N + (e - IPW * P);
        sCW[wsw(e)] = *reinterpret_cast<const float4*>(a.conv_w + (int64_t)ch * 4);
        sCB[e] = a.conv_b ? a.conv_b[ch] : 0.f;
    }

    const int nch = (int)((L + Q - 1) / Q);
    const int64_t cbase = s0 / Q + seq;   // entry-state slot of the sequence's first chunk
    // this workgroup's chunks: all of them, or segment seg_k's (a later segment
    // starts from zero; its first entry slot belongs to the segment before)
    // (the last level runs to the sequence's end)
    const int cfirst = seg_k * a.seg;
    const int cend = a.seg > 0 && seg_k < a.seg_levels - 1 ? (cfirst + a.seg < nch ? cfirst + a.seg : nch) : nch;

    // One raw piece (4 rows x 8 channels, rows 4 rg .. of half h) of chunk c,
    // refilled a chunk ahead; and its conv + SiLU into the unit's LDS planes,
    // times the rows' weights when wt is given (x) or not (B).  Only the
    // workgroup's first unit can hold a sequence's first row: the staging
    // calls after it pass first = false, which folds the carried-halo path
    // (its loads, its 24 registers and the window's selects) out of the loop.
    const int rg = (lane & 7) + 8 * (wave & 1);   // row group of both roles' pieces
    auto load_piece = [&](RawBuf& b, const uint16_t* col, int64_t ld, int c, int h) __attribute__((always_inline)) {
        c = c < cend ? c : cend - 1;
        load_raw_piece(col + (s0 + (int64_t)c * Q) * ld, (int)ld, h * QH + 4 * rg, (int)(-(int64_t)c * Q),
                       (int)(L - 1 - (int64_t)c * Q), (lane & 7) == 0, b.r);
    };
    auto conv_store = [&](RawBuf& b, int c, int h, int ch, int lw, const float* wt, u16* dh, u16* dl, int cg,
                          bool first) __attribute__((always_inline)) {
        const int row0 = QH * h + 4 * rg;                    // first row of the piece in the chunk
        const bool start = first && c == 0 && row0 == 0;    // the piece starts the sequence
        raw_halo(b.r, lane);
        float hv[3][8];
        if (start) load_halo(a.conv_state, a.conv_dim, slot, init, ch, hv);
        float wx[RR] = {1.f, 1.f, 1.f, 1.f};
        if (wt) {
            const float4 w4 = *reinterpret_cast<const float4*>(wt + row0);
            wx[0] = w4.x; wx[1] = w4.y; wx[2] = w4.z; wx[3] = w4.w;
        }
        const ConvW cw = read_convw(sCW, sCB, lw);
        float4 wv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) wv[k] = cw.w(k);
        float u[8][RR];
        conv_piece8(b.r, start, hv, wv, cw.b, u);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t wh[RR / 2], wl[RR / 2];
#pragma unroll
            for (int m = 0; m < RR / 2; ++m)
                split2(u[k][2 * m] * wx[2 * m], u[k][2 * m + 1] * wx[2 * m + 1], wh[m], wl[m]);
            store_tokens<RR>(dh + (8 * cg + k) * RH + 4 * rg, wh);
            store_tokens<RR>(dl + (8 * cg + k) * RH + 4 * rg, wl);
        }
    };

    if (wave < 4) {
        // ---------------------------------------------------------- producers
        const int hp = wave >> 1;              // the head of this wave's x pieces
        const int head = head0 + hp;
        const float Ah = a.A[head];
        const int xcg = lane >> 3;             // x channel group (8 channels)
        const uint16_t* xcol = static_cast<const uint16_t*>(a.x) + head * a.hs_x + 8 * xcg;
        const int xch = head * P + 8 * xcg, xlw = hp * P + 8 * xcg;   // first xBC channel, its weights in LDS
        RawBuf bx0, bx1;             // the pieces of each half
        float d0, d1;                // dt of the next chunk to start (rows 2 lane, 2 lane + 1)
        double lrun = 0.0;           // log decay from the segment's start
        auto load_dt = [&](int c) __attribute__((always_inline)) {
            c = c < cend ? c : cend - 1;
            const int64_t r0 = s0 + (int64_t)c * Q;
            const int S = (int)((L - (int64_t)c * Q) < Q ? (L - (int64_t)c * Q) : Q);
            d0 = a.dt[(r0 + (2 * lane < S ? 2 * lane : S - 1)) * a.ld_dt + head];
            d1 = a.dt[(r0 + (2 * lane + 1 < S ? 2 * lane + 1 : S - 1)) * a.ld_dt + head];
        };
        // a chunk's start: gamma of this wave's head, the weights w_i = dt_i
        // e(gamma_S - gamma_i) into this wave's table, the decay for the consumers
        auto start_chunk = [&](int c) __attribute__((always_inline)) {
            const int S = (int)((L - (int64_t)c * Q) < Q ? (L - (int64_t)c * Q) : Q);
            if (2 * lane >= S) d0 = 0.f;
            if (2 * lane + 1 >= S) d1 = 0.f;
            double g0, g1;
            gamma_scan(d0, d1, Ah, g0, g1);
            const double gS = ((S - 1) & 1) ? readlane_f64(g1, (S - 1) >> 1) : readlane_f64(g0, (S - 1) >> 1);
            // (read back by this wave's own lanes: its LDS operations complete in order)
            *reinterpret_cast<float2*>(&sW[wave][2 * lane]) = float2{d0 * expc(gS - g0), d1 * expc(gS - g1)};
            if ((wave & 1) == 0 && lane == 0) {
                sDecay[hp] = expc(gS);
                if (seg_k > 0 && c > cfirst) a.cum[(cbase + c) * a.nheads + head] = lrun;
            }
            lrun += gS;
            load_dt(c + 1);
        };
        auto stage_x = [&](RawBuf& b, int c, int h, bool first) __attribute__((always_inline)) {
            conv_store(b, c, h, xch, xlw, sW[wave], sXH[h][hp], sXL[h][hp], xcg, first);
        };

        load_dt(cfirst);
        __builtin_amdgcn_sched_barrier(0);
        load_piece(bx0, xcol, a.ld_x, cfirst, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_piece(bx1, xcol, a.ld_x, cfirst, 1);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();   // conv weights
        start_chunk(cfirst);
        stage_x(bx0, cfirst, 0, true);
        load_piece(bx0, xcol, a.ld_x, cfirst + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();   // unit (cfirst, 0) staged
        for (int c = cfirst; c < cend; ++c) {
            stage_x(bx1, c, 1, false);
            load_piece(bx1, xcol, a.ld_x, c + 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();   // unit (c, 0) multiplied, (c, 1) staged
            if (c + 1 < cend) {
                start_chunk(c + 1);
                stage_x(bx0, c + 1, 0, false);
                load_piece(bx0, xcol, a.ld_x, c + 2, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();   // unit (c, 1) multiplied, (c + 1, 0) staged
        }
        if (seg_k > 0 && (wave & 1) == 0 && lane == 0) a.lam[(cbase + cfirst) * a.nheads + head] = lrun;
    } else {
        // ---------------------------------------------------------- consumers
        const int cw = wave - 4;   // n tile of both heads' states
        const int bcg = (lane >> 3) + 8 * (cw >> 1);   // B channel group (of 16) of this thread's pieces
        const uint16_t* bcol = static_cast<const uint16_t*>(a.B) + grp * a.gs_B + 8 * bcg;
        const int bch = d_inner + grp * N + 8 * bcg, blw = IPW * P + 8 * bcg;
        RawBuf bb0, bb1;
        auto stage_b = [&](RawBuf& b, int c, int h, bool first) __attribute__((always_inline)) {
            conv_store(b, c, h, bch, blw, nullptr, sBTh[h], sBTl[h], bcg, first);
        };
        // acc[hh][pt]: head hh, p tile pt; lane l has p = 32 pt + l % 32 and, in
        // registers 4m .. 4m + 3, n = 32 cw + 8m + 4 (l / 32) + 0..3
        f32x16_t acc[IPW][2];
        auto soff = [&](int pt, int m) { return (32 * pt + l32) * N + 32 * cw + 8 * m + 4 * g32; };
        // entry states in accumulator order: float4 ((tile * 4 + m) * 64 + lane), tile = 2 cw + pt
        auto eoff = [&](int pt, int m) { return 4 * (((2 * cw + pt) * 4 + m) * 64 + lane); };
        load_piece(bb0, bcol, a.ld_B, cfirst, 0);
        __builtin_amdgcn_sched_barrier(0);
        load_piece(bb1, bcol, a.ld_B, cfirst, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hh = 0; hh < IPW; ++hh) {
            const float* st = a.ssm_state + ((int64_t)slot * a.nheads + head0 + hh) * (int64_t)(P * N);
#pragma unroll
            for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float4 v = float4{0.f, 0.f, 0.f, 0.f};
                    if (init && seg_k == 0) v = *reinterpret_cast<const float4*>(st + soff(pt, m));
                    acc[hh][pt][4 * m + 0] = v.x; acc[hh][pt][4 * m + 1] = v.y;
                    acc[hh][pt][4 * m + 2] = v.z; acc[hh][pt][4 * m + 3] = v.w;
                }
        }
        // h^T += B^T (w x) over the 16-row K blocks of a staged half.  Rows past
        // the sequence's end have weight 0 (their (w x) is 0) and finite B
        // rows, so every block is multiplied: no branch splits the products
        // from the conv beside them.
        auto multiply = [&](int h) __attribute__((always_inline)) {
#pragma unroll
            for (int k = 0; k < QH / 16; ++k) {
                const int bo = (32 * cw + l32) * RH + 16 * k + 8 * g32;
                const bf16x8_t bh = as_bf16x8(lds128(sBTh[h] + bo));
                const bf16x8_t bl = as_bf16x8(lds128(sBTl[h] + bo));
#pragma unroll
                for (int hh = 0; hh < IPW; ++hh)
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt) {
                        const int xo = (32 * pt + l32) * RH + 16 * k + 8 * g32;
                        const bf16x8_t xh = as_bf16x8(lds128(sXH[h][hh] + xo));
                        const bf16x8_t xl = as_bf16x8(lds128(sXL[h][hh] + xo));
                        mma32<true, true>(acc[hh][pt], bh, bl, xh, xl);
                    }
            }
        };
        __syncthreads();   // conv weights
        stage_b(bb0, cfirst, 0, true);
        load_piece(bb0, bcol, a.ld_B, cfirst + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();   // unit (cfirst, 0) staged
        for (int c = cfirst; c < cend; ++c) {
            // entry state of this chunk, then h <- e(gamma_S) h
            const bool store = seg_k == 0 || c > cfirst;
#pragma unroll
            for (int hh = 0; hh < IPW; ++hh) {
                float* he = a.states + ((cbase + c) * a.nheads + head0 + hh) * (int64_t)(P * N);
                const float decay = sDecay[hh];
                if constexpr (Q16) {
                    if (store) store_entry_q16(he, acc[hh], cw, lane);
                }
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    if (!Q16 && store) {
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            *reinterpret_cast<float4*>(he + eoff(pt, m)) =
                                float4{acc[hh][pt][4 * m], acc[hh][pt][4 * m + 1], acc[hh][pt][4 * m + 2],
                                       acc[hh][pt][4 * m + 3]};
                    }
                    acc[hh][pt] *= decay;
                }
            }
            // unit (c, 0): its products beside the conv of (c, 1)'s B
            multiply(0);
            stage_b(bb1, c, 1, false);
            load_piece(bb1, bcol, a.ld_B, c + 1, 1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
            // unit (c, 1): its products beside the conv of (c + 1, 0)'s B
            multiply(1);
            if (c + 1 < cend) {
                stage_b(bb0, c + 1, 0, false);
                load_piece(bb0, bcol, a.ld_B, c + 2, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            __syncthreads();
        }
        // The end state: the sequence's final state when this is its only segment;
        // otherwise a local end state, left in the next segment's first entry slot
        // (for segment 0 that is already the true entry state there) or, for the
        // last segment, in seg_end, for the carry kernel to complete.
#pragma unroll
        for (int hh = 0; hh < IPW; ++hh) {
            const int head = head0 + hh;
            if (cend == nch && seg_k == 0) {
                float* st = a.ssm_state + ((int64_t)slot * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        *reinterpret_cast<float4*>(st + soff(pt, m)) =
                            float4{acc[hh][pt][4 * m], acc[hh][pt][4 * m + 1], acc[hh][pt][4 * m + 2],
                                   acc[hh][pt][4 * m + 3]};
            } else {
                float* he = cend < nch ? a.states + ((cbase + cend) * a.nheads + head) * (int64_t)(P * N)
                                       : a.seg_end + ((int64_t)seq * a.nheads + head) * (int64_t)(P * N);
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        *reinterpret_cast<float4*>(he + eoff(pt, m)) =
                            float4{acc[hh][pt][4 * m], acc[hh][pt][4 * m + 1], acc[hh][pt][4 * m + 2],
                                   acc[hh][pt][4 * m + 3]};
            }
        }
    }
}

template <int N, typename Tin>
hipError_t launch_pass(const ScanArgs& a, hipStream_t stream) {
    const unsigned levels = a.seg > 0 ? (unsigned)a.seg_levels : 1u;
    if constexpr (N == 128) {
        if ((a.nheads / a.ngroups) % 2 == 0) {
            if constexpr (is_raw<Tin>()) {
                // 16-bit entry states unless sequences are split into segments
                // (the segment carry joins fp32 states)
                if (a.seg == 0)
                    hipLaunchKernelGGL((ssd_state_pass_raw_kernel<N, true>), dim3(a.nheads * a.batch / 2 * levels),
                                       dim3(512), 0, stream, a);
                else
                    hipLaunchKernelGGL((ssd_state_pass_raw_kernel<N, false>), dim3(a.nheads * a.batch / 2 * levels),
                                       dim3(512), 0, stream, a);
            }
            else
                hipLaunchKernelGGL((ssd_state_pass_kernel<N, 2, Tin>), dim3(a.nheads * a.batch / 2 * levels),
                                   dim3(512), 0, stream, a);
            return hipGetLastError();
        }
    }
    if constexpr (is_raw<Tin>() && N == 128) {
        return hipErrorInvalidValue;   // raw pieces at dstate 128 need two heads per workgroup
    } else {
        hipLaunchKernelGGL((ssd_state_pass_kernel<N, 1, Tin>), dim3(a.nheads * a.batch * levels), dim3(256), 0,
                           stream, a);
        return hipGetLastError();
    }
}

template <int N>
hipError_t launch_carry(const ScanArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(segment_carry_kernel<N>, dim3(a.nheads * a.batch), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int N, typename Tin>
hipError_t launch_out(const ScanArgs& a, int64_t total_tokens, hipStream_t stream) {
    const int64_t slots = total_tokens / Q + a.batch;
    const int split = a.out_split > 1 ? a.out_split : 1;
    const dim3 grid((unsigned)(slots * a.ngroups * split));
    if constexpr (is_raw<Tin>()) {
        // the entry-state format the raw state pass wrote: 16-bit at dstate 128
        // unless sequences are split into segments
        if (N == 128 && a.seg == 0)
            hipLaunchKernelGGL((ssd_chunk_out_raw_kernel<N, N == 128>), grid, dim3(512), 0, stream, a);
        else
            hipLaunchKernelGGL((ssd_chunk_out_raw_kernel<N, false>), grid, dim3(512), 0, stream, a);
    }
    else
        hipLaunchKernelGGL((ssd_chunk_out_kernel<N, Tin>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

bool chunked_scan_supported(int policy, int nheads, int ngroups, int headdim, int dstate, int chunk) {
    return policy == kPolicyBf16x3 && headdim == P && (dstate == 64 || dstate == 128) && chunk == Q &&
           ngroups > 0 && nheads % ngroups == 0 && nheads / ngroups <= MAXHPG;
}

bool chunked_raw_supported(int nheads, int ngroups, int headdim, int dstate, int chunk) {
    if (!chunked_scan_supported(kPolicyBf16x3, nheads, ngroups, headdim, dstate, chunk)) return false;
    return dstate == 64 || (dstate == 128 && (nheads / ngroups) % 2 == 0);
}

static size_t r256(size_t v) { return (v + 255) / 256 * 256; }

static size_t entry_states_bytes(int64_t total_tokens, int batch, int nheads, int headdim, int dstate) {
    return r256((size_t)(total_tokens / Q + batch) * (size_t)nheads * (size_t)headdim * (size_t)dstate *
                sizeof(float));
}

// Splitting sequences into segments: only when the (sequence, head) walks fill
// fewer than SEG_TARGET state-pass workgroups (one per CU), into segments of at
// least SEG_MIN chunks.  Then batch * nheads < 2 * SEG_TARGET, which bounds the
// end states the last segments leave for the carry kernel.  At one workgroup
// per CU already (8 x 4096 tokens, 64 heads), splitting in two cost more in the
// chunk output's extra entry-state reads (0.40 -> 0.45 ms) than it saved.
constexpr int SEG_TARGET = 256;
constexpr int SEG_MIN = 4;
constexpr int SEG_END_MAX = 2 * SEG_TARGET;

static size_t seg_end_bytes(int batch, int nheads, int headdim, int dstate) {
    const int64_t n = (int64_t)batch * nheads < SEG_END_MAX ? (int64_t)batch * nheads : SEG_END_MAX;
    return r256((size_t)n * headdim * dstate * sizeof(float));
}

size_t chunked_scan_states_bytes(int64_t total_tokens, int batch, int nheads, int headdim, int dstate) {
    const size_t slots = (size_t)(total_tokens / Q + batch) * (size_t)nheads;
    return entry_states_bytes(total_tokens, batch, nheads, headdim, dstate) +
           r256((size_t)batch * sizeof(int32_t)) + seg_end_bytes(batch, nheads, headdim, dstate) +
           2 * r256(slots * sizeof(double));
}

ScanSplit chunked_scan_split(int64_t total_tokens, int batch, int nheads, int ngroups, int dstate, int max_seqlen) {
    ScanSplit sp{1, 0, 1};
    const int hpg = nheads / ngroups;
    // chunk output: fewer (chunk, group) workgroups than CUs split the group's
    // heads over up to hpg workgroups (a 137-token prompt has 16 such pairs)
    {
        const int64_t wgs = (total_tokens / Q + batch) * (int64_t)ngroups;
        int split = 1;
        while (hpg % (2 * split) == 0 && wgs * 2 * split <= 256) split *= 2;
        sp.out_split = split;
    }
    const int ipw = (dstate == 128 && hpg % 2 == 0) ? 2 : 1;
    const int64_t level = (int64_t)nheads * batch / ipw;
    const int nch = (int)(((int64_t)max_seqlen + Q - 1) / Q);
    if (level >= SEG_TARGET || (int64_t)batch * nheads > SEG_END_MAX) return sp;
    int nseg = (int)((SEG_TARGET + level - 1) / level);
    if (nseg > nch / SEG_MIN) nseg = nch / SEG_MIN;
    if (nseg < 2) return sp;
    sp.seg = (nch + nseg - 1) / nseg;
    sp.seg_levels = (nch + sp.seg - 1) / sp.seg;
    return sp;
}

void chunked_scan_plan(ScanArgs& a, int64_t total_tokens, int max_seqlen) {
    const ScanSplit sp = chunked_scan_split(total_tokens, a.batch, a.nheads, a.ngroups, a.dstate, max_seqlen);
    a.out_split = sp.out_split;
    a.seg = sp.seg;
    a.seg_levels = sp.seg_levels;
    char* p = reinterpret_cast<char*>(a.order) + r256((size_t)a.batch * sizeof(int32_t));
    a.seg_end = reinterpret_cast<float*>(p);
    p += seg_end_bytes(a.batch, a.nheads, a.headdim, a.dstate);
    const size_t slots = (size_t)(total_tokens / Q + a.batch) * (size_t)a.nheads;
    a.lam = reinterpret_cast<double*>(p);
    a.cum = reinterpret_cast<double*>(p + r256(slots * sizeof(double)));
}

int32_t* chunked_scan_order(float* states, int64_t total_tokens, int batch, int nheads, int headdim,
                            int dstate) {
    return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(states) +
                                      entry_states_bytes(total_tokens, batch, nheads, headdim, dstate));
}

hipError_t launch_ssd_state_pass(const ScanArgs& a, hipStream_t stream) {
    if (a.order) {
        hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((a.batch + ORD_NT - 1) / ORD_NT)), dim3(ORD_NT), 0,
                           stream, a.cu_seqlens, a.batch, a.order);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const bool f = a.act_dtype == kF32;
    hipError_t e = hipErrorInvalidValue;
    if (a.raw_conv) {
        // (launch_pass picks two heads per workgroup for dstate 128, which the
        // raw pieces need; chunked_raw_supported admits only those shapes)
        if (a.dstate == 128) e = launch_pass<128, RawBf16>(a, stream);
        if (a.dstate == 64) e = launch_pass<64, RawBf16>(a, stream);
    } else {
        if (a.dstate == 128) e = f ? launch_pass<128, float>(a, stream) : launch_pass<128, u16>(a, stream);
        if (a.dstate == 64) e = f ? launch_pass<64, float>(a, stream) : launch_pass<64, u16>(a, stream);
    }
    if (e != hipSuccess || a.seg == 0) return e;
    return a.dstate == 128 ? launch_carry<128>(a, stream) : launch_carry<64>(a, stream);
}

hipError_t launch_ssd_chunk_out(const ScanArgs& a, int64_t total_tokens, hipStream_t stream) {
    if (a.raw_conv) {
        if (a.dstate == 128) return launch_out<128, RawBf16>(a, total_tokens, stream);
        if (a.dstate == 64) return launch_out<64, RawBf16>(a, total_tokens, stream);
        return hipErrorInvalidValue;
    }
    const bool f = a.act_dtype == kF32;
    if (a.dstate == 128) return f ? launch_out<128, float>(a, total_tokens, stream) : launch_out<128, u16>(a, total_tokens, stream);
    if (a.dstate == 64) return f ? launch_out<64, float>(a, total_tokens, stream) : launch_out<64, u16>(a, total_tokens, stream);
    return hipErrorInvalidValue;
}

}  // namespace m2
