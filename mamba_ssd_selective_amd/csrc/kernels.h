// Internal host-side interface between the C ABI layer (m2ssd_api.cpp) and the
// kernel translation units.  Argument validation happens in the API layer; the
// launchers assume valid, supported arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m2 {

// Element types; kF64 is internal (the fp32 path's post-conv workspace).
enum DType : int { kF32 = 0, kBF16 = 1, kF64 = 2 };

// Matrix-core arithmetic of the scan: fp64 products (fp32 inputs), or bf16
// products on a (high, low) split of each fp32 operand (bf16 inputs).
enum Policy : int { kPolicyF64 = 0, kPolicyBf16x3 = 1 };

struct ConvArgs {
    const void* seg_ptr[3];     // x, B, C segments
    int64_t seg_ld[3];          // row strides (elements)
    int seg_ch[3];              // channels per segment
    int nseg;
    int act_dtype;
    const float* conv_w;        // [conv_dim, 4]
    const float* conv_b;        // [conv_dim] or null
    int conv_dim;
    float* conv_state;          // [n_slots, 3, conv_dim]
    const int32_t* cu_seqlens;  // [batch+1]
    int batch;
    int64_t total_tokens;
    const int32_t* state_idx;   // [batch] or null
    const uint8_t* has_init;    // [batch] or null
    int apply_silu;
    // Output: channel c of segment s (c counted within the segment) in row t is
    // element (c / out_bw[s]) * out_bs[s] + t * out_ld[s] + c % out_bw[s] of
    // out_ptr[s].  Row-major output: out_bw = the segment's channels, out_bs = 0;
    // the prefill's blocked layout: one block per head (x) or group (B, C).
    void* out_ptr[3];
    int64_t out_ld[3];
    int64_t out_bs[3];
    int out_bw[3];
    int out_dtype;
};

struct ScanArgs {
    // x[t, head, p] = x + t * ld_x + head * hs_x + p; B[t, g, n] = B + t * ld_B + g * gs_B + n
    // (row-major: hs_x = headdim, gs_B = gs_C = dstate)
    const void* x; int64_t ld_x; int64_t hs_x;
    const void* B; int64_t ld_B; int64_t gs_B;
    const void* C; int64_t ld_C; int64_t gs_C;
    int act_dtype;              // storage type of x, B, C
    int policy;                 // Policy
    const float* dt; int64_t ld_dt;
    const float* A;
    const float* D;             // or null
    float* ssm_state;           // [n_slots, H, P, N]
    const int32_t* cu_seqlens;
    int batch;
    const int32_t* state_idx;
    const uint8_t* has_init;
    int nheads, headdim, dstate, ngroups, chunk;
    float* y; int64_t ld_y;
    float* states;              // chunk-parallel path: entry state of every chunk
    int32_t* order;             // chunk-parallel path: sequences by length, longest first [batch]
    // Chunk-parallel path, long sequences split into segments of `seg` chunks
    // (0 = not split): segment k >= 1 of a sequence starts from a zero state.
    int seg;
    int seg_levels;             // segments of the longest sequence (state-pass grid levels)
    double* lam;                // per (first chunk slot of a segment, head): its total log decay
    double* cum;                // per (chunk slot, head): log decay from its segment's start
    float* seg_end;             // [batch * nheads] local end states of last segments
    int out_split;              // chunk output: workgroups per (chunk, group), each a run of heads
    // Chunk-parallel path, raw_conv set: x, B, C are the raw (pre-conv) bf16
    // xBC rows and both scan kernels compute the conv (width 4) + SiLU
    // themselves, reading the 3 rows before a sequence's first row from
    // conv_state (zeros when has_init is 0).  conv_w [conv_dim, 4], conv_b
    // [conv_dim] or null; x channel (h, p) is xBC channel h*headdim + p, B
    // channel (g, n) is d_inner + g*dstate + n, C channel (g, n) is
    // d_inner + ngroups*dstate + g*dstate + n.  conv_state is only read.
    int raw_conv;
    const float* conv_w;
    const float* conv_b;
    const float* conv_state;
    int conv_dim;
    // Raw chunk output, fuse_norm set (out_split 1): after its heads, each
    // workgroup applies the grouped gated RMSNorm (norm group = its SSM group)
    // to its chunk's rows of y, with z (bf16, rows of ld_z), norm_w, eps and
    // the gate order, writing norm_out (out_dtype; rows of ld_out, may be y
    // itself for fp32).  The group width (heads per group x headdim) is at
    // most 2048 and every row 16-byte aligned.
    int fuse_norm;
    const void* z; int64_t ld_z;
    const float* norm_w;
    float eps;
    int norm_before_gate;
    void* norm_out; int64_t ld_out; int out_dtype;
    // One-pass fp64 path, few long sequences split into segments of `seg` steps
    // (seg_levels of them at most; lam holds each segment's total log decay):
    // per (segment, sequence, head) the local end state, then the true one
    // after the carry, P x N fp64 each.
    double* seg_state;
};

struct NormArgs {
    const float* y; int64_t ld_y;
    const void* z; int64_t ld_z; int z_dtype;
    const float* norm_w;
    float eps;
    int ngroups;
    int norm_before_gate;
    int64_t total_tokens;
    int d_inner;
    void* out; int64_t ld_out; int out_dtype;
};

struct DecodeArgs {
    // One row per sequence: x [batch, nheads*headdim], B and C [batch, ngroups*dstate],
    // z [batch, nheads*headdim] (act_dtype), dt [batch, nheads]: fp32 step sizes,
    // or with dt_softplus set raw values of act_dtype that give
    // dt = softplus(raw + dt_bias[h]) (dt_bias null = 0).
    const void* x; int64_t ld_x;
    const void* B; int64_t ld_B;
    const void* C; int64_t ld_C;
    const void* z; int64_t ld_z;
    int act_dtype;
    const void* dt; int64_t ld_dt;
    int dt_softplus;
    const float* dt_bias;
    const float* A;
    const float* D;             // or null
    const float* conv_w;        // [conv_dim, 4]
    const float* conv_b;        // or null
    const float* norm_w;        // [nheads*headdim]
    float eps;
    int norm_before_gate;
    float* conv_state;          // [n_slots, 3, conv_dim]
    float* ssm_state;           // [n_slots, H, P, N]
    int batch;
    const int32_t* state_idx;   // or null
    const uint8_t* has_init;    // or null
    int nheads, headdim, dstate, ngroups;
    void* y; int64_t ld_y; int y_dtype;
    int split;                  // set by the launcher: workgroups per (sequence, group)
};

// Each launcher enqueues its kernel(s) on `stream` and returns the launch status.
hipError_t launch_conv_rows(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_state_update(const ConvArgs& a, hipStream_t stream);
hipError_t launch_ssd_scan(const ScanArgs& a, hipStream_t stream);
hipError_t launch_gated_norm(const NormArgs& a, hipStream_t stream);

// Single-token decode step (decode_step.hip): one fused kernel, one workgroup
// per (sequence, group).
bool decode_supported(int nheads, int ngroups, int headdim, int dstate);
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t stream);

// Packed in-projection rows (inproj.hip): dt [T, nheads] fp32 = softplus(raw +
// bias[h]) from the raw column run of each row (bias null = 0); and the row
// offsets (and, with slot_out, the identity slot map) of sequences first ..
// first+count of a batch whose first `first` sequences are one row each.
hipError_t launch_step_size(const void* raw, int64_t ld_raw, int act_dtype, const float* bias,
                            int nheads, int64_t total_tokens, float* dt, hipStream_t stream);
hipError_t launch_rebase(const int32_t* cu, int first, int count, int32_t rows, int32_t* out,
                         int32_t* slot_out, hipStream_t stream);

// True when a scan kernel is compiled for this (headdim, dstate).
bool scan_supported(int headdim, int dstate);
// One-pass fp64 path (ssd_scan.hip): workspace bytes for splitting few long
// sequences into segments (0 when the policy or the item count never splits),
// and the split itself: sets a.seg, a.seg_levels, a.seg_state and a.lam from
// the longest sequence, with ws (at least one_pass_seg_bytes) behind them; no
// split without ws.
size_t one_pass_seg_bytes(int batch, int nheads, int headdim, int dstate, int policy);
void one_pass_plan(ScanArgs& a, int max_seqlen, void* ws);

// Chunk-parallel scan (ssd_chunked.hip) for PolicyBf16x3 (x/B/C stored as bf16
// or fp32), headdim 64, dstate 64 or 128, chunk 128, at most 256 heads per group.  The state pass writes the entry state of every chunk to
// `states` ([total_tokens/128 + batch chunk slots, H] blocks of P x N fp32, each
// block in the state pass's accumulator order; sequence b's chunk c is slot
// cu_seqlens[b]/128 + b + c) and the final states; the chunk
// pass reads them and writes y.
// The workspace holds the entry states (256-byte rounded) and then the int32
// order of the sequences, longest first, that the state pass deals work in.
bool chunked_scan_supported(int policy, int nheads, int ngroups, int headdim, int dstate, int chunk);
// True when the chunk-parallel kernels also take raw bf16 xBC rows (raw_conv):
// dstate 64, or dstate 128 with an even number of heads per group.
bool chunked_raw_supported(int nheads, int ngroups, int headdim, int dstate, int chunk);
size_t chunked_scan_states_bytes(int64_t total_tokens, int batch, int nheads, int headdim, int dstate);
int32_t* chunked_scan_order(float* states, int64_t total_tokens, int batch, int nheads, int headdim,
                            int dstate);
// The chunk-parallel scan's split of the work (host only): chunk-output
// workgroups per (chunk, group), and the segments long sequences are split
// into when the (sequence, head) walks alone would leave CUs idle (seg chunks
// each, 0 = not split; seg_levels segments cover max_seqlen, the last level
// runs to a sequence's end).
struct ScanSplit {
    int out_split, seg, seg_levels;
};
ScanSplit chunked_scan_split(int64_t total_tokens, int batch, int nheads, int ngroups, int dstate, int max_seqlen);
// Sets out_split, seg, seg_levels (chunked_scan_split) and the buffers behind them.
void chunked_scan_plan(ScanArgs& a, int64_t total_tokens, int max_seqlen);
hipError_t launch_ssd_state_pass(const ScanArgs& a, hipStream_t stream);
hipError_t launch_ssd_chunk_out(const ScanArgs& a, int64_t total_tokens, hipStream_t stream);

}  // namespace m2
