/*
 * m2ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 mixer-core prefill library.
 *
 * The library runs the prefill hot path of one Mamba-2 (SSD) layer of a
 * Nemotron-H model on one GPU:
 *   1. causal depthwise conv1d (width 4) + SiLU over the carried conv state
 *      followed by the new rows ("add_short_conv_rows", page "perf(nemotron_h):
 *      prefill single-GPU prompts in multi-token chunks", section
 *      Implementation; "conv1d(xBC) -> SiLU", page "Nemotron-H", section 3);
 *   2. the chunked selective scan with no sequential step inside a chunk:
 *      a_t = dt_t * A_h, gamma = inclusive cumulative sum of a over the chunk,
 *      chunk total gamma_S = the LAST element of that sum, every exponent
 *      clamped at 0 (same page, section Implementation), with the recurrent
 *      state carried across chunks and across calls (page "Nemotron-H",
 *      section 4.1 "Mamba2 SSM layer" gives the token recurrence it equals);
 *   3. the grouped gated RMSNorm with z (page "Nemotron-H", section 4.1:
 *      GroupRMSNorm(y, ssm_norm.weight), then the SiLU(z) gate; the NemotronH
 *      decode page names the op RmsNormGatedGroup(n_groups));
 * and the single-token decode step of the same layer at cache slots
 * (mamba2_decode), which continues the states a prefill left; the same
 * operations taking packed in-projection rows with the raw step size
 * (mamba2_prefill_inproj, mamba2_decode_inproj), and batches mixing decode rows
 * and prefill sequences (mamba2_mixed_inproj).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is DEVICE memory owned by the caller, except where
 *   stated.  The library never frees or retains caller memory and performs no
 *   allocation on the hot path; scratch memory is the caller's `workspace`.
 * - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *   null stream).  A call returns after enqueueing.
 * - Matrices are row-major.  `ld_*` arguments are row strides in ELEMENTS; the
 *   inner (channel) stride is always 1.  Activations (x, B, C, z, xBC) are
 *   M2_F32 or M2_BF16 as given by `act_dtype` / `*_dtype`; dt, A, D, weights
 *   and both recurrent states are always fp32 (a state held in bf16 would be
 *   silently halved; the ABI rejects nothing else because it takes no state
 *   dtype argument).
 * - Varlen batches are packed: sequence b owns rows cu_seqlens[b] ..
 *   cu_seqlens[b+1]-1 of every token-indexed array.  cu_seqlens is int32
 *   [batch+1] in device memory, non-decreasing, cu_seqlens[0] == 0,
 *   cu_seqlens[batch] == total_tokens, and no sequence is longer than
 *   max_seqlen (a host value).  Empty sequences are allowed; with
 *   total_tokens == 0 the token-indexed arrays (x, B, C, z, dt, y, the
 *   in-projection rows) are not read and may be NULL, and the call only
 *   resets the states of fresh slots (has_init == 0).
 * - Recurrent states live in caller pools indexed by slot:
 *     conv_state [n_slots, width-1, conv_dim] fp32, row j = the raw xBC input
 *       that is (width-1-j) steps older than the next new row (oldest first);
 *     ssm_state  [n_slots, nheads, headdim, dstate] fp32 (dstate fastest).
 *   Sequence b uses slot state_idx[b] (int32 device array; NULL = slot b).
 *   Slots used in one call must be distinct.  has_init[b] (uint8 device
 *   array; NULL = all 1) == 0 makes sequence b start from zero states.
 *   States are ADVANCED IN PLACE: after the call slot state_idx[b] holds the
 *   state after the last row of sequence b.  If a call fails after launch
 *   (M2_ERR_HIP) the states are unspecified; callers that need retry keep a
 *   copy (the recurrent state cannot be rewound).
 * - Argument errors are detected on the host before any launch; the call then
 *   returns a negative status and has no side effects.  m2_last_error()
 *   returns a thread-local message for the last failing call on this thread.
 * - Device-side contents (cu_seqlens, state_idx, has_init, dt >= 0, A <= 0)
 *   are not read by the host; violating their contracts gives unspecified
 *   results but never out-of-bounds access for cu_seqlens within
 *   [0, total_tokens] and state_idx within [0, n_slots).
 * - Debug mode (environment variable M2SSD_DEBUG=1, read at every call): after
 *   the argument checks and before any launch, the call copies its device
 *   metadata to the host (synchronously) and returns M2_ERR_SHAPE, with no
 *   side effects, for: cu_seqlens not starting at 0 and ending at
 *   total_tokens, or a length outside [0, max_seqlen]; a state_idx entry
 *   outside [0, n_slots) or repeated; an A entry above 0 or not finite; and,
 *   where the entry takes the final step size (mamba2_prefill,
 *   ssd_chunk_scan, mamba2_decode), a dt entry below 0 or not finite.
 * - Results are deterministic: equal inputs give bitwise-equal outputs.
 */
#ifndef M2SSD_H
#define M2SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (negative on failure). */
#define M2_OK               0
#define M2_ERR_NULL        -1   /* a required pointer is NULL */
#define M2_ERR_SHAPE       -2   /* a dimension is non-positive or inconsistent */
#define M2_ERR_DTYPE       -3   /* dtype code not in {M2_F32, M2_BF16} */
#define M2_ERR_CHUNK       -4   /* chunk_size not a multiple of 16 in [16, 128] */
#define M2_ERR_STRIDE      -5   /* a row stride is smaller than the row width */
#define M2_ERR_ALIGN       -6   /* a pointer or stride breaks 16-byte row alignment */
#define M2_ERR_UNSUPPORTED -7   /* (headdim, dstate) or width has no compiled kernel */
#define M2_ERR_WORKSPACE   -8   /* workspace NULL or smaller than the query returned */
#define M2_ERR_HIP         -9   /* a HIP runtime call or kernel launch failed */

/* Activation / output element types. */
#define M2_F32   0
#define M2_BF16  1

/* Thread-local message describing the last failing call on this thread ("" if none). */
const char* m2_last_error(void);

/* Library version string (static storage). */
const char* m2_version(void);

/*
 * mamba2_conv_rows -- causal depthwise conv1d (+ optional SiLU) over the xBC
 * stream of a packed varlen batch, advancing the conv state in place.
 * (Page "perf(nemotron_h): prefill single-GPU prompts in multi-token chunks",
 * section Implementation: the short-conv rows of a chunk read the conv state
 * carried from earlier rows ahead of the chunk's own rows; page "Nemotron-H",
 * section 3 for the SiLU after conv1d(xBC) and section 10 for the width - 1
 * rows the conv state keeps per channel.)
 *
 * For sequence b of length L with padded stream xpad = [conv_state[slot] (width-1
 * rows, or zeros if has_init[b]==0) ; the L new rows]:
 *   out[t, c]  = act(conv_b[c] + sum_{k<width} conv_w[c, k] * xpad[t + k, c])
 *   new state  = the last width-1 rows of xpad (so for L < width-1 the old rows
 *                shift and are kept).
 * Weight column width-1 multiplies the current row.
 *
 * The conv_dim input channels come in three row-strided segments, in order:
 *   x [T, d_x] (ld_x), B [T, d_b] (ld_B), C [T, d_b] (ld_C), conv_dim = d_x + 2*d_b.
 * They may be views into one in-projection row (e.g. B == x + d_x, C == B + d_b).
 * Pass d_b = 0 (B, C ignored) to convolve a single segment of d_x channels.
 *
 *   act_dtype    element type of x, B, C (M2_F32 / M2_BF16)
 *   conv_w       [conv_dim, width] fp32;  conv_b [conv_dim] fp32 or NULL (0)
 *   width        must be 4
 *   conv_state   [n_slots, width-1, conv_dim] fp32, read and advanced in place
 *   apply_silu   nonzero: act = SiLU, zero: identity
 *   out          [T, conv_dim] with row stride ld_out, element type out_dtype;
 *                must not overlap the inputs or the state.
 * Alignment: every pointer 16-byte aligned; row strides times element size
 * multiples of 16 bytes; d_x and d_b multiples of 8.
 */
int mamba2_conv_rows(const void* x, int64_t ld_x, const void* B, int64_t ld_B,
                     const void* C, int64_t ld_C, int d_x, int d_b, int act_dtype,
                     const float* conv_w, const float* conv_b, int width,
                     float* conv_state, int n_slots,
                     const int32_t* cu_seqlens, int batch, int64_t total_tokens,
                     int max_seqlen, const int32_t* state_idx, const uint8_t* has_init,
                     int apply_silu, void* out, int64_t ld_out, int out_dtype,
                     void* stream);

/*
 * ssd_chunk_scan -- chunked selective scan (Mamba-2 SSD) of a packed varlen
 * batch, from post-conv x, B, C; writes the pre-norm output and advances the
 * SSM state in place.  (Page "perf(nemotron_h): prefill single-GPU prompts in
 * multi-token chunks", section Implementation: the SSD rows of a chunk with no
 * sequential step, a_t = dt_t * A, the in-chunk cumulative sum, the chunk total
 * read from its last element and every exponent clamped at 0; page
 * "Nemotron-H", section 4.1 for the token recurrence the chunk form equals.)
 *
 * Per sequence, per head h (group g = h / (nheads/ngroups)), in chunks of
 * chunk_size rows counted from the sequence's first row, with
 * a_t = dt[t,h] * A[h], gamma_t the inclusive cumulative sum of a over the
 * chunk, gamma_S its last element and e(v) = exp(min(v, 0)):
 *   y[t,h,:] = e(gamma_t) * C_t . h_in
 *              + sum_{i<=t} e(gamma_t - gamma_i) * (C_t . B_i) * dt_i * x_i
 *              + D[h] * x_t
 *   h_out    = e(gamma_S) * h_in + sum_i e(gamma_S - gamma_i) * dt_i * x_i (outer) B_i
 * which equals the token recurrence h <- exp(dt*A) h + dt x (outer) B,
 * y = h . C + D x up to rounding.
 *
 *   x   [T, nheads*headdim] (ld_x);  B, C [T, ngroups*dstate] (ld_B, ld_C);
 *       element type act_dtype.
 *   dt  [T, nheads] fp32 (ld_dt), the final step size (softplus and bias
 *       already applied), expected >= 0;  A [nheads] fp32, expected <= 0;
 *   D   [nheads] fp32 or NULL (0).
 *   ssm_state [n_slots, nheads, headdim, dstate] fp32, read and advanced in place.
 *   y   [T, nheads*headdim] fp32 (ld_y), must not overlap any input.
 *   chunk_size: multiple of 16 in [16, 128].
 *   workspace: device memory of at least ssd_chunk_scan_workspace_size()
 *     bytes, 16-byte aligned (NULL allowed when that size is 0); its contents
 *     on entry do not matter and are undefined on return.
 * Alignment: x, B, C, y, ssm_state 16-byte aligned; ld_x, ld_B, ld_C times
 * the element size and ld_y * 4 multiples of 16 bytes.
 * Supported (headdim, dstate): (16,16), (32,64), (64,64), (64,128).
 * Arithmetic:
 *   bf16 inputs, headdim 64, dstate 64 or 128, chunk_size 128 (chunk-parallel
 *     path): x, B, C enter bf16 matrix instructions as they are; the computed
 *     operands (dt-weighted x, the masked decay matrix, the carried state) are
 *     split into (high, low) bf16 pairs and enter two products; fp32
 *     accumulation.  The workspace holds the state entering every chunk.
 *   other bf16 shapes (one-pass path): every fp32 operand split into a (high,
 *     low) bf16 pair, three products per tile, fp32 accumulation; no workspace.
 *   fp32 inputs: computed in fp64 (fp64 matrix instructions, chunks evaluated
 *     64 rows at a time -- the same function of the inputs).  With fewer than
 *     256 (sequence, head) pairs, long sequences are split into segments that
 *     run in parallel from a zero state; a carry pass joins their end states
 *     (the recurrence is linear in its state) and adds the carried-in state's
 *     readout to the later segments' rows.  The workspace holds one fp64 state
 *     and one fp64 log decay per (segment, sequence, head).
 * Cumulative sums and exponent differences are fp64 on every path.
 */
int ssd_chunk_scan(const void* x, int64_t ld_x, const void* B, int64_t ld_B,
                   const void* C, int64_t ld_C, int act_dtype,
                   const float* dt, int64_t ld_dt, const float* A, const float* D,
                   float* ssm_state, int n_slots,
                   const int32_t* cu_seqlens, int batch, int64_t total_tokens,
                   int max_seqlen, const int32_t* state_idx, const uint8_t* has_init,
                   int nheads, int headdim, int dstate, int ngroups, int chunk_size,
                   float* y, int64_t ld_y, void* workspace, size_t ws_bytes, void* stream);

/*
 * Bytes of device workspace ssd_chunk_scan needs for these sizes (0 when the
 * shape runs on a path without workspace, or on bad arguments): on the
 * chunk-parallel path the state entering every chunk, (total_tokens/128 +
 * batch) * nheads * headdim * dstate * 4 bytes, then the order in which the
 * sequences' carries are dealt out (batch int32), then the buffers of long
 * sequences split into segments; for fp32 inputs with items = batch * nheads
 * below 256, ceil(256 / items) * items fp64 states of headdim * dstate and as
 * many fp64 log decays; each part rounded up to 256 bytes.
 */
size_t ssd_chunk_scan_workspace_size(int64_t total_tokens, int batch, int nheads, int headdim,
                                     int dstate, int ngroups, int chunk_size, int act_dtype);

/*
 * ssd_chunk_scan_plan -- how ssd_chunk_scan and mamba2_prefill split the
 * chunk-parallel scan (of page "perf(nemotron_h): prefill single-GPU prompts
 * in multi-token chunks", section Implementation) for these sizes; host only,
 * no device work.  *out_split: chunk-output workgroups per (chunk, group) (a
 * small grid splits a group's heads over several; the norm then runs as its
 * own kernel).  *seg: chunks per segment when long sequences are split so
 * that their state walks fill the CUs (0 = not split); *seg_levels: segments
 * of a max_seqlen-long sequence, the last of which takes every chunk from its
 * start to the sequence's end (a sequence longer than max_seqlen is still
 * covered).  Returns M2_OK, or an error (M2_ERR_SHAPE for sizes that take the
 * one-pass scan, which has no chunk plan); the outputs are written on M2_OK
 * only.
 */
int ssd_chunk_scan_plan(int64_t total_tokens, int batch, int max_seqlen, int nheads, int headdim,
                        int dstate, int ngroups, int chunk_size, int act_dtype, int* out_split,
                        int* seg, int* seg_levels);

/*
 * gated_rmsnorm_group -- grouped RMSNorm with the SiLU(z) gate.  (Page
 * "Nemotron-H", section 4.1: the scan output is normalised per group with the
 * ssm_norm weight and multiplied by the SiLU(z) gate; page "NemotronH decodes
 * on the single-step recurrent kernels", PR description, names the op
 * RmsNormGatedGroup(n_groups).)
 *
 * Per token t and group j (channels j*d_inner/ngroups .. (j+1)*d_inner/ngroups-1):
 *   norm_before_gate != 0:  out = y / sqrt(mean_j(y^2) + eps) * w * silu(z)
 *   norm_before_gate == 0:  v = y * silu(z);  out = v / sqrt(mean_j(v^2) + eps) * w
 *   y  [T, d_inner] fp32 (ld_y);  z [T, d_inner] (ld_z, z_dtype);
 *   norm_w [d_inner] fp32;  out [T, d_inner] (ld_out, out_dtype).
 * out may alias y exactly (same pointer and stride) for an in-place update.
 * The group width d_inner / ngroups must be at most 2048.
 */
int gated_rmsnorm_group(const float* y, int64_t ld_y, const void* z, int64_t ld_z,
                        int z_dtype, const float* norm_w, float eps, int ngroups,
                        int norm_before_gate, int64_t total_tokens, int d_inner,
                        void* out, int64_t ld_out, int out_dtype, void* stream);

/*
 * Bytes of device workspace mamba2_prefill needs for these sizes and this
 * activation dtype (0 on bad arguments).  The workspace holds the fp32
 * pre-norm output (used when y is not fp32) and the scan's own workspace
 * (ssd_chunk_scan_workspace_size()), and, when the prefill runs as the
 * four-kernel chain, the post-conv activations of the batch before them (fp32
 * for bf16 inputs, fp64 for fp32 inputs; on the chunk-parallel scan path
 * blocked per head and per group).  bf16 inputs at headdim 64, dstate 64 or
 * 128 (an even number of heads per group at 128) and chunk 128 have the scan
 * kernels convolve the raw rows themselves, so no post-conv activations are
 * stored; M2SSD_PREFILL_CHAIN=1 in the environment (read at every call, here
 * and in mamba2_prefill alike) selects the chain instead.
 */
size_t mamba2_prefill_workspace_size(int64_t total_tokens, int batch, int max_seqlen,
                                     int nheads, int headdim, int dstate, int ngroups,
                                     int chunk_size, int act_dtype);

/*
 * mamba2_prefill -- the whole mixer core of one layer for a packed varlen batch:
 * conv (+SiLU) over [conv_state ; rows] of x | B | C, the chunked scan with
 * carried ssm_state, the D skip and the grouped gated RMSNorm with z.  (Page
 * "Nemotron-H", section 3: the Mamba-2 layer's conv1d -> SiLU -> SSM -> gated
 * norm sequence, and section 4.1 for each step; page "perf(nemotron_h): prefill
 * single-GPU prompts in multi-token chunks", section Implementation: a layer's
 * conv rows and SSD rows run in one prefill pass over the chunked prompt, the
 * states committed after it.)
 * Arguments mean what they mean for the three calls above; additionally
 *   z [T, nheads*headdim] (ld_z) of act_dtype;
 *   conv_w [conv_dim, 4], conv_b [conv_dim] or NULL, norm_w [nheads*headdim];
 *   y [T, nheads*headdim] (ld_y), element type y_dtype (fp32 recommended:
 *     a bf16 output alone carries a relative rounding of 2^-9);
 *   workspace: device memory of at least mamba2_prefill_workspace_size() bytes,
 *     16-byte aligned (NULL allowed when that size is 0).
 * Both states are advanced in place.  The kernels that run depend on the
 * shape (the counters tell): on the raw-row path the chunk output applies the
 * norm itself when each of its workgroups holds whole norm groups and every
 * row is 16-byte aligned, and the norm kernel runs otherwise; the results do
 * not depend on which ran.
 */
int mamba2_prefill(const void* x, int64_t ld_x, const void* B, int64_t ld_B,
                   const void* C, int64_t ld_C, const void* z, int64_t ld_z, int act_dtype,
                   const float* dt, int64_t ld_dt, const float* A, const float* D,
                   const float* conv_w, const float* conv_b, const float* norm_w,
                   float eps, int norm_before_gate,
                   float* conv_state, float* ssm_state, int n_slots,
                   const int32_t* cu_seqlens, int batch, int64_t total_tokens,
                   int max_seqlen, const int32_t* state_idx, const uint8_t* has_init,
                   int nheads, int headdim, int dstate, int ngroups, int chunk_size,
                   void* y, int64_t ld_y, int y_dtype,
                   void* workspace, size_t ws_bytes, void* stream);

/*
 * mamba2_prefill_noalloc -- mamba2_prefill for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and bitwise the same results.  Its scratch is a fixed device array
 * inside the library, mamba2_prefill_noalloc_scratch_bytes() bytes (64 MiB),
 * one copy per GPU the library runs on, held until the process ends; its
 * device address is looked up on the first call on each device.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   Sizes whose mamba2_prefill_workspace_size() exceeds the scratch are
 *   refused with M2_ERR_WORKSPACE before any launch, with no side effects.
 *   Every call on one GPU shares that GPU's scratch, which keeps the last
 *   call's contents (nothing in it needs to start at zero): calls that overlap
 *   on one GPU -- on different streams, or from different threads -- race and
 *   must be serialized by the caller.
 */
size_t mamba2_prefill_noalloc_scratch_bytes(void);
int mamba2_prefill_noalloc(const void* x, int64_t ld_x, const void* B, int64_t ld_B,
                           const void* C, int64_t ld_C, const void* z, int64_t ld_z, int act_dtype,
                           const float* dt, int64_t ld_dt, const float* A, const float* D,
                           const float* conv_w, const float* conv_b, const float* norm_w,
                           float eps, int norm_before_gate,
                           float* conv_state, float* ssm_state, int n_slots,
                           const int32_t* cu_seqlens, int batch, int64_t total_tokens,
                           int max_seqlen, const int32_t* state_idx, const uint8_t* has_init,
                           int nheads, int headdim, int dstate, int ngroups, int chunk_size,
                           void* y, int64_t ld_y, int y_dtype, void* stream);

/*
 * mamba2_decode -- one new token for each of `batch` sequences, at their cache
 * slots: the conv update, the selective state update with its readout and the
 * grouped gated RMSNorm, in one fused kernel (for a small batch with an fp32
 * y: the state update split over more workgroups, then one launch for the conv
 * state and the norm) (page "NemotronH decodes on the
 * single-step recurrent kernels", PR description: decode rows take the
 * single-step conv update and state update at their slots, in place, with no
 * gather or scatter; page "Nemotron-H", section 4.1 for the recurrence and the
 * norm).  Row b of every token-indexed argument is sequence b's new token; the
 * result equals mamba2_prefill over one-token sequences (cu_seqlens = 0, 1, ..,
 * batch) up to rounding.  Per sequence b with slot s = state_idx[b] (NULL:
 * s = b), all states zero when has_init[b] == 0, group g = h / (nheads/ngroups)
 * and e(v) = exp(min(v, 0)):
 *   xpad      = [conv_state[s] (3 rows) ; the new x | B | C row]
 *   u[c]      = SiLU(conv_b[c] + sum_k conv_w[c, k] * xpad[k, c]),  split into x, B, C
 *   conv_state[s] <- rows 1..3 of xpad
 *   h[h,p,:]  <- e(dt[b,h] * A[h]) * h[h,p,:] + dt[b,h] * x[h,p] * B[g,:]
 *   ypre[h,p] = C[g,:] . h[h,p,:] + D[h] * x[h,p]
 *   y         = the gated grouped RMSNorm of ypre with z, as in gated_rmsnorm_group
 *
 *   x [batch, nheads*headdim] (ld_x), B, C [batch, ngroups*dstate] (ld_B, ld_C),
 *     z [batch, nheads*headdim] (ld_z): element type act_dtype;
 *   dt [batch, nheads] fp32 (ld_dt), the final step size, expected >= 0;
 *   A, D, conv_w, conv_b, norm_w, eps, norm_before_gate: as for mamba2_prefill;
 *   conv_state [n_slots, 3, conv_dim], ssm_state [n_slots, nheads, headdim,
 *     dstate] fp32, read and advanced in place;
 *   y [batch, nheads*headdim] (ld_y), element type y_dtype; must not overlap
 *     an input or a state.
 * batch == 0 is a no-op (after the dtype, shape and stride checks; the
 * pointers may then be NULL).  Slots used in one call must be distinct.  Alignment:
 * conv_w and ssm_state 16-byte aligned (the other arrays are read per element).
 * Supported (headdim, dstate): (16,16), (32,64), (64,64), (64,128), with a
 * group width (nheads/ngroups)*headdim of at most 2048.  No workspace.
 * Arithmetic: fp32, one rounding order fixed per shape (deterministic).
 */
int mamba2_decode(const void* x, int64_t ld_x, const void* B, int64_t ld_B,
                  const void* C, int64_t ld_C, const void* z, int64_t ld_z, int act_dtype,
                  const float* dt, int64_t ld_dt, const float* A, const float* D,
                  const float* conv_w, const float* conv_b, const float* norm_w,
                  float eps, int norm_before_gate,
                  float* conv_state, float* ssm_state, int n_slots, int batch,
                  const int32_t* state_idx, const uint8_t* has_init,
                  int nheads, int headdim, int dstate, int ngroups,
                  void* y, int64_t ld_y, int y_dtype, void* stream);

/*
 * Packed in-projection rows.  A Mamba-2 layer's in-projection emits one row per
 * token holding, in this order, z (d_inner = nheads*headdim channels), xBC
 * (conv_dim = d_inner + 2*ngroups*dstate channels: x | B | C) and the RAW step
 * size (nheads channels) (page "NemotronH decodes on the single-step recurrent
 * kernels", PR description: in_proj -> QkvSplit(z | xBC | dt), three outputs of
 * widths (I, conv_dim, num_heads) from the head, the middle and the tail of an
 * in_proj row).  The entries below read those rows in place and compute the
 * step size themselves (page "Nemotron-H", section 4.1: softplus of dt plus
 * the per-head ssm_dt.bias):
 *   dt[t, h] = softplus(raw[t, h] + dt_bias[h]),  softplus(v) = log(1 + e^v).
 *
 *   zxbcdt   [rows, ld_row] of act_dtype; ld_row >= 2*d_inner + 2*ngroups*dstate
 *            + nheads (padding after the raw step size is ignored).  Alignment:
 *            zxbcdt 16-byte aligned, ld_row * element size and d_inner *
 *            element size multiples of 16 bytes (as the views x, B, C, z need).
 *   dt_bias  [nheads] fp32, or NULL (0).
 * Everything else means what it means for mamba2_prefill / mamba2_decode.
 */

/*
 * Bytes of device workspace mamba2_prefill_inproj needs (0 on bad arguments):
 * mamba2_prefill_workspace_size() plus the fp32 step sizes [total_tokens, nheads]
 * (256-byte rounded, at least one row).  Always nonzero for valid arguments.
 */
size_t mamba2_prefill_inproj_workspace_size(int64_t total_tokens, int batch, int max_seqlen,
                                            int nheads, int headdim, int dstate, int ngroups,
                                            int chunk_size, int act_dtype);

/*
 * mamba2_prefill_inproj -- mamba2_prefill over a packed varlen batch given as
 * in-projection rows: the same conv, scan, D skip and gated norm, with dt
 * computed on the device from the rows' raw step sizes and dt_bias.
 * workspace is required (mamba2_prefill_inproj_workspace_size() bytes).
 */
int mamba2_prefill_inproj(const void* zxbcdt, int64_t ld_row, int act_dtype, const float* dt_bias,
                          const float* A, const float* D, const float* conv_w, const float* conv_b,
                          const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                          float* ssm_state, int n_slots, const int32_t* cu_seqlens, int batch,
                          int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                          const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                          int chunk_size, void* y, int64_t ld_y, int y_dtype, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * mamba2_decode_inproj -- mamba2_decode with row b of zxbcdt as sequence b's
 * new token; the step size softplus(raw + dt_bias) is formed inside the fused
 * decode kernel.  No workspace.  batch == 0 is a no-op.
 */
int mamba2_decode_inproj(const void* zxbcdt, int64_t ld_row, int act_dtype, const float* dt_bias,
                         const float* A, const float* D, const float* conv_w, const float* conv_b,
                         const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                         float* ssm_state, int n_slots, int batch, const int32_t* state_idx,
                         const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                         void* y, int64_t ld_y, int y_dtype, void* stream);

/*
 * Bytes of device workspace mamba2_mixed_inproj needs (0 on bad arguments):
 * mamba2_prefill_inproj_workspace_size() for the whole batch plus the prefill
 * part's row offsets and slot map, and for fp32 inputs room for the segment
 * buffers of any smaller prefill part (a sub-batch can be split into segments
 * where the whole batch would not be).
 */
size_t mamba2_mixed_inproj_workspace_size(int64_t total_tokens, int batch, int max_seqlen,
                                          int nheads, int headdim, int dstate, int ngroups,
                                          int chunk_size, int act_dtype);

/*
 * mamba2_mixed_inproj -- one layer step over a batch that mixes decode rows and
 * prefill sequences (page "NemotronH decodes on the single-step recurrent
 * kernels", PR description: decode rows take the single-step conv and state
 * updates at their cache slots, prefill rows keep the chunk scan, and the split
 * is the metadata's num_decodes, never the token count -- a fresh one-token
 * prompt is a prefill).  Sequences 0 .. num_decodes-1 are decode sequences of
 * exactly one row each, rows 0 .. num_decodes-1 (cu_seqlens[b] == b for
 * b <= num_decodes: a contract on device data, checked only with
 * M2SSD_DEBUG=1); sequences num_decodes .. batch-1 are prefills.  The decode
 * rows run the decode kernel, the prefill sequences the prefill chain; when
 * both are present the decode rows run on a second stream the library keeps
 * per thread and device (default priority), forked from `stream` and joined
 * back into it before the call's work is complete on `stream`; the result
 * equals mamba2_prefill_inproj over the whole batch up to rounding.  cu_seqlens, state_idx, has_init cover all `batch`
 * sequences; state_idx NULL means slot b for sequence b (needs n_slots >= batch).
 * 0 <= num_decodes <= batch; workspace is required.
 */
int mamba2_mixed_inproj(const void* zxbcdt, int64_t ld_row, int act_dtype, const float* dt_bias,
                        const float* A, const float* D, const float* conv_w, const float* conv_b,
                        const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                        float* ssm_state, int n_slots, const int32_t* cu_seqlens, int batch,
                        int num_decodes, int64_t total_tokens, int max_seqlen,
                        const int32_t* state_idx, const uint8_t* has_init, int nheads, int headdim,
                        int dstate, int ngroups, int chunk_size, void* y, int64_t ld_y, int y_dtype,
                        void* workspace, size_t ws_bytes, void* stream);

/* Launch counters (process-wide, atomic): which kernels ran, per instantiation. */
typedef struct {
    uint64_t conv_launches;        /* conv kernel launches */
    uint64_t conv_state_launches;  /* conv-state update launches */
    uint64_t scan_f64_launches;    /* scan launches, fp64 matrix path (fp32 inputs) */
    uint64_t scan_bf16x3_launches; /* scan launches, one-pass split-bf16 path (bf16 inputs) */
    uint64_t norm_launches;        /* gated norm launches */
    uint64_t prefill_calls;        /* successful mamba2_prefill calls */
    uint64_t scan_chunked_launches; /* scan launches, chunk-parallel path (bf16 inputs) */
    uint64_t decode_launches;      /* fused decode-step launches */
} m2_counters;

/* Copy the counters into *out (M2_ERR_NULL if out is NULL). */
int m2_get_counters(m2_counters* out);
/* Zero the counters. */
void m2_reset_counters(void);

/*
 * Kernel timing of mamba2_prefill with HIP events on the caller's stream.
 * m2_timing_enable(n) with n > 0 creates n event sets (host-side HIP objects,
 * no device allocation) and makes each following mamba2_prefill call record
 * events between its kernel launches, up to n calls; n == 0 stops recording.
 * m2_timing_read() waits for the recorded events, returns the summed kernel
 * times and the number of recorded calls, and rewinds the recorder.
 * Not thread-safe: one timing session per process.
 */
typedef struct {
    double conv_ms;        /* conv kernel */
    double conv_state_ms;  /* conv-state update */
    double scan_pass_ms;   /* scan state pass (the whole scan on the one-pass paths) */
    double scan_out_ms;    /* scan chunk-output kernel (0 on the one-pass paths) */
    double norm_ms;        /* gated norm */
    uint64_t calls;        /* recorded prefill calls */
} m2_kernel_times;

int m2_timing_enable(int max_calls);
int m2_timing_read(m2_kernel_times* out);

#ifdef __cplusplus
}
#endif

#endif /* M2SSD_H */
