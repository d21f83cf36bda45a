// C ABI of the Mamba-2 mixer-core prefill library: argument validation (all of
// it on the host, before any launch), dispatch to the kernel launchers, the
// fused prefill chain, launch counters and the thread-local error message.
// The operations are defined in include/m2ssd.h.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/m2ssd.h"
#include "kernels.h"

namespace {

thread_local std::string g_last_error;
// Set while a mixed batch runs its parts: the whole batch's index arrays were
// debug-checked already, and the prefill part's row offsets are computed on
// the device by then, so the parts skip the per-call debug reads.
thread_local bool g_parts_of_checked_batch = false;

struct Counters {
    std::atomic<uint64_t> conv{0}, conv_state{0}, scan_f64{0}, scan_bf16x3{0}, norm{0}, prefill{0},
        scan_chunked{0}, decode{0};
} g_counters;

// Event recorder for m2_timing_*: set k holds kEv events around the kernel
// stages of call k (conv, conv state, scan state pass, scan output, norm).
// Interval k (events k -> k + 1, in stream order) of a call is stage
// stage[call][k]: 0 conv, 1 conv state, 2 scan state pass, 3 scan output, 4 norm.
constexpr int kEv = 6;
struct Timing {
    std::vector<hipEvent_t> ev;
    std::vector<int> stage;
    int max_calls = 0;
    int used = 0;
    // event set for the next prefill call (its intervals in stream order are the
    // stages `order`), or null when off / full
    hipEvent_t* next(const int (&order)[kEv - 1]) {
        if (used >= max_calls) return nullptr;
        for (int k = 0; k < kEv - 1; ++k) stage[(size_t)(kEv - 1) * used + k] = order[k];
        return &ev[kEv * used++];
    }
} g_timing;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    g_last_error.clear();
    return M2_OK;
}

int64_t round256(int64_t v) { return (v + 255) / 256 * 256; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int elem_size(int dtype) { return dtype == M2_BF16 ? 2 : 4; }
bool valid_dtype(int d) { return d == M2_F32 || d == M2_BF16; }

// Debug checks of device-side index arrays, enabled per call by M2SSD_DEBUG=1.
bool debug_enabled() {
    if (g_parts_of_checked_batch) return false;
    const char* e = std::getenv("M2SSD_DEBUG");
    return e && e[0] == '1';
}

int debug_check_indices(const int32_t* cu, int batch, int64_t total, int max_seqlen,
                        const int32_t* idx, int n_slots) {
    std::vector<int32_t> hcu(batch + 1), hidx;
    if (hipMemcpy(hcu.data(), cu, sizeof(int32_t) * (batch + 1), hipMemcpyDeviceToHost) != hipSuccess)
        return fail(M2_ERR_HIP, "debug: reading cu_seqlens failed");
    if (hcu[0] != 0 || hcu[batch] != total)
        return fail(M2_ERR_SHAPE, "debug: cu_seqlens must start at 0 and end at total_tokens=%lld",
                    (long long)total);
    for (int b = 0; b < batch; ++b) {
        const int64_t L = (int64_t)hcu[b + 1] - hcu[b];
        if (L < 0 || L > max_seqlen)
            return fail(M2_ERR_SHAPE, "debug: sequence %d has length %lld (max_seqlen %d)", b,
                        (long long)L, max_seqlen);
    }
    if (idx) {
        hidx.resize(batch);
        if (hipMemcpy(hidx.data(), idx, sizeof(int32_t) * batch, hipMemcpyDeviceToHost) != hipSuccess)
            return fail(M2_ERR_HIP, "debug: reading state_idx failed");
        std::vector<char> seen(n_slots, 0);
        for (int b = 0; b < batch; ++b) {
            if (hidx[b] < 0 || hidx[b] >= n_slots)
                return fail(M2_ERR_SHAPE, "debug: state_idx[%d]=%d outside [0, %d)", b, hidx[b], n_slots);
            if (seen[hidx[b]]++)
                return fail(M2_ERR_SHAPE, "debug: state_idx[%d]=%d repeats a slot", b, hidx[b]);
        }
    }
    return M2_OK;
}

int check_batch(const int32_t* cu, int batch, int64_t total, int max_seqlen, const int32_t* idx,
                int n_slots) {
    if (!cu) return fail(M2_ERR_NULL, "cu_seqlens is NULL");
    if (batch <= 0) return fail(M2_ERR_SHAPE, "batch must be positive (got %d)", batch);
    if (total < 0 || max_seqlen < 0) return fail(M2_ERR_SHAPE, "total_tokens and max_seqlen must be >= 0");
    if ((int64_t)max_seqlen * batch < total)
        return fail(M2_ERR_SHAPE, "total_tokens %lld exceeds batch * max_seqlen", (long long)total);
    if (total > ((int64_t)1 << 31) - 1) return fail(M2_ERR_SHAPE, "total_tokens must fit in int32");
    if (n_slots <= 0) return fail(M2_ERR_SHAPE, "n_slots must be positive");
    if (!idx && n_slots < batch) return fail(M2_ERR_SHAPE, "state_idx NULL needs n_slots >= batch");
    if (debug_enabled()) return debug_check_indices(cu, batch, total, max_seqlen, idx, n_slots);
    return M2_OK;
}

// Debug check of the step sizes and decay rates the exponents are built from:
// A finite and <= 0 for every head; dt (when given final, rows x nheads with
// row stride ld_dt) finite and >= 0.  A decay rate above 0 or a negative step
// would be clamped silently by the kernels.
int debug_check_dt_A(const float* dt, int64_t ld_dt, int64_t rows, int nheads, const float* A) {
    std::vector<float> hA(nheads);
    if (hipMemcpy(hA.data(), A, sizeof(float) * nheads, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(M2_ERR_HIP, "debug: reading A failed");
    for (int h = 0; h < nheads; ++h)
        if (!(hA[h] <= 0.f) || !std::isfinite(hA[h]))
            return fail(M2_ERR_SHAPE, "debug: A[%d]=%g must be finite and <= 0", h, (double)hA[h]);
    if (!dt || rows <= 0) return M2_OK;
    std::vector<float> hdt((size_t)rows * nheads);
    if (hipMemcpy2D(hdt.data(), sizeof(float) * nheads, dt, sizeof(float) * ld_dt, sizeof(float) * nheads,
                    (size_t)rows, hipMemcpyDeviceToHost) != hipSuccess)
        return fail(M2_ERR_HIP, "debug: reading dt failed");
    for (int64_t t = 0; t < rows; ++t)
        for (int h = 0; h < nheads; ++h) {
            const float v = hdt[(size_t)t * nheads + h];
            if (!(v >= 0.f) || !std::isfinite(v))
                return fail(M2_ERR_SHAPE, "debug: dt[%lld][%d]=%g must be finite and >= 0", (long long)t, h,
                            (double)v);
        }
    return M2_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(M2_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return M2_OK;
}

// ---- per-operation validation (no side effects) ----

int validate_conv(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                  int64_t ld_C, int d_x, int d_b, int act_dtype, const float* conv_w,
                  const float* conv_b, int width, float* conv_state, int n_slots,
                  const int32_t* cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                  const int32_t* state_idx, const void* out, int64_t ld_out, int out_dtype) {
    const bool rows = total_tokens > 0;   // token-indexed arrays are read only when there are rows
    if ((rows && (!x || !out)) || !conv_w || !conv_state)
        return fail(M2_ERR_NULL, "conv: x, conv_w, conv_state and out are required");
    if (rows && d_b > 0 && (!B || !C)) return fail(M2_ERR_NULL, "conv: B and C are required when d_b > 0");
    if (!valid_dtype(act_dtype) || !valid_dtype(out_dtype)) return fail(M2_ERR_DTYPE, "conv: dtype must be M2_F32 or M2_BF16");
    if (width != 4) return fail(M2_ERR_UNSUPPORTED, "conv: width must be 4 (got %d)", width);
    if (d_x <= 0 || d_b < 0 || d_x % 8 || d_b % 8)
        return fail(M2_ERR_SHAPE, "conv: d_x > 0 and d_b >= 0 must be multiples of 8 (got %d, %d)", d_x, d_b);
    const int conv_dim = d_x + 2 * d_b;
    if (ld_x < d_x || (d_b > 0 && (ld_B < d_b || ld_C < d_b)) || ld_out < conv_dim)
        return fail(M2_ERR_STRIDE, "conv: a row stride is smaller than its row width");
    const int es = elem_size(act_dtype);
    if (!aligned16(x) || (d_b > 0 && (!aligned16(B) || !aligned16(C))) || !aligned16(out) ||
        !aligned16(conv_w) || !aligned16(conv_state) || (conv_b && !aligned16(conv_b)))
        return fail(M2_ERR_ALIGN, "conv: pointers must be 16-byte aligned");
    if ((ld_x * es) % 16 || (d_b > 0 && ((ld_B * es) % 16 || (ld_C * es) % 16)) ||
        (ld_out * elem_size(out_dtype)) % 16)
        return fail(M2_ERR_ALIGN, "conv: row strides must be multiples of 16 bytes");
    return check_batch(cu_seqlens, batch, total_tokens, max_seqlen, state_idx, n_slots);
}

int validate_scan_dims(int nheads, int headdim, int dstate, int ngroups, int chunk_size) {
    if (nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return fail(M2_ERR_SHAPE, "scan: nheads, headdim, dstate, ngroups must be positive");
    if (nheads % ngroups) return fail(M2_ERR_SHAPE, "scan: nheads %% ngroups != 0 (%d, %d)", nheads, ngroups);
    if (chunk_size < 16 || chunk_size > 128 || chunk_size % 16)
        return fail(M2_ERR_CHUNK, "chunk_size must be a multiple of 16 in [16, 128] (got %d)", chunk_size);
    if (!m2::scan_supported(headdim, dstate))
        return fail(M2_ERR_UNSUPPORTED, "no scan kernel for headdim=%d dstate=%d", headdim, dstate);
    return M2_OK;
}

int validate_scan(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                  int64_t ld_C, int act_dtype, const float* dt, int64_t ld_dt, const float* A,
                  const float* D, float* ssm_state, int n_slots, const int32_t* cu_seqlens,
                  int batch, int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                  int nheads, int headdim, int dstate, int ngroups, int chunk_size,
                  const float* y, int64_t ld_y) {
    (void)D;
    if ((total_tokens > 0 && (!x || !B || !C || !dt || !y)) || !A || !ssm_state)
        return fail(M2_ERR_NULL, "scan: x, B, C, dt, A, ssm_state and y are required");
    if (!valid_dtype(act_dtype)) return fail(M2_ERR_DTYPE, "scan: act_dtype must be M2_F32 or M2_BF16");
    int st = validate_scan_dims(nheads, headdim, dstate, ngroups, chunk_size);
    if (st) return st;
    const int64_t di = (int64_t)nheads * headdim, gn = (int64_t)ngroups * dstate;
    if (ld_x < di || ld_B < gn || ld_C < gn || ld_dt < nheads || ld_y < di)
        return fail(M2_ERR_STRIDE, "scan: a row stride is smaller than its row width");
    const int es = elem_size(act_dtype);
    if (!aligned16(x) || !aligned16(B) || !aligned16(C) || !aligned16(y) || !aligned16(ssm_state))
        return fail(M2_ERR_ALIGN, "scan: x, B, C, y and ssm_state must be 16-byte aligned");
    if ((ld_x * es) % 16 || (ld_B * es) % 16 || (ld_C * es) % 16 || (ld_y * 4) % 16)
        return fail(M2_ERR_ALIGN, "scan: ld_x, ld_B, ld_C and ld_y must be multiples of 16 bytes");
    return check_batch(cu_seqlens, batch, total_tokens, max_seqlen, state_idx, n_slots);
}

int validate_norm(const float* y, int64_t ld_y, const void* z, int64_t ld_z, int z_dtype,
                  const float* norm_w, int ngroups, int64_t total_tokens, int d_inner,
                  const void* out, int64_t ld_out, int out_dtype) {
    if ((total_tokens > 0 && (!y || !z || !out)) || !norm_w)
        return fail(M2_ERR_NULL, "norm: y, z, norm_w and out are required");
    if (!valid_dtype(z_dtype) || !valid_dtype(out_dtype)) return fail(M2_ERR_DTYPE, "norm: dtype must be M2_F32 or M2_BF16");
    if (d_inner <= 0 || ngroups <= 0 || d_inner % ngroups || total_tokens < 0)
        return fail(M2_ERR_SHAPE, "norm: need d_inner > 0 divisible by ngroups > 0, total_tokens >= 0");
    if (d_inner / ngroups > 2048) return fail(M2_ERR_UNSUPPORTED, "norm: group width above 2048");
    if (ld_y < d_inner || ld_z < d_inner || ld_out < d_inner)
        return fail(M2_ERR_STRIDE, "norm: a row stride is smaller than d_inner");
    if (static_cast<const void*>(y) == out && (ld_out != ld_y || out_dtype != M2_F32))
        return fail(M2_ERR_STRIDE, "norm: in-place use needs out == y with the same stride and fp32 output");
    return M2_OK;
}

// Scan launch: the chunk-parallel kernels when a.states is set (it points at the
// entry-state buffer; the caller sets it only for shapes those kernels cover),
// else the one-pass kernel.  ev_mid (optional) is recorded after the state pass,
// or after the whole one-pass scan.
int launch_scan(m2::ScanArgs& a, int64_t total_tokens, hipStream_t s, hipEvent_t ev_mid) {
    int st;
    if (a.states) {
        if ((st = hip_status(m2::launch_ssd_state_pass(a, s), "scan state pass launch"))) return st;
        if (ev_mid) (void)hipEventRecord(ev_mid, s);
        if ((st = hip_status(m2::launch_ssd_chunk_out(a, total_tokens, s), "scan chunk output launch"))) return st;
        g_counters.scan_chunked++;
        return M2_OK;
    }
    if ((st = hip_status(m2::launch_ssd_scan(a, s), "scan launch"))) return st;
    if (ev_mid) (void)hipEventRecord(ev_mid, s);
    (a.policy == m2::kPolicyBf16x3 ? g_counters.scan_bf16x3 : g_counters.scan_f64)++;
    return M2_OK;
}

size_t scan_states_bytes(int64_t total_tokens, int batch, int nheads, int headdim, int dstate,
                         int ngroups, int chunk_size, int act_dtype) {
    const int policy = act_dtype == M2_BF16 ? m2::kPolicyBf16x3 : m2::kPolicyF64;
    if (!m2::chunked_scan_supported(policy, nheads, ngroups, headdim, dstate, chunk_size)) return 0;
    return m2::chunked_scan_states_bytes(total_tokens, batch, nheads, headdim, dstate);
}

// The scan's whole workspace: the chunk-parallel path's buffers, or the
// one-pass fp64 path's segment buffers (0 for paths that need none).
size_t scan_ws_bytes(int64_t total_tokens, int batch, int nheads, int headdim, int dstate, int ngroups,
                     int chunk_size, int act_dtype) {
    const size_t chunked = scan_states_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups,
                                             chunk_size, act_dtype);
    if (chunked > 0) return chunked;
    const int policy = act_dtype == M2_BF16 ? m2::kPolicyBf16x3 : m2::kPolicyF64;
    return m2::one_pass_seg_bytes(batch, nheads, headdim, dstate, policy);
}

// Row-major conv output: segment s starts at its channel offset within each row.
void set_rowmajor_out(m2::ConvArgs& a, void* out, int64_t ld_out, int elt) {
    int64_t c = 0;
    for (int k = 0; k < 3; ++k) {
        a.out_ptr[k] = static_cast<char*>(out) + c * elt;
        a.out_ld[k] = ld_out;
        a.out_bs[k] = 0;
        a.out_bw[k] = a.seg_ch[k] > 0 ? a.seg_ch[k] : 1;
        c += a.seg_ch[k];
    }
}

// The prefill's scan convolves the raw bf16 rows itself (no post-conv
// activations in the workspace) wherever the chunk-parallel kernels take raw
// rows; M2SSD_PREFILL_CHAIN=1 (read at every call) runs the four-kernel chain
// with the post-conv activations in the workspace instead.
bool prefill_raw(int act_dtype, int nheads, int headdim, int dstate, int ngroups, int chunk_size) {
    if (act_dtype != M2_BF16) return false;
    if (nheads <= 0 || ngroups <= 0 || nheads % ngroups) return false;
    if (!m2::chunked_raw_supported(nheads, ngroups, headdim, dstate, chunk_size)) return false;
    const char* e = std::getenv("M2SSD_PREFILL_CHAIN");
    return !(e && e[0] == '1');
}

}  // namespace

extern "C" {

const char* m2_last_error(void) { return g_last_error.c_str(); }

const char* m2_version(void) { return "m2ssd 0.1 (gfx950)"; }

int m2_get_counters(m2_counters* out) {
    if (!out) return fail(M2_ERR_NULL, "m2_get_counters: out is NULL");
    out->conv_launches = g_counters.conv.load();
    out->conv_state_launches = g_counters.conv_state.load();
    out->scan_f64_launches = g_counters.scan_f64.load();
    out->scan_bf16x3_launches = g_counters.scan_bf16x3.load();
    out->norm_launches = g_counters.norm.load();
    out->prefill_calls = g_counters.prefill.load();
    out->scan_chunked_launches = g_counters.scan_chunked.load();
    out->decode_launches = g_counters.decode.load();
    return ok();
}

void m2_reset_counters(void) {
    g_counters.conv = 0;
    g_counters.conv_state = 0;
    g_counters.scan_f64 = 0;
    g_counters.scan_bf16x3 = 0;
    g_counters.norm = 0;
    g_counters.prefill = 0;
    g_counters.scan_chunked = 0;
    g_counters.decode = 0;
}

int mamba2_conv_rows(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                     int64_t ld_C, int d_x, int d_b, int act_dtype, const float* conv_w,
                     const float* conv_b, int width, float* conv_state, int n_slots,
                     const int32_t* cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                     const int32_t* state_idx, const uint8_t* has_init, int apply_silu, void* out,
                     int64_t ld_out, int out_dtype, void* stream) {
    int st = validate_conv(x, ld_x, B, ld_B, C, ld_C, d_x, d_b, act_dtype, conv_w, conv_b, width,
                           conv_state, n_slots, cu_seqlens, batch, total_tokens, max_seqlen,
                           state_idx, out, ld_out, out_dtype);
    if (st) return st;
    m2::ConvArgs a{};
    a.seg_ptr[0] = x; a.seg_ld[0] = ld_x; a.seg_ch[0] = d_x;
    a.seg_ptr[1] = B; a.seg_ld[1] = ld_B; a.seg_ch[1] = d_b;
    a.seg_ptr[2] = C; a.seg_ld[2] = ld_C; a.seg_ch[2] = d_b;
    a.nseg = d_b > 0 ? 3 : 1;
    a.act_dtype = act_dtype;
    a.conv_w = conv_w; a.conv_b = conv_b;
    a.conv_dim = d_x + 2 * d_b;
    a.conv_state = conv_state;
    a.cu_seqlens = cu_seqlens; a.batch = batch; a.total_tokens = total_tokens;
    a.state_idx = state_idx; a.has_init = has_init;
    a.apply_silu = apply_silu; a.out_dtype = out_dtype;
    set_rowmajor_out(a, out, ld_out, elem_size(out_dtype));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (total_tokens > 0) {
        if ((st = hip_status(m2::launch_conv_rows(a, s), "conv launch"))) return st;
        g_counters.conv++;
    }
    if ((st = hip_status(m2::launch_conv_state_update(a, s), "conv state launch"))) return st;
    g_counters.conv_state++;
    return ok();
}

size_t ssd_chunk_scan_workspace_size(int64_t total_tokens, int batch, int nheads, int headdim,
                                     int dstate, int ngroups, int chunk_size, int act_dtype) {
    if (total_tokens < 0 || batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || !valid_dtype(act_dtype))
        return 0;
    return scan_ws_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype);
}

int ssd_chunk_scan_plan(int64_t total_tokens, int batch, int max_seqlen, int nheads, int headdim, int dstate,
                        int ngroups, int chunk_size, int act_dtype, int* out_split, int* seg, int* seg_levels) {
    if (!out_split || !seg || !seg_levels) return fail(M2_ERR_NULL, "scan plan: out_split, seg and seg_levels are required");
    int st = validate_scan_dims(nheads, headdim, dstate, ngroups, chunk_size);
    if (st) return st;
    if (!valid_dtype(act_dtype)) return fail(M2_ERR_DTYPE, "scan plan: act_dtype must be M2_F32 or M2_BF16");
    if (total_tokens < 0 || batch <= 0 || max_seqlen < 0)
        return fail(M2_ERR_SHAPE, "scan plan: batch must be > 0, total_tokens and max_seqlen >= 0");
    if ((int64_t)max_seqlen * batch < total_tokens)
        return fail(M2_ERR_SHAPE, "scan plan: total_tokens %lld exceeds batch * max_seqlen", (long long)total_tokens);
    if (scan_states_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype) == 0)
        return fail(M2_ERR_SHAPE, "scan plan: these sizes take the one-pass scan, which has no chunk plan");
    const m2::ScanSplit sp = m2::chunked_scan_split(total_tokens, batch, nheads, ngroups, dstate, max_seqlen);
    *out_split = sp.out_split;
    *seg = sp.seg;
    *seg_levels = sp.seg_levels;
    return ok();
}

int ssd_chunk_scan(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                   int64_t ld_C, int act_dtype, const float* dt, int64_t ld_dt, const float* A,
                   const float* D, float* ssm_state, int n_slots, const int32_t* cu_seqlens,
                   int batch, int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                   const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                   int chunk_size, float* y, int64_t ld_y, void* workspace, size_t ws_bytes,
                   void* stream) {
    int st = validate_scan(x, ld_x, B, ld_B, C, ld_C, act_dtype, dt, ld_dt, A, D, ssm_state,
                           n_slots, cu_seqlens, batch, total_tokens, max_seqlen, state_idx, nheads,
                           headdim, dstate, ngroups, chunk_size, y, ld_y);
    if (st) return st;
    if (debug_enabled() && (st = debug_check_dt_A(dt, ld_dt, total_tokens, nheads, A))) return st;
    const size_t chunked_need = scan_states_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype);
    const size_t need = scan_ws_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(M2_ERR_WORKSPACE, "scan: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (need > 0 && !aligned16(workspace)) return fail(M2_ERR_ALIGN, "scan: workspace must be 16-byte aligned");
    m2::ScanArgs a{};
    a.x = x; a.ld_x = ld_x; a.hs_x = headdim;
    a.B = B; a.ld_B = ld_B; a.gs_B = dstate;
    a.C = C; a.ld_C = ld_C; a.gs_C = dstate;
    a.act_dtype = act_dtype; a.policy = act_dtype == M2_BF16 ? m2::kPolicyBf16x3 : m2::kPolicyF64;
    a.dt = dt; a.ld_dt = ld_dt; a.A = A; a.D = D; a.ssm_state = ssm_state;
    a.cu_seqlens = cu_seqlens; a.batch = batch; a.state_idx = state_idx; a.has_init = has_init;
    a.nheads = nheads; a.headdim = headdim; a.dstate = dstate; a.ngroups = ngroups;
    a.chunk = chunk_size; a.y = y; a.ld_y = ld_y;
    a.states = chunked_need > 0 ? static_cast<float*>(workspace) : nullptr;
    a.order = a.states ? m2::chunked_scan_order(a.states, total_tokens, batch, nheads, headdim, dstate) : nullptr;
    if (a.states) m2::chunked_scan_plan(a, total_tokens, max_seqlen);
    else m2::one_pass_plan(a, max_seqlen, need > 0 ? workspace : nullptr);
    // one sequence, or all of one length (batch * max_seqlen tokens): the
    // identity order is already longest first (the order only sets the state
    // pass's dispatch; a sequence past max_seqlen would only be dealt later)
    if (batch == 1 || total_tokens == (int64_t)batch * max_seqlen) a.order = nullptr;
    if ((st = launch_scan(a, total_tokens, static_cast<hipStream_t>(stream), nullptr))) return st;
    return ok();
}

int gated_rmsnorm_group(const float* y, int64_t ld_y, const void* z, int64_t ld_z, int z_dtype,
                        const float* norm_w, float eps, int ngroups, int norm_before_gate,
                        int64_t total_tokens, int d_inner, void* out, int64_t ld_out,
                        int out_dtype, void* stream) {
    int st = validate_norm(y, ld_y, z, ld_z, z_dtype, norm_w, ngroups, total_tokens, d_inner, out,
                           ld_out, out_dtype);
    if (st) return st;
    if (total_tokens == 0) return ok();
    m2::NormArgs a{};
    a.y = y; a.ld_y = ld_y; a.z = z; a.ld_z = ld_z; a.z_dtype = z_dtype; a.norm_w = norm_w;
    a.eps = eps; a.ngroups = ngroups; a.norm_before_gate = norm_before_gate;
    a.total_tokens = total_tokens; a.d_inner = d_inner; a.out = out; a.ld_out = ld_out;
    a.out_dtype = out_dtype;
    if ((st = hip_status(m2::launch_gated_norm(a, static_cast<hipStream_t>(stream)), "norm launch"))) return st;
    g_counters.norm++;
    return ok();
}

size_t mamba2_prefill_workspace_size(int64_t total_tokens, int batch, int max_seqlen, int nheads,
                                     int headdim, int dstate, int ngroups, int chunk_size,
                                     int act_dtype) {
    (void)max_seqlen;
    if (total_tokens < 0 || batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
        ngroups <= 0 || !valid_dtype(act_dtype))
        return 0;
    const int64_t conv_dim = (int64_t)nheads * headdim + 2 * (int64_t)ngroups * dstate;
    const int64_t di = (int64_t)nheads * headdim;
    // post-conv activations (fp32 for bf16 inputs, fp64 for fp32 inputs; none
    // when the scan convolves the raw rows itself), the pre-norm output (fp32;
    // used when y is not fp32) and the scan's entry states
    const int64_t ues = act_dtype == M2_BF16 ? 4 : 8;
    const bool raw = prefill_raw(act_dtype, nheads, headdim, dstate, ngroups, chunk_size);
    return (size_t)((raw ? 0 : round256(total_tokens * conv_dim * ues)) + round256(total_tokens * di * 4)) +
           scan_ws_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype);
}

}  // extern "C"

namespace {

// The prefill chain.  Every argument check runs first; with launch == false the
// call stops there (a dry run used by the entries that launch a step of their
// own before the chain), so a failing check never leaves side effects.
int prefill_run(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                int64_t ld_C, const void* z, int64_t ld_z, int act_dtype, const float* dt,
                int64_t ld_dt, const float* A, const float* D, const float* conv_w,
                const float* conv_b, const float* norm_w, float eps, int norm_before_gate,
                float* conv_state, float* ssm_state, int n_slots, const int32_t* cu_seqlens,
                int batch, int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                int chunk_size, void* y, int64_t ld_y, int y_dtype, void* workspace,
                size_t ws_bytes, void* stream, bool launch) {
    int st = validate_scan_dims(nheads, headdim, dstate, ngroups, chunk_size);
    if (st) return st;
    const int d_x = nheads * headdim, d_b = ngroups * dstate;
    const int conv_dim = d_x + 2 * d_b;
    if ((total_tokens > 0 && (!z || !y)) || !norm_w) return fail(M2_ERR_NULL, "prefill: z, norm_w and y are required");
    if (!valid_dtype(y_dtype)) return fail(M2_ERR_DTYPE, "prefill: y_dtype must be M2_F32 or M2_BF16");
    if (!valid_dtype(act_dtype)) return fail(M2_ERR_DTYPE, "prefill: act_dtype must be M2_F32 or M2_BF16");
    const size_t need = mamba2_prefill_workspace_size(total_tokens, batch, max_seqlen, nheads,
                                                      headdim, dstate, ngroups, chunk_size, act_dtype);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(M2_ERR_WORKSPACE, "prefill: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (workspace && !aligned16(workspace)) return fail(M2_ERR_ALIGN, "prefill: workspace must be 16-byte aligned");
    // Post-conv activations: fp32 for bf16 inputs, fp64 for fp32 inputs (the
    // fp64 scan path reads them without an fp32 rounding in between).  They are
    // not rounded to bf16: y and the state reach max|err|/RMS ~ 0.05 from that
    // rounding alone, where the largest outputs are tens of times the RMS.
    const int u_dtype = act_dtype == M2_BF16 ? m2::kF32 : m2::kF64;
    const int ues = u_dtype == m2::kF64 ? 8 : 4;
    const bool raw = prefill_raw(act_dtype, nheads, headdim, dstate, ngroups, chunk_size);
    const int64_t u_bytes = raw ? 0 : round256((int64_t)total_tokens * conv_dim * ues);
    const int64_t ypre_bytes = round256((int64_t)total_tokens * d_x * 4);
    char* wsb = static_cast<char*>(workspace);
    void* u = raw ? nullptr : wsb;
    float* ypre_ws = wsb ? reinterpret_cast<float*>(wsb + u_bytes) : nullptr;
    const bool chunked = scan_states_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype) > 0;
    float* states_ws = (wsb && chunked) ? reinterpret_cast<float*>(wsb + u_bytes + ypre_bytes) : nullptr;
    // one-pass path: its segment buffers (if any) take the same place
    void* seg_ws = (wsb && !chunked &&
                    scan_ws_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups, chunk_size, act_dtype) > 0)
                       ? static_cast<void*>(wsb + u_bytes + ypre_bytes) : nullptr;
    if ((st = validate_conv(x, ld_x, B, ld_B, C, ld_C, d_x, d_b, act_dtype, conv_w, conv_b, 4,
                            conv_state, n_slots, cu_seqlens, batch, total_tokens, max_seqlen,
                            state_idx, u ? u : y, conv_dim, M2_F32)))
        return st;
    if ((total_tokens > 0 && !dt) || !A || !ssm_state) return fail(M2_ERR_NULL, "prefill: dt, A and ssm_state are required");
    if (ld_dt < nheads) return fail(M2_ERR_STRIDE, "prefill: ld_dt < nheads");
    if (!aligned16(ssm_state)) return fail(M2_ERR_ALIGN, "prefill: ssm_state must be 16-byte aligned");
    // (the norm's input: the pre-norm output, in y itself when y is fp32)
    const bool pre_in_y = y_dtype == M2_F32 || !ypre_ws;
    if ((st = validate_norm(pre_in_y ? static_cast<const float*>(y) : ypre_ws, pre_in_y ? ld_y : d_x, z, ld_z,
                            act_dtype, norm_w, ngroups, total_tokens, d_x, y, ld_y,
                            pre_in_y ? M2_F32 : y_dtype)))
        return st;
    if (y_dtype == M2_F32 && (ld_y * 4) % 16) return fail(M2_ERR_ALIGN, "prefill: ld_y must be a multiple of 16 bytes");
    if (!aligned16(y)) return fail(M2_ERR_ALIGN, "prefill: y must be 16-byte aligned");
    if (!launch) return M2_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    // stages in stream order: the chain runs conv, conv state, state pass, chunk
    // output, norm; with raw rows the scan comes first and the conv state after it
    // (both scan kernels read the old conv state)
    static const int kChainOrder[kEv - 1] = {0, 1, 2, 3, 4};
    static const int kRawOrder[kEv - 1] = {2, 3, 1, 4, 0};
    hipEvent_t* tev = g_timing.next(raw ? kRawOrder : kChainOrder);
    auto mark = [&](int k) { if (tev) (void)hipEventRecord(tev[k], s); };
    mark(0);
    m2::ConvArgs ca{};
    ca.seg_ptr[0] = x; ca.seg_ld[0] = ld_x; ca.seg_ch[0] = d_x;
    ca.seg_ptr[1] = B; ca.seg_ld[1] = ld_B; ca.seg_ch[1] = d_b;
    ca.seg_ptr[2] = C; ca.seg_ld[2] = ld_C; ca.seg_ch[2] = d_b;
    ca.nseg = 3; ca.act_dtype = act_dtype; ca.conv_w = conv_w; ca.conv_b = conv_b;
    ca.conv_dim = conv_dim; ca.conv_state = conv_state; ca.cu_seqlens = cu_seqlens;
    ca.batch = batch; ca.total_tokens = total_tokens; ca.state_idx = state_idx;
    ca.has_init = has_init; ca.apply_silu = 1; ca.out_dtype = u_dtype;
    // Post-conv layout.  Chunked scan: blocked, x as [head][token][headdim] and B, C
    // as [group][token][dstate], so each (chunk, head) and (chunk, group) tile the
    // scan reads is one contiguous run (row-major rows scattered the reads over
    // DRAM pages: both scan kernels ran ~7% slower).  Otherwise row-major.
    const int64_t T = total_tokens;
    char* ub = static_cast<char*>(u);
    m2::ScanArgs sa{};
    if (raw) {
        set_rowmajor_out(ca, nullptr, conv_dim, ues);   // (no conv output: only the state advance runs)
        sa.x = x; sa.ld_x = ld_x; sa.hs_x = headdim;
        sa.B = B; sa.ld_B = ld_B; sa.gs_B = dstate;
        sa.C = C; sa.ld_C = ld_C; sa.gs_C = dstate;
        sa.raw_conv = 1; sa.conv_w = conv_w; sa.conv_b = conv_b; sa.conv_state = conv_state;
        sa.conv_dim = conv_dim;
    } else if (chunked) {
        const int64_t off[3] = {0, (int64_t)d_x * T * ues, (int64_t)(d_x + d_b) * T * ues};
        const int bw[3] = {headdim, dstate, dstate};
        for (int k = 0; k < 3; ++k) {
            ca.out_ptr[k] = ub + off[k]; ca.out_ld[k] = bw[k]; ca.out_bw[k] = bw[k]; ca.out_bs[k] = T * bw[k];
        }
        sa.x = ub; sa.ld_x = headdim; sa.hs_x = T * headdim;
        sa.B = ub + off[1]; sa.ld_B = dstate; sa.gs_B = T * dstate;
        sa.C = ub + off[2]; sa.ld_C = dstate; sa.gs_C = T * dstate;
    } else {
        set_rowmajor_out(ca, u, conv_dim, ues);
        sa.x = ub; sa.ld_x = conv_dim; sa.hs_x = headdim;
        sa.B = ub + (int64_t)d_x * ues; sa.ld_B = conv_dim; sa.gs_B = dstate;
        sa.C = ub + (int64_t)(d_x + d_b) * ues; sa.ld_C = conv_dim; sa.gs_C = dstate;
    }
    if (!raw) {
        if (total_tokens > 0) {
            if ((st = hip_status(m2::launch_conv_rows(ca, s), "prefill conv launch"))) return st;
            g_counters.conv++;
        }
        mark(1);
        if ((st = hip_status(m2::launch_conv_state_update(ca, s), "prefill conv state launch"))) return st;
        g_counters.conv_state++;
        mark(2);
    }

    float* ypre = (y_dtype == M2_F32) ? static_cast<float*>(y) : ypre_ws;
    const int64_t ld_pre = (y_dtype == M2_F32) ? ld_y : d_x;
    sa.act_dtype = raw ? m2::kBF16 : u_dtype;
    sa.policy = act_dtype == M2_BF16 ? m2::kPolicyBf16x3 : m2::kPolicyF64;
    sa.dt = dt; sa.ld_dt = ld_dt; sa.A = A; sa.D = D; sa.ssm_state = ssm_state;
    sa.cu_seqlens = cu_seqlens; sa.batch = batch; sa.state_idx = state_idx; sa.has_init = has_init;
    sa.nheads = nheads; sa.headdim = headdim; sa.dstate = dstate; sa.ngroups = ngroups;
    sa.chunk = chunk_size; sa.y = ypre; sa.ld_y = ld_pre;
    sa.states = states_ws;
    sa.order = states_ws ? m2::chunked_scan_order(states_ws, total_tokens, batch, nheads, headdim, dstate) : nullptr;
    if (states_ws) m2::chunked_scan_plan(sa, total_tokens, max_seqlen);
    else m2::one_pass_plan(sa, max_seqlen, seg_ws);
    // one sequence, or all of one length: no order to compute (see ssd_chunk_scan)
    if (batch == 1 || total_tokens == (int64_t)batch * max_seqlen) sa.order = nullptr;
    // The raw chunk output applies the norm itself when each of its workgroups
    // holds a whole norm group (out_split 1) and every row is 16-byte aligned.
    {
        const int gs = d_x / ngroups;
        const int oes = y_dtype == M2_BF16 ? 2 : 4;
        const bool al = aligned16(ypre) && aligned16(z) && aligned16(y) && aligned16(norm_w) &&
                        (ld_pre * 4) % 16 == 0 && (ld_z * 2) % 16 == 0 && (ld_y * oes) % 16 == 0;
        if (raw && sa.out_split <= 1 && gs % 8 == 0 && gs <= 2048 && al && total_tokens > 0) {
            sa.fuse_norm = 1;
            sa.z = z; sa.ld_z = ld_z; sa.norm_w = norm_w; sa.eps = eps; sa.norm_before_gate = norm_before_gate;
            sa.norm_out = y; sa.ld_out = ld_y; sa.out_dtype = y_dtype;
        }
    }
    if ((st = launch_scan(sa, total_tokens, s, tev ? tev[raw ? 1 : 3] : nullptr))) return st;
    if (raw) {
        mark(2);
        if ((st = hip_status(m2::launch_conv_state_update(ca, s), "prefill conv state launch"))) return st;
        g_counters.conv_state++;
        mark(3);
    } else {
        mark(4);
    }

    if (total_tokens > 0 && !sa.fuse_norm) {
        m2::NormArgs na{};
        na.y = ypre; na.ld_y = ld_pre; na.z = z; na.ld_z = ld_z; na.z_dtype = act_dtype;
        na.norm_w = norm_w; na.eps = eps; na.ngroups = ngroups; na.norm_before_gate = norm_before_gate;
        na.total_tokens = total_tokens; na.d_inner = d_x; na.out = y; na.ld_out = ld_y;
        na.out_dtype = y_dtype;
        if ((st = hip_status(m2::launch_gated_norm(na, s), "prefill norm launch"))) return st;
        g_counters.norm++;
    }
    if (raw) {
        mark(4);
        mark(5);
    } else {
        mark(5);
    }
    g_counters.prefill++;
    return ok();
}

// The fused decode step; dt is fp32 step sizes, or (dt_softplus) raw values of
// act_dtype with dt_bias.  launch == false: checks only, as for prefill_run.
int decode_run(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
               int64_t ld_C, const void* z, int64_t ld_z, int act_dtype, const void* dt,
               int64_t ld_dt, int dt_softplus, const float* dt_bias, const float* A,
               const float* D, const float* conv_w, const float* conv_b, const float* norm_w,
               float eps, int norm_before_gate, float* conv_state, float* ssm_state, int n_slots,
               int batch, const int32_t* state_idx, const uint8_t* has_init, int nheads,
               int headdim, int dstate, int ngroups, void* y, int64_t ld_y, int y_dtype,
               void* stream, bool launch) {
    if (!valid_dtype(act_dtype) || !valid_dtype(y_dtype))
        return fail(M2_ERR_DTYPE, "decode: act_dtype and y_dtype must be M2_F32 or M2_BF16");
    if (batch < 0 || n_slots <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return fail(M2_ERR_SHAPE, "decode: batch must be >= 0 and n_slots, nheads, headdim, dstate, ngroups positive");
    if (nheads % ngroups) return fail(M2_ERR_SHAPE, "decode: nheads %% ngroups != 0 (%d, %d)", nheads, ngroups);
    if (!state_idx && n_slots < batch) return fail(M2_ERR_SHAPE, "decode: state_idx NULL needs n_slots >= batch");
    if (!m2::decode_supported(nheads, ngroups, headdim, dstate))
        return fail(M2_ERR_UNSUPPORTED, "decode: no kernel for headdim=%d dstate=%d with group width %d",
                    headdim, dstate, nheads / ngroups * headdim);
    const int64_t di = (int64_t)nheads * headdim, gn = (int64_t)ngroups * dstate;
    if (ld_x < di || ld_B < gn || ld_C < gn || ld_z < di || ld_dt < nheads || ld_y < di)
        return fail(M2_ERR_STRIDE, "decode: a row stride is smaller than its row width");
    if (batch == 0) return M2_OK;
    if (!x || !B || !C || !z || !dt || !A || !conv_w || !norm_w || !conv_state || !ssm_state || !y)
        return fail(M2_ERR_NULL, "decode: x, B, C, z, dt, A, conv_w, norm_w, both states and y are required");
    if (!aligned16(conv_w) || !aligned16(ssm_state))
        return fail(M2_ERR_ALIGN, "decode: conv_w and ssm_state must be 16-byte aligned");
    if (debug_enabled() && state_idx) {
        std::vector<int32_t> hidx(batch);
        if (hipMemcpy(hidx.data(), state_idx, sizeof(int32_t) * batch, hipMemcpyDeviceToHost) != hipSuccess)
            return fail(M2_ERR_HIP, "debug: reading state_idx failed");
        std::vector<char> seen(n_slots, 0);
        for (int b = 0; b < batch; ++b) {
            if (hidx[b] < 0 || hidx[b] >= n_slots)
                return fail(M2_ERR_SHAPE, "debug: state_idx[%d]=%d outside [0, %d)", b, hidx[b], n_slots);
            if (seen[hidx[b]]++)
                return fail(M2_ERR_SHAPE, "debug: state_idx[%d]=%d repeats a slot", b, hidx[b]);
        }
    }
    if (!launch) return M2_OK;
    m2::DecodeArgs a{};
    a.x = x; a.ld_x = ld_x; a.B = B; a.ld_B = ld_B; a.C = C; a.ld_C = ld_C; a.z = z; a.ld_z = ld_z;
    a.act_dtype = act_dtype; a.dt = dt; a.ld_dt = ld_dt; a.dt_softplus = dt_softplus;
    a.dt_bias = dt_bias; a.A = A; a.D = D;
    a.conv_w = conv_w; a.conv_b = conv_b; a.norm_w = norm_w; a.eps = eps;
    a.norm_before_gate = norm_before_gate; a.conv_state = conv_state; a.ssm_state = ssm_state;
    a.batch = batch; a.state_idx = state_idx; a.has_init = has_init;
    a.nheads = nheads; a.headdim = headdim; a.dstate = dstate; a.ngroups = ngroups;
    a.y = y; a.ld_y = ld_y; a.y_dtype = y_dtype;
    int st;
    if ((st = hip_status(m2::launch_decode_step(a, static_cast<hipStream_t>(stream)), "decode launch"))) return st;
    g_counters.decode++;
    return M2_OK;
}

// Views of one packed in-projection row: z | x | B | C | raw dt, in that order.
struct RowViews {
    const char *z, *x, *B, *C, *dt;
};
RowViews row_views(const void* row, int es, int nheads, int headdim, int dstate, int ngroups) {
    const int64_t di = (int64_t)nheads * headdim, gn = (int64_t)ngroups * dstate;
    const char* r = static_cast<const char*>(row);
    return RowViews{r, r + di * es, r + 2 * di * es, r + (2 * di + gn) * es, r + (2 * di + 2 * gn) * es};
}

// A second stream for the decode rows of a mixed batch, so that they stream
// their states while the prefill chain runs its latency-bound phases.  One per
// thread and device, created on first use at the default priority (with the
// fork / join events) and kept until the process ends; nullptr when it cannot
// be made, and the decode rows then run on the caller's stream.
struct SideStream {
    hipStream_t s;
    hipEvent_t fork, join;
};
SideStream* side_stream() {
    thread_local std::vector<SideStream> sides;   // by device
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
    if ((int)sides.size() <= dev) sides.resize(dev + 1, SideStream{nullptr, nullptr, nullptr});
    SideStream& sd = sides[dev];
    if (sd.s) return &sd;
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
        if (f) (void)hipEventDestroy(f);
        (void)hipStreamDestroy(st);
        return nullptr;
    }
    sd = SideStream{st, f, j};
    return &sd;
}

int64_t row_width(int nheads, int headdim, int dstate, int ngroups) {
    return 2 * (int64_t)nheads * headdim + 2 * (int64_t)ngroups * dstate + nheads;
}

size_t step_size_bytes(int64_t total_tokens, int nheads) {
    return (size_t)round256((total_tokens > 0 ? total_tokens : 1) * (int64_t)nheads * 4);
}

// Prefill from packed rows: the step-size kernel writes fp32 dt after the
// prefill's own workspace, then the chain runs with it.
int prefill_inproj_run(const void* row, int64_t ld_row, int act_dtype, const float* dt_bias,
                       const float* A, const float* D, const float* conv_w, const float* conv_b,
                       const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                       float* ssm_state, int n_slots, const int32_t* cu_seqlens, int batch,
                       int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                       const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                       int chunk_size, void* y, int64_t ld_y, int y_dtype, void* workspace,
                       size_t ws_bytes, void* stream, bool launch) {
    if (!row && total_tokens > 0) return fail(M2_ERR_NULL, "prefill_inproj: the in-projection rows are required");
    if (!valid_dtype(act_dtype)) return fail(M2_ERR_DTYPE, "prefill_inproj: act_dtype must be M2_F32 or M2_BF16");
    if (nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return fail(M2_ERR_SHAPE, "prefill_inproj: nheads, headdim, dstate, ngroups must be positive");
    if (ld_row < row_width(nheads, headdim, dstate, ngroups))
        return fail(M2_ERR_STRIDE, "prefill_inproj: ld_row %lld is below the row width %lld",
                    (long long)ld_row, (long long)row_width(nheads, headdim, dstate, ngroups));
    const size_t pws = mamba2_prefill_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim,
                                                     dstate, ngroups, chunk_size, act_dtype);
    const size_t need = pws + step_size_bytes(total_tokens, nheads);
    if (!workspace || ws_bytes < need)
        return fail(M2_ERR_WORKSPACE, "prefill_inproj: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (!aligned16(workspace)) return fail(M2_ERR_ALIGN, "prefill_inproj: workspace must be 16-byte aligned");
    float* dt = reinterpret_cast<float*>(static_cast<char*>(workspace) + pws);
    const RowViews v = row ? row_views(row, elem_size(act_dtype), nheads, headdim, dstate, ngroups)
                           : RowViews{nullptr, nullptr, nullptr, nullptr, nullptr};
    auto chain = [&](bool go) {
        return prefill_run(v.x, ld_row, v.B, ld_row, v.C, ld_row, v.z, ld_row, act_dtype, dt, nheads,
                           A, D, conv_w, conv_b, norm_w, eps, norm_before_gate, conv_state,
                           ssm_state, n_slots, cu_seqlens, batch, total_tokens, max_seqlen,
                           state_idx, has_init, nheads, headdim, dstate, ngroups, chunk_size, y,
                           ld_y, y_dtype, workspace, pws, stream, go);
    };
    int st = chain(false);
    if (st || !launch) return st;
    if ((st = hip_status(m2::launch_step_size(v.dt, ld_row, act_dtype, dt_bias, nheads, total_tokens, dt,
                                              static_cast<hipStream_t>(stream)),
                         "step size launch")))
        return st;
    return chain(true);
}

int decode_inproj_run(const void* row, int64_t ld_row, int act_dtype, const float* dt_bias,
                      const float* A, const float* D, const float* conv_w, const float* conv_b,
                      const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                      float* ssm_state, int n_slots, int batch, const int32_t* state_idx,
                      const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                      void* y, int64_t ld_y, int y_dtype, void* stream, bool launch) {
    if (!valid_dtype(act_dtype)) return fail(M2_ERR_DTYPE, "decode_inproj: act_dtype must be M2_F32 or M2_BF16");
    if (nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0)
        return fail(M2_ERR_SHAPE, "decode_inproj: nheads, headdim, dstate, ngroups must be positive");
    if (ld_row < row_width(nheads, headdim, dstate, ngroups))
        return fail(M2_ERR_STRIDE, "decode_inproj: ld_row %lld is below the row width %lld",
                    (long long)ld_row, (long long)row_width(nheads, headdim, dstate, ngroups));
    if (batch > 0 && !row) return fail(M2_ERR_NULL, "decode_inproj: the in-projection rows are required");
    const RowViews v = row ? row_views(row, elem_size(act_dtype), nheads, headdim, dstate, ngroups)
                           : RowViews{nullptr, nullptr, nullptr, nullptr, nullptr};
    return decode_run(v.x, ld_row, v.B, ld_row, v.C, ld_row, v.z, ld_row, act_dtype, v.dt, ld_row, 1,
                      dt_bias, A, D, conv_w, conv_b, norm_w, eps, norm_before_gate, conv_state,
                      ssm_state, n_slots, batch, state_idx, has_init, nheads, headdim, dstate,
                      ngroups, y, ld_y, y_dtype, stream, launch);
}

}  // namespace

extern "C" {

int mamba2_prefill(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                   int64_t ld_C, const void* z, int64_t ld_z, int act_dtype, const float* dt,
                   int64_t ld_dt, const float* A, const float* D, const float* conv_w,
                   const float* conv_b, const float* norm_w, float eps, int norm_before_gate,
                   float* conv_state, float* ssm_state, int n_slots, const int32_t* cu_seqlens,
                   int batch, int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                   const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                   int chunk_size, void* y, int64_t ld_y, int y_dtype, void* workspace,
                   size_t ws_bytes, void* stream) {
    auto run = [&](bool launch) {
        return prefill_run(x, ld_x, B, ld_B, C, ld_C, z, ld_z, act_dtype, dt, ld_dt, A, D, conv_w, conv_b,
                           norm_w, eps, norm_before_gate, conv_state, ssm_state, n_slots, cu_seqlens,
                           batch, total_tokens, max_seqlen, state_idx, has_init, nheads, headdim,
                           dstate, ngroups, chunk_size, y, ld_y, y_dtype, workspace, ws_bytes, stream,
                           launch);
    };
    int st;
    if (debug_enabled()) {  // the arguments are checked before dt and A are read
        if ((st = run(false)) || (st = debug_check_dt_A(dt, ld_dt, total_tokens, nheads, A))) return st;
    }
    st = run(true);
    return st ? st : ok();
}

}  // extern "C"

namespace {

// Scratch of mamba2_prefill_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never uses
// its name as an address (on the host it is a stand-in symbol); the device
// address of each GPU's copy is looked up once per device and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // by device ordinal; nullptr until looked up

// The current device's copy of `scratch`, or nullptr (with the error set).
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        fail(M2_ERR_HIP, "prefill_noalloc: hipGetDevice failed");
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(M2_ERR_HIP, "prefill_noalloc: hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t mamba2_prefill_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

int mamba2_prefill_noalloc(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                           int64_t ld_C, const void* z, int64_t ld_z, int act_dtype, const float* dt,
                           int64_t ld_dt, const float* A, const float* D, const float* conv_w,
                           const float* conv_b, const float* norm_w, float eps, int norm_before_gate,
                           float* conv_state, float* ssm_state, int n_slots, const int32_t* cu_seqlens,
                           int batch, int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                           const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                           int chunk_size, void* y, int64_t ld_y, int y_dtype, void* stream) {
    const size_t need = mamba2_prefill_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim,
                                                      dstate, ngroups, chunk_size, act_dtype);
    if (need > kNoAllocScratchBytes)
        return fail(M2_ERR_WORKSPACE,
                    "prefill_noalloc: these sizes need %zu bytes of scratch, above the library's %zu",
                    need, kNoAllocScratchBytes);
    // every argument check runs before the device scratch is looked up
    auto run = [&](bool launch, void* ws) {
        return prefill_run(x, ld_x, B, ld_B, C, ld_C, z, ld_z, act_dtype, dt, ld_dt, A, D, conv_w, conv_b,
                           norm_w, eps, norm_before_gate, conv_state, ssm_state, n_slots, cu_seqlens,
                           batch, total_tokens, max_seqlen, state_idx, has_init, nheads, headdim,
                           dstate, ngroups, chunk_size, y, ld_y, y_dtype, ws,
                           ws ? kNoAllocScratchBytes : 0, stream, launch);
    };
    int st;
    // The argument checks run first, also on a machine without a GPU: a dry run
    // (no launch, nothing dereferenced) with a host stand-in for the workspace.
    alignas(256) static unsigned char dry_ws[256];
    if ((st = run(false, need > 0 ? dry_ws : nullptr))) return st;
    if (debug_enabled() && (st = debug_check_dt_A(dt, ld_dt, total_tokens, nheads, A))) return st;
    void* ws = nullptr;
    if (need > 0 && !(ws = scratch_on_current_device())) return M2_ERR_HIP;
    st = run(true, ws);
    return st ? st : ok();
}

int mamba2_decode(const void* x, int64_t ld_x, const void* B, int64_t ld_B, const void* C,
                  int64_t ld_C, const void* z, int64_t ld_z, int act_dtype, const float* dt,
                  int64_t ld_dt, const float* A, const float* D, const float* conv_w,
                  const float* conv_b, const float* norm_w, float eps, int norm_before_gate,
                  float* conv_state, float* ssm_state, int n_slots, int batch,
                  const int32_t* state_idx, const uint8_t* has_init, int nheads, int headdim,
                  int dstate, int ngroups, void* y, int64_t ld_y, int y_dtype, void* stream) {
    auto run = [&](bool launch) {
        return decode_run(x, ld_x, B, ld_B, C, ld_C, z, ld_z, act_dtype, dt, ld_dt, 0, nullptr, A, D,
                          conv_w, conv_b, norm_w, eps, norm_before_gate, conv_state, ssm_state, n_slots,
                          batch, state_idx, has_init, nheads, headdim, dstate, ngroups, y, ld_y,
                          y_dtype, stream, launch);
    };
    int st;
    if (debug_enabled() && batch > 0) {
        if ((st = run(false)) || (st = debug_check_dt_A(dt, ld_dt, batch, nheads, A))) return st;
    }
    st = run(true);
    return st ? st : ok();
}

size_t mamba2_prefill_inproj_workspace_size(int64_t total_tokens, int batch, int max_seqlen,
                                            int nheads, int headdim, int dstate, int ngroups,
                                            int chunk_size, int act_dtype) {
    const size_t pws = mamba2_prefill_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim,
                                                     dstate, ngroups, chunk_size, act_dtype);
    if (pws == 0 && (total_tokens < 0 || batch <= 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 ||
                     ngroups <= 0 || !valid_dtype(act_dtype)))
        return 0;
    return pws + step_size_bytes(total_tokens, nheads);
}

int mamba2_prefill_inproj(const void* zxbcdt, int64_t ld_row, int act_dtype, const float* dt_bias,
                          const float* A, const float* D, const float* conv_w, const float* conv_b,
                          const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                          float* ssm_state, int n_slots, const int32_t* cu_seqlens, int batch,
                          int64_t total_tokens, int max_seqlen, const int32_t* state_idx,
                          const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                          int chunk_size, void* y, int64_t ld_y, int y_dtype, void* workspace,
                          size_t ws_bytes, void* stream) {
    auto run = [&](bool launch) {
        return prefill_inproj_run(zxbcdt, ld_row, act_dtype, dt_bias, A, D, conv_w, conv_b, norm_w, eps,
                                  norm_before_gate, conv_state, ssm_state, n_slots, cu_seqlens, batch,
                                  total_tokens, max_seqlen, state_idx, has_init, nheads, headdim, dstate,
                                  ngroups, chunk_size, y, ld_y, y_dtype, workspace, ws_bytes, stream,
                                  launch);
    };
    int st;
    if (debug_enabled()) {  // raw step sizes take any sign; A is checked
        if ((st = run(false)) || (st = debug_check_dt_A(nullptr, 0, 0, nheads, A))) return st;
    }
    st = run(true);
    return st ? st : ok();
}

int mamba2_decode_inproj(const void* zxbcdt, int64_t ld_row, int act_dtype, const float* dt_bias,
                         const float* A, const float* D, const float* conv_w, const float* conv_b,
                         const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                         float* ssm_state, int n_slots, int batch, const int32_t* state_idx,
                         const uint8_t* has_init, int nheads, int headdim, int dstate, int ngroups,
                         void* y, int64_t ld_y, int y_dtype, void* stream) {
    auto run = [&](bool launch) {
        return decode_inproj_run(zxbcdt, ld_row, act_dtype, dt_bias, A, D, conv_w, conv_b, norm_w, eps,
                                 norm_before_gate, conv_state, ssm_state, n_slots, batch, state_idx,
                                 has_init, nheads, headdim, dstate, ngroups, y, ld_y, y_dtype, stream,
                                 launch);
    };
    int st;
    if (debug_enabled() && batch > 0) {
        if ((st = run(false)) || (st = debug_check_dt_A(nullptr, 0, 0, nheads, A))) return st;
    }
    st = run(true);
    return st ? st : ok();
}

size_t mamba2_mixed_inproj_workspace_size(int64_t total_tokens, int batch, int max_seqlen,
                                          int nheads, int headdim, int dstate, int ngroups,
                                          int chunk_size, int act_dtype) {
    const size_t pws = mamba2_prefill_inproj_workspace_size(total_tokens, batch, max_seqlen, nheads,
                                                            headdim, dstate, ngroups, chunk_size,
                                                            act_dtype);
    if (pws == 0) return 0;
    // The prefill part is a sub-batch of batch - num_decodes sequences, and the
    // fp64 path's segment buffers do not grow with the batch (a smaller batch
    // can be split where a larger one is not): room for the largest of them.
    size_t seg_any = 0;
    if (act_dtype == M2_F32 && scan_states_bytes(total_tokens, batch, nheads, headdim, dstate, ngroups,
                                                 chunk_size, act_dtype) == 0) {
        for (int b = 1; b <= batch && (int64_t)b * nheads < 256; ++b) {
            const size_t v = m2::one_pass_seg_bytes(b, nheads, headdim, dstate, m2::kPolicyF64);
            if (v > seg_any) seg_any = v;
        }
    }
    return (size_t)(round256((int64_t)(batch + 1) * 4) + round256((int64_t)batch * 4)) + pws + seg_any;
}

int mamba2_mixed_inproj(const void* zxbcdt, int64_t ld_row, int act_dtype, const float* dt_bias,
                        const float* A, const float* D, const float* conv_w, const float* conv_b,
                        const float* norm_w, float eps, int norm_before_gate, float* conv_state,
                        float* ssm_state, int n_slots, const int32_t* cu_seqlens, int batch,
                        int num_decodes, int64_t total_tokens, int max_seqlen,
                        const int32_t* state_idx, const uint8_t* has_init, int nheads, int headdim,
                        int dstate, int ngroups, int chunk_size, void* y, int64_t ld_y, int y_dtype,
                        void* workspace, size_t ws_bytes, void* stream) {
    if (batch <= 0) return fail(M2_ERR_SHAPE, "mixed: batch must be positive (got %d)", batch);
    if (num_decodes < 0 || num_decodes > batch)
        return fail(M2_ERR_SHAPE, "mixed: num_decodes %d outside [0, batch=%d]", num_decodes, batch);
    if (total_tokens < num_decodes)
        return fail(M2_ERR_SHAPE, "mixed: total_tokens %lld is below num_decodes %d", (long long)total_tokens,
                    num_decodes);
    if (!cu_seqlens) return fail(M2_ERR_NULL, "mixed: cu_seqlens is required");
    if (!state_idx && n_slots < batch) return fail(M2_ERR_SHAPE, "mixed: state_idx NULL needs n_slots >= batch");
    if (!valid_dtype(act_dtype) || !valid_dtype(y_dtype))
        return fail(M2_ERR_DTYPE, "mixed: act_dtype and y_dtype must be M2_F32 or M2_BF16");
    const size_t need = mamba2_mixed_inproj_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim,
                                                           dstate, ngroups, chunk_size, act_dtype);
    if (need == 0) return fail(M2_ERR_SHAPE, "mixed: nheads, headdim, dstate, ngroups must be positive");
    if (!workspace || ws_bytes < need)
        return fail(M2_ERR_WORKSPACE, "mixed: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (!aligned16(workspace)) return fail(M2_ERR_ALIGN, "mixed: workspace must be 16-byte aligned");
    if (debug_enabled()) {
        int st = debug_check_indices(cu_seqlens, batch, total_tokens, max_seqlen, state_idx, n_slots);
        if (st) return st;
        std::vector<int32_t> hcu(num_decodes + 1);
        if (hipMemcpy(hcu.data(), cu_seqlens, sizeof(int32_t) * (num_decodes + 1), hipMemcpyDeviceToHost) != hipSuccess)
            return fail(M2_ERR_HIP, "debug: reading cu_seqlens failed");
        for (int b = 0; b <= num_decodes; ++b)
            if (hcu[b] != b) return fail(M2_ERR_SHAPE, "debug: decode sequence %d is not one row at row %d", b, b);
        if (A && (st = debug_check_dt_A(nullptr, 0, 0, nheads, A))) return st;
    }
    const int np = batch - num_decodes;
    const int64_t tp = total_tokens - num_decodes;
    const int es = elem_size(act_dtype);
    char* wsb = static_cast<char*>(workspace);
    int32_t* cu_p = reinterpret_cast<int32_t*>(wsb);
    int32_t* slot_p = reinterpret_cast<int32_t*>(wsb + round256((int64_t)(batch + 1) * 4));
    char* pws = wsb + round256((int64_t)(batch + 1) * 4) + round256((int64_t)batch * 4);
    const size_t pws_bytes = ws_bytes - (size_t)(pws - wsb);
    const char* row_p = zxbcdt ? static_cast<const char*>(zxbcdt) + (int64_t)num_decodes * ld_row * es : nullptr;
    char* y_p = y ? static_cast<char*>(y) + (int64_t)num_decodes * ld_y * elem_size(y_dtype) : nullptr;
    const int32_t* idx_p = state_idx ? state_idx + num_decodes : slot_p;
    const uint8_t* init_p = has_init ? has_init + num_decodes : nullptr;
    struct Scope {  // the parts skip per-call debug reads (checked above)
        Scope() { g_parts_of_checked_batch = true; }
        ~Scope() { g_parts_of_checked_batch = false; }
    } scope;
    auto decode_part = [&](bool go, void* strm) {
        return decode_inproj_run(zxbcdt, ld_row, act_dtype, dt_bias, A, D, conv_w, conv_b, norm_w, eps,
                                 norm_before_gate, conv_state, ssm_state, n_slots, num_decodes,
                                 state_idx, has_init, nheads, headdim, dstate, ngroups, y, ld_y,
                                 y_dtype, strm, go);
    };
    auto prefill_part = [&](bool go) {
        return prefill_inproj_run(row_p, ld_row, act_dtype, dt_bias, A, D, conv_w, conv_b, norm_w, eps,
                                  norm_before_gate, conv_state, ssm_state, n_slots, cu_p, np, tp,
                                  max_seqlen, idx_p, init_p, nheads, headdim, dstate, ngroups,
                                  chunk_size, y_p, ld_y, y_dtype, pws, pws_bytes, stream, go);
    };
    int st;
    if (num_decodes > 0 && (st = decode_part(false, stream))) return st;
    if (np > 0 && (st = prefill_part(false))) return st;
    // The two parts touch disjoint rows, slots and workspace: with both present
    // the decode rows go to the side stream, forked from and joined back into
    // the caller's stream.
    hipStream_t cs = static_cast<hipStream_t>(stream);
    SideStream* sd = (num_decodes > 0 && np > 0) ? side_stream() : nullptr;
    if (sd) {
        if ((st = hip_status(hipEventRecord(sd->fork, cs), "mixed fork record"))) return st;
        if ((st = hip_status(hipStreamWaitEvent(sd->s, sd->fork, 0), "mixed fork wait"))) return st;
        if ((st = decode_part(true, sd->s))) return st;
        if ((st = hip_status(hipEventRecord(sd->join, sd->s), "mixed join record"))) return st;
    } else if (num_decodes > 0 && (st = decode_part(true, stream))) {
        return st;
    }
    if (np > 0) {
        st = hip_status(m2::launch_rebase(cu_seqlens, num_decodes, np, (int32_t)tp, cu_p,
                                          state_idx ? nullptr : slot_p, cs),
                        "mixed rebase launch");
        if (!st) st = prefill_part(true);
    }
    // join even after a failed prefill launch, so the caller's stream never runs ahead
    if (sd) {
        const int sj = hip_status(hipStreamWaitEvent(cs, sd->join, 0), "mixed join wait");
        if (!st) st = sj;
    }
    return st ? st : ok();
}

int m2_timing_enable(int max_calls) {
    if (max_calls < 0) return fail(M2_ERR_SHAPE, "m2_timing_enable: max_calls < 0");
    for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
    g_timing.ev.clear();
    g_timing.used = 0;
    g_timing.max_calls = 0;
    if (max_calls == 0) return ok();
    g_timing.ev.resize((size_t)kEv * max_calls);
    g_timing.stage.assign((size_t)(kEv - 1) * max_calls, 0);
    for (auto& e : g_timing.ev) {
        const hipError_t r = hipEventCreate(&e);
        if (r != hipSuccess) {
            g_timing.ev.clear();
            return fail(M2_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(r));
        }
    }
    g_timing.max_calls = max_calls;
    return ok();
}

int m2_timing_read(m2_kernel_times* out) {
    if (!out) return fail(M2_ERR_NULL, "m2_timing_read: out is NULL");
    *out = m2_kernel_times{};
    double* dst[kEv - 1] = {&out->conv_ms, &out->conv_state_ms, &out->scan_pass_ms, &out->scan_out_ms,
                            &out->norm_ms};
    for (int c = 0; c < g_timing.used; ++c) {
        hipEvent_t* e = &g_timing.ev[kEv * c];
        const hipError_t r = hipEventSynchronize(e[kEv - 1]);
        if (r != hipSuccess) return fail(M2_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(r));
        for (int k = 0; k < kEv - 1; ++k) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, e[k], e[k + 1]) != hipSuccess) ms = 0.f;
            *dst[g_timing.stage[(size_t)(kEv - 1) * c + k]] += ms;
        }
    }
    out->calls = (uint64_t)g_timing.used;
    g_timing.used = 0;
    return ok();
}

}  // extern "C"
