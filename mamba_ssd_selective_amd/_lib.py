"""ctypes binding of libm2ssd.so (the C ABI declared in include/m2ssd.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.
There is no fallback: if the library is missing or a call fails, this raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# M2SSD_LIB names another build of the same library (the ABI tests load the
# host-sanitized one this way); by default the in-tree libm2ssd.so.
LIB_PATH = os.environ.get("M2SSD_LIB") or os.path.join(_PKG, "libm2ssd.so")

M2_F32 = 0
M2_BF16 = 1

_STATUS = {0: "M2_OK", -1: "M2_ERR_NULL", -2: "M2_ERR_SHAPE", -3: "M2_ERR_DTYPE",
           -4: "M2_ERR_CHUNK", -5: "M2_ERR_STRIDE", -6: "M2_ERR_ALIGN",
           -7: "M2_ERR_UNSUPPORTED", -8: "M2_ERR_WORKSPACE", -9: "M2_ERR_HIP"}


class M2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Counters(ctypes.Structure):
    _fields_ = [("conv_launches", ctypes.c_uint64), ("conv_state_launches", ctypes.c_uint64),
                ("scan_f64_launches", ctypes.c_uint64), ("scan_bf16x3_launches", ctypes.c_uint64),
                ("norm_launches", ctypes.c_uint64), ("prefill_calls", ctypes.c_uint64),
                ("scan_chunked_launches", ctypes.c_uint64), ("decode_launches", ctypes.c_uint64)]


class KernelTimes(ctypes.Structure):
    _fields_ = [("conv_ms", ctypes.c_double), ("conv_state_ms", ctypes.c_double),
                ("scan_pass_ms", ctypes.c_double), ("scan_out_ms", ctypes.c_double),
                ("norm_ms", ctypes.c_double),
                ("calls", ctypes.c_uint64)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "m2_last_error": (ctypes.c_char_p, []),
    "m2_version": (ctypes.c_char_p, []),
    "m2_get_counters": (_I, [ctypes.POINTER(Counters)]),
    "m2_reset_counters": (None, []),
    "m2_timing_enable": (_I, [_I]),
    "m2_timing_read": (_I, [ctypes.POINTER(KernelTimes)]),
    "mamba2_conv_rows": (_I, [_P, _L, _P, _L, _P, _L, _I, _I, _I, _P, _P, _I, _P, _I,
                              _P, _I, _L, _I, _P, _P, _I, _P, _L, _I, _P]),
    "ssd_chunk_scan": (_I, [_P, _L, _P, _L, _P, _L, _I, _P, _L, _P, _P, _P, _I,
                            _P, _I, _L, _I, _P, _P, _I, _I, _I, _I, _I, _P, _L, _P,
                            ctypes.c_size_t, _P]),
    "ssd_chunk_scan_workspace_size": (ctypes.c_size_t, [_L, _I, _I, _I, _I, _I, _I, _I]),
    "ssd_chunk_scan_plan": (_I, [_L, _I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(_I), ctypes.POINTER(_I),
                                 ctypes.POINTER(_I)]),
    "gated_rmsnorm_group": (_I, [_P, _L, _P, _L, _I, _P, _F, _I, _I, _L, _I, _P, _L, _I, _P]),
    "mamba2_prefill_workspace_size": (ctypes.c_size_t, [_L, _I, _I, _I, _I, _I, _I, _I, _I]),
    "mamba2_prefill": (_I, [_P, _L, _P, _L, _P, _L, _P, _L, _I, _P, _L, _P, _P, _P, _P, _P,
                            _F, _I, _P, _P, _I, _P, _I, _L, _I, _P, _P, _I, _I, _I, _I, _I,
                            _P, _L, _I, _P, ctypes.c_size_t, _P]),
    "mamba2_prefill_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "mamba2_prefill_noalloc": (_I, [_P, _L, _P, _L, _P, _L, _P, _L, _I, _P, _L, _P, _P, _P, _P, _P,
                                    _F, _I, _P, _P, _I, _P, _I, _L, _I, _P, _P, _I, _I, _I, _I, _I,
                                    _P, _L, _I, _P]),
    "mamba2_decode": (_I, [_P, _L, _P, _L, _P, _L, _P, _L, _I, _P, _L, _P, _P, _P, _P, _P,
                           _F, _I, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _L, _I, _P]),
    "mamba2_prefill_inproj_workspace_size": (ctypes.c_size_t, [_L, _I, _I, _I, _I, _I, _I, _I, _I]),
    "mamba2_prefill_inproj": (_I, [_P, _L, _I, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _I, _P, _I,
                                   _L, _I, _P, _P, _I, _I, _I, _I, _I, _P, _L, _I, _P,
                                   ctypes.c_size_t, _P]),
    "mamba2_decode_inproj": (_I, [_P, _L, _I, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _I, _I, _P,
                                  _P, _I, _I, _I, _I, _P, _L, _I, _P]),
    "mamba2_mixed_inproj_workspace_size": (ctypes.c_size_t, [_L, _I, _I, _I, _I, _I, _I, _I, _I]),
    "mamba2_mixed_inproj": (_I, [_P, _L, _I, _P, _P, _P, _P, _P, _P, _F, _I, _P, _P, _I, _P, _I, _I,
                                 _L, _I, _P, _P, _I, _I, _I, _I, _I, _P, _L, _I, _P,
                                 ctypes.c_size_t, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libm2ssd.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mamba_ssd_selective_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise M2Error(status, load().m2_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return M2_F32
    if t.dtype == torch.bfloat16:
        return M2_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a 2-D tensor with unit inner stride on the GPU."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() == 2 and t.numel() == 0:
        return t.size(1)   # no rows to read: any stride will do (torch may report 0)
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit inner stride")
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _vec(t: Optional[torch.Tensor], name: str, dtype) -> None:
    if t is None:
        return
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def cu_seqlens_of(seq_lens: Sequence[int], device) -> torch.Tensor:
    """Packed-batch row offsets [0, L0, L0+L1, ...] as int32 on `device` (host cumsum)."""
    cu = [0]
    for L in seq_lens:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def version() -> str:
    return load().m2_version().decode()


def get_counters() -> dict:
    c = Counters()
    _check(load().m2_get_counters(ctypes.byref(c)))
    return {f: getattr(c, f) for f, _ in Counters._fields_}


def reset_counters() -> None:
    load().m2_reset_counters()


def timing_enable(max_calls: int) -> None:
    """Record HIP events around each kernel of the next `max_calls` mamba2_prefill calls."""
    _check(load().m2_timing_enable(int(max_calls)))


def timing_read() -> dict:
    """Summed per-kernel milliseconds and the number of recorded calls (waits for the events)."""
    t = KernelTimes()
    _check(load().m2_timing_read(ctypes.byref(t)))
    return {f: getattr(t, f) for f, _ in KernelTimes._fields_}


def mamba2_conv_rows(x, B, C, conv_w, conv_b, conv_state, cu_seqlens, max_seqlen,
                     state_idx=None, has_init=None, apply_silu=True, out=None,
                     out_dtype=torch.float32):
    """Causal depthwise conv1d (+SiLU) of x | B | C; advances conv_state in place.

    x [T, d_x], B and C [T, d_b] (or None with d_b = 0), conv_w [conv_dim, 4],
    conv_b [conv_dim] or None, conv_state [n_slots, 3, conv_dim] fp32.
    Returns out [T, conv_dim].
    """
    lib = load()
    T = x.size(0)
    d_x = x.size(1)
    d_b = 0 if B is None else B.size(1)
    conv_dim = d_x + 2 * d_b
    if out is None:
        out = torch.empty((T, conv_dim), dtype=out_dtype, device=x.device)
    _vec(conv_w, "conv_w", torch.float32)
    _vec(conv_b, "conv_b", torch.float32)
    _vec(conv_state, "conv_state", torch.float32)
    _vec(cu_seqlens, "cu_seqlens", torch.int32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    st = lib.mamba2_conv_rows(
        _ptr(x), _rows(x, "x"), _ptr(B), _rows(B, "B") if B is not None else 0,
        _ptr(C), _rows(C, "C") if C is not None else 0, d_x, d_b, _dtype_code(x),
        _ptr(conv_w), _ptr(conv_b), conv_w.size(1), _ptr(conv_state), conv_state.size(0),
        _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, int(max_seqlen), _ptr(state_idx),
        _ptr(has_init), int(bool(apply_silu)), _ptr(out), _rows(out, "out"), _dtype_code(out),
        _stream())
    _check(st)
    return out


def ssd_chunk_scan_workspace_size(total_tokens, batch, nheads, headdim, dstate, ngroups,
                                  chunk_size=128, act_dtype=torch.bfloat16) -> int:
    code = M2_BF16 if act_dtype == torch.bfloat16 else M2_F32
    return int(load().ssd_chunk_scan_workspace_size(total_tokens, batch, nheads, headdim, dstate,
                                                    ngroups, chunk_size, code))


def ssd_chunk_scan_plan(total_tokens, batch, max_seqlen, nheads, headdim, dstate, ngroups,
                        chunk_size=128, act_dtype=torch.bfloat16):
    """The chunk-parallel scan's work split for these sizes: (out_split, seg, seg_levels)."""
    code = M2_BF16 if act_dtype == torch.bfloat16 else M2_F32
    o, sg, lv = _I(0), _I(0), _I(0)
    _check(load().ssd_chunk_scan_plan(total_tokens, batch, max_seqlen, nheads, headdim, dstate, ngroups,
                                      chunk_size, code, ctypes.byref(o), ctypes.byref(sg), ctypes.byref(lv)))
    return o.value, sg.value, lv.value


def ssd_chunk_scan(x, B, C, dt, A, D, ssm_state, cu_seqlens, max_seqlen, nheads, headdim,
                   dstate, ngroups, chunk_size=128, state_idx=None, has_init=None, y=None,
                   workspace=None):
    """Chunked selective scan from post-conv x [T, H*P], B, C [T, G*N]; returns pre-norm y (fp32).

    workspace: uint8 device tensor of at least ssd_chunk_scan_workspace_size() bytes
    (allocated here when None and the size is nonzero).
    """
    lib = load()
    T = x.size(0)
    batch = cu_seqlens.numel() - 1
    need = ssd_chunk_scan_workspace_size(T, batch, nheads, headdim, dstate, ngroups, chunk_size,
                                         x.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if y is None:
        y = torch.empty((T, nheads * headdim), dtype=torch.float32, device=x.device)
    for t, n in ((A, "A"), (D, "D"), (ssm_state, "ssm_state")):
        _vec(t, n, torch.float32)
    _vec(cu_seqlens, "cu_seqlens", torch.int32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if dt.dtype != torch.float32:
        raise ValueError("dt must be float32")
    if B.dtype != x.dtype or C.dtype != x.dtype:
        raise ValueError("x, B and C must share one dtype")
    st = lib.ssd_chunk_scan(
        _ptr(x), _rows(x, "x"), _ptr(B), _rows(B, "B"), _ptr(C), _rows(C, "C"), _dtype_code(x),
        _ptr(dt), _rows(dt, "dt"), _ptr(A), _ptr(D), _ptr(ssm_state), ssm_state.size(0),
        _ptr(cu_seqlens), cu_seqlens.numel() - 1, T, int(max_seqlen), _ptr(state_idx),
        _ptr(has_init), nheads, headdim, dstate, ngroups, chunk_size, _ptr(y), _rows(y, "y"),
        _ptr(workspace), ws_bytes, _stream())
    _check(st)
    return y


def gated_rmsnorm_group(y, z, norm_w, ngroups, eps=1e-5, norm_before_gate=True, out=None,
                        out_dtype=torch.float32):
    """Grouped RMSNorm of y [T, d] with the SiLU(z) gate; out may be y itself (fp32)."""
    lib = load()
    T, d = y.shape
    if out is None:
        out = torch.empty((T, d), dtype=out_dtype, device=y.device)
    if y.dtype != torch.float32:
        raise ValueError("y must be float32")
    _vec(norm_w, "norm_w", torch.float32)
    st = lib.gated_rmsnorm_group(
        _ptr(y), _rows(y, "y"), _ptr(z), _rows(z, "z"), _dtype_code(z), _ptr(norm_w),
        float(eps), ngroups, int(bool(norm_before_gate)), T, d, _ptr(out), _rows(out, "out"),
        _dtype_code(out), _stream())
    _check(st)
    return out


def mamba2_prefill_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim, dstate,
                                  ngroups, chunk_size=128, act_dtype=torch.bfloat16) -> int:
    code = M2_BF16 if act_dtype == torch.bfloat16 else M2_F32
    return int(load().mamba2_prefill_workspace_size(total_tokens, batch, max_seqlen, nheads,
                                                    headdim, dstate, ngroups, chunk_size, code))


def mamba2_prefill(x, B, C, z, dt, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                   cu_seqlens, max_seqlen, nheads, headdim, dstate, ngroups, chunk_size=128,
                   state_idx=None, has_init=None, eps=1e-5, norm_before_gate=True, y=None,
                   y_dtype=torch.float32, workspace=None):
    """The whole mixer core (conv + SiLU, chunked scan, D skip, gated group norm).

    x [T, H*P], B, C [T, G*N], z [T, H*P] (one activation dtype), dt [T, H] fp32,
    states advanced in place.  Returns y [T, H*P].
    """
    lib = load()
    T = x.size(0)
    batch = cu_seqlens.numel() - 1
    if y is None:
        y = torch.empty((T, nheads * headdim), dtype=y_dtype, device=x.device)
    need = mamba2_prefill_workspace_size(T, batch, max_seqlen, nheads, headdim, dstate,
                                         ngroups, chunk_size, x.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    for t, n in ((A, "A"), (D, "D"), (conv_w, "conv_w"), (conv_b, "conv_b"), (norm_w, "norm_w"),
                 (conv_state, "conv_state"), (ssm_state, "ssm_state")):
        _vec(t, n, torch.float32)
    _vec(cu_seqlens, "cu_seqlens", torch.int32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if dt.dtype != torch.float32:
        raise ValueError("dt must be float32")
    if not (x.dtype == B.dtype == C.dtype == z.dtype):
        raise ValueError("x, B, C and z must share one dtype")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.mamba2_prefill(
        _ptr(x), _rows(x, "x"), _ptr(B), _rows(B, "B"), _ptr(C), _rows(C, "C"),
        _ptr(z), _rows(z, "z"), _dtype_code(x), _ptr(dt), _rows(dt, "dt"), _ptr(A), _ptr(D),
        _ptr(conv_w), _ptr(conv_b), _ptr(norm_w), float(eps), int(bool(norm_before_gate)),
        _ptr(conv_state), _ptr(ssm_state), conv_state.size(0), _ptr(cu_seqlens), batch, T,
        int(max_seqlen), _ptr(state_idx), _ptr(has_init), nheads, headdim, dstate, ngroups,
        chunk_size, _ptr(y), _rows(y, "y"), _dtype_code(y), _ptr(workspace), ws_bytes, _stream())
    _check(st)
    return y


def mamba2_prefill_noalloc_scratch_bytes() -> int:
    """Size of the library's fixed device scratch used by mamba2_prefill_noalloc."""
    return int(load().mamba2_prefill_noalloc_scratch_bytes())


def mamba2_prefill_noalloc(x, B, C, z, dt, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                           cu_seqlens, max_seqlen, nheads, headdim, dstate, ngroups, chunk_size=128,
                           state_idx=None, has_init=None, eps=1e-5, norm_before_gate=True, y=None,
                           y_dtype=torch.float32):
    """mamba2_prefill with the library's own fixed device scratch instead of a
    workspace (no device allocation in the library; y is allocated here only
    when not given)."""
    lib = load()
    T = x.size(0)
    batch = cu_seqlens.numel() - 1
    if y is None:
        y = torch.empty((T, nheads * headdim), dtype=y_dtype, device=x.device)
    for t, n in ((A, "A"), (D, "D"), (conv_w, "conv_w"), (conv_b, "conv_b"), (norm_w, "norm_w"),
                 (conv_state, "conv_state"), (ssm_state, "ssm_state")):
        _vec(t, n, torch.float32)
    _vec(cu_seqlens, "cu_seqlens", torch.int32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if dt.dtype != torch.float32:
        raise ValueError("dt must be float32")
    if not (x.dtype == B.dtype == C.dtype == z.dtype):
        raise ValueError("x, B, C and z must share one dtype")
    st = lib.mamba2_prefill_noalloc(
        _ptr(x), _rows(x, "x"), _ptr(B), _rows(B, "B"), _ptr(C), _rows(C, "C"),
        _ptr(z), _rows(z, "z"), _dtype_code(x), _ptr(dt), _rows(dt, "dt"), _ptr(A), _ptr(D),
        _ptr(conv_w), _ptr(conv_b), _ptr(norm_w), float(eps), int(bool(norm_before_gate)),
        _ptr(conv_state), _ptr(ssm_state), conv_state.size(0), _ptr(cu_seqlens), batch, T,
        int(max_seqlen), _ptr(state_idx), _ptr(has_init), nheads, headdim, dstate, ngroups,
        chunk_size, _ptr(y), _rows(y, "y"), _dtype_code(y), _stream())
    _check(st)
    return y


def mamba2_decode(x, B, C, z, dt, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                  nheads, headdim, dstate, ngroups, state_idx=None, has_init=None, eps=1e-5,
                  norm_before_gate=True, y=None, y_dtype=torch.float32):
    """One decode token per sequence at its cache slot (conv update, state update,
    readout, D skip, gated group norm), both states advanced in place.

    x [batch, H*P], B, C [batch, G*N], z [batch, H*P] (one activation dtype),
    dt [batch, H] fp32.  Returns y [batch, H*P].
    """
    lib = load()
    batch = x.size(0)
    if y is None:
        y = torch.empty((batch, nheads * headdim), dtype=y_dtype, device=x.device)
    for t, n in ((A, "A"), (D, "D"), (conv_w, "conv_w"), (conv_b, "conv_b"), (norm_w, "norm_w"),
                 (conv_state, "conv_state"), (ssm_state, "ssm_state")):
        _vec(t, n, torch.float32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if dt.dtype != torch.float32:
        raise ValueError("dt must be float32")
    if not (x.dtype == B.dtype == C.dtype == z.dtype):
        raise ValueError("x, B, C and z must share one dtype")
    if conv_state.size(0) != ssm_state.size(0):
        raise ValueError("conv_state and ssm_state must have the same number of slots")
    st = lib.mamba2_decode(
        _ptr(x), _rows(x, "x"), _ptr(B), _rows(B, "B"), _ptr(C), _rows(C, "C"),
        _ptr(z), _rows(z, "z"), _dtype_code(x), _ptr(dt), _rows(dt, "dt"), _ptr(A), _ptr(D),
        _ptr(conv_w), _ptr(conv_b), _ptr(norm_w), float(eps), int(bool(norm_before_gate)),
        _ptr(conv_state), _ptr(ssm_state), conv_state.size(0), batch, _ptr(state_idx),
        _ptr(has_init), nheads, headdim, dstate, ngroups, _ptr(y), _rows(y, "y"),
        _dtype_code(y), _stream())
    _check(st)
    return y


def _inproj_common(row, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state, nheads,
                   headdim, dstate, ngroups):
    width = 2 * nheads * headdim + 2 * ngroups * dstate + nheads
    ld_row = _rows(row, "zxbcdt")
    if row.size(1) < width:
        raise ValueError(f"zxbcdt rows have {row.size(1)} channels, below z | xBC | dt = {width}")
    for t, n in ((dt_bias, "dt_bias"), (A, "A"), (D, "D"), (conv_w, "conv_w"), (conv_b, "conv_b"),
                 (norm_w, "norm_w"), (conv_state, "conv_state"), (ssm_state, "ssm_state")):
        _vec(t, n, torch.float32)
    if conv_state.size(0) != ssm_state.size(0):
        raise ValueError("conv_state and ssm_state must have the same number of slots")
    return ld_row


def mamba2_prefill_inproj_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim, dstate,
                                         ngroups, chunk_size=128, act_dtype=torch.bfloat16) -> int:
    code = M2_BF16 if act_dtype == torch.bfloat16 else M2_F32
    return int(load().mamba2_prefill_inproj_workspace_size(total_tokens, batch, max_seqlen, nheads,
                                                           headdim, dstate, ngroups, chunk_size, code))


def mamba2_prefill_inproj(zxbcdt, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                          cu_seqlens, max_seqlen, nheads, headdim, dstate, ngroups, chunk_size=128,
                          state_idx=None, has_init=None, eps=1e-5, norm_before_gate=True, y=None,
                          y_dtype=torch.float32, workspace=None):
    """The mixer core over packed in-projection rows zxbcdt [T, >= 2*H*P + 2*G*N + H]
    (z | x | B | C | raw dt); dt = softplus(raw + dt_bias) is formed on the device.
    States advance in place.  Returns y [T, H*P]."""
    lib = load()
    T = zxbcdt.size(0)
    batch = cu_seqlens.numel() - 1
    ld_row = _inproj_common(zxbcdt, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                            nheads, headdim, dstate, ngroups)
    _vec(cu_seqlens, "cu_seqlens", torch.int32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if y is None:
        y = torch.empty((T, nheads * headdim), dtype=y_dtype, device=zxbcdt.device)
    if workspace is None:
        need = mamba2_prefill_inproj_workspace_size(T, batch, max_seqlen, nheads, headdim, dstate,
                                                    ngroups, chunk_size, zxbcdt.dtype)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=zxbcdt.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.mamba2_prefill_inproj(
        _ptr(zxbcdt), ld_row, _dtype_code(zxbcdt), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(conv_w),
        _ptr(conv_b), _ptr(norm_w), float(eps), int(bool(norm_before_gate)), _ptr(conv_state),
        _ptr(ssm_state), conv_state.size(0), _ptr(cu_seqlens), batch, T, int(max_seqlen),
        _ptr(state_idx), _ptr(has_init), nheads, headdim, dstate, ngroups, chunk_size, _ptr(y),
        _rows(y, "y"), _dtype_code(y), _ptr(workspace), ws_bytes, _stream())
    _check(st)
    return y


def mamba2_decode_inproj(zxbcdt, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                         nheads, headdim, dstate, ngroups, state_idx=None, has_init=None, eps=1e-5,
                         norm_before_gate=True, y=None, y_dtype=torch.float32):
    """One decode token per sequence from packed in-projection rows (row b = sequence b),
    with dt = softplus(raw + dt_bias) formed in the decode kernel.  Returns y [batch, H*P]."""
    lib = load()
    batch = zxbcdt.size(0)
    ld_row = _inproj_common(zxbcdt, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                            nheads, headdim, dstate, ngroups)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if y is None:
        y = torch.empty((batch, nheads * headdim), dtype=y_dtype, device=zxbcdt.device)
    st = lib.mamba2_decode_inproj(
        _ptr(zxbcdt), ld_row, _dtype_code(zxbcdt), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(conv_w),
        _ptr(conv_b), _ptr(norm_w), float(eps), int(bool(norm_before_gate)), _ptr(conv_state),
        _ptr(ssm_state), conv_state.size(0), batch, _ptr(state_idx), _ptr(has_init), nheads,
        headdim, dstate, ngroups, _ptr(y), _rows(y, "y"), _dtype_code(y), _stream())
    _check(st)
    return y


def mamba2_mixed_inproj_workspace_size(total_tokens, batch, max_seqlen, nheads, headdim, dstate,
                                       ngroups, chunk_size=128, act_dtype=torch.bfloat16) -> int:
    code = M2_BF16 if act_dtype == torch.bfloat16 else M2_F32
    return int(load().mamba2_mixed_inproj_workspace_size(total_tokens, batch, max_seqlen, nheads,
                                                         headdim, dstate, ngroups, chunk_size, code))


def mamba2_mixed_inproj(zxbcdt, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                        cu_seqlens, num_decodes, max_seqlen, nheads, headdim, dstate, ngroups,
                        chunk_size=128, state_idx=None, has_init=None, eps=1e-5,
                        norm_before_gate=True, y=None, y_dtype=torch.float32, workspace=None):
    """A batch whose first num_decodes sequences are one decode row each (rows
    0 .. num_decodes-1) and whose other sequences are prefills, from packed
    in-projection rows.  Decode rows run the fused decode kernel, prefills the
    chunked chain.  Returns y [T, H*P]."""
    lib = load()
    T = zxbcdt.size(0)
    batch = cu_seqlens.numel() - 1
    ld_row = _inproj_common(zxbcdt, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                            nheads, headdim, dstate, ngroups)
    _vec(cu_seqlens, "cu_seqlens", torch.int32)
    _vec(state_idx, "state_idx", torch.int32)
    _vec(has_init, "has_init", torch.uint8)
    if y is None:
        y = torch.empty((T, nheads * headdim), dtype=y_dtype, device=zxbcdt.device)
    if workspace is None:
        need = mamba2_mixed_inproj_workspace_size(T, batch, max_seqlen, nheads, headdim, dstate,
                                                  ngroups, chunk_size, zxbcdt.dtype)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=zxbcdt.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.mamba2_mixed_inproj(
        _ptr(zxbcdt), ld_row, _dtype_code(zxbcdt), _ptr(dt_bias), _ptr(A), _ptr(D), _ptr(conv_w),
        _ptr(conv_b), _ptr(norm_w), float(eps), int(bool(norm_before_gate)), _ptr(conv_state),
        _ptr(ssm_state), conv_state.size(0), _ptr(cu_seqlens), batch, int(num_decodes), T,
        int(max_seqlen), _ptr(state_idx), _ptr(has_init), nheads, headdim, dstate, ngroups,
        chunk_size, _ptr(y), _rows(y, "y"), _dtype_code(y), _ptr(workspace), ws_bytes, _stream())
    _check(st)
    return y
