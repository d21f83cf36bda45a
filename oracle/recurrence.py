"""fp64 token-by-token oracle of the Mamba-2 mixer-core prefill.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the bench's CPU
baseline use this module; the library never does.

Everything here is the plain definition, one token at a time, in float64
with inputs upcast exactly from their fp32/bf16 storage:

1. causal depthwise conv (width K, bias, SiLU) over the carried conv state
   followed by the new rows: the chunked-prefill page ("perf(nemotron_h):
   prefill single-GPU prompts in multi-token chunks", section Implementation)
   runs the short conv of each chunk on the carried state ahead of the
   chunk's rows; the "Nemotron-H" page (section 2 block diagram, section 3
   "Forward graph") applies SiLU to the conv1d output of xBC;
2. split of the conv output into x | B | C (page "feat(#1311 A2-D1): NemotronH
   decodes on the single-step recurrent kernels ...", the mixer op sequence
   QkvSplit(x | B | C); page "Nemotron-H", section 4.1);
3. the selective-state recurrence, state update before read-out (page
   "Nemotron-H", section 4.1 "Mamba2 SSM layer"):
       h <- exp(dt*A) * h + dt * x (outer) B,     y = h . C + D * x
   with A < 0 supplied by the caller (the chunked-prefill page writes the
   log-decay as a_t = dt_t * A with every exponent <= 0; the sign reading is
   listed with the other readings of the pages in the design notes);
   head h reads group h // (nheads / ngroups) (the group-index mutation
   min(h/hpg, 1) named on the NemotronH decode page implies g = h / hpg);
4. grouped gated RMSNorm with z: per token and per group of
   d_inner / ngroups contiguous channels (page "Nemotron-H", section 4.1:
   the scan output goes through a per-group RMS normalization with the
   ssm_norm weight and is then multiplied by the SiLU(z) gate; the other
   order is available by flag).

Layouts (all row-major):
  xbc [T, conv_dim] with channels [x (H*P) | B (G*N) | C (G*N)];
  z [T, H*P]; dt [T, H]; conv_w [conv_dim, K]; conv_state [slots, K-1, conv_dim]
  (row j holds the raw input j+1 steps older than the newest of the last K-1,
  i.e. oldest first); ssm_state [slots, H, P, N].
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np


def silu(v: np.ndarray) -> np.ndarray:
    """v * sigmoid(v) = v / (1 + exp(-v)), computed without overflow warnings."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])
    out[~pos] = v[~pos] * e / (1.0 + e)
    return out


def conv_rows_seq(xbc: np.ndarray, conv_w: np.ndarray, conv_b: Optional[np.ndarray],
                  conv_state_in: np.ndarray, apply_silu: bool = True
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Causal depthwise conv of one sequence over [carried state ; new rows].

    xbc [L, C]; conv_w [C, K]; conv_b [C] or None; conv_state_in [K-1, C].
    Output row t uses padded rows t .. t+K-1, where the padded stream is the
    K-1 carried rows followed by the L new rows; weight column K-1 multiplies
    the current row.  Returns (u [L, C], conv_state_out [K-1, C]) with the
    new state = the last K-1 rows of the padded stream.
    """
    xbc = np.asarray(xbc, dtype=np.float64)
    w = np.asarray(conv_w, dtype=np.float64)
    L, Cd = xbc.shape
    K = w.shape[1]
    xpad = np.concatenate([np.asarray(conv_state_in, dtype=np.float64), xbc], axis=0)
    pre = np.zeros((L, Cd), dtype=np.float64)
    if conv_b is not None:
        pre += np.asarray(conv_b, dtype=np.float64)[None, :]
    for t in range(L):
        for k in range(K):
            pre[t] += w[:, k] * xpad[t + k]
    u = silu(pre) if apply_silu else pre
    return u, xpad[L:L + K - 1].copy()


def ssd_recurrence_seq(x: np.ndarray, B: np.ndarray, C: np.ndarray, dt: np.ndarray,
                       A: np.ndarray, D: Optional[np.ndarray], h0: np.ndarray
                       ) -> Tuple[np.ndarray, np.ndarray]:
    """Token-by-token selective-state recurrence of one sequence.

    x [L, H, P]; B, C [L, G, N]; dt [L, H]; A [H]; D [H] or None; h0 [H, P, N].
    For each token: alpha = exp(dt*A); h = alpha*h + (dt*x) outer B[group];
    y = sum_n C[group, n] * h[:, :, n] + D*x.  Returns (y [L, H, P], h [H, P, N]).
    """
    x = np.asarray(x, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    L, H, P = x.shape
    G = B.shape[1]
    grp = np.arange(H) // (H // G)
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    h = np.array(h0, dtype=np.float64, copy=True)
    y = np.zeros((L, H, P), dtype=np.float64)
    for t in range(L):
        alpha = np.exp(dt[t] * A)                                   # [H]
        Bt = B[t, grp]                                              # [H, N]
        Ct = C[t, grp]                                              # [H, N]
        h = alpha[:, None, None] * h + (dt[t][:, None] * x[t])[:, :, None] * Bt[:, None, :]
        y[t] = np.einsum("hpn,hn->hp", h, Ct) + Dv[:, None] * x[t]
    return y, h


def gated_rmsnorm_group(y: np.ndarray, z: np.ndarray, norm_w: np.ndarray, eps: float,
                        ngroups: int, norm_before_gate: bool = True) -> np.ndarray:
    """Grouped RMSNorm of y with the SiLU(z) gate.

    y, z [T, d]; norm_w [d].  Groups are ngroups runs of d/ngroups contiguous
    channels.  norm_before_gate: out = y / rms_group(y) * w * silu(z);
    otherwise v = y * silu(z), out = v / rms_group(v) * w.
    """
    y = np.asarray(y, dtype=np.float64)
    gate = silu(np.asarray(z, dtype=np.float64))
    T, d = y.shape
    v = y if norm_before_gate else y * gate
    vg = v.reshape(T, ngroups, d // ngroups)
    rstd = 1.0 / np.sqrt(np.mean(vg * vg, axis=-1) + eps)
    out = (vg * rstd[:, :, None]).reshape(T, d) * np.asarray(norm_w, dtype=np.float64)[None, :]
    if norm_before_gate:
        out = out * gate
    return out


def split_xbc(u: np.ndarray, nheads: int, headdim: int, ngroups: int, dstate: int):
    """Views x [L, H, P], B [L, G, N], C [L, G, N] of a conv output with channels [x | B | C]."""
    L = u.shape[0]
    di = nheads * headdim
    gn = ngroups * dstate
    x = u[:, :di].reshape(L, nheads, headdim)
    B = u[:, di:di + gn].reshape(L, ngroups, dstate)
    C = u[:, di + gn:di + 2 * gn].reshape(L, ngroups, dstate)
    return x, B, C


def prefill(inp: Dict[str, np.ndarray], nheads: int, headdim: int, dstate: int, ngroups: int,
            eps: float = 1e-5, norm_before_gate: bool = True, apply_norm: bool = True,
            seqs=None) -> Dict[str, np.ndarray]:
    """The whole mixer core over a packed varlen batch, in fp64.

    ``inp`` holds the arrays of workloads.make_inputs.  States are read at
    state_idx[b] (zero when has_init[b] == 0) and the advanced states are
    returned as full copies of the pools with the touched slots replaced.
    ``seqs`` restricts the work to a subset of sequences (the other rows of
    y stay NaN).  Returns y [T, d_inner] (normed, or pre-norm if
    apply_norm=False), u [T, conv_dim] (conv output), conv_state, ssm_state.
    """
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int64)
    nseq = len(cu) - 1
    T = int(cu[-1])
    d_inner = nheads * headdim
    conv_state = np.array(inp["conv_state"], dtype=np.float64, copy=True)
    ssm_state = np.array(inp["ssm_state"], dtype=np.float64, copy=True)
    idx = inp.get("state_idx")
    has_init = inp.get("has_init")
    y = np.full((T, d_inner), np.nan)
    u_all = np.full((T, inp["xbc"].shape[1]), np.nan)
    for b in (range(nseq) if seqs is None else seqs):
        lo, hi = int(cu[b]), int(cu[b + 1])
        slot = b if idx is None else int(idx[b])
        init = True if has_init is None else bool(has_init[b])
        cs = conv_state[slot] if init else np.zeros_like(conv_state[slot])
        h0 = ssm_state[slot] if init else np.zeros_like(ssm_state[slot])
        u, cs_out = conv_rows_seq(inp["xbc"][lo:hi], inp["conv_w"], inp.get("conv_b"), cs)
        x, Bm, Cm = split_xbc(u, nheads, headdim, ngroups, dstate)
        ys, h = ssd_recurrence_seq(x, Bm, Cm, inp["dt"][lo:hi], inp["A"], inp.get("D"), h0)
        ys = ys.reshape(hi - lo, d_inner)
        if apply_norm:
            ys = gated_rmsnorm_group(ys, inp["z"][lo:hi], inp["norm_w"], eps, ngroups,
                                     norm_before_gate)
        y[lo:hi] = ys
        u_all[lo:hi] = u
        conv_state[slot] = cs_out
        ssm_state[slot] = h
    return dict(y=y, u=u_all, conv_state=conv_state, ssm_state=ssm_state)
