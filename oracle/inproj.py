"""fp64 oracle of the packed in-projection row, the step size dt, and mixed
decode + prefill batches.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the bench's CPU
baseline use this module; the library never does.

1. The in-projection of a Mamba-2 layer emits one row per token that holds,
   in this order, z (d_inner channels), xBC (conv_dim = d_inner + 2*G*N
   channels, themselves x | B | C) and the raw step size (nheads channels):
   page "feat(#1311 A2-D1): NemotronH decodes on the single-step recurrent
   kernels ..." names the op sequence in_proj -> QkvSplit(z | xBC | dt) ->
   CausalConv1dFwd(silu) -> QkvSplit(x | B | C), and describes the split as
   three outputs of widths (I, conv_dim, num_heads) taken from the head, the
   middle and the tail of an in_proj row.
2. The step size is dt = softplus(dt_raw + dt_bias[h]): page "Nemotron-H",
   section 4.1 "Mamba2 SSM layer" (the decay uses softplus of dt plus the
   ssm_dt.bias weight), section 6 (ssm_dt.bias has one value per head).
3. A mixed batch holds num_decodes one-token decode rows first, then prefill
   sequences; the decode rows continue their slots' states (page "feat(#1311
   A2-D1) ...": the split into decode and prefill rows is chosen by the
   metadata's num_decodes, never by the token count, so a one-token prefill of
   a fresh request stays a prefill).  A decode row is a one-token sequence of
   the same recurrence, so the whole batch is the prefill driver of
   oracle.recurrence over all sequences.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import recurrence as R


def softplus(v: np.ndarray) -> np.ndarray:
    """log(1 + e^v) in fp64, written as max(v, 0) + log1p(e^-|v|) so that
    neither large positive nor large negative v overflows."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def step_size(dt_raw: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """dt[t, h] = softplus(dt_raw[t, h] + dt_bias[h]) (fp64)."""
    raw = np.asarray(dt_raw, dtype=np.float64)
    return softplus(raw + np.asarray(dt_bias, dtype=np.float64)[None, :])


def row_width(nheads: int, headdim: int, dstate: int, ngroups: int) -> int:
    """Used channels of one in-projection row: d_inner + conv_dim + nheads."""
    d_inner = nheads * headdim
    return 2 * d_inner + 2 * ngroups * dstate + nheads


def split_inproj_row(row: np.ndarray, nheads: int, headdim: int, dstate: int, ngroups: int):
    """Views z [T, d_inner], xbc [T, conv_dim], dt_raw [T, nheads] of rows [T, >= width]."""
    d_inner = nheads * headdim
    conv_dim = d_inner + 2 * ngroups * dstate
    if row.shape[1] < d_inner + conv_dim + nheads:
        raise ValueError("in-projection row narrower than z | xBC | dt")
    z = row[:, :d_inner]
    xbc = row[:, d_inner:d_inner + conv_dim]
    dt_raw = row[:, d_inner + conv_dim:d_inner + conv_dim + nheads]
    return z, xbc, dt_raw


def prefill_inproj(inp: Dict[str, np.ndarray], nheads: int, headdim: int, dstate: int,
                   ngroups: int, eps: float = 1e-5, norm_before_gate: bool = True,
                   seqs=None) -> Dict[str, np.ndarray]:
    """The mixer core over a packed batch whose activations arrive as one
    in-projection row per token (``inp["row"]``) with the raw step size in its
    tail and ``inp["dt_bias"]``; everything else as for recurrence.prefill."""
    z, xbc, dt_raw = split_inproj_row(inp["row"], nheads, headdim, dstate, ngroups)
    full = {k: v for k, v in inp.items() if k not in ("row", "dt_bias")}
    full.update(z=z, xbc=xbc, dt=step_size(dt_raw, inp["dt_bias"]))
    return R.prefill(full, nheads, headdim, dstate, ngroups, eps=eps,
                     norm_before_gate=norm_before_gate, seqs=seqs)


def mixed_batch(inp: Dict[str, np.ndarray], num_decodes: int, nheads: int, headdim: int,
                dstate: int, ngroups: int, eps: float = 1e-5,
                norm_before_gate: bool = True) -> Dict[str, np.ndarray]:
    """A batch of num_decodes decode rows (sequences 0 .. num_decodes-1, one
    row each, rows 0 .. num_decodes-1) followed by prefill sequences."""
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int64)
    if num_decodes < 0 or num_decodes > len(cu) - 1:
        raise ValueError("num_decodes outside [0, batch]")
    if not np.array_equal(cu[:num_decodes + 1], np.arange(num_decodes + 1)):
        raise ValueError("decode rows must come first, one row per decode sequence")
    return prefill_inproj(inp, nheads, headdim, dstate, ngroups, eps=eps,
                          norm_before_gate=norm_before_gate)
