"""Seeded synthetic inputs for the Mamba-2 mixer-core prefill workloads.

This module holds no arithmetic of the method itself: it only draws the
inputs (raw conv/SSM streams, dt, A, D, weights, carried states, varlen
layout) that both the oracle and the HIP path consume.  dt is drawn already
passed through softplus, because the library takes the final dt >= 0 as an
input (the softplus(dt + bias) step of the Nemotron-H page, section 4.1
"Mamba2 SSM layer", happens before this path).

Shapes follow the Nemotron-H layer dimensions (page "Nemotron-H",
section 5 "Parameters and settings" and section 6 "Weight naming
convention"): the xBC stream has d_inner + 2*ngroups*dstate channels in the
order [x | B | C], z has d_inner channels and dt has nheads.

Value distributions:
  * raw x, B, C, z ~ N(0, 1), rounded to bf16 (round-to-nearest-even) when
    the activation dtype is bf16;
  * dt = softplus(dt_raw + bias_h), dt_raw ~ N(0, 1), bias_h ~ U(-4, -2);
  * A_h = -exp(U(0, ln 16)) in [-16, -1];  D_h ~ N(0, 1);
  * conv weight and bias ~ U(-1/2, 1/2); norm weight ~ 1 + 0.1 N(0, 1);
  * carried states (when nonzero): ssm ~ N(0, 0.1^2), conv ~ N(0, 1)
    (conv state values rounded like the activations, since the conv state
    holds past raw inputs);
  * decay-stress dt: |dt*A| = 10^U(-3, 6) per (token, head), with 5% of the
    (token, head) entries set to exactly 1e6.

Every sequence draws its token-indexed arrays from its own SeedSequence
substream, so one sequence can be regenerated alone.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class LayerShape:
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    width: int = 4

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def conv_dim(self) -> int:
        return self.d_inner + 2 * self.ngroups * self.dstate


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    seqlens: tuple              # per-sequence token counts (None: drawn, see varlen_*)
    act: str                    # "f32" or "bf16" for x/B/C/z
    init: str                   # "zero", "random" (per sequence) or "pool"
    dt_mode: str = "softplus"   # "softplus" or "stress"
    chunk_size: int = 128
    n_slots: Optional[int] = None
    varlen_count: int = 0       # >0: draw this many lengths uniform in [1, varlen_max]
    varlen_max: int = 0
    eps: float = 1e-5
    description: str = ""


_BLOCK = 512

NANO = LayerShape(nheads=64, headdim=64, dstate=128, ngroups=8)
H8B = LayerShape(nheads=128, headdim=64, dstate=128, ngroups=8)
TINY = LayerShape(nheads=4, headdim=16, dstate=16, ngroups=2)

WORKLOADS: Dict[int, Workload] = {
    0: Workload("tiny_f32_11tok", TINY, (11,), "f32", "zero", chunk_size=16,
                description="1 x 11 tokens, fp32; prefilled as 7+4 and as 11 single steps"),
    1: Workload("nano_137tok_bf16", NANO, (137,), "bf16", "zero",
                description="1 x 137 tokens (128 + 9), Nemotron-nano layer shape"),
    2: Workload("nano_8x4096_bf16", NANO, (4096,) * 8, "bf16", "random",
                description="8 x 4096 tokens, chunk 128, nonzero carried states"),
    3: Workload("decay_stress_2x2048_f32", NANO, (2048,) * 2, "f32", "zero", dt_mode="stress",
                description="2 x 2048 tokens fp32, |dt*A| log-uniform in [1e-3, 1e6], 5% at 1e6"),
    4: Workload("h8b_varlen16_bf16", H8B, None, "bf16", "pool", n_slots=64,
                varlen_count=16, varlen_max=8192,
                description="16 packed sequences, lengths U[1, 8192], states from a 64-slot pool"),
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    t = u >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t &= np.uint32(0xFFFF0000)
    return t.view(np.float32)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


def _substream(ss: np.random.SeedSequence, j: int) -> np.random.SeedSequence:
    """Child j of ``ss`` (what ss.spawn would hand out j-th), built without spawning."""
    return np.random.SeedSequence(ss.entropy, spawn_key=tuple(ss.spawn_key) + (j,))


def seqlens_of(w: Workload, seed: int) -> List[int]:
    if w.seqlens is not None:
        return list(w.seqlens)
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xC0FFEE]))
    return [int(v) for v in rng.integers(1, w.varlen_max + 1, size=w.varlen_count)]


def make_inputs(w: Workload, seed: int, seqlens: Optional[List[int]] = None,
                only_seq: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every input of one prefill call.

    Returns float32 arrays (bf16-representable where the activation dtype is
    bf16) and int32/uint8 index arrays:
      xbc [T, conv_dim], z [T, d_inner], dt [T, H], A [H], D [H],
      conv_w [conv_dim, width], conv_b [conv_dim], norm_w [d_inner],
      conv_state [n_slots, width-1, conv_dim], ssm_state [n_slots, H, P, N],
      cu_seqlens [B+1], state_idx [B], has_init [B].
    With ``only_seq`` set, only that sequence's token arrays are drawn (the
    others are left zero), which lets a sampled check regenerate one sequence.
    """
    s = w.shape
    H, P, N, G, K = s.nheads, s.headdim, s.dstate, s.ngroups, s.width
    if seqlens is None:
        seqlens = seqlens_of(w, seed)
    nseq = len(seqlens)
    cu = np.zeros(nseq + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])

    root = np.random.SeedSequence(seed)
    params_ss, states_ss, seq_root = root.spawn(3)
    seq_ss = seq_root.spawn(nseq)

    prm = np.random.default_rng(params_ss)
    A = (-np.exp(prm.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    D = prm.standard_normal(H).astype(np.float32)
    dt_bias = prm.uniform(-4.0, -2.0, size=H)
    conv_w = prm.uniform(-0.5, 0.5, size=(s.conv_dim, K)).astype(np.float32)
    conv_b = prm.uniform(-0.5, 0.5, size=s.conv_dim).astype(np.float32)
    norm_w = (1.0 + 0.1 * prm.standard_normal(s.d_inner)).astype(np.float32)

    act_round = round_bf16 if w.act == "bf16" else (lambda a: a.astype(np.float32))

    n_slots = w.n_slots if w.n_slots is not None else nseq
    conv_state = np.zeros((n_slots, K - 1, s.conv_dim), dtype=np.float32)
    ssm_state = np.zeros((n_slots, H, P, N), dtype=np.float32)
    if w.init == "pool":
        srng = np.random.default_rng(states_ss)
        state_idx = srng.permutation(n_slots)[:nseq].astype(np.int32)
        conv_state[:] = act_round(srng.standard_normal(conv_state.shape, dtype=np.float32))
        ssm_state[:] = (0.1 * srng.standard_normal(ssm_state.shape, dtype=np.float32))
        has_init = np.ones(nseq, dtype=np.uint8)
    else:
        state_idx = np.arange(nseq, dtype=np.int32)
        has_init = np.zeros(nseq, dtype=np.uint8) if w.init == "zero" else np.ones(nseq, dtype=np.uint8)

    xbc = np.zeros((T, s.conv_dim), dtype=np.float32)
    z = np.zeros((T, s.d_inner), dtype=np.float32)
    dt = np.zeros((T, H), dtype=np.float32)

    # Token arrays are drawn in blocks of _BLOCK rows; block j of sequence b
    # uses substream j of sequence b's SeedSequence, so the values do not
    # depend on how many threads fill them.
    def fill(b: int, j: int) -> None:
        r = np.random.default_rng(_substream(seq_ss[b], j))
        L = seqlens[b]
        lo = int(cu[b]) + j * _BLOCK
        n = min(_BLOCK, L - j * _BLOCK)
        xbc[lo:lo + n] = act_round(r.standard_normal((n, s.conv_dim), dtype=np.float32))
        z[lo:lo + n] = act_round(r.standard_normal((n, s.d_inner), dtype=np.float32))
        if w.dt_mode == "stress":
            m = 10.0 ** r.uniform(-3.0, 6.0, size=(n, H))
            m[r.random((n, H)) < 0.05] = 1e6
            dt[lo:lo + n] = (m / np.abs(A.astype(np.float64))[None, :]).astype(np.float32)
        else:
            raw = r.standard_normal((n, H))
            dt[lo:lo + n] = _softplus(raw + dt_bias[None, :]).astype(np.float32)

    jobs = []
    for b in range(nseq):
        if only_seq is not None and b != only_seq:
            continue
        jobs += [(b, j) for j in range((seqlens[b] + _BLOCK - 1) // _BLOCK)]
        if w.init == "random":
            r = np.random.default_rng(_substream(seq_ss[b], 1 << 20))
            slot = int(state_idx[b])
            conv_state[slot] = act_round(r.standard_normal((K - 1, s.conv_dim), dtype=np.float32))
            ssm_state[slot] = 0.1 * r.standard_normal((H, P, N), dtype=np.float32)
    nthreads = max(1, min(16, len(os.sched_getaffinity(0)), len(jobs)))
    if nthreads == 1:
        for job in jobs:
            fill(*job)
    else:
        with concurrent.futures.ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(lambda job: fill(*job), jobs))

    return dict(xbc=xbc, z=z, dt=dt, A=A, D=D, conv_w=conv_w, conv_b=conv_b, norm_w=norm_w,
                conv_state=conv_state, ssm_state=ssm_state, cu_seqlens=cu,
                state_idx=state_idx, has_init=has_init)


def small_shape_inputs(shape: LayerShape, seqlens: List[int], seed: int, act: str = "f32",
                       init: str = "random", n_slots: Optional[int] = None,
                       dt_mode: str = "softplus") -> Dict[str, np.ndarray]:
    """Inputs for an ad-hoc shape (tests of ragged tails, group maps, edge cases)."""
    w = Workload("adhoc", shape, tuple(seqlens), act, init, dt_mode=dt_mode, n_slots=n_slots)
    return make_inputs(w, seed)


def group_channels(shape: LayerShape, g: int):
    """Heads, x/z channels and conv channels (x | B | C order) owned by SSM group g."""
    hpg = shape.nheads // shape.ngroups
    P, N = shape.headdim, shape.dstate
    di, gn = shape.d_inner, shape.ngroups * shape.dstate
    heads = np.arange(g * hpg, (g + 1) * hpg)
    xch = np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])
    bch = di + g * N + np.arange(N)
    cch = di + gn + g * N + np.arange(N)
    return heads, xch, np.concatenate([xch, bch, cch])


def slice_group(inp: Dict[str, np.ndarray], shape: LayerShape, g: int):
    """Inputs of the one-group problem (ngroups = 1, nheads = heads per group) for group g.

    Groups never interact in the mixer core (each owns its heads, its B/C, x, z
    and conv channels and its norm group), so this is an exact sub-problem."""
    heads, xch, ch = group_channels(shape, g)
    out = dict(inp)
    out["xbc"] = inp["xbc"][:, ch]
    out["z"] = inp["z"][:, xch]
    out["dt"] = inp["dt"][:, heads]
    out["A"] = inp["A"][heads]
    out["D"] = inp["D"][heads]
    out["conv_w"] = inp["conv_w"][ch]
    out["conv_b"] = inp["conv_b"][ch]
    out["norm_w"] = inp["norm_w"][xch]
    out["conv_state"] = inp["conv_state"][:, :, ch]
    out["ssm_state"] = inp["ssm_state"][:, heads]
    return out, LayerShape(len(heads), shape.headdim, shape.dstate, 1, shape.width)


def inproj_inputs(shape: LayerShape, seqlens: List[int], seed: int, act: str = "bf16",
                  init: str = "random", n_slots: Optional[int] = None,
                  pad: int = 8) -> Dict[str, np.ndarray]:
    """Inputs whose activations arrive as one in-projection row per token.

    The row holds z (d_inner), xBC (conv_dim) and the raw step size (nheads), in
    that order, then zero padding up to a multiple of ``pad`` channels (so bf16
    rows stay 16-byte aligned).  dt_raw ~ N(0, 1) is rounded like the other
    activations; dt_bias ~ U(-4, -2) per head (fp32).  Nothing here applies the
    step-size function: the oracle and the library each do that themselves.
    Returns the arrays of make_inputs without xbc, z and dt, plus
    row [T, ld_row] (float32 values, bf16-representable for bf16) and dt_bias [H].
    """
    base = small_shape_inputs(shape, seqlens, seed, act=act, init=init, n_slots=n_slots)
    T = base["xbc"].shape[0]
    H = shape.nheads
    width = shape.d_inner + shape.conv_dim + H
    ld_row = (width + pad - 1) // pad * pad
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0xD7]))
    act_round = round_bf16 if act == "bf16" else (lambda a: a.astype(np.float32))
    dt_raw = act_round(rng.standard_normal((T, H), dtype=np.float32))
    dt_bias = rng.uniform(-4.0, -2.0, size=H).astype(np.float32)
    row = np.zeros((T, ld_row), dtype=np.float32)
    row[:, :shape.d_inner] = base["z"]
    row[:, shape.d_inner:shape.d_inner + shape.conv_dim] = base["xbc"]
    row[:, shape.d_inner + shape.conv_dim:width] = dt_raw
    out = {k: v for k, v in base.items() if k not in ("xbc", "z", "dt")}
    out.update(row=row, dt_bias=dt_bias)
    return out
