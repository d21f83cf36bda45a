"""Precision model of the prefill's storage and product choices (error budget).

TEST INFRASTRUCTURE ONLY (see oracle/recurrence.py).

The library keeps three quantities wider than its bf16 inputs, and each of
those choices costs HBM traffic or matrix-core work:
  * the post-conv activations u = SiLU(conv(xBC)) are fp32 (or never leave the
    chip), not bf16 or fp16;
  * the state entering each chunk, handed from the state pass to the chunk
    output, is fp32;
  * every fp32 operand of a bf16 matrix product enters as a (hi, lo) pair,
    three products per tile.
This module measures what the narrower alternative would do to the results,
by running the fp64 definitions with exactly one rounding inserted:

  conv_output_rounded   the oracle's prefill (recurrence.py) with the conv output
                        rounded channel-range by channel-range before the scan;
  entry_state_rounded   the chunk form (chunked.py's closed form, restated with a
                        hook) with the entry state rounded for the chunk's
                        read-out only, the carried state staying exact;
  split_product_error   one bf16 matrix product emulated with single bf16
                        operands or with (hi, lo) pairs.

Each returns max|err| / RMS of the affected output against the unrounded fp64
result: the metric the GPU parity checks apply (the bar is 2e-2 for bf16
inputs), so a rounding whose effect alone comes near the bar is ruled out.
The rounding functions follow the formats' definitions: round to nearest,
ties to even, of the fp32 value (bf16: 8 significant bits; fp16: 11, with its
range).
"""
from __future__ import annotations

from typing import Callable, Dict, Tuple

import numpy as np

from . import recurrence as R


def round_fp32(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_fp16(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of the fp32 rounding of v, as fp64."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64).astype(np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_fp16_block(v: np.ndarray) -> np.ndarray:
    """fp16 of the whole block v scaled by one power of two 2^k, chosen so the
    block's largest magnitude lands in [2^14, 2^15): the scaling is exact, so
    only fp16's rounding (11 significant bits) and its subnormal floor remain,
    with the range set by the block instead of by fp16's 65504."""
    v = np.asarray(v, dtype=np.float64)
    m = float(np.max(np.abs(v))) if v.size else 0.0
    if m == 0.0 or not np.isfinite(m):
        return round_fp16(v)
    k = 14 - int(np.floor(np.log2(m)))
    return np.ldexp(round_fp16(np.ldexp(v, k)), -k)


def round_q16_rows(v: np.ndarray, run: int = 32) -> np.ndarray:
    """16-bit fixed point with one scale per run of `run` values along the last
    axis (for a P x N state: per p and n tile of 32): s = fp32(max |v| of the
    run), q = round-half-even(clip(v / s, -1, 1) * 32767), read back as
    q * (s / 32767).  Absolute error at most s / 65534 per value: each run
    keeps 15 bits below its largest magnitude, whatever the exponent spread."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    for n0 in range(0, v.shape[-1], run):
        r = v[..., n0:n0 + run]
        sc = np.max(np.abs(r), axis=-1, keepdims=True).astype(np.float32).astype(np.float64)
        safe = np.where(sc > 0.0, sc, 1.0)
        q = np.round(np.clip(r / safe, -1.0, 1.0) * 32767.0)
        out[..., n0:n0 + run] = np.where(sc > 0.0, q * (sc / 32767.0), 0.0)
    return out


FORMATS: Dict[str, Callable[[np.ndarray], np.ndarray]] = {
    "fp64": lambda v: np.asarray(v, dtype=np.float64), "fp32": round_fp32,
    "fp16": round_fp16, "bf16": round_bf16, "fp16_block": round_fp16_block,
    "q16_rows": round_q16_rows}


def rel_max(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / RMS(ref)."""
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / np.sqrt(np.mean(ref * ref)))


def conv_output_rounded(inp: Dict[str, np.ndarray], nheads: int, headdim: int, dstate: int,
                        ngroups: int, x_fmt: str, bc_fmt: str, eps: float = 1e-5
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """The oracle's prefill (every sequence, carried states as given) with the
    conv output's x channels stored in x_fmt and its B, C channels in bc_fmt.
    Returns (y [T, d_inner] after the gated norm, final SSM states [nseq, H, P, N])."""
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int64)
    di = nheads * headdim
    ys, hs = [], []
    for b in range(len(cu) - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        slot = int(inp["state_idx"][b])
        init = bool(inp["has_init"][b])
        cs = inp["conv_state"][slot] if init else np.zeros_like(inp["conv_state"][slot])
        h0 = inp["ssm_state"][slot] if init else np.zeros_like(inp["ssm_state"][slot])
        u, _ = R.conv_rows_seq(inp["xbc"][lo:hi], inp["conv_w"], inp["conv_b"], cs)
        u = np.concatenate([FORMATS[x_fmt](u[:, :di]), FORMATS[bc_fmt](u[:, di:])], axis=1)
        x, Bm, Cm = R.split_xbc(u, nheads, headdim, ngroups, dstate)
        y, h = R.ssd_recurrence_seq(x, Bm, Cm, inp["dt"][lo:hi], inp["A"], inp["D"], h0)
        ys.append(R.gated_rmsnorm_group(y.reshape(hi - lo, di), inp["z"][lo:hi], inp["norm_w"], eps,
                                        ngroups, True))
        hs.append(h)
    return np.concatenate(ys), np.stack(hs)


def entry_state_rounded(x: np.ndarray, B: np.ndarray, C: np.ndarray, dt: np.ndarray, A: np.ndarray,
                        D: np.ndarray, h0: np.ndarray, chunk: int, fmt: str) -> np.ndarray:
    """Pre-norm y [L, H, P] of one sequence by the chunk form (see chunked.py),
    with the state entering each chunk stored in `fmt` for that chunk's
    read-out e(gamma_t) C_t . h_in; the state carried to the next chunk stays
    exact (it lives on chip).  exp(min(v, 0)) throughout."""
    x, B, C, dt, A, D = (np.asarray(v, dtype=np.float64) for v in (x, B, C, dt, A, D))
    L, H, P = x.shape
    G = B.shape[1]
    hpg = H // G
    rnd = FORMATS[fmt]
    h = np.array(h0, dtype=np.float64, copy=True)
    y = np.zeros((L, H, P))
    e = lambda v: np.exp(np.minimum(v, 0.0))
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        S = c1 - c0
        for hh in range(H):
            g = hh // hpg
            gam = np.cumsum(dt[c0:c1, hh] * A[hh])
            Lm = np.where(np.tri(S, dtype=bool), e(gam[:, None] - gam[None, :]), 0.0)
            Cc, Bc = C[c0:c1, g], B[c0:c1, g]
            xdt = x[c0:c1, hh] * dt[c0:c1, hh][:, None]
            y[c0:c1, hh] = (Lm * (Cc @ Bc.T)) @ xdt + e(gam)[:, None] * (Cc @ rnd(h[hh]).T) \
                + D[hh] * x[c0:c1, hh]
            h[hh] = e(gam[-1]) * h[hh] + (xdt * e(gam[-1] - gam)[:, None]).T @ Bc
    return y


def split_product_error(a: np.ndarray, b: np.ndarray, split: bool) -> float:
    """max|a @ b - emulated| / RMS(a @ b) for one bf16 matrix product with fp64
    accumulation: single bf16 operands, or (hi, lo) pairs with hi = bf16(v),
    lo = bf16(v - hi) and the product hi.hi + hi.lo + lo.hi (lo.lo dropped)."""
    a = round_fp32(a)
    b = round_fp32(b)
    ah, bh = round_bf16(a), round_bf16(b)
    if split:
        al, bl = round_bf16(a - ah), round_bf16(b - bh)
        got = ah @ bh + ah @ bl + al @ bh
    else:
        got = ah @ bh
    return rel_max(got, a @ b)
