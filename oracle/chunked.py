"""Brute-force chunked evaluation of the selective scan (fp64), a second CPU form.

TEST INFRASTRUCTURE ONLY (see oracle/recurrence.py).

The chunked-prefill page ("perf(nemotron_h): prefill single-GPU prompts in
multi-token chunks", section Implementation) runs the Mamba-2 mixer over S
rows without a sequential step: with a_t = dt_t * A and gamma_t the inclusive
cumulative sum of a over the chunk, every exponent is at most 0, the chunk
total gamma_S is the LAST element of that cumulative sum (not a separate
reduction), and exponents are clamped at 0.  The display equations of that
section are lost from the page text; they are restated here from the
recurrence of the "Nemotron-H" page (section 4.1) unrolled over one chunk
with carried state h_in:

    y_t  = exp(min(gamma_t, 0)) * C_t . h_in
           + sum_{i<=t} exp(min(gamma_t - gamma_i, 0)) * (C_t . B_i) * dt_i * x_i
           + D * x_t
    h_out = exp(min(gamma_S, 0)) * h_in
           + sum_i exp(min(gamma_S - gamma_i, 0)) * dt_i * x_i (outer) B_i

Two evaluations are offered:
  * ``chunk_scan_seq``: the closed form above, chunk by chunk, with every
    exponent checked to be <= 0 before the clamp is applied;
  * ``dual_form_seq``: the fully materialised quadratic ("SSD dual") form of
    one whole sequence, y = (Lmask * C B^T) (dt x) + decay-weighted C h_0 + D x,
    with Lmask[t, i] = exp(sum_{k=i+1..t} a_k) built from explicit segment sums
    rather than from differences of a cumulative sum.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


class PositiveExponent(AssertionError):
    """Raised when an exponent of the chunk form is positive before clamping."""


def _check_nonpositive(v: np.ndarray, what: str) -> None:
    if np.any(v > 0):
        raise PositiveExponent(f"{what}: max exponent {float(np.max(v))!r} > 0")


def chunk_scan_seq(x: np.ndarray, B: np.ndarray, C: np.ndarray, dt: np.ndarray,
                   A: np.ndarray, D: Optional[np.ndarray], h0: np.ndarray, chunk: int,
                   check_exponents: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """Closed-form chunked scan of one sequence.

    x [L, H, P]; B, C [L, G, N]; dt [L, H]; A [H]; D [H] or None; h0 [H, P, N].
    Returns (y [L, H, P], h_out [H, P, N]).
    """
    x = np.asarray(x, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    L, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    hpg = H // G
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    y = np.zeros((L, H, P))
    h = np.array(h0, dtype=np.float64, copy=True)
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        S = c1 - c0
        for hh in range(H):
            g = hh // hpg
            a = dt[c0:c1, hh] * A[hh]                     # [S], <= 0
            gam = np.cumsum(a)                             # inclusive, sequential
            gam_S = gam[-1]
            seg = gam[:, None] - gam[None, :]              # gamma_t - gamma_i
            causal = np.tri(S, dtype=bool)                 # i <= t
            if check_exponents:
                _check_nonpositive(gam, "gamma_t")
                _check_nonpositive(seg[causal], "gamma_t - gamma_i")
                _check_nonpositive(gam_S - gam, "gamma_S - gamma_i")
            Lmask = np.where(causal, np.exp(np.minimum(seg, 0.0)), 0.0)
            Cc, Bc = C[c0:c1, g], B[c0:c1, g]              # [S, N]
            xdt = x[c0:c1, hh] * dt[c0:c1, hh][:, None]    # [S, P]
            G_tt = Cc @ Bc.T                               # [S, S]
            y_intra = (Lmask * G_tt) @ xdt
            y_inter = np.exp(np.minimum(gam, 0.0))[:, None] * (Cc @ h[hh].T)
            y[c0:c1, hh] = y_intra + y_inter + Dv[hh] * x[c0:c1, hh]
            dec = np.exp(np.minimum(gam_S - gam, 0.0))     # [S]
            h[hh] = np.exp(min(gam_S, 0.0)) * h[hh] + (xdt * dec[:, None]).T @ Bc
    return y, h


def dual_form_seq(x: np.ndarray, B: np.ndarray, C: np.ndarray, dt: np.ndarray,
                  A: np.ndarray, D: Optional[np.ndarray], h0: np.ndarray
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Quadratic materialised form of one whole sequence (tiny inputs only).

    Lmask[t, i] = exp(sum_{k=i+1}^{t} a_k) for i <= t (the empty sum is 0),
    each entry summed on its own; decay of the initial state to row t is
    exp(sum_{k=0}^{t} a_k).  Returns (y [L, H, P], h_out [H, P, N]).
    """
    x = np.asarray(x, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    L, H, P = x.shape
    G = B.shape[1]
    hpg = H // G
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    y = np.zeros((L, H, P))
    h_out = np.zeros_like(np.asarray(h0, dtype=np.float64))
    for hh in range(H):
        g = hh // hpg
        a = dt[:, hh] * A[hh]
        Lmask = np.zeros((L, L))
        for t in range(L):
            for i in range(t + 1):
                Lmask[t, i] = np.exp(np.sum(a[i + 1:t + 1]))
        to_start = np.array([np.exp(np.sum(a[:t + 1])) for t in range(L)])
        xdt = x[:, hh] * dt[:, hh][:, None]
        M = Lmask * (C[:, g] @ B[:, g].T)
        y[:, hh] = M @ xdt + to_start[:, None] * (C[:, g] @ np.asarray(h0, dtype=np.float64)[hh].T) \
            + Dv[hh] * x[:, hh]
        to_end = np.array([np.exp(np.sum(a[i + 1:])) for i in range(L)])
        h_out[hh] = np.exp(np.sum(a)) * h0[hh] + (xdt * to_end[:, None]).T @ B[:, g]
    return y, h_out
