"""Planted mistakes in the oracle (CPU only): each one must turn at least one of
the oracle's pins red, so that a plausible slip in the oracle cannot pass
unnoticed.  The mutations are those a port of this method typically makes:

  1. the head -> group map clamped as min(h / hpg, 1) (the NemotronH decode
     page's own mutation of the group index);
  2. the in-chunk cumulative decay summed in fp32 with no clamp at 0;
  3. the carry dropped (every call starts from a zero SSM state);
  4. the conv state shifted by one row;
  5. the gate order swapped;
  6. the chunk treated as dense (the causal predicate dropped);
  7. B and C read from each other's channel runs of the conv output;
  8. (in-projection rows) the dt bias dropped, softplus confused with e^v or
     with log(1 + e^-v), and the row read in the wrong order.

Each mutant wraps or replaces one oracle function through monkeypatch; the
pins are the functions of test_oracle_pins, called as they are.
"""
import numpy as np
import pytest

import test_oracle_pins as PINS
from oracle import chunked as Ch
from oracle import recurrence as R


def _red(pins):
    """Number of pins that fail (AssertionError) among [(fn, args), ...]."""
    red = 0
    for fn, args in pins:
        try:
            fn(*args)
        except AssertionError:
            red += 1
    return red


def _mutant_chunk_form(x, B, C, dt, A, D, h0, chunk, fp32_gamma=False, dense=False):
    """The closed chunk form with one planted mistake: gamma summed in fp32 and
    no exponent clamped (fp32_gamma), or every (t, i) pair of the chunk used
    (dense)."""
    x, B, C, dt, A = (np.asarray(v, dtype=np.float64) for v in (x, B, C, dt, A))
    L, H, P = x.shape
    G = B.shape[1]
    hpg = H // G
    Dv = np.zeros(H) if D is None else np.asarray(D, dtype=np.float64)
    y = np.zeros((L, H, P))
    h = np.array(h0, dtype=np.float64, copy=True)
    for c0 in range(0, L, chunk):
        c1 = min(L, c0 + chunk)
        S = c1 - c0
        for hh in range(H):
            g = hh // hpg
            a = dt[c0:c1, hh] * A[hh]
            if fp32_gamma:
                gam = np.cumsum(a.astype(np.float32)).astype(np.float64)
                clamp = lambda v: v
            else:
                gam = np.cumsum(a)
                clamp = lambda v: np.minimum(v, 0.0)
            seg = gam[:, None] - gam[None, :]
            keep = np.ones((S, S), dtype=bool) if dense else np.tri(S, dtype=bool)
            Lmask = np.where(keep, np.exp(clamp(seg)), 0.0)
            Cc, Bc = C[c0:c1, g], B[c0:c1, g]
            xdt = x[c0:c1, hh] * dt[c0:c1, hh][:, None]
            y[c0:c1, hh] = (Lmask * (Cc @ Bc.T)) @ xdt + np.exp(clamp(gam))[:, None] * (Cc @ h[hh].T) \
                + Dv[hh] * x[c0:c1, hh]
            dec = np.exp(clamp(gam[-1] - gam))
            h[hh] = np.exp(clamp(gam[-1])) * h[hh] + (xdt * dec[:, None]).T @ Bc
    return y, h


def test_mutation_group_index_clamped(monkeypatch):
    real = R.ssd_recurrence_seq

    def mutant(x, B, C, dt, A, D, h0):
        # heads of group j >= 2 read group 1: the same as indexing min(h / hpg, 1)
        G = np.asarray(B).shape[1]
        pick = np.minimum(np.arange(G), 1)
        return real(x, np.asarray(B)[:, pick], np.asarray(C)[:, pick], dt, A, D, h0)
    monkeypatch.setattr(R, "ssd_recurrence_seq", mutant)
    assert _red([(PINS.test_group_map_is_contiguous_heads, ())]) == 1


def test_mutation_gamma_fp32_unclamped(monkeypatch):
    monkeypatch.setattr(Ch, "chunk_scan_seq",
                        lambda *a, **k: _mutant_chunk_form(*a[:8], fp32_gamma=True))
    with np.errstate(over="ignore", invalid="ignore"):   # the unclamped mutant overflows
        assert _red([(PINS.test_decay_stress_small_shape_finite_and_chunk_form_agrees, ())]) == 1


def test_mutation_carry_dropped(monkeypatch):
    real = R.ssd_recurrence_seq
    monkeypatch.setattr(R, "ssd_recurrence_seq",
                        lambda x, B, C, dt, A, D, h0: real(x, B, C, dt, A, D, np.zeros_like(h0)))
    assert _red([(PINS.test_split_7_plus_4_equals_11_equals_11_single_steps, ()),
                 (PINS.test_scalar_recurrence_closed_form_products, ())]) >= 1


def test_mutation_conv_state_off_by_one(monkeypatch):
    real = R.conv_rows_seq

    def mutant(xbc, conv_w, conv_b, conv_state_in, apply_silu=True):
        u, _ = real(xbc, conv_w, conv_b, conv_state_in, apply_silu)
        xpad = np.concatenate([np.asarray(conv_state_in, np.float64), np.asarray(xbc, np.float64)])
        L = np.asarray(xbc).shape[0]
        return u, xpad[L - 1:L + 2]          # one row early: should be xpad[L:L + 3]
    monkeypatch.setattr(R, "conv_rows_seq", mutant)
    assert _red([(PINS.test_conv_matches_numpy_convolve, (L,)) for L in (2, 4, 9)] +
                [(PINS.test_split_7_plus_4_equals_11_equals_11_single_steps, ())]) >= 1


def test_mutation_gate_order_swapped(monkeypatch):
    real = R.gated_rmsnorm_group
    monkeypatch.setattr(R, "gated_rmsnorm_group",
                        lambda y, z, w, eps, ngroups, nbg=True: real(y, z, w, eps, ngroups, not nbg))
    assert _red([(PINS.test_norm_single_group_matches_torch_rms_norm, (True,)),
                 (PINS.test_norm_single_group_matches_torch_rms_norm, (False,)),
                 (PINS.test_golden_gated_norm, ())]) >= 2


@pytest.mark.parametrize("chunk", [3, 7, 16])
def test_mutation_dense_chunk(monkeypatch, chunk):
    monkeypatch.setattr(Ch, "chunk_scan_seq",
                        lambda *a, **k: _mutant_chunk_form(*a[:8], dense=True))
    assert _red([(PINS.test_recurrence_equals_chunk_form, (4, 2, chunk))]) == 1


def test_mutation_B_and_C_swapped(monkeypatch):
    """The conv output's B and C channel runs read the other way round."""
    def mutant(u, nheads, headdim, ngroups, dstate):
        L = u.shape[0]
        di, gn = nheads * headdim, ngroups * dstate
        x = u[:, :di].reshape(L, nheads, headdim)
        C = u[:, di:di + gn].reshape(L, ngroups, dstate)
        B = u[:, di + gn:di + 2 * gn].reshape(L, ngroups, dstate)
        return x, B, C
    monkeypatch.setattr(R, "split_xbc", mutant)
    assert _red([(PINS.test_split_xbc_takes_x_then_B_then_C, ()),
                 (PINS.test_one_token_roles_of_B_and_C, ())]) == 2


def test_unmutated_pins_pass():
    """The same pins, unmutated, are green (so a red above is the mutation's)."""
    assert _red([(PINS.test_group_map_is_contiguous_heads, ()),
                 (PINS.test_split_xbc_takes_x_then_B_then_C, ()),
                 (PINS.test_one_token_roles_of_B_and_C, ()),
                 (PINS.test_decay_stress_small_shape_finite_and_chunk_form_agrees, ()),
                 (PINS.test_split_7_plus_4_equals_11_equals_11_single_steps, ()),
                 (PINS.test_conv_matches_numpy_convolve, (4,)),
                 (PINS.test_norm_single_group_matches_torch_rms_norm, (True,)),
                 (PINS.test_golden_gated_norm, ()),
                 (PINS.test_recurrence_equals_chunk_form, (4, 2, 7))]) == 0


# ------------------------------------------------------------------ in-projection rows
#
# Planted mistakes in oracle.inproj, each caught by the pins of
# test_oracle_inproj_pins: the dt bias dropped, softplus confused with e^v or
# with its mirror log(1 + e^-v), and the row read in the wrong order (xBC
# before z, or the raw step size taken from the head of the row).

import test_oracle_inproj_pins as IPINS
from oracle import inproj as IP

INPROJ_PINS = [(IPINS.test_softplus_closed_forms, ()),
               (IPINS.test_step_size_inverts_and_biases_per_head, ()),
               (IPINS.test_split_takes_head_middle_tail_of_the_row, ()),
               (IPINS.test_packed_prefill_equals_prefill_of_the_pieces, (True,)),
               (IPINS.test_mixed_batch_is_independent_sequences_with_decodes_first, ())]


def test_inproj_mutation_bias_dropped(monkeypatch):
    monkeypatch.setattr(IP, "step_size", lambda raw, bias: IP.softplus(np.asarray(raw, np.float64)))
    assert _red(INPROJ_PINS) >= 2


@pytest.mark.parametrize("wrong", ["exp", "mirror"])
def test_inproj_mutation_softplus(monkeypatch, wrong):
    real = IP.softplus
    fn = (lambda v: np.exp(np.minimum(np.asarray(v, np.float64), 700.0))) if wrong == "exp" \
        else (lambda v: real(-np.asarray(v, np.float64)))
    monkeypatch.setattr(IP, "softplus", fn)
    with np.errstate(over="ignore", invalid="ignore"):
        assert _red(INPROJ_PINS) >= 2


@pytest.mark.parametrize("order", ["xbc_first", "dt_at_head"])
def test_inproj_mutation_row_order(monkeypatch, order):
    def mutant(row, nheads, headdim, dstate, ngroups):
        di = nheads * headdim
        cd = di + 2 * ngroups * dstate
        if row.shape[1] < di + cd + nheads:
            raise ValueError("in-projection row narrower than z | xBC | dt")
        if order == "xbc_first":
            return row[:, cd:cd + di], row[:, :cd], row[:, di + cd:di + cd + nheads]
        return row[:, nheads:nheads + di], row[:, nheads + di:nheads + di + cd], row[:, :nheads]
    monkeypatch.setattr(IP, "split_inproj_row", mutant)
    assert _red(INPROJ_PINS) >= 2


def test_inproj_unmutated_pins_pass():
    assert _red(INPROJ_PINS) == 0
