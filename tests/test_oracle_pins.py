"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties one oracle function to a hand-derived fixture, a closed form,
an invariant of the method, a library routine, or a second formulation of the
chunk algorithm, chosen so that a plausible slip (a dropped term, a wrong
sign or index, a transposed operand, a wrong group map, state read-out before
the update, a reversed conv) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import chunked as Ch
from oracle import recurrence as R
from workloads import TINY, WORKLOADS, LayerShape, make_inputs, small_shape_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_scan_inputs(rng, L, H, P, N, G, dt_scale=1.0, h0_scale=0.3):
    x = rng.standard_normal((L, H, P))
    B = rng.standard_normal((L, G, N))
    C = rng.standard_normal((L, G, N))
    dt = dt_scale * np.log1p(np.exp(rng.standard_normal((L, H)) - 1.0))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=H))
    D = rng.standard_normal(H)
    h0 = h0_scale * rng.standard_normal((H, P, N))
    return x, B, C, dt, A, D, h0


# ---------------------------------------------------------------- golden fixtures

def test_golden_scalar_recurrence():
    g = _golden("scalar_recurrence.json")
    i = g["inputs"]
    L = len(i["dt"])
    x = np.array(i["x"]).reshape(L, 1, 1)
    B = np.array(i["B"]).reshape(L, 1, 1)
    C = np.array(i["C"]).reshape(L, 1, 1)
    dt = np.array(i["dt"]).reshape(L, 1)
    y, h = R.ssd_recurrence_seq(x, B, C, dt, np.array([i["A"]]), np.array([i["D"]]),
                                np.full((1, 1, 1), i["h0"]))
    tol = g["tolerance_abs"]
    np.testing.assert_allclose(y.ravel(), g["expected"]["y"], rtol=0, atol=tol)
    np.testing.assert_allclose(h.ravel(), [g["expected"]["h_final"]], rtol=0, atol=tol)
    # The chunk form reaches the same numbers at every chunking.
    for q in (1, 2, 3, 4):
        yc, hc = Ch.chunk_scan_seq(x, B, C, dt, np.array([i["A"]]), np.array([i["D"]]),
                                   np.full((1, 1, 1), i["h0"]), q)
        np.testing.assert_allclose(yc.ravel(), g["expected"]["y"], rtol=0, atol=tol)
        np.testing.assert_allclose(hc.ravel(), [g["expected"]["h_final"]], rtol=0, atol=tol)


def test_golden_conv_rows():
    g = _golden("conv_rows.json")
    i = g["inputs"]
    rows = np.array(i["rows"]).reshape(-1, 1)
    state = np.array(i["state"]).reshape(-1, 1)
    w = np.array(i["w"]).reshape(1, -1)
    u, st = R.conv_rows_seq(rows, w, np.array([i["b"]]), state, apply_silu=False)
    assert np.array_equal(u.ravel(), np.array(g["expected"]["pre_activation"]))
    assert np.array_equal(st.ravel(), np.array(g["expected"]["state_out"]))


def test_golden_gated_norm():
    g = _golden("gated_norm.json")
    i = g["inputs"]
    y = np.array(i["y"]).reshape(1, -1)
    z = np.array(i["z"]).reshape(1, -1)
    for key, nbg in (("norm_before_gate", True), ("gate_before_norm", False)):
        out = R.gated_rmsnorm_group(y, z, np.array(i["w"]), i["eps"], i["ngroups"], nbg)
        np.testing.assert_allclose(out.ravel(), g["expected"][key], rtol=0,
                                   atol=g["tolerance_abs"])


# ---------------------------------------------------------------- recurrence vs chunk forms

@pytest.mark.parametrize("H,G", [(2, 2), (4, 2), (8, 1), (16, 2)])
@pytest.mark.parametrize("chunk", [1, 3, 7, 16])
def test_recurrence_equals_chunk_form(H, G, chunk):
    rng = np.random.default_rng(100 * H + chunk)
    L, P, N = 23, 4, 5
    x, B, C, dt, A, D, h0 = _rand_scan_inputs(rng, L, H, P, N, G)
    y1, h1 = R.ssd_recurrence_seq(x, B, C, dt, A, D, h0)
    y2, h2 = Ch.chunk_scan_seq(x, B, C, dt, A, D, h0, chunk)
    assert np.max(np.abs(y2 - y1)) <= 1e-12 * np.max(np.abs(y1))
    assert np.max(np.abs(h2 - h1)) <= 1e-12 * np.max(np.abs(h1))


@pytest.mark.parametrize("H,G", [(2, 1), (4, 2), (8, 1)])
def test_recurrence_equals_materialized_dual_form(H, G):
    rng = np.random.default_rng(7 + H)
    L, P, N = 12, 3, 4
    x, B, C, dt, A, D, h0 = _rand_scan_inputs(rng, L, H, P, N, G)
    y1, h1 = R.ssd_recurrence_seq(x, B, C, dt, A, D, h0)
    y2, h2 = Ch.dual_form_seq(x, B, C, dt, A, D, h0)
    assert np.max(np.abs(y2 - y1)) <= 1e-12 * np.max(np.abs(y1))
    assert np.max(np.abs(h2 - h1)) <= 1e-12 * np.max(np.abs(h1))


# ---------------------------------------------------------------- closed forms

def test_no_decay_is_causal_linear_attention():
    """A = 0, D = 0: y_t = C_t . sum_{i<=t} dt_i x_i (outer) B_i, via numpy cumsum."""
    rng = np.random.default_rng(3)
    L, H, P, N, G = 17, 4, 3, 5, 2
    x, B, C, dt, _, _, _ = _rand_scan_inputs(rng, L, H, P, N, G)
    A = np.zeros(H)
    h0 = np.zeros((H, P, N))
    y, h = R.ssd_recurrence_seq(x, B, C, dt, A, None, h0)
    grp = np.arange(H) // (H // G)
    kv = (dt[:, :, None, None] * x[:, :, :, None]) * B[:, grp][:, :, None, :]   # [L,H,P,N]
    S = np.cumsum(kv, axis=0)
    ref = np.einsum("lhpn,lhn->lhp", S, C[:, grp])
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(h, S[-1], rtol=1e-12, atol=1e-12)


def test_huge_decay_is_memoryless_and_finite():
    """|dt*A| = 1e6 on every row: y_t = (C_t.B_t) dt_t x_t + D x_t; h_out = dt x (outer) B of the last row."""
    rng = np.random.default_rng(4)
    L, H, P, N, G = 9, 4, 3, 5, 2
    x, B, C, _, A, D, h0 = _rand_scan_inputs(rng, L, H, P, N, G)
    dt = np.broadcast_to(1e6 / np.abs(A)[None, :], (L, H)).copy()
    grp = np.arange(H) // (H // G)
    ref_y = np.einsum("lhn,lhn->lh", C[:, grp], B[:, grp])[:, :, None] * dt[:, :, None] * x \
        + D[None, :, None] * x
    ref_h = (dt[-1][:, None] * x[-1])[:, :, None] * B[-1, grp][:, None, :]
    for fn in (lambda: R.ssd_recurrence_seq(x, B, C, dt, A, D, h0),
               lambda: Ch.chunk_scan_seq(x, B, C, dt, A, D, h0, 4)):
        y, h = fn()
        assert np.all(np.isfinite(y)) and np.all(np.isfinite(h))
        np.testing.assert_allclose(y, ref_y, rtol=1e-12, atol=1e-9)
        np.testing.assert_allclose(h, ref_h, rtol=1e-12, atol=1e-9)


def test_scalar_recurrence_closed_form_products():
    """H = P = N = 1: h_t = (prod_{k<=t} alpha_k) h0 + sum_i (prod_{i<k<=t} alpha_k) beta_i."""
    rng = np.random.default_rng(5)
    L = 30
    x, B, C, dt, A, D, h0 = _rand_scan_inputs(rng, L, 1, 1, 1, 1)
    y, h = R.ssd_recurrence_seq(x, B, C, dt, A, D, h0)
    alpha = np.exp(dt[:, 0] * A[0])
    beta = dt[:, 0] * x[:, 0, 0] * B[:, 0, 0]
    hs = np.empty(L)
    for t in range(L):
        hs[t] = np.prod(alpha[:t + 1]) * h0[0, 0, 0] + sum(
            np.prod(alpha[i + 1:t + 1]) * beta[i] for i in range(t + 1))
    np.testing.assert_allclose(y[:, 0, 0], hs * C[:, 0, 0] + D[0] * x[:, 0, 0], rtol=1e-12)
    np.testing.assert_allclose(h[0, 0, 0], hs[-1], rtol=1e-12)


@pytest.mark.parametrize("zero", ["B", "C"])
def test_zero_B_or_C_leaves_only_skip(zero):
    rng = np.random.default_rng(6)
    L, H, P, N, G = 8, 4, 3, 5, 2
    x, B, C, dt, A, D, _ = _rand_scan_inputs(rng, L, H, P, N, G)
    h0 = np.zeros((H, P, N))
    if zero == "B":
        B[:] = 0
    else:
        C[:] = 0
    y, _ = R.ssd_recurrence_seq(x, B, C, dt, A, D, h0)
    np.testing.assert_allclose(y, D[None, :, None] * x, rtol=0, atol=0)


def test_group_map_is_contiguous_heads():
    """6 heads in 3 groups (2 heads per group); only group 1 has nonzero B, so only heads 2 and 3 carry SSM output."""
    rng = np.random.default_rng(8)
    L, H, P, N, G = 6, 6, 2, 3, 3
    x, B, C, dt, A, D, _ = _rand_scan_inputs(rng, L, H, P, N, G)
    B[:, [0, 2]] = 0.0
    y, _ = R.ssd_recurrence_seq(x, B, C, dt, A, D, np.zeros((H, P, N)))
    ssm = y - D[None, :, None] * x
    hpg = H // G
    for h in range(H):
        if h // hpg == 1:
            assert np.max(np.abs(ssm[:, h])) > 1e-3
        else:
            assert np.max(np.abs(ssm[:, h])) == 0.0


def test_positive_exponent_is_detected():
    """The chunk form asserts every exponent <= 0; a growing mode (A > 0) must trip it."""
    rng = np.random.default_rng(9)
    x, B, C, dt, A, D, h0 = _rand_scan_inputs(rng, 5, 2, 2, 2, 1)
    with pytest.raises(Ch.PositiveExponent):
        Ch.chunk_scan_seq(x, B, C, dt, np.abs(A), D, h0, 4)


# ---------------------------------------------------------------- the x | B | C split of the conv output
#
# Page "feat(#1311 A2-D1): NemotronH decodes on the single-step recurrent
# kernels ...", PR description: the conv output is split as QkvSplit(x | B | C);
# page "Nemotron-H", section 4.1: xBC is the joint (x, B, C) stream, B enters
# the state update and C the read-out.

def test_split_xbc_takes_x_then_B_then_C():
    """Channel c of a conv-output row carries the value c: the split must give
    x = channels [0, H*P), B = [H*P, H*P + G*N), C = [H*P + G*N, H*P + 2*G*N),
    with x[t, h, p] = u[t, h*P + p] and B[t, g, n] = u[t, H*P + g*N + n]."""
    H, P, G, N, L = 4, 3, 2, 5, 3
    di, gn = H * P, G * N
    u = np.arange(L)[:, None] * 1000.0 + np.arange(di + 2 * gn)[None, :]
    x, B, C = R.split_xbc(u, H, P, G, N)
    assert x.shape == (L, H, P) and B.shape == (L, G, N) and C.shape == (L, G, N)
    for t in range(L):
        for h in range(H):
            for p in range(P):
                assert x[t, h, p] == 1000.0 * t + h * P + p
        for g in range(G):
            for n in range(N):
                assert B[t, g, n] == 1000.0 * t + di + g * N + n
                assert C[t, g, n] == 1000.0 * t + di + gn + g * N + n


def test_one_token_roles_of_B_and_C():
    """One token through the whole prefill driver, identity conv tap (u =
    silu(xBC)) and a carried state h0: the new state is e^{dt A} h0 + dt x (outer)
    B with B = silu of the middle channel run, and the pre-norm output is
    C . h + D x with C = silu of the last run.  B and C hold different values,
    so reading them the other way round changes both."""
    H, P, N, G = 2, 3, 4, 1
    di, gn = H * P, G * N
    cd = di + 2 * gn
    row = np.concatenate([np.linspace(-1.0, 1.0, di), np.arange(1, N + 1) * 0.5,
                          -np.arange(1, N + 1) * 0.25])[None, :]
    w = np.zeros((cd, 4))
    w[:, 3] = 1.0
    rng = np.random.default_rng(91)
    h0 = rng.standard_normal((1, H, P, N))
    dt = np.array([[0.3, 0.7]])
    A = np.array([-1.5, -0.5])
    D = np.array([0.25, -2.0])
    inp = dict(xbc=row, conv_w=w, conv_b=np.zeros(cd), conv_state=np.zeros((1, 3, cd)),
               ssm_state=h0, dt=dt, A=A, D=D, z=np.zeros((1, di)), norm_w=np.ones(di),
               cu_seqlens=np.array([0, 1]), state_idx=np.array([0]), has_init=np.array([1]))
    out = R.prefill(inp, H, P, N, G, apply_norm=False)
    sx = row[0, :di] / (1.0 + np.exp(-row[0, :di]))
    sb = row[0, di:di + gn] / (1.0 + np.exp(-row[0, di:di + gn]))
    sc = row[0, di + gn:] / (1.0 + np.exp(-row[0, di + gn:]))
    for h in range(H):
        xh = sx[h * P:(h + 1) * P]
        want_h = math.exp(dt[0, h] * A[h]) * h0[0, h] + dt[0, h] * np.outer(xh, sb)
        np.testing.assert_allclose(out["ssm_state"][0, h], want_h, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(out["y"][0, h * P:(h + 1) * P], want_h @ sc + D[h] * xh,
                                   rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- conv and norm vs library routines

def test_conv_identity_tap_is_silu():
    rng = np.random.default_rng(10)
    L, Cd = 7, 5
    xs = rng.standard_normal((L, Cd))
    w = np.zeros((Cd, 4))
    w[:, 3] = 1.0
    u, _ = R.conv_rows_seq(xs, w, None, rng.standard_normal((3, Cd)))
    np.testing.assert_allclose(u, xs / (1.0 + np.exp(-xs)), rtol=1e-14)


@pytest.mark.parametrize("L", [1, 2, 3, 4, 9])
def test_conv_matches_numpy_convolve(L):
    rng = np.random.default_rng(11 + L)
    Cd = 6
    xs = rng.standard_normal((L, Cd))
    w = rng.standard_normal((Cd, 4))
    b = rng.standard_normal(Cd)
    st = rng.standard_normal((3, Cd))
    u, st_out = R.conv_rows_seq(xs, w, b, st, apply_silu=False)
    for c in range(Cd):
        stream = np.concatenate([st[:, c], xs[:, c]])
        # np.convolve flips its kernel; flipping w back makes w[3] hit the newest row.
        full = np.convolve(stream, w[c, ::-1], mode="valid")
        np.testing.assert_allclose(u[:, c], full + b[c], rtol=1e-13, atol=1e-13)
        np.testing.assert_array_equal(st_out[:, c], stream[-3:])


@pytest.mark.parametrize("nbg", [True, False])
def test_norm_single_group_matches_torch_rms_norm(nbg):
    rng = np.random.default_rng(12)
    T, d = 5, 32
    y = rng.standard_normal((T, d))
    z = rng.standard_normal((T, d))
    w = 1 + 0.1 * rng.standard_normal(d)
    eps = 1e-5
    out = R.gated_rmsnorm_group(y, z, w, eps, 1, nbg)
    yt, zt, wt = (torch.tensor(a, dtype=torch.float64) for a in (y, z, w))
    gate = torch.nn.functional.silu(zt)
    if nbg:
        ref = torch.nn.functional.rms_norm(yt, (d,), wt, eps) * gate
    else:
        ref = torch.nn.functional.rms_norm(yt * gate, (d,), wt, eps)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_norm_groups_are_independent_contiguous_runs():
    rng = np.random.default_rng(13)
    T, d, G = 4, 24, 3
    y = rng.standard_normal((T, d))
    z = rng.standard_normal((T, d))
    w = rng.standard_normal(d)
    out = R.gated_rmsnorm_group(y, z, w, 1e-6, G, True)
    g = d // G
    for j in range(G):
        sl = slice(j * g, (j + 1) * g)
        np.testing.assert_allclose(out[:, sl], R.gated_rmsnorm_group(y[:, sl], z[:, sl], w[sl],
                                                                     1e-6, 1, True), rtol=1e-14)


# ---------------------------------------------------------------- invariants of the whole core

def _split_call(inp, cuts, shape, seq_rows):
    """Run the oracle prefill on the rows of one sequence cut into consecutive pieces, carrying states."""
    s = shape
    cs = np.array(inp["conv_state"], copy=True)
    ss = np.array(inp["ssm_state"], copy=True)
    ys = []
    lo = 0
    has_init = inp["has_init"].copy()
    for n in cuts:
        piece = dict(inp)
        piece["xbc"] = inp["xbc"][lo:lo + n]
        piece["z"] = inp["z"][lo:lo + n]
        piece["dt"] = inp["dt"][lo:lo + n]
        piece["cu_seqlens"] = np.array([0, n], dtype=np.int32)
        piece["conv_state"] = cs
        piece["ssm_state"] = ss
        piece["has_init"] = has_init
        out = R.prefill(piece, s.nheads, s.headdim, s.dstate, s.ngroups)
        ys.append(out["y"])
        cs, ss = out["conv_state"], out["ssm_state"]
        has_init = np.ones_like(has_init)
        lo += n
    assert lo == seq_rows
    return np.concatenate(ys), cs, ss


def test_split_7_plus_4_equals_11_equals_11_single_steps():
    """The 11-token prompt: chunks 7 + 4 and 11 one-token calls give the 11-token result."""
    w = WORKLOADS[0]
    inp = make_inputs(w, 0)
    s = w.shape
    full = R.prefill(inp, s.nheads, s.headdim, s.dstate, s.ngroups)
    for cuts in ([7, 4], [1] * 11, [11]):
        y, cs, ss = _split_call(inp, cuts, s, 11)
        np.testing.assert_allclose(y, full["y"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(cs, full["conv_state"], rtol=0, atol=0)
        np.testing.assert_allclose(ss, full["ssm_state"], rtol=1e-12, atol=1e-12)


def test_has_init_zero_equals_zero_states():
    shape = LayerShape(4, 8, 8, 2)
    inp = small_shape_inputs(shape, [5, 3], seed=21, init="random")
    a = dict(inp)
    a["has_init"] = np.array([0, 1], dtype=np.uint8)
    b = dict(inp)
    b["conv_state"] = inp["conv_state"].copy()
    b["ssm_state"] = inp["ssm_state"].copy()
    b["conv_state"][0] = 0
    b["ssm_state"][0] = 0
    oa = R.prefill(a, 4, 8, 8, 2)
    ob = R.prefill(b, 4, 8, 8, 2)
    for k in ("y", "conv_state", "ssm_state"):
        np.testing.assert_array_equal(oa[k], ob[k])


def test_decay_stress_small_shape_finite_and_chunk_form_agrees():
    """Decay-stress distribution (|dt A| up to 1e6, 5% at 1e6) on a small shape: finite, and both forms agree."""
    shape = LayerShape(4, 8, 16, 2)
    inp = small_shape_inputs(shape, [300], seed=3, dt_mode="stress", init="zero")
    out = R.prefill(inp, 4, 8, 16, 2, apply_norm=False)
    assert np.all(np.isfinite(out["y"])) and np.all(np.isfinite(out["ssm_state"]))
    x, B, C = R.split_xbc(out["u"], 4, 8, 2, 16)
    yc, hc = Ch.chunk_scan_seq(x, B, C, inp["dt"], inp["A"], inp["D"],
                               np.zeros((4, 8, 16)), 128)
    y_rec = out["y"].reshape(300, 4, 8)
    # gamma reaches ~1e8 inside a chunk here, so each exponent difference
    # gamma_t - gamma_i carries an fp64 absolute error near 1e8 * 2^-53 ~ 1e-8:
    # the two forms agree to about that relative size of the largest terms.
    assert np.max(np.abs(yc - y_rec)) <= 1e-9 * np.max(np.abs(y_rec))
    assert np.max(np.abs(hc - out["ssm_state"][0])) <= 1e-9 * np.max(np.abs(hc))


def test_varlen_batch_equals_per_sequence_runs():
    shape = LayerShape(4, 8, 8, 2)
    lens = [5, 1, 0, 9]
    inp = small_shape_inputs(shape, lens, seed=31, init="random")
    full = R.prefill(inp, 4, 8, 8, 2)
    cu = inp["cu_seqlens"]
    for b, L in enumerate(lens):
        one = dict(inp)
        one["xbc"] = inp["xbc"][cu[b]:cu[b + 1]]
        one["z"] = inp["z"][cu[b]:cu[b + 1]]
        one["dt"] = inp["dt"][cu[b]:cu[b + 1]]
        one["cu_seqlens"] = np.array([0, L], dtype=np.int32)
        one["state_idx"] = inp["state_idx"][b:b + 1]
        one["has_init"] = inp["has_init"][b:b + 1]
        o = R.prefill(one, 4, 8, 8, 2)
        np.testing.assert_array_equal(o["y"], full["y"][cu[b]:cu[b + 1]])
        slot = inp["state_idx"][b]
        np.testing.assert_array_equal(o["ssm_state"][slot], full["ssm_state"][slot])
        np.testing.assert_array_equal(o["conv_state"][slot], full["conv_state"][slot])


# ---------------------------------------------------------------- segment carry

@pytest.mark.parametrize("cuts", [(7,), (5, 13), (1, 2, 20)])
def test_segment_carry_identity(cuts):
    """A sequence cut into segments, each later segment run from a zero state,
    joined back: with E_k the segment's end state from its own start and
    lambda_k = sum of dt*A over it, T_0 = E_0, T_k = exp(lambda_k) T_{k-1} + E_k
    is the true end state, and the true outputs of segment k add
    exp(sum of dt*A from the segment's start through t) * C_t . T_{k-1} to
    the local ones.  This is the carry both scan paths use for long sequences
    (the bf16 state pass, and the fp64 one-pass path with its readout fix) and
    the rank-level carry of a sequence split over devices."""
    rng = np.random.default_rng(81)
    L, H, P, N, G = 24, 4, 3, 5, 2
    x, B, C, dt, A, D, h0 = _rand_scan_inputs(rng, L, H, P, N, G)
    y_ref, h_ref = R.ssd_recurrence_seq(x, B, C, dt, A, D, h0)
    grp = np.arange(H) // (H // G)
    bounds = [0, *cuts, L]
    T = None
    y = np.zeros_like(y_ref)
    for k in range(len(bounds) - 1):
        lo, hi = bounds[k], bounds[k + 1]
        start = h0 if k == 0 else np.zeros_like(h0)
        yk, Ek = R.ssd_recurrence_seq(x[lo:hi], B[lo:hi], C[lo:hi], dt[lo:hi], A, D, start)
        if k > 0:
            a = dt[lo:hi] * A[None, :]                       # [S, H]
            decay_t = np.exp(np.cumsum(a, axis=0))           # through row t, inclusive
            inter = np.einsum("hpn,thn->thp", T, C[lo:hi][:, grp])
            yk = yk + decay_t[:, :, None] * inter
            Ek = np.exp(a.sum(axis=0))[:, None, None] * T + Ek
        y[lo:hi] = yk
        T = Ek
    np.testing.assert_allclose(y, y_ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(T, h_ref, rtol=1e-11, atol=1e-12)
