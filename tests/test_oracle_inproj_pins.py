"""Pins of oracle.inproj (CPU only): the step-size function, the split of the
in-projection row, the packed-row prefill and the mixed decode + prefill batch.

Each pin checks the oracle against something other than itself: closed forms of
softplus, an independently computed inverse, the layout of a row built from
known pieces, and the separately pinned recurrence driver.
"""
import math

import numpy as np
import pytest

from oracle import inproj as IP
from oracle import recurrence as R
from workloads import LayerShape, inproj_inputs


def test_softplus_closed_forms():
    assert IP.softplus(np.array([0.0]))[0] == pytest.approx(math.log(2.0), abs=1e-16)
    v = np.linspace(-50.0, 50.0, 1001)
    # softplus(v) - softplus(-v) = v  (log((1 + e^v) / (1 + e^-v)) = v)
    np.testing.assert_allclose(IP.softplus(v) - IP.softplus(-v), v, rtol=0, atol=1e-13)
    # the naive definition where it neither overflows nor loses digits in 1 + e^v
    m = np.linspace(-5.0, 30.0, 701)
    np.testing.assert_allclose(IP.softplus(m), np.log(1.0 + np.exp(m)), rtol=1e-13)
    # no overflow at the ends: softplus(800) = 800, softplus(-700) = e^-700 > 0
    assert IP.softplus(np.array([800.0]))[0] == 800.0
    far = IP.softplus(np.array([-700.0]))[0]
    assert far > 0 and far == pytest.approx(math.exp(-700.0), rel=1e-12)
    # derivative is the logistic function
    h = 1e-5
    d = (IP.softplus(m + h) - IP.softplus(m - h)) / (2 * h)
    np.testing.assert_allclose(d, 1.0 / (1.0 + np.exp(-m)), rtol=0, atol=1e-9)


def test_step_size_inverts_and_biases_per_head():
    rng = np.random.default_rng(3)
    T, H = 5, 3
    target = rng.uniform(1e-4, 5.0, size=(T, H))
    bias = np.array([-4.0, -2.5, -3.25])
    raw = np.log(np.expm1(target)) - bias[None, :]  # inverse of softplus, computed by numpy
    np.testing.assert_allclose(IP.step_size(raw, bias), target, rtol=1e-12)
    # raw = 0: every row of column h is softplus(bias_h)
    z = IP.step_size(np.zeros((T, H)), bias)
    np.testing.assert_allclose(z, np.broadcast_to(np.log1p(np.exp(bias))[None, :], (T, H)), rtol=1e-15)


def test_split_takes_head_middle_tail_of_the_row():
    H, P, N, G = 4, 16, 16, 2
    di, cd = H * P, H * P + 2 * G * N
    T, ld = 3, IP.row_width(H, P, N, G) + 5
    row = np.full((T, ld), -1.0)
    row[:, :di] = 100 + np.arange(di)
    row[:, di:di + cd] = 200 + np.arange(cd)
    row[:, di + cd:di + cd + H] = 300 + np.arange(H)
    z, xbc, dt_raw = IP.split_inproj_row(row, H, P, N, G)
    assert z.shape == (T, di) and xbc.shape == (T, cd) and dt_raw.shape == (T, H)
    assert np.all(z == 100 + np.arange(di)) and np.all(xbc == 200 + np.arange(cd))
    assert np.all(dt_raw == 300 + np.arange(H))
    with pytest.raises(ValueError):
        IP.split_inproj_row(row[:, :di + cd + H - 1], H, P, N, G)


@pytest.mark.parametrize("nbg", [True, False])
def test_packed_prefill_equals_prefill_of_the_pieces(nbg):
    shape = LayerShape(4, 16, 16, 2)
    inp = inproj_inputs(shape, [9, 1, 20], seed=11, act="f32")
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    di, cd = shape.d_inner, shape.conv_dim
    # choose the step sizes, and write the raw values that produce them into the row
    rng = np.random.default_rng(4)
    T = inp["row"].shape[0]
    target = rng.uniform(0.01, 2.0, size=(T, H))
    row = inp["row"].astype(np.float64)
    row[:, di + cd:di + cd + H] = np.log(np.expm1(target)) - inp["dt_bias"].astype(np.float64)[None, :]
    got = IP.prefill_inproj(dict(inp, row=row), H, P, N, G, norm_before_gate=nbg)
    pieces = {k: v for k, v in inp.items() if k not in ("row", "dt_bias")}
    pieces.update(z=row[:, :di], xbc=row[:, di:di + cd], dt=target)
    want = R.prefill(pieces, H, P, N, G, norm_before_gate=nbg)
    for k in ("y", "conv_state", "ssm_state"):
        np.testing.assert_allclose(got[k], want[k], rtol=1e-11, atol=1e-12)


def test_mixed_batch_is_independent_sequences_with_decodes_first():
    shape = LayerShape(4, 16, 16, 2)
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    lens = [1, 1, 1, 6, 1, 13]  # three decode rows, then prefills (one of them T == 1)
    inp = inproj_inputs(shape, lens, seed=2, act="f32", init="random")
    inp["has_init"] = np.array([1, 1, 1, 0, 0, 1], dtype=np.uint8)
    got = IP.mixed_batch(inp, 3, H, P, N, G)
    cu = inp["cu_seqlens"]
    for b in range(len(lens)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        one = dict(inp, row=inp["row"][lo:hi], cu_seqlens=np.array([0, hi - lo], np.int32),
                   state_idx=inp["state_idx"][b:b + 1], has_init=inp["has_init"][b:b + 1])
        alone = IP.prefill_inproj(one, H, P, N, G)
        np.testing.assert_allclose(got["y"][lo:hi], alone["y"], rtol=1e-12, atol=1e-13)
        s = int(inp["state_idx"][b])
        np.testing.assert_allclose(got["ssm_state"][s], alone["ssm_state"][s], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got["conv_state"][s], alone["conv_state"][s], rtol=0, atol=0)
    with pytest.raises(ValueError):
        IP.mixed_batch(inp, 4, H, P, N, G)  # sequence 3 has 6 rows: not a decode row
