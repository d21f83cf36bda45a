"""GPU parity of the single-token decode step (mamba2_decode, through the C ABI)
against the fp64 oracle.

A decode row is one step of the token recurrence the oracle is written as, so
the reference for a batch of decode rows is the oracle's prefill over
one-token sequences (cu_seqlens = 0, 1, ..., batch).  Metric and bars as for
the prefill: max|gpu - oracle| / RMS(oracle) per tensor, 1e-4 for fp32 inputs,
2e-2 for bf16 inputs.  The cases cover every compiled (headdim, dstate), the
production 8 heads per group (where a wrong group index would first show),
permuted cache slots, fresh slots (has_init = 0), both gate orders, a bf16
output, decode steps continuing a chunked prefill, a full-size batch at the
Nemotron-nano layer shape, and bitwise repeatability.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from oracle import recurrence as R
from workloads import NANO, LayerShape, WORKLOADS, make_inputs, small_shape_inputs
from parity_util import TOL, rel_err, split_views, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    m2.load()


def gpu_decode(d, shape, nbg=True, y_dtype=torch.float32, rows=slice(None), state_idx="inp",
               has_init="inp"):
    """One mamba2_decode call on rows `rows` of the device inputs `d` (states in place)."""
    x, B, C = split_views(d["xbc"][rows], shape)
    si = d["state_idx"] if state_idx == "inp" else state_idx
    hi = d["has_init"] if has_init == "inp" else has_init
    y = m2.mamba2_decode(x, B, C, d["z"][rows], d["dt"][rows], d["A"], d["D"], d["conv_w"],
                         d["conv_b"], d["norm_w"], d["conv_state"], d["ssm_state"], shape.nheads,
                         shape.headdim, shape.dstate, shape.ngroups, si, hi, 1e-5, nbg,
                         y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y


def check_decode(inp, shape, act, nbg=True):
    d = to_device(inp, act)
    y = gpu_decode(d, shape, nbg)
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups,
                    norm_before_gate=nbg)
    batch = len(inp["cu_seqlens"]) - 1
    tol = TOL[act]
    assert rel_err(y, ref["y"], "y", batch * shape.d_inner) <= tol
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= tol
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol


DECODE_CASES = [
    # (shape, batch, n_slots)
    (LayerShape(4, 16, 16, 2), 3, 5),
    (LayerShape(8, 32, 64, 2), 5, 9),
    (LayerShape(16, 64, 64, 4), 4, 4),
    (LayerShape(16, 64, 128, 2), 6, 11),      # 8 heads per group
    (LayerShape(64, 64, 128, 8), 3, 7),       # Nemotron-nano layer shape
    (LayerShape(128, 64, 128, 8), 2, 2),      # 16 heads per group (8B shape)
    (LayerShape(32, 64, 128, 1), 2, 3),       # group width 2048, the largest supported
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_batch_at_slots(case, act):
    shape, batch, n_slots = DECODE_CASES[case]
    inp = small_shape_inputs(shape, [1] * batch, seed=100 + case, act=act, init="pool",
                             n_slots=n_slots)
    # a mix of carried and fresh slots; the fresh ones start from zero states
    inp["has_init"] = (np.arange(batch) % 3 != 1).astype(np.uint8)
    print(f" shape={shape} batch={batch} slots={inp['state_idx'].tolist()}")
    check_decode(inp, shape, act)


@pytest.mark.parametrize("nbg", [True, False])
def test_decode_gate_orders(nbg):
    shape = LayerShape(16, 64, 128, 2)
    inp = small_shape_inputs(shape, [1] * 5, seed=120 + nbg, act="bf16", init="pool", n_slots=6)
    check_decode(inp, shape, "bf16", nbg)


def test_decode_bf16_output():
    """bf16 y: each element within one bf16 rounding of the fp32 result of the same call."""
    shape = NANO
    inp = small_shape_inputs(shape, [1] * 4, seed=130, act="bf16", init="pool", n_slots=4)
    d32 = to_device(inp, "bf16")
    d16 = to_device(inp, "bf16")
    y32 = gpu_decode(d32, shape)
    y16 = gpu_decode(d16, shape, y_dtype=torch.bfloat16)
    assert y16.dtype == torch.bfloat16
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert torch.equal(d16["ssm_state"], d32["ssm_state"])


def test_decode_continues_chunked_prefill_at_8_heads_per_group():
    """Nemotron-nano shape (8 heads per group): a 137-token chunked prefill
    (128 + 9) followed by 3 decode steps equals the oracle over 140 tokens."""
    shape = NANO
    inp = small_shape_inputs(shape, [140], seed=140, act="bf16", init="random")
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    d = to_device(inp, "bf16")
    x, B, C = split_views(d["xbc"], shape)
    cu = torch.tensor([0, 137], dtype=torch.int32, device="cuda")
    yp = m2.mamba2_prefill(x[:137], B[:137], C[:137], d["z"][:137], d["dt"][:137], d["A"], d["D"],
                           d["conv_w"], d["conv_b"], d["norm_w"], d["conv_state"], d["ssm_state"],
                           cu, 137, shape.nheads, shape.headdim, shape.dstate, shape.ngroups, 128,
                           d["state_idx"], d["has_init"])
    ys = [yp]
    for t in range(137, 140):
        ys.append(gpu_decode(d, shape, rows=slice(t, t + 1)))
    y = torch.cat(ys)
    tol = TOL["bf16"]
    assert rel_err(y[137:], ref["y"][137:], "y (decode rows)", 3 * shape.d_inner) <= tol
    assert rel_err(y, ref["y"], "y", 140 * shape.d_inner) <= tol
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= tol
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol


def test_decode_tiny_7_prefill_plus_4_steps_and_11_steps():
    """The tiny fp32 workload: 7 prefilled tokens + 4 decode steps, and 11 decode
    steps from zero states, both against the oracle over the 11 tokens."""
    w = WORKLOADS[0]
    s = w.shape
    inp = make_inputs(w, 0)
    ref = R.prefill(inp, s.nheads, s.headdim, s.dstate, s.ngroups)
    tol = TOL["f32"]
    for n_pre in (7, 0):
        d = to_device(inp, "f32")
        ys = []
        if n_pre:
            x, B, C = split_views(d["xbc"], s)
            cu = torch.tensor([0, n_pre], dtype=torch.int32, device="cuda")
            ys.append(m2.mamba2_prefill(x[:n_pre], B[:n_pre], C[:n_pre], d["z"][:n_pre],
                                        d["dt"][:n_pre], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                        d["norm_w"], d["conv_state"], d["ssm_state"], cu, n_pre,
                                        s.nheads, s.headdim, s.dstate, s.ngroups, w.chunk_size,
                                        d["state_idx"], d["has_init"]))
        one = torch.ones(1, dtype=torch.uint8, device="cuda")
        for t in range(n_pre, 11):
            hi = d["has_init"] if t == 0 else one
            ys.append(gpu_decode(d, s, rows=slice(t, t + 1), has_init=hi))
        print(f" prefill {n_pre} + {11 - n_pre} decode steps")
        assert rel_err(torch.cat(ys), ref["y"], "y", 11 * s.d_inner) <= tol
        assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= tol
        assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol


def test_decode_nano_full_batch_from_pool():
    """256 decode rows at the Nemotron-nano layer shape, slots permuted within a
    512-slot pool (every row checked), then repeated bitwise."""
    shape = NANO
    inp = small_shape_inputs(shape, [1] * 256, seed=150, act="bf16", init="pool", n_slots=512)
    d = to_device(inp, "bf16")
    cs0, ss0 = d["conv_state"].clone(), d["ssm_state"].clone()
    y = gpu_decode(d, shape)
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    tol = TOL["bf16"]
    assert rel_err(y, ref["y"], "y", 256 * shape.d_inner) <= tol
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= tol
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol
    # untouched slots keep their bits
    used = torch.as_tensor(inp["state_idx"], device="cuda", dtype=torch.long)
    free = torch.ones(512, dtype=torch.bool, device="cuda")
    free[used] = False
    assert torch.equal(d["ssm_state"][free], ss0[free]) and torch.equal(d["conv_state"][free], cs0[free])
    # same inputs and states again: the same bits
    cs1, ss1 = d["conv_state"].clone(), d["ssm_state"].clone()
    d["conv_state"].copy_(cs0)
    d["ssm_state"].copy_(ss0)
    m2.reset_counters()
    y2 = gpu_decode(d, shape)
    assert torch.equal(y2, y) and torch.equal(d["ssm_state"], ss1) and torch.equal(d["conv_state"], cs1)
    assert m2.get_counters()["decode_launches"] == 1


def test_decode_empty_batch_and_errors():
    shape = LayerShape(4, 16, 16, 2)
    inp = small_shape_inputs(shape, [1, 1], seed=160, act="f32", init="pool", n_slots=2)
    d = to_device(inp, "f32")
    cs0, ss0 = d["conv_state"].clone(), d["ssm_state"].clone()
    y = gpu_decode(d, shape, rows=slice(0, 0), state_idx=None, has_init=None)
    assert y.shape == (0, shape.d_inner)
    assert torch.equal(d["conv_state"], cs0) and torch.equal(d["ssm_state"], ss0)
    x, B, C = split_views(d["xbc"], shape)
    with pytest.raises(m2.M2Error, match="M2_ERR_UNSUPPORTED"):
        m2.mamba2_decode(x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                         d["norm_w"], d["conv_state"], d["ssm_state"], 2, 32, 16, 2)
    with pytest.raises(m2.M2Error, match="M2_ERR_SHAPE"):
        m2.mamba2_decode(x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                         d["norm_w"], d["conv_state"], d["ssm_state"], 4, 16, 16, 3)
