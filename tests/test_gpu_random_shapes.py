"""Seeded random layer shapes and batches through mamba2_prefill, against the fp64 oracle.

Each case draws, from its own seed: the activation dtype, heads, groups and
a (headdim, dstate) pair the library has kernels for (bf16 at headdim 64
takes the chunk-parallel path, smaller pairs and fp32 inputs the one-pass
scan), 1 to 6 sequences of
0 to 700 tokens (with chunk-boundary and one-token lengths mixed in), zero,
random or slot-pool initial states (pool slots in random order, some marked
fresh), the gate order and the output dtype.  Whichever kernels the shape
selects (raw-row scan kernels with or without the fused norm, the chain, the
one-pass scan), y, the conv state and the ssm state must meet the bars the
other parity tests use (bf16 outputs: one bf16 rounding on top).  The decode
sweep draws the same way for mamba2_decode: a supported (headdim, dstate) pair,
groups, heads per group up to the 2048-channel group width, 1 to 300 one-token
rows at shuffled pool slots (some fresh), the gate order and the output dtype.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from oracle import recurrence as R
from workloads import LayerShape, small_shape_inputs
from parity_util import TOL, rel_err, split_views, to_device
from test_gpu_parity import gpu_prefill

pytestmark = pytest.mark.gpu

SPECIAL_LENS = [0, 1, 2, 3, 127, 128, 129, 255, 256, 257]


def draw_case(seed):
    r = np.random.default_rng(1000 + seed)
    act = "f32" if seed % 4 == 3 else "bf16"
    # the (headdim, dstate) pairs the library has scan kernels for; bf16 mostly
    # at headdim 64 (the chunk-parallel path), sometimes smaller (the one-pass scan)
    pairs = [(64, 64), (64, 128)] * (3 if act == "bf16" else 1) + [(16, 16), (32, 64)]
    headdim, dstate = pairs[int(r.integers(0, len(pairs)))]
    ngroups = int(r.choice([1, 2, 4]))
    hpg = int(r.choice([1, 2, 3, 4, 8]))
    nheads = ngroups * hpg
    batch = int(r.integers(1, 7))
    lens = [int(r.choice(SPECIAL_LENS)) if r.random() < 0.4 else int(r.integers(0, 701)) for _ in range(batch)]
    if sum(lens) == 0:
        lens[0] = int(r.integers(1, 300))
    init = str(r.choice(["zero", "random", "pool"]))
    nbg = bool(r.random() < 0.5)
    y_dtype = torch.bfloat16 if (act == "bf16" and r.random() < 0.3) else torch.float32
    return act, LayerShape(nheads, headdim, dstate, ngroups), lens, init, nbg, y_dtype, r


@pytest.mark.parametrize("seed", range(48))
def test_random_shape_against_oracle(seed):
    act, shape, lens, init, nbg, y_dtype, r = draw_case(seed)
    print(f" act={act} shape={shape} lens={lens} init={init} nbg={nbg} y={y_dtype}", flush=True)
    n_slots = len(lens) + 3
    inp = small_shape_inputs(shape, lens, seed=5000 + seed, act=act, init=init, n_slots=n_slots)
    if init == "pool":
        inp["has_init"] = (r.random(len(lens)) < 0.6).astype(np.uint8)
    y, cs, ss = gpu_prefill(inp, shape, act, nbg=nbg, y_dtype=y_dtype)
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups, norm_before_gate=nbg)
    tol = TOL[act]
    T = sum(lens)
    if y_dtype == torch.float32:
        assert rel_err(y, ref["y"], "y", T * shape.d_inner) <= tol
    else:
        yr = ref["y"]
        g = y.double().cpu().numpy()
        assert g.shape == yr.shape
        bound = 2.0 ** -8 * np.abs(yr) + tol * np.sqrt(np.mean(yr * yr))
        worst = float(np.max(np.abs(g - yr) - bound))
        print(f"  y (bf16): worst excess over the bound {worst:.3e}", flush=True)
        assert worst <= 0.0
    assert rel_err(cs, ref["conv_state"], "conv_state") <= tol
    assert rel_err(ss, ref["ssm_state"], "ssm_state") <= tol


def draw_decode_case(seed):
    r = np.random.default_rng(2000 + seed)
    act = "f32" if seed % 3 == 2 else "bf16"
    headdim, dstate = [(64, 64), (64, 128), (64, 128), (16, 16), (32, 64)][int(r.integers(0, 5))]
    ngroups = int(r.choice([1, 2, 4, 8]))
    # heads per group up to a group width (hpg * headdim) of 2048, the decode's limit
    hpg = int(r.choice([1, 2, 3, 5, 8, 16, 32]))
    while hpg * headdim > 2048:
        hpg //= 2
    batch = int(r.integers(1, 301))
    n_slots = batch + int(r.integers(0, 8))
    nbg = bool(r.random() < 0.5)
    y_dtype = torch.bfloat16 if (act == "bf16" and r.random() < 0.3) else torch.float32
    return act, LayerShape(ngroups * hpg, headdim, dstate, ngroups), batch, n_slots, nbg, y_dtype, r


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_batch_against_oracle(seed):
    """mamba2_decode on a seeded random shape and batch (1 to 300 rows at
    permuted pool slots, some fresh), against the oracle's one-token prefill."""
    act, shape, batch, n_slots, nbg, y_dtype, r = draw_decode_case(seed)
    print(f" act={act} shape={shape} batch={batch} slots={n_slots} nbg={nbg} y={y_dtype}", flush=True)
    inp = small_shape_inputs(shape, [1] * batch, seed=6000 + seed, act=act, init="pool", n_slots=n_slots)
    inp["has_init"] = (r.random(batch) < 0.7).astype(np.uint8)
    d = to_device(inp, act)
    x, B, C = split_views(d["xbc"], shape)
    y = m2.mamba2_decode(x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"], d["norm_w"],
                         d["conv_state"], d["ssm_state"], shape.nheads, shape.headdim, shape.dstate,
                         shape.ngroups, d["state_idx"], d["has_init"], 1e-5, nbg, y_dtype=y_dtype)
    torch.cuda.synchronize()
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups, norm_before_gate=nbg)
    tol = TOL[act]
    if y_dtype == torch.float32:
        assert rel_err(y, ref["y"], "y", batch * shape.d_inner) <= tol
    else:
        yr = ref["y"]
        g = y.double().cpu().numpy()
        bound = 2.0 ** -8 * np.abs(yr) + tol * np.sqrt(np.mean(yr * yr))
        assert float(np.max(np.abs(g - yr) - bound)) <= 0.0
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= tol
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol
