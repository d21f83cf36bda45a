"""The prefill's scan kernels convolving the raw bf16 rows themselves, against
the four-kernel chain (conv kernel, fp32 post-conv activations in the
workspace, selected with M2SSD_PREFILL_CHAIN=1).  Both compute the conv with
the same operations in the same order and feed the same (hi, lo) products, so
the conv state must be bitwise equal, and y and the SSM state agree to the
rounding of the split products (the compiler may fuse the dt weighting of x
into the low part of the split differently in the two kernels; where that
moves a value across a bf16 rounding boundary its (hi, lo) pair changes and
the product with it, at ~1e-5 of the values -- measured: both paths are as far
from the oracle as from each other; the check allows 1e-3 of the RMS); each is
also checked against the fp64 oracle at the bf16 bar.  Cases: sequences shorter than the conv's 3-row
halo (their first rows read the carried conv state), ragged chunk tails,
empty sequences, dstate 64 (one head per state-pass workgroup), long
sequences split into segments, the 137-token prompt (chunk output split over
heads), both gate orders, a fresh slot next to carried ones.

Where each chunk-output workgroup holds a whole norm group (no split over
heads) the chunk output also applies the gated norm to its rows and the norm
kernel does not run; the chain always runs it.  The last three cases take that
path: group widths 512 and 128 (lanes past the group's 8-channel blocks idle),
fp32 and bf16 outputs, both gate orders."""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from oracle import recurrence as R
from workloads import LayerShape, small_shape_inputs
from parity_util import TOL, rel_err, split_views, to_device
from test_gpu_parity import gpu_prefill

pytestmark = pytest.mark.gpu

SHORT_LENS = [1 + (7 * b) % 24 for b in range(130)]
MANY_LENS = [1 + (5 * b) % 9 for b in range(1500)]

CASES = [
    # (shape, lengths, init, norm_before_gate, output dtype, norm fused into the chunk output)
    (LayerShape(16, 64, 128, 2), [300, 1, 2, 3, 129, 0, 257], "random", True, torch.float32, False),
    (LayerShape(16, 64, 128, 2), [300, 1, 2, 3, 129, 0, 257], "random", False, torch.float32, False),
    (LayerShape(8, 64, 64, 4), [513, 3, 0, 128], "pool", True, torch.float32, False),
    (LayerShape(16, 64, 128, 2), [2000, 700, 1, 0], "pool", True, torch.float32, False),
    (LayerShape(64, 64, 128, 8), [137], "zero", True, torch.float32, False),
    (LayerShape(32, 64, 128, 2), [4096], "random", True, torch.float32, False),
    (LayerShape(64, 64, 128, 8), [1500, 700, 3, 0, 129], "pool", True, torch.bfloat16, True),
    (LayerShape(64, 64, 128, 8), [1500, 700, 3, 0, 129], "random", False, torch.float32, True),
    (LayerShape(8, 64, 64, 4), [4200, 100], "random", True, torch.float32, True),
    # norm groups of 2048 and 1024 channels (4 and 2 eight-channel blocks per
    # lane in the fused norm), over 130 short sequences so that the chunk
    # output has enough (chunk, group) items to keep whole groups per workgroup
    (LayerShape(32, 64, 64, 1), SHORT_LENS, "pool", False, torch.float32, True),
    (LayerShape(16, 64, 128, 1), SHORT_LENS, "random", True, torch.bfloat16, True),
    # more sequences than the length ranking stages at once (1024), each a
    # few tokens, every one from its own slot of the pool
    (LayerShape(8, 64, 64, 2), MANY_LENS, "pool", True, torch.float32, True),
    # odd heads per group (3) and one head per group, at dstate 64
    (LayerShape(12, 64, 64, 4), [300, 130, 5], "random", True, torch.float32, True),
    (LayerShape(4, 64, 64, 4), [257, 1, 64], "random", False, torch.float32, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_raw_conv_scan_equals_chain_and_oracle(case, monkeypatch):
    m2.load()
    shape, lens, init, nbg, ydt, fused = CASES[case]
    inp = small_shape_inputs(shape, lens, seed=200 + case, act="bf16", init=init,
                             n_slots=len(lens) + 2)
    if init == "pool":
        inp["has_init"] = np.array([(b + 1) % 3 != 0 for b in range(len(lens))], dtype=np.uint8)
    shown = lens if len(lens) <= 16 else f"{len(lens)} sequences, {sum(lens)} tokens"
    print(f" shape={shape} lens={shown} init={init} nbg={nbg} y={ydt} fused norm={fused}", flush=True)
    m2.reset_counters()
    y, cs, ss = gpu_prefill(inp, shape, "bf16", nbg=nbg, y_dtype=ydt)
    c = m2.get_counters()
    assert c["conv_launches"] == 0 and c["scan_chunked_launches"] == 1 and c["conv_state_launches"] == 1
    assert c["norm_launches"] == (0 if fused else 1)
    monkeypatch.setenv("M2SSD_PREFILL_CHAIN", "1")
    y2, cs2, ss2 = gpu_prefill(inp, shape, "bf16", nbg=nbg, y_dtype=ydt)
    c = m2.get_counters()
    assert c["conv_launches"] == 1 and c["norm_launches"] == (1 if fused else 2)
    monkeypatch.delenv("M2SSD_PREFILL_CHAIN")
    assert torch.equal(cs, cs2)
    assert rel_err(ss, ss2.double().cpu().numpy(), "ssm_state raw vs chain") <= 1e-3
    if ydt == torch.float32:
        assert rel_err(y, y2.double().cpu().numpy(), "y raw vs chain") <= 1e-3
    else:
        # bf16 outputs: where the fp32 values differ across a rounding boundary the
        # stored values differ by one bf16 step (2^-8 of the value at most)
        a, b = y.double().cpu().numpy(), y2.double().cpu().numpy()
        rms = float(np.sqrt(np.mean(b * b)))
        assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-3 * rms)
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups,
                    norm_before_gate=nbg)
    tol = TOL["bf16"]
    if ydt == torch.float32:
        assert rel_err(y, ref["y"], "y", sum(lens) * shape.d_inner) <= tol
    else:
        # one bf16 rounding (2^-9 relative) on top of the fp32 path's error
        yr = ref["y"]
        g = y.double().cpu().numpy()
        assert g.shape == yr.shape
        bound = 2.0 ** -8 * np.abs(yr) + tol * np.sqrt(np.mean(yr * yr))
        worst = float(np.max(np.abs(g - yr) - bound))
        print(f"  y (bf16): worst excess over the bound {worst:.3e}", flush=True)
        assert worst <= 0.0
    assert rel_err(cs, ref["conv_state"], "conv_state") == 0.0
    assert rel_err(ss, ref["ssm_state"], "ssm_state") <= tol


@pytest.mark.parametrize("chain", [False, True])
def test_sequence_longer_than_planned_levels(chain, monkeypatch):
    """max_seqlen is an upper bound the caller states; the segment plan is made
    from it.  A sequence longer than that bound (2000 tokens against 1024 here,
    still within batch * max_seqlen) has more chunks than the planned segment
    levels: the state pass's last level runs to the sequence's end and the
    carry and chunk-output kernels cap the segment index, so every chunk is
    still computed and the results match the oracle."""
    m2.load()
    shape = LayerShape(16, 64, 128, 2)
    lens = [2000, 100, 100, 100]
    inp = small_shape_inputs(shape, lens, seed=301, act="bf16", init="random", n_slots=6)
    if chain:
        monkeypatch.setenv("M2SSD_PREFILL_CHAIN", "1")
    d = to_device(inp, "bf16")
    x, B, C = split_views(d["xbc"], shape)
    y = m2.mamba2_prefill(x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"], d["norm_w"],
                          d["conv_state"], d["ssm_state"], d["cu_seqlens"], 1024, shape.nheads, shape.headdim,
                          shape.dstate, shape.ngroups, 128, d["state_idx"], d["has_init"], 1e-5, True)
    torch.cuda.synchronize()
    ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    tol = TOL["bf16"]
    assert rel_err(y, ref["y"], "y", sum(lens) * shape.d_inner) <= tol
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") == 0.0
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol
