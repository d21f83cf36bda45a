"""mamba2_prefill_noalloc (the entry for callers that cannot allocate device
memory) against mamba2_prefill with a caller workspace, through the C ABI: the
same kernels, so the results must be bitwise equal, and both within the bar
of the fp64 oracle.  Two calls in a row on the library's fixed scratch, the
second with a smaller input, then a batch too large for the scratch, which is
refused before any launch."""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from oracle import recurrence as R
from workloads import LayerShape, small_shape_inputs
from parity_util import TOL, rel_err, split_views, to_device

pytestmark = pytest.mark.gpu


def _args(d, shape):
    x, B, C = split_views(d["xbc"], shape)
    return (x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"], d["norm_w"])


def _run_both(inp, shape, act, chunk):
    lens = np.diff(inp["cu_seqlens"])
    dims = (shape.nheads, shape.headdim, shape.dstate, shape.ngroups, chunk)
    ref_d, na_d = to_device(inp, act), to_device(inp, act)
    y_ref = m2.mamba2_prefill(*_args(ref_d, shape), ref_d["conv_state"], ref_d["ssm_state"],
                              ref_d["cu_seqlens"], int(lens.max()), *dims, ref_d["state_idx"],
                              ref_d["has_init"])
    y_na = m2.mamba2_prefill_noalloc(*_args(na_d, shape), na_d["conv_state"], na_d["ssm_state"],
                                     na_d["cu_seqlens"], int(lens.max()), *dims, na_d["state_idx"],
                                     na_d["has_init"])
    torch.cuda.synchronize()
    return y_ref, ref_d, y_na, na_d


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_noalloc_equals_workspace_entry_on_two_calls(act):
    m2.load()
    shape = LayerShape(16, 64, 128, 2)
    cases = [([300, 37, 129], 128, 91), ([20, 1], 128, 92)]   # the second call is smaller
    for lens, chunk, seed in cases:
        inp = small_shape_inputs(shape, lens, seed=seed, act=act, init="random")
        need = m2.mamba2_prefill_workspace_size(sum(lens), len(lens), max(lens), shape.nheads,
                                                shape.headdim, shape.dstate, shape.ngroups, chunk,
                                                torch.bfloat16 if act == "bf16" else torch.float32)
        assert need <= m2.mamba2_prefill_noalloc_scratch_bytes()
        print(f" {act} lens={lens} workspace {need} bytes", flush=True)
        y_ref, ref_d, y_na, na_d = _run_both(inp, shape, act, chunk)
        assert torch.equal(y_na, y_ref)
        assert torch.equal(na_d["conv_state"], ref_d["conv_state"])
        assert torch.equal(na_d["ssm_state"], ref_d["ssm_state"])
        ref = R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
        tol = TOL[act]
        assert rel_err(y_na, ref["y"], "y", sum(lens) * shape.d_inner) <= tol
        assert rel_err(na_d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol
        assert rel_err(na_d["conv_state"], ref["conv_state"], "conv_state") <= tol


def test_noalloc_refuses_sizes_beyond_its_scratch():
    m2.load()
    shape = LayerShape(64, 64, 128, 8)
    lens = [4096] * 8
    need = m2.mamba2_prefill_workspace_size(sum(lens), len(lens), 4096, 64, 64, 128, 8, 128,
                                            torch.bfloat16)
    assert need > m2.mamba2_prefill_noalloc_scratch_bytes()
    T = sum(lens)
    dev = "cuda"
    xbc = torch.zeros((T, shape.conv_dim), dtype=torch.bfloat16, device=dev)
    z = torch.zeros((T, shape.d_inner), dtype=torch.bfloat16, device=dev)
    dt = torch.zeros((T, 64), device=dev)
    f = lambda *s: torch.zeros(s, device=dev)
    cs, ss = f(8, 3, shape.conv_dim), f(8, 64, 64, 128)
    cs_before, ss_before = cs.clone(), ss.clone()
    x, B, C = split_views(xbc, shape)
    cu = m2.cu_seqlens_of(lens, dev)
    with pytest.raises(m2.M2Error, match="M2_ERR_WORKSPACE"):
        m2.mamba2_prefill_noalloc(x, B, C, z, dt, f(64), f(64), f(shape.conv_dim, 4), f(shape.conv_dim),
                                  f(shape.d_inner), cs, ss, cu, 4096, 64, 64, 128, 8)
    torch.cuda.synchronize()
    assert torch.equal(cs, cs_before) and torch.equal(ss, ss_before)
