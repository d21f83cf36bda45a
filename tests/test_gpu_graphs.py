"""HIP graph capture of the library's entries (through torch.cuda.graph on the
launch stream): a decode step, a prefill with sequences split into segments,
and a mixed batch (whose decode rows fork onto the library's second stream
and join back).  Each graph is replayed several times with eager work and
synchronizations between the replays (the states are reset to their inputs
eagerly before every replay), and every replay must reproduce the eager call
bit for bit: same kernels, same inputs, same order.

Workspaces and outputs are allocated before capture; the library itself
allocates nothing and makes no host synchronization outside its debug mode.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from workloads import LayerShape, inproj_inputs
from parity_util import act_torch, tdev

pytestmark = pytest.mark.gpu

SHAPE = LayerShape(16, 64, 128, 2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    m2.load()


def device_inputs(lens, seed):
    inp = inproj_inputs(SHAPE, lens, seed=seed, act="bf16", init="pool", n_slots=len(lens) + 2)
    d = {k: tdev(inp[k]) for k in ("dt_bias", "A", "D", "conv_w", "conv_b", "norm_w", "conv_state",
                                   "ssm_state")}
    d["row"] = tdev(inp["row"], act_torch("bf16"))
    d["cu_seqlens"] = tdev(inp["cu_seqlens"], torch.int32)
    d["state_idx"] = tdev(inp["state_idx"], torch.int32)
    d["has_init"] = tdev(inp["has_init"], torch.uint8)
    return d


def check_graph(d, run, replays=3):
    """run(d) -> y.  Eager once from the input states, then capture and replay."""
    cs0, ss0 = d["conv_state"].clone(), d["ssm_state"].clone()
    y_e = run(d).clone()
    torch.cuda.synchronize()
    cs_e, ss_e = d["conv_state"].clone(), d["ssm_state"].clone()
    # warm-up on a side stream, as graph capture expects, then capture
    d["conv_state"].copy_(cs0)
    d["ssm_state"].copy_(ss0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(d)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    d["conv_state"].copy_(cs0)
    d["ssm_state"].copy_(ss0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        y_g = run(d)
    for k in range(replays):
        d["conv_state"].copy_(cs0)          # eager work between the replays
        d["ssm_state"].copy_(ss0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), f"replay {k}: y differs"
        assert torch.equal(d["conv_state"], cs_e), f"replay {k}: conv_state differs"
        assert torch.equal(d["ssm_state"], ss_e), f"replay {k}: ssm_state differs"


def test_graph_decode_step():
    H, P, N, G = SHAPE.nheads, SHAPE.headdim, SHAPE.dstate, SHAPE.ngroups
    d = device_inputs([1] * 6, seed=91)
    y = torch.empty((6, SHAPE.d_inner), device="cuda")

    def run(d):
        return m2.mamba2_decode_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                       d["norm_w"], d["conv_state"], d["ssm_state"], H, P, N, G,
                                       d["state_idx"], d["has_init"], y=y)
    check_graph(d, run)


def test_graph_prefill_split_sequences():
    H, P, N, G = SHAPE.nheads, SHAPE.headdim, SHAPE.dstate, SHAPE.ngroups
    lens = [1100, 300, 0]
    d = device_inputs(lens, seed=92)
    T = sum(lens)
    y = torch.empty((T, SHAPE.d_inner), device="cuda")
    ws = torch.empty(m2.mamba2_prefill_inproj_workspace_size(T, len(lens), max(lens), H, P, N, G, 128,
                                                             torch.bfloat16), dtype=torch.uint8, device="cuda")

    def run(d):
        return m2.mamba2_prefill_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                        d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"],
                                        max(lens), H, P, N, G, 128, d["state_idx"], d["has_init"],
                                        y=y, workspace=ws)
    check_graph(d, run)


def test_graph_mixed_batch():
    H, P, N, G = SHAPE.nheads, SHAPE.headdim, SHAPE.dstate, SHAPE.ngroups
    lens = [1, 1, 1, 1, 700, 9]
    d = device_inputs(lens, seed=93)
    T = sum(lens)
    y = torch.empty((T, SHAPE.d_inner), device="cuda")
    ws = torch.empty(m2.mamba2_mixed_inproj_workspace_size(T, len(lens), max(lens), H, P, N, G, 128,
                                                           torch.bfloat16), dtype=torch.uint8, device="cuda")

    def run(d):
        return m2.mamba2_mixed_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                      d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"], 4,
                                      max(lens), H, P, N, G, 128, d["state_idx"], d["has_init"], y=y,
                                      workspace=ws)
    check_graph(d, run)
