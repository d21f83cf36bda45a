"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
slicing one SSM group out of a workload (groups are independent through the
whole mixer core: each group owns its heads, its B/C channels, its x and z
channels, its conv channels and its norm group), and the comparison metric
max|gpu - oracle| / RMS(oracle) with the element count asserted."""
from __future__ import annotations

import numpy as np
import torch

from workloads import LayerShape, group_channels, slice_group  # noqa: F401

TOL = {"f32": 1e-4, "bf16": 2e-2}


def tdev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def act_torch(act: str):
    return torch.bfloat16 if act == "bf16" else torch.float32


def to_device(inp: dict, act: str) -> dict:
    """Device copies of a workloads.make_inputs dict (activations in `act`, exact)."""
    at = act_torch(act)
    d = {
        "xbc": tdev(inp["xbc"], at), "z": tdev(inp["z"], at), "dt": tdev(inp["dt"]),
        "A": tdev(inp["A"]), "D": tdev(inp["D"]), "conv_w": tdev(inp["conv_w"]),
        "conv_b": tdev(inp["conv_b"]), "norm_w": tdev(inp["norm_w"]),
        "conv_state": tdev(inp["conv_state"]), "ssm_state": tdev(inp["ssm_state"]),
        "cu_seqlens": tdev(inp["cu_seqlens"], torch.int32),
        "state_idx": tdev(inp["state_idx"], torch.int32),
        "has_init": tdev(inp["has_init"], torch.uint8),
    }
    return d


def split_views(xbc: torch.Tensor, shape: LayerShape):
    di = shape.d_inner
    gn = shape.ngroups * shape.dstate
    return xbc[:, :di], xbc[:, di:di + gn], xbc[:, di + gn:di + 2 * gn]


def rel_err(gpu, ref, name: str, expect_count: int = None) -> float:
    """max|gpu - ref| / RMS(ref); asserts finiteness and the element count."""
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if torch.is_tensor(gpu) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    if expect_count is not None:
        assert r.size == expect_count, f"{name}: {r.size} elements compared, expected {expect_count}"
    assert r.size > 0, f"{name}: nothing to compare"
    assert np.all(np.isfinite(g)), f"{name}: non-finite GPU values"
    rms = float(np.sqrt(np.mean(r * r)))
    err = float(np.max(np.abs(g - r)))
    rel = err / rms if rms > 0 else err
    print(f"  {name}: n={r.size} max|err|={err:.3e} rms={rms:.3e} rel={rel:.3e}", flush=True)
    return rel
