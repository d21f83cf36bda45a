"""GPU parity of the packed in-projection entries (mamba2_prefill_inproj,
mamba2_decode_inproj) and of mixed decode + prefill batches
(mamba2_mixed_inproj), through the C ABI, against the fp64 oracle
(oracle.inproj: the row split, dt = softplus(raw + bias), then the token
recurrence).

Metric and bars as for the other parity tests: max|gpu - oracle| / RMS(oracle)
per tensor (y, final conv_state, final ssm_state), 1e-4 for fp32 inputs, 2e-2
for bf16 inputs, element counts asserted.  Cases: ragged varlen batches with
empty and one-row sequences on both scan paths, a missing dt_bias, rows padded
past their width, decode rows at permuted and fresh slots, mixed batches with
decode rows first (including a fresh one-row prefill, which stays a prefill),
the all-decode and all-prefill extremes, and a Nemotron-nano-shaped mixed batch.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from oracle import inproj as IP
from workloads import NANO, LayerShape, inproj_inputs
from parity_util import TOL, act_torch, rel_err, tdev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    m2.load()


def to_device(inp, act):
    d = {k: tdev(inp[k]) for k in ("A", "D", "conv_w", "conv_b", "norm_w", "conv_state",
                                   "ssm_state", "dt_bias")}
    d["row"] = tdev(inp["row"], act_torch(act))
    d["cu_seqlens"] = tdev(inp["cu_seqlens"], torch.int32)
    d["state_idx"] = tdev(inp["state_idx"], torch.int32)
    d["has_init"] = tdev(inp["has_init"], torch.uint8)
    return d


def compare(d, y, ref, shape, act, rows):
    tol = TOL[act]
    assert rel_err(y, ref["y"], "y", rows * shape.d_inner) <= tol
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= tol
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= tol


PREFILL_CASES = [
    # (shape, lengths, act, chunk)
    (LayerShape(4, 16, 16, 2), [11, 0, 1, 37], "f32", 16),
    (LayerShape(16, 64, 128, 2), [150, 0, 1, 129, 7], "bf16", 128),   # chunk-parallel scan
    (LayerShape(8, 32, 64, 2), [70, 3], "bf16", 32),                  # one-pass scan
    (NANO, [137, 2], "bf16", 128),
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_inproj_matches_oracle(case):
    shape, lens, act, chunk = PREFILL_CASES[case]
    inp = inproj_inputs(shape, lens, seed=300 + case, act=act, init="random")
    print(f" shape={shape} lens={lens} act={act} ld_row={inp['row'].shape[1]}", flush=True)
    d = to_device(inp, act)
    y = m2.mamba2_prefill_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                 d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"],
                                 max(lens), shape.nheads, shape.headdim, shape.dstate,
                                 shape.ngroups, chunk, d["state_idx"], d["has_init"])
    torch.cuda.synchronize()
    ref = IP.prefill_inproj(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    compare(d, y, ref, shape, act, sum(lens))


def test_prefill_inproj_without_bias_and_padded_rows():
    """dt_bias NULL means a zero bias; channels past the row width are ignored."""
    shape = LayerShape(4, 16, 16, 2)
    inp = inproj_inputs(shape, [20, 5], seed=7, act="f32", init="zero", pad=64)
    width = IP.row_width(4, 16, 16, 2)
    inp["row"][:, width:] = np.nan  # padding must never be read into the result
    inp["dt_bias"] = np.zeros_like(inp["dt_bias"])
    d = to_device(inp, "f32")
    y = m2.mamba2_prefill_inproj(d["row"], None, d["A"], d["D"], d["conv_w"], d["conv_b"],
                                 d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"], 20,
                                 4, 16, 16, 2, 16, d["state_idx"], d["has_init"])
    torch.cuda.synchronize()
    ref = IP.prefill_inproj(inp, 4, 16, 16, 2)
    compare(d, y, ref, shape, "f32", 25)


DECODE_CASES = [
    (LayerShape(4, 16, 16, 2), 5, 9, "f32"),
    (LayerShape(16, 64, 128, 2), 4, 6, "bf16"),
    (NANO, 6, 11, "bf16"),
    (NANO, 3, 3, "f32"),
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_inproj_matches_oracle(case):
    shape, batch, n_slots, act = DECODE_CASES[case]
    inp = inproj_inputs(shape, [1] * batch, seed=400 + case, act=act, init="pool", n_slots=n_slots)
    inp["has_init"] = (np.arange(batch) % 3 != 2).astype(np.uint8)
    print(f" shape={shape} batch={batch} slots={inp['state_idx'].tolist()} act={act}", flush=True)
    d = to_device(inp, act)
    y = m2.mamba2_decode_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                d["norm_w"], d["conv_state"], d["ssm_state"], shape.nheads,
                                shape.headdim, shape.dstate, shape.ngroups, d["state_idx"],
                                d["has_init"])
    torch.cuda.synchronize()
    ref = IP.prefill_inproj(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    compare(d, y, ref, shape, act, batch)


MIXED_CASES = [
    # (shape, lengths (decode rows first), num_decodes, act, chunk, n_slots, has_init)
    (LayerShape(4, 16, 16, 2), [1, 1, 1, 9, 1, 30], 3, "f32", 16, 8, [1, 1, 0, 1, 0, 1]),
    (LayerShape(16, 64, 128, 2), [1, 1, 140, 1, 0, 60], 2, "bf16", 128, 9, [1, 0, 1, 0, 1, 1]),
    (LayerShape(16, 64, 128, 2), [1, 1, 1, 1], 4, "bf16", 128, 4, [1, 1, 1, 0]),   # decode only
    (LayerShape(16, 64, 128, 2), [33, 1, 200], 0, "bf16", 128, 3, [1, 0, 1]),     # prefill only
    (NANO, [1] * 16 + [300, 129, 1], 16, "bf16", 128, 40, None),
    # fp32: 20 sequences x 16 heads would not be split, but the prefill part's
    # 2 x 16 are, so its segment buffers come from the mixed workspace
    (LayerShape(16, 64, 128, 2), [1] * 18 + [1300, 700], 18, "f32", 128, 24, None),
]


@pytest.mark.parametrize("case", range(len(MIXED_CASES)))
def test_mixed_batch_matches_oracle(case):
    shape, lens, nd, act, chunk, n_slots, init = MIXED_CASES[case]
    inp = inproj_inputs(shape, lens, seed=500 + case, act=act, init="pool", n_slots=n_slots)
    if init is not None:
        inp["has_init"] = np.array(init, dtype=np.uint8)
    print(f" shape={shape} lens={lens} num_decodes={nd} act={act}", flush=True)
    d = to_device(inp, act)
    m2.reset_counters()
    y = m2.mamba2_mixed_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                               d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"], nd,
                               max(lens), shape.nheads, shape.headdim, shape.dstate, shape.ngroups,
                               chunk, d["state_idx"], d["has_init"])
    torch.cuda.synchronize()
    c = m2.get_counters()
    assert c["decode_launches"] == (1 if nd > 0 else 0)
    assert c["prefill_calls"] == (1 if nd < len(lens) else 0)
    ref = IP.mixed_batch(inp, nd, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    compare(d, y, ref, shape, act, sum(lens))


def test_mixed_batch_identity_slots_and_repeatability():
    """state_idx NULL: sequence b uses slot b, in both parts; equal inputs give equal bits."""
    shape = LayerShape(16, 64, 128, 2)
    lens = [1, 1, 1, 77, 140]
    inp = inproj_inputs(shape, lens, seed=77, act="bf16", init="random")
    inp["state_idx"] = np.arange(len(lens), dtype=np.int32)
    outs = []
    for _ in range(2):
        d = to_device(inp, "bf16")
        y = m2.mamba2_mixed_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"],
                                   d["conv_b"], d["norm_w"], d["conv_state"], d["ssm_state"],
                                   d["cu_seqlens"], 3, max(lens), shape.nheads, shape.headdim,
                                   shape.dstate, shape.ngroups, 128, None, d["has_init"])
        torch.cuda.synchronize()
        outs.append((y.cpu(), d["conv_state"].cpu(), d["ssm_state"].cpu()))
    ref = IP.mixed_batch(inp, 3, shape.nheads, shape.headdim, shape.dstate, shape.ngroups)
    compare(d, y, ref, shape, "bf16", sum(lens))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_mixed_batch_full_size_sampled():
    """The mixed step at the size the bench times: 256 decode rows, then two
    4096-token prefills (which the state pass splits into segments), nano shape.
    Every decode row is checked in full; the prefills on sampled (sequence,
    group) slices, each an exact sub-problem of the mixer core."""
    from oracle import recurrence as R
    from workloads import group_channels, slice_group
    s = NANO
    H, P, N, G = s.nheads, s.headdim, s.dstate, s.ngroups
    nd = 256
    lens = [1] * nd + [4096, 4096]
    inp = inproj_inputs(s, lens, seed=22, act="bf16", init="pool", n_slots=len(lens))
    d = to_device(inp, "bf16")
    y = m2.mamba2_mixed_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                               d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"], nd,
                               4096, H, P, N, G, 128, d["state_idx"], d["has_init"])
    torch.cuda.synchronize()
    assert torch.isfinite(y).all()
    tol = TOL["bf16"]
    cu = inp["cu_seqlens"]
    # decode rows: the oracle over those sequences only
    ref = IP.prefill_inproj(inp, H, P, N, G, seqs=range(nd))
    slots = inp["state_idx"][:nd]
    assert rel_err(y[:nd], ref["y"][:nd], "decode y", nd * s.d_inner) <= tol
    assert rel_err(d["ssm_state"][torch.as_tensor(slots, device="cuda", dtype=torch.long)],
                   ref["ssm_state"][slots], "decode ssm_state") <= tol
    assert rel_err(d["conv_state"][torch.as_tensor(slots, device="cuda", dtype=torch.long)],
                   ref["conv_state"][slots], "decode conv_state") <= tol
    # prefill sequences: sampled groups
    z, xbc, dt_raw = IP.split_inproj_row(inp["row"], H, P, N, G)
    dt = IP.step_size(dt_raw, inp["dt_bias"])
    for b, g in ((nd, 0), (nd, 5), (nd + 1, 7)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        slot = int(inp["state_idx"][b])
        one = {k: v for k, v in inp.items() if k not in ("row", "dt_bias")}
        one.update(xbc=xbc[lo:hi], z=z[lo:hi], dt=dt[lo:hi], cu_seqlens=np.array([0, hi - lo], np.int32),
                   conv_state=inp["conv_state"][slot:slot + 1], ssm_state=inp["ssm_state"][slot:slot + 1],
                   state_idx=np.zeros(1, np.int32), has_init=inp["has_init"][b:b + 1])
        sub_inp, sub = slice_group(one, s, g)
        r = R.prefill(sub_inp, sub.nheads, sub.headdim, sub.dstate, 1)
        heads, xch, ch = group_channels(s, g)
        ht, xt, ct = (torch.as_tensor(v, device="cuda") for v in (heads, xch, ch))
        print(f" prefill seq {b} (slot {slot}) group {g}", flush=True)
        assert rel_err(y[lo:hi][:, xt], r["y"], "y", (hi - lo) * len(xch)) <= tol
        assert rel_err(d["ssm_state"][slot][ht], r["ssm_state"][0], "ssm_state") <= tol
        assert rel_err(d["conv_state"][slot][:, ct], r["conv_state"][0], "conv_state") <= tol


def test_mixed_batch_debug_checks(monkeypatch):
    """With M2SSD_DEBUG=1 the host reads the index arrays before any launch: a
    'decode' sequence of two rows and a repeated slot are refused with
    M2_ERR_SHAPE and leave the states untouched; a valid batch still matches."""
    monkeypatch.setenv("M2SSD_DEBUG", "1")
    shape = LayerShape(4, 16, 16, 2)
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    lens = [1, 1, 9, 20]
    inp = inproj_inputs(shape, lens, seed=31, act="f32", init="pool", n_slots=6)

    def call(d, nd, cu=None, idx=None):
        return m2.mamba2_mixed_inproj(d["row"], d["dt_bias"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                      d["norm_w"], d["conv_state"], d["ssm_state"],
                                      d["cu_seqlens"] if cu is None else cu, nd, max(lens), H, P, N, G, 16,
                                      d["state_idx"] if idx is None else idx, d["has_init"])

    d = to_device(inp, "f32")
    ss0, cs0 = d["ssm_state"].clone(), d["conv_state"].clone()
    # sequence 1 declared a decode row but given two rows
    bad_cu = tdev(np.array([0, 1, 3, 11, 31], np.int32), torch.int32)
    with pytest.raises(m2.M2Error) as e:
        call(d, 2, cu=bad_cu)
    assert e.value.status == -2
    rep = tdev(np.array([0, 1, 1, 2], np.int32), torch.int32)
    with pytest.raises(m2.M2Error) as e:
        call(d, 2, idx=rep)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert torch.equal(d["ssm_state"], ss0) and torch.equal(d["conv_state"], cs0)
    y = call(d, 2)
    torch.cuda.synchronize()
    ref = IP.mixed_batch(inp, 2, H, P, N, G)
    compare(d, y, ref, shape, "f32", sum(lens))
