"""GPU parity of the HIP path (called through the C ABI) against the fp64 oracle.

Metric: max|gpu - oracle| / RMS(oracle) per tensor (y, final conv_state, final
ssm_state), with the element count asserted.  Bars: 1e-4 for fp32 inputs,
2e-2 for bf16 inputs.  Small shapes span several 16-row tiles, several chunks
and ragged tails; the full-size workloads are checked on every (sequence,
group) pair, each an exact sub-problem the oracle computes in seconds
(groups are independent through the whole mixer core), in a pool of host
processes.
"""
import numpy as np
import pytest
import torch

import mamba_ssd_selective_amd as m2
from oracle import recurrence as R
from workloads import LayerShape, Workload, WORKLOADS, make_inputs, round_bf16, seqlens_of, small_shape_inputs
from parity_util import TOL, group_channels, rel_err, slice_group, split_views, tdev, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    m2.load()


def gpu_prefill(inp, shape, act, chunk=128, nbg=True, y_dtype=torch.float32, eps=1e-5):
    d = to_device(inp, act)
    x, B, C = split_views(d["xbc"], shape)
    lens = np.diff(inp["cu_seqlens"])
    y = m2.mamba2_prefill(x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"],
                          d["norm_w"], d["conv_state"], d["ssm_state"], d["cu_seqlens"],
                          int(lens.max()) if len(lens) else 0, shape.nheads, shape.headdim,
                          shape.dstate, shape.ngroups, chunk, d["state_idx"], d["has_init"],
                          eps, nbg, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y, d["conv_state"], d["ssm_state"]


def oracle_prefill(inp, shape, nbg=True, eps=1e-5):
    return R.prefill(inp, shape.nheads, shape.headdim, shape.dstate, shape.ngroups, eps=eps,
                     norm_before_gate=nbg)


def check_all(inp, shape, act, chunk=128, nbg=True):
    y, cs, ss = gpu_prefill(inp, shape, act, chunk, nbg)
    ref = oracle_prefill(inp, shape, nbg)
    T = int(inp["cu_seqlens"][-1])
    tol = TOL[act]
    assert rel_err(y, ref["y"], "y", T * shape.d_inner) <= tol
    assert rel_err(cs, ref["conv_state"], "conv_state") <= tol
    assert rel_err(ss, ref["ssm_state"], "ssm_state") <= tol


# ------------------------------------------------------------------ conv

@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_conv_rows_varlen(act):
    shape = LayerShape(4, 16, 16, 2)
    lens = [5, 0, 1, 2, 40, 3, 17]
    inp = small_shape_inputs(shape, lens, seed=1, act=act, init="random", n_slots=9)
    inp["state_idx"] = np.array([8, 0, 3, 5, 1, 7, 2], dtype=np.int32)
    inp["has_init"] = np.array([1, 0, 0, 1, 1, 0, 1], dtype=np.uint8)
    d = to_device(inp, act)
    x, B, C = split_views(d["xbc"], shape)
    out = m2.mamba2_conv_rows(x, B, C, d["conv_w"], d["conv_b"], d["conv_state"], d["cu_seqlens"],
                              max(lens), d["state_idx"], d["has_init"])
    torch.cuda.synchronize()
    ref = R.prefill(inp, 4, 16, 16, 2)
    T = sum(lens)
    assert rel_err(out, ref["u"], "u", T * shape.conv_dim) <= 1e-5
    assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") == 0.0


def test_conv_rows_bf16_output_and_identity_activation():
    shape = LayerShape(8, 16, 16, 2)
    inp = small_shape_inputs(shape, [33, 7], seed=2, act="bf16", init="random")
    d = to_device(inp, "bf16")
    x, B, C = split_views(d["xbc"], shape)
    out = m2.mamba2_conv_rows(x, B, C, d["conv_w"], d["conv_b"], d["conv_state"].clone(),
                              d["cu_seqlens"], 33, d["state_idx"], d["has_init"],
                              apply_silu=False, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    pre = []
    for b in range(2):
        lo, hi = inp["cu_seqlens"][b], inp["cu_seqlens"][b + 1]
        u, _ = R.conv_rows_seq(inp["xbc"][lo:hi], inp["conv_w"], inp["conv_b"],
                               inp["conv_state"][b], apply_silu=False)
        pre.append(u)
    assert rel_err(out, np.concatenate(pre), "pre-activation (bf16 out)") <= 2e-2


# ------------------------------------------------------------------ scan alone

SCAN_CASES = [
    (LayerShape(4, 16, 16, 2), [11], 16),
    (LayerShape(4, 16, 16, 1), [1, 0, 37, 16, 2], 16),
    (LayerShape(8, 32, 64, 2), [130, 5, 77], 48),
    (LayerShape(16, 64, 64, 2), [200, 1, 129], 128),
    (LayerShape(16, 64, 128, 2), [300, 37], 128),
    (LayerShape(16, 64, 128, 1), [161], 64),
    # chunk-parallel path (bf16): empty, 1-row, exact-multiple and ragged sequences
    (LayerShape(16, 64, 128, 1), [128, 0, 1, 257, 255], 128),
    (LayerShape(8, 64, 64, 4), [513, 3, 0], 128),
    (LayerShape(64, 64, 128, 8), [129, 384], 128),
    # few long sequences: the state pass splits them into segments
    (LayerShape(16, 64, 128, 2), [1500, 40], 128),
]


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("case", range(len(SCAN_CASES)))
def test_ssd_chunk_scan(case, act):
    shape, lens, chunk = SCAN_CASES[case]
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    inp = small_shape_inputs(shape, lens, seed=10 + case, act=act, init="random")
    # post-conv inputs: the oracle's conv output, stored in the activation dtype
    u = R.prefill(inp, H, P, N, G, apply_norm=False)["u"].astype(np.float32)
    if act == "bf16":
        u = round_bf16(u)
    ud = tdev(u, torch.bfloat16 if act == "bf16" else torch.float32)
    x, B, C = split_views(ud, shape)
    d = to_device(inp, act)
    y = m2.ssd_chunk_scan(x, B, C, d["dt"], d["A"], d["D"], d["ssm_state"], d["cu_seqlens"],
                          max(lens), H, P, N, G, chunk, d["state_idx"], d["has_init"])
    torch.cuda.synchronize()
    cu = inp["cu_seqlens"]
    y_ref = np.zeros((int(cu[-1]), H * P))
    ss_ref = inp["ssm_state"].astype(np.float64).copy()
    for b in range(len(lens)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        xs, Bs, Cs = R.split_xbc(u[lo:hi].astype(np.float64), H, P, G, N)
        slot = int(inp["state_idx"][b])
        h0 = ss_ref[slot] if inp["has_init"][b] else np.zeros((H, P, N))
        yb, hb = R.ssd_recurrence_seq(xs, Bs, Cs, inp["dt"][lo:hi], inp["A"], inp["D"], h0)
        y_ref[lo:hi] = yb.reshape(hi - lo, H * P)
        ss_ref[slot] = hb
    tol = TOL[act]
    assert rel_err(y, y_ref, "y_pre", int(cu[-1]) * H * P) <= tol
    assert rel_err(d["ssm_state"], ss_ref, "ssm_state") <= tol


# ------------------------------------------------------------------ norm alone

@pytest.mark.parametrize("gw", [32, 512, 1024])
@pytest.mark.parametrize("nbg", [True, False])
@pytest.mark.parametrize("zdt", ["f32", "bf16"])
def test_gated_rmsnorm_group(gw, nbg, zdt):
    rng = np.random.default_rng(gw + 7 * nbg)
    T, G = 37, 4
    d = gw * G
    y = rng.standard_normal((T, d)).astype(np.float32)
    z = rng.standard_normal((T, d)).astype(np.float32)
    if zdt == "bf16":
        z = round_bf16(z)
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    yd = tdev(y)
    out = m2.gated_rmsnorm_group(yd, tdev(z, torch.bfloat16 if zdt == "bf16" else torch.float32),
                                 tdev(w), G, 1e-5, nbg)
    torch.cuda.synchronize()
    ref = R.gated_rmsnorm_group(y, z, w, 1e-5, G, nbg)
    assert rel_err(out, ref, "norm out", T * d) <= 1e-5
    # in place on y gives the same bits
    out2 = m2.gated_rmsnorm_group(yd, tdev(z, torch.bfloat16 if zdt == "bf16" else torch.float32),
                                  tdev(w), G, 1e-5, nbg, out=yd)
    torch.cuda.synchronize()
    assert torch.equal(out2, out)


# ------------------------------------------------------------------ the fused prefill

def test_prefill_tiny_split_7_plus_4_and_single_steps():
    """11 tokens as one call, as 7 + 4 and as 11 one-token calls, all against the 11-token oracle."""
    w = WORKLOADS[0]
    s = w.shape
    inp = make_inputs(w, 0)
    ref = oracle_prefill(inp, s)
    for cuts in ([11], [7, 4], [1] * 11):
        d = to_device(inp, "f32")
        x, B, C = split_views(d["xbc"], s)
        ys = []
        lo = 0
        for i, n in enumerate(cuts):
            cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
            hi_ = torch.tensor([0 if i == 0 else 1], dtype=torch.uint8, device="cuda")
            ys.append(m2.mamba2_prefill(x[lo:lo + n], B[lo:lo + n], C[lo:lo + n], d["z"][lo:lo + n],
                                        d["dt"][lo:lo + n], d["A"], d["D"], d["conv_w"], d["conv_b"],
                                        d["norm_w"], d["conv_state"], d["ssm_state"], cu, n,
                                        s.nheads, s.headdim, s.dstate, s.ngroups, w.chunk_size,
                                        None, hi_))
            lo += n
        torch.cuda.synchronize()
        print(f" cuts={cuts}")
        assert rel_err(torch.cat(ys), ref["y"], "y", 11 * s.d_inner) <= TOL["f32"]
        assert rel_err(d["conv_state"], ref["conv_state"], "conv_state") <= TOL["f32"]
        assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= TOL["f32"]


@pytest.mark.parametrize("nbg", [True, False])
def test_prefill_small_varlen_both_gate_orders(nbg):
    shape = LayerShape(16, 64, 128, 2)
    lens = [0, 1, 2, 3, 130, 45]
    inp = small_shape_inputs(shape, lens, seed=44, act="bf16", init="random", n_slots=8)
    inp["state_idx"] = np.array([7, 2, 0, 5, 1, 6], dtype=np.int32)
    inp["has_init"] = np.array([0, 1, 0, 1, 1, 0], dtype=np.uint8)
    check_all(inp, shape, "bf16", 128, nbg)


@pytest.mark.parametrize("nbg", [True, False])
def test_prefill_bf16_output(nbg):
    """bf16 y on the chunk-parallel path (pre-norm values in the fp32 workspace): every
    element within about one bf16 rounding of the oracle; states as with fp32 y."""
    shape = LayerShape(16, 64, 128, 2)
    lens = [129, 0, 70, 256]
    inp = small_shape_inputs(shape, lens, seed=46 + nbg, act="bf16", init="random", n_slots=4)
    y, cs, ss = gpu_prefill(inp, shape, "bf16", 128, nbg, y_dtype=torch.bfloat16)
    ref = oracle_prefill(inp, shape, nbg)
    yr = ref["y"]
    scale = np.sqrt(np.mean(yr ** 2))
    g = y.float().cpu().numpy().astype(np.float64)
    # one bf16 rounding (2^-9 relative) on top of the fp32 path's error (2e-2 of the RMS)
    bound = 2.0 ** -8 * np.abs(yr) + TOL["bf16"] * scale
    worst = np.max(np.abs(g - yr) - bound)
    print(f"  worst excess over the bound: {worst:.3e} (RMS {scale:.3e})")
    assert worst <= 0.0
    assert rel_err(cs, ref["conv_state"], "conv_state") <= TOL["bf16"]
    assert rel_err(ss, ref["ssm_state"], "ssm_state") <= TOL["bf16"]


@pytest.mark.parametrize("hpg_case", [(16, 1), (8, 8), (4, 4)])
def test_prefill_head_group_maps(hpg_case):
    """Heads per group 16, 1 and 1: the group index h // hpg, at the real 8 heads per group as well."""
    H, G = hpg_case
    shape = LayerShape(H, 64, 128, G)
    inp = small_shape_inputs(shape, [150, 20], seed=50 + H + G, act="f32", init="random")
    check_all(inp, shape, "f32", 64)


def test_prefill_nano_137_tokens():
    w = WORKLOADS[1]
    inp = make_inputs(w, 1)
    check_all(inp, w.shape, "bf16", w.chunk_size)


def _check_pairs(inp, s, y, cs, ss, pairs, act):
    """Each (sequence, group) pair of the device results against the oracle run
    on that sequence's rows and that group alone."""
    cu = inp["cu_seqlens"]
    tol = TOL[act]
    for b, g in pairs:
        heads, xch, ch = group_channels(s, g)
        heads_t, xch_t, ch_t = (torch.as_tensor(v, device="cuda") for v in (heads, xch, ch))
        lo, hi = int(cu[b]), int(cu[b + 1])
        one = {k: v for k, v in inp.items()}
        for k in ("xbc", "z", "dt"):
            one[k] = inp[k][lo:hi]
        one["cu_seqlens"] = np.array([0, hi - lo], dtype=np.int32)
        one["state_idx"] = inp["state_idx"][b:b + 1]
        one["has_init"] = inp["has_init"][b:b + 1]
        sub_inp, sub = slice_group(one, s, g)
        ref = R.prefill(sub_inp, sub.nheads, sub.headdim, sub.dstate, 1)
        slot = int(inp["state_idx"][b])
        print(f" seq {b} (len {hi - lo}, slot {slot}) group {g}")
        assert rel_err(y[lo:hi][:, xch_t], ref["y"], "y", (hi - lo) * len(xch)) <= tol
        assert rel_err(ss[slot][heads_t], ref["ssm_state"][slot], "ssm_state") <= tol
        assert rel_err(cs[slot][:, ch_t], ref["conv_state"][slot], "conv_state") <= tol


# Few long sequences leave most CUs idle if each (sequence, head) walks its
# chunks alone, so the state pass splits them into segments that start from a
# zero state and a carry pass joins them.  Cases: ragged last chunk and
# segment, an empty and a one-row sequence next to long ones, an exact
# multiple of the segment length, dstate 64 (one head per workgroup), a fresh
# slot on a long sequence.
SEGMENT_CASES = [
    # (shape, lengths, has_init)
    (LayerShape(16, 64, 128, 2), [2000, 700, 1, 0], [1, 0, 1, 1]),
    (LayerShape(8, 64, 64, 4), [1029, 512], [1, 1]),
    (LayerShape(16, 64, 128, 2), [4096], [1]),
    (LayerShape(16, 64, 128, 2), [1300, 2600], [0, 1]),
]


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("case", range(len(SEGMENT_CASES)))
def test_prefill_long_sequences_split_into_segments(case, act):
    """bf16: the chunk-parallel path's segments; f32: the fp64 one-pass path's
    (segments of 64-row steps, the carry kernel and the readout fix of later
    segments)."""
    shape, lens, init = SEGMENT_CASES[case]
    inp = small_shape_inputs(shape, lens, seed=60 + case, act=act, init="pool",
                             n_slots=len(lens) + 3)
    inp["has_init"] = np.array(init, dtype=np.uint8)
    print(f" shape={shape} lens={lens} slots={inp['state_idx'].tolist()}")
    check_all(inp, shape, act)


def test_prefill_bf16_decay_stress_split_sequences():
    """|dt A| log-uniform in [1e-3, 1e6] (5% at 1e6) on the bf16 chunk-parallel
    path, with a sequence long enough to be split into segments: every clamped
    exponent (in-chunk, chunk totals, segment totals, segment-relative decays)
    must stay finite and the outputs match the oracle."""
    shape = LayerShape(16, 64, 128, 2)
    inp = small_shape_inputs(shape, [1500, 200], seed=71, act="bf16", init="random",
                             dt_mode="stress")
    check_all(inp, shape, "bf16")


def test_prefill_all_sequences_empty():
    """total_tokens = 0: no rows to convolve or scan; a fresh slot (has_init = 0)
    is reset to zero states, a carried one is left as it was."""
    shape = LayerShape(16, 64, 128, 2)
    inp = small_shape_inputs(shape, [0, 0, 0], seed=72, act="bf16", init="pool", n_slots=5)
    inp["has_init"] = np.array([0, 1, 0], dtype=np.uint8)
    y, cs, ss = gpu_prefill(inp, shape, "bf16")
    ref = oracle_prefill(inp, shape)
    assert y.shape[0] == 0
    fresh = [int(inp["state_idx"][b]) for b in (0, 2)]
    assert float(ss[fresh].abs().max()) == 0.0 and float(cs[fresh].abs().max()) == 0.0
    assert rel_err(ss, ref["ssm_state"], "ssm_state") == 0.0
    assert rel_err(cs, ref["conv_state"], "conv_state") == 0.0


def test_prefill_many_heads_per_group():
    """32 heads per group: the widest norm group the library takes (32 x 64 =
    2048 channels), 32-head loops in the scan kernels, and the head split of
    the chunk output on a small grid."""
    shape = LayerShape(64, 64, 128, 2)
    inp = small_shape_inputs(shape, [300, 5], seed=73, act="bf16", init="random")
    check_all(inp, shape, "bf16")


def _all_pairs(w, seed, act, tmp_path):
    """The full-size workload on the GPU (the launch configuration the bench
    times), then every (sequence, group) pair against the fp64 oracle, element by
    element, in a pool of host processes (tests/oracle_pool.py)."""
    import oracle_pool
    inp = make_inputs(w, seed)
    s = w.shape
    y, cs, ss = gpu_prefill(inp, s, act, w.chunk_size)
    assert torch.isfinite(y).all() and torch.isfinite(ss).all() and torch.isfinite(cs).all()
    np.save(tmp_path / "y.npy", y.cpu().numpy())
    np.save(tmp_path / "ssm_state.npy", ss.cpu().numpy())
    np.save(tmp_path / "conv_state.npy", cs.cpu().numpy())
    T = int(inp["cu_seqlens"][-1])
    del inp, y, cs, ss
    res = oracle_pool.all_pairs(w, seed, str(tmp_path))
    tol = TOL[act]
    assert len(res) == len(seqlens_of(w, seed)) * s.ngroups
    assert sum(r["y"]["n"] for r in res) == T * s.d_inner
    worst = {}
    for r in res:
        for name in ("y", "ssm_state", "conv_state"):
            m = r[name]
            assert m["finite"], f"non-finite {name} at sequence {r['seq']} group {r['group']}"
            rel = m["err"] / m["rms"] if m["rms"] > 0 else m["err"]
            if rel > worst.get(name, (-1.0,))[0]:
                worst[name] = (rel, r["seq"], r["group"], r["len"])
            assert rel <= tol, f"{name} sequence {r['seq']} group {r['group']}: {rel:.3e} > {tol}"
    for name, (rel, b, g, L) in worst.items():
        print(f"  {name}: worst max|err|/rms {rel:.3e} at sequence {b} (len {L}) group {g}; "
              f"{len(res)} pairs", flush=True)


def test_prefill_decay_stress_full_size_all_pairs(tmp_path):
    _all_pairs(WORKLOADS[3], 3, "f32", tmp_path)


def test_prefill_decay_stress_full_size_nonzero_initial_states(tmp_path):
    """The decay-stress configuration from carried (nonzero) conv and SSM states."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS[3], name="decay_stress_2x2048_f32_carried", init="random")
    _all_pairs(w, 33, "f32", tmp_path)


def test_prefill_nano_8x4096_full_size_all_pairs(tmp_path):
    _all_pairs(WORKLOADS[2], 2, "bf16", tmp_path)


def test_prefill_h8b_varlen_full_size_all_pairs(tmp_path):
    _all_pairs(WORKLOADS[4], 4, "bf16", tmp_path)


def test_prefill_offsets_past_4_gib():
    """88 sequences of 4096 tokens at the 8 x 4096 layer shape (360,448 tokens):
    the last sequence's xBC rows start 4.4 GB into the input, its y rows 5.8 GB
    into the output, and its post-conv x blocks and entry states lie more than
    4 GiB into the workspace, so every offset past 32 bits is taken.  The last
    sequence is drawn by the workload generator and checked on two groups; the
    others are filler drawn on the device (finite, their own slots)."""
    s = WORKLOADS[2].shape
    lens = [4096] * 88
    last = len(lens) - 1
    w = Workload("offsets", s, tuple(lens), "bf16", "random")
    inp = make_inputs(w, 81, only_seq=last)      # token arrays of the last sequence only
    cu = inp["cu_seqlens"]
    T, lo, hi = int(cu[-1]), int(cu[last]), int(cu[last + 1])
    assert lo * s.conv_dim * 2 > 2 ** 32 and lo * s.d_inner * 4 > 2 ** 32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(81)
    xbc = torch.randn((T, s.conv_dim), generator=gen, device="cuda", dtype=torch.bfloat16)
    z = torch.randn((T, s.d_inner), generator=gen, device="cuda", dtype=torch.bfloat16)
    dt = torch.nn.functional.softplus(torch.randn((T, s.nheads), generator=gen, device="cuda") - 3.0)
    xbc[lo:hi] = tdev(inp["xbc"][lo:hi], torch.bfloat16)
    z[lo:hi] = tdev(inp["z"][lo:hi], torch.bfloat16)
    dt[lo:hi] = tdev(inp["dt"][lo:hi])
    d = {k: tdev(inp[k]) for k in ("A", "D", "conv_w", "conv_b", "norm_w", "conv_state", "ssm_state")}
    x, B, C = split_views(xbc, s)
    y = m2.mamba2_prefill(x, B, C, z, dt, d["A"], d["D"], d["conv_w"], d["conv_b"], d["norm_w"],
                          d["conv_state"], d["ssm_state"], tdev(cu, torch.int32), 4096, s.nheads,
                          s.headdim, s.dstate, s.ngroups, 128, tdev(inp["state_idx"], torch.int32),
                          tdev(inp["has_init"], torch.uint8))
    torch.cuda.synchronize()
    assert torch.isfinite(y).all() and torch.isfinite(d["ssm_state"]).all()
    del xbc, z, dt
    _check_pairs(inp, s, y, d["conv_state"], d["ssm_state"], [(last, 0), (last, 6)], "bf16")


# ------------------------------------------------------------------ properties

def test_deterministic_and_counters():
    w = WORKLOADS[1]
    inp = make_inputs(w, 1)
    m2.reset_counters()
    y1, c1, s1 = gpu_prefill(inp, w.shape, "bf16")
    y2, c2, s2 = gpu_prefill(inp, w.shape, "bf16")
    assert torch.equal(y1, y2) and torch.equal(c1, c2) and torch.equal(s1, s2)
    c = m2.get_counters()
    assert c["prefill_calls"] == 2 and c["scan_chunked_launches"] == 2 and c["norm_launches"] == 2
    assert c["scan_bf16x3_launches"] == 0 and c["scan_f64_launches"] == 0
    inp0 = make_inputs(WORKLOADS[0], 0)
    gpu_prefill(inp0, WORKLOADS[0].shape, "f32", 16)
    assert m2.get_counters()["scan_f64_launches"] == 1


def test_carried_state_matters():
    """A carried state must change the outputs (the zeroed twin differs by far more than the tolerance)."""
    shape = LayerShape(16, 64, 128, 2)
    inp = small_shape_inputs(shape, [40], seed=60, act="bf16", init="random")
    y1, _, s1 = gpu_prefill(inp, shape, "bf16")
    zero = dict(inp)
    zero["has_init"] = np.zeros_like(inp["has_init"])
    y0, _, s0 = gpu_prefill(zero, shape, "bf16")
    sep_y = (y1 - y0).abs().max().item() / y1.pow(2).mean().sqrt().item()
    print(f"  carried-vs-zeroed separation of y: {sep_y:.3e}")
    assert sep_y > 50 * TOL["bf16"]


def test_debug_mode_rejects_bad_step_sizes_and_decays(monkeypatch):
    """With M2SSD_DEBUG=1 the host reads dt and A before any launch: a negative
    or NaN step size, or a positive decay rate, is refused with M2_ERR_SHAPE
    and no state changes (prefill, scan alone, decode); the packed-row entries
    take raw step sizes of any sign but still refuse a positive A; valid
    inputs run and match the oracle."""
    monkeypatch.setenv("M2SSD_DEBUG", "1")
    shape = LayerShape(4, 16, 16, 2)
    H, P, N, G = shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    inp = small_shape_inputs(shape, [9, 5], seed=74, act="f32", init="random")
    d = to_device(inp, "f32")
    x, B, C = split_views(d["xbc"], shape)
    cs0, ss0 = d["conv_state"].clone(), d["ssm_state"].clone()

    def prefill(dt, A):
        return m2.mamba2_prefill(x, B, C, d["z"], dt, A, d["D"], d["conv_w"], d["conv_b"], d["norm_w"],
                                 d["conv_state"], d["ssm_state"], d["cu_seqlens"], 9, H, P, N, G, 16,
                                 d["state_idx"], d["has_init"])

    def refused(fn, *args):
        with pytest.raises(m2.M2Error) as e:
            fn(*args)
        assert e.value.status == -2, e.value
        torch.cuda.synchronize()
        assert torch.equal(d["conv_state"], cs0) and torch.equal(d["ssm_state"], ss0)

    neg, nan, posA = d["dt"].clone(), d["dt"].clone(), d["A"].clone()
    neg[11, 2] = -1e-3
    nan[3, 0] = float("nan")
    posA[1] = 0.5
    refused(prefill, neg, d["A"])
    refused(prefill, nan, d["A"])
    refused(prefill, d["dt"], posA)
    u = tdev(R.prefill(inp, H, P, N, G, apply_norm=False)["u"])
    ux, uB, uC = split_views(u, shape)
    refused(lambda: m2.ssd_chunk_scan(ux, uB, uC, neg, d["A"], d["D"], d["ssm_state"], d["cu_seqlens"], 9,
                                      H, P, N, G, 16, d["state_idx"], d["has_init"]))
    refused(lambda: m2.mamba2_decode(x[:2], B[:2], C[:2], d["z"][:2], neg[10:12], d["A"], d["D"],
                                     d["conv_w"], d["conv_b"], d["norm_w"], d["conv_state"],
                                     d["ssm_state"], H, P, N, G, d["state_idx"], d["has_init"]))
    # packed rows: any raw step-size sign is valid, a positive A is not
    from workloads import inproj_inputs
    pinp = inproj_inputs(shape, [9, 5], seed=75, act="f32", init="pool", n_slots=4)
    raw0 = shape.d_inner + shape.conv_dim
    assert (pinp["row"][:, raw0:raw0 + H] < 0).any()
    pd = {k: tdev(pinp[k]) for k in ("row", "dt_bias", "A", "D", "conv_w", "conv_b", "norm_w",
                                     "conv_state", "ssm_state")}
    pidx, pinit = tdev(pinp["state_idx"], torch.int32), tdev(pinp["has_init"], torch.uint8)
    pcu = tdev(pinp["cu_seqlens"], torch.int32)

    def packed(A):
        return m2.mamba2_prefill_inproj(pd["row"], pd["dt_bias"], A, pd["D"], pd["conv_w"], pd["conv_b"],
                                        pd["norm_w"], pd["conv_state"], pd["ssm_state"], pcu, 9, H, P, N,
                                        G, 16, pidx, pinit)
    pcs0, pss0 = pd["conv_state"].clone(), pd["ssm_state"].clone()
    with pytest.raises(m2.M2Error) as e:
        packed(posA)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert torch.equal(pd["conv_state"], pcs0) and torch.equal(pd["ssm_state"], pss0)
    packed(pd["A"])
    torch.cuda.synchronize()
    # valid split-view inputs still run, and match the oracle
    y = prefill(d["dt"], d["A"])
    torch.cuda.synchronize()
    ref = oracle_prefill(inp, shape)
    assert rel_err(y, ref["y"], "y", 14 * shape.d_inner) <= TOL["f32"]
    assert rel_err(d["ssm_state"], ref["ssm_state"], "ssm_state") <= TOL["f32"]


def test_argument_errors_raise():
    shape = LayerShape(4, 16, 16, 2)
    inp = small_shape_inputs(shape, [8], seed=70, act="f32", init="zero")
    d = to_device(inp, "f32")
    x, B, C = split_views(d["xbc"], shape)
    args = (x, B, C, d["z"], d["dt"], d["A"], d["D"], d["conv_w"], d["conv_b"], d["norm_w"],
            d["conv_state"], d["ssm_state"], d["cu_seqlens"], 8)
    with pytest.raises(m2.M2Error, match="M2_ERR_CHUNK"):
        m2.mamba2_prefill(*args, 4, 16, 16, 2, 144)
    with pytest.raises(m2.M2Error, match="M2_ERR_UNSUPPORTED"):
        m2.mamba2_prefill(*args, 2, 32, 16, 2, 128)
    with pytest.raises(m2.M2Error, match="M2_ERR_SHAPE"):
        m2.mamba2_prefill(*args, 4, 16, 16, 3, 128)
