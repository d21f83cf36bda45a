#!/usr/bin/env python3
"""Prefill throughput of one Mamba-2 (SSD) mixer-core layer on one MI355X.

A step is one mamba2_prefill call (causal conv + SiLU, chunked selective scan
with carried state, D skip, grouped gated RMSNorm) over one batch of seeded
synthetic Nemotron-nano-shaped input already resident in HBM: 8 sequences of
4096 tokens, 64 heads x headdim 64, dstate 128, 8 groups, chunk 128, bf16
activations, fp32 dt/A/D/states, fp32 output.  States advance in place each
step, so every step does identical work.

Prints one JSON line on stdout (progress goes to stderr):
  value        tokens/s of the whole step (sum of sequence lengths / step time)
  roofline     step_frac: the step's method bytes (read x|B|C, z, dt and the
               states; write y and the states) over the step time, against
               8 TB/s HBM; frac: the dominant kernel's method bytes per launch
               (kernel_bytes) over its average launch time (HIP events the
               library records on the launch stream during the timed steps);
               design_extra_bytes: what that kernel moves beyond its method
               bytes because of this design's decomposition; traffic: the
               counter-measured HBM bytes of that kernel (profiles/)
  cpu_baseline the fp64 oracle on a bounded sample of the same input, on the
               host cores, in a process pool over (sequence, group) slices

--mode selects another step of the same layer (default: prefill, the line above):
  prefill_inproj  the same prefill taking packed in-projection rows
                  (z | x | B | C | raw dt) with dt = softplus(raw + bias) on the
                  device (mamba2_prefill_inproj)
  decode          one decode token for each of 256 sequences at cache slots of a
                  256-slot fp32 state pool, from packed rows (mamba2_decode_inproj:
                  the fused decode kernel, step size formed in it)
  mixed           a serving step: 256 decode rows then 2 prefill sequences of
                  4096 tokens, from packed rows (mamba2_mixed_inproj); its
                  roofline is the whole step's algorithmic bytes over its time,
                  since the decode rows overlap the prefill chain
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SSD prefill tokens/s per Mamba-2 layer @chunk128; HBM GB/s & MFMA % of peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16
FP64_PEAK_TFLOPS = 78.6     # fp64 matrix
WORKLOAD_ID = 2   # 8 x 4096 tokens, the Nemotron-nano layer shape


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- CPU baseline (oracle)

def _oracle_item(args):
    sub, H, P, N = args
    from oracle import recurrence as R
    t = time.perf_counter()
    R.prefill(sub, H, P, N, 1)
    return time.perf_counter() - t


def cpu_baseline(inp, w, seqs=tuple(range(8)), tokens=1536):
    """Oracle on the first `tokens` rows of `seqs`, all groups, one (sequence, group) slice per task."""
    import multiprocessing as mp
    import concurrent.futures as cf
    import numpy as np
    from workloads import slice_group
    s = w.shape
    items = []
    cu = inp["cu_seqlens"]
    ntok = 0
    for b in seqs:
        lo = int(cu[b])
        n = min(tokens, int(cu[b + 1]) - lo)
        ntok += n
        slot = int(inp["state_idx"][b])
        one = dict(inp)
        for k in ("xbc", "z", "dt"):
            one[k] = inp[k][lo:lo + n]
        one["cu_seqlens"] = np.array([0, n], dtype=np.int32)
        one["conv_state"] = inp["conv_state"][slot:slot + 1]
        one["ssm_state"] = inp["ssm_state"][slot:slot + 1]
        one["state_idx"] = np.zeros(1, dtype=np.int32)
        one["has_init"] = inp["has_init"][b:b + 1]
        for g in range(s.ngroups):
            sub, sh = slice_group(one, s, g)
            items.append((sub, sh.nheads, sh.headdim, sh.dstate))
    cores = max(1, min(16, len(os.sched_getaffinity(0)), len(items)))
    os.environ["OMP_NUM_THREADS"] = "1"
    t = time.perf_counter()
    with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as ex:
        busy = sum(ex.map(_oracle_item, items))
    wall = time.perf_counter() - t
    return {"value": ntok / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {tokens} tokens of sequences {list(seqs)} ({ntok} tokens, all "
                      f"{s.ngroups} groups / {s.nheads} heads) of the same input; fp64 "
                      f"token-by-token oracle, {len(items)} (sequence, group) tasks; "
                      f"wall {wall:.2f} s, summed task time {busy:.1f} s"}


# ---------------------------------------------------------------- algorithmic work per kernel

def kernel_bytes(w, T, nseq, raw=True, fused=False):
    """Method bytes of one launch of each prefill kernel: the layer's own inputs and
    outputs a kernel reads or writes, each counted once at its storage width (bf16
    x|B|C and z, fp32 dt, y and states), plus the stage boundaries the separate
    kernels keep: the pre-norm output y_pre (fp32, written by the scan, read by
    the norm) and, on the four-kernel chain, the conv's fp32 output (written by
    the conv, read by the scan kernels).  Each kernel counts every input it needs
    for its own function.  The state entering every chunk (written by the state
    pass, read by the chunk output: the staged carry this design chose) is not
    a method byte: design_extra_bytes() counts it.

    raw (the default prefill at bf16: the scan kernels convolve the raw rows)
      conv_state   read the old and write the new conv state of each sequence
      scan_pass    read raw x, B and dt; read the initial, write the final SSM state
      scan_out     read raw x, B, C and dt; write y_pre
      norm         read y_pre and z, write y
    raw + fused (each chunk-output workgroup holds whole norm groups: it applies
    the norm itself and the norm kernel does not run)
      scan_out     read raw x, B, C, dt and z; write y
    chain (M2SSD_PREFILL_CHAIN=1, fp32 inputs)
      conv         read x|B|C, write the post-conv activations (fp32; fp64 for fp32 inputs)
      scan_pass    read post-conv x, B and dt; states as above (fp32 inputs: the
                   one-pass scan, which also reads C and writes y_pre)
      scan_out     read post-conv x, B, C and dt; write y_pre
      norm         as above
    """
    s = w.shape
    act = 2 if w.act == "bf16" else 4
    di, cd, gn, H = s.d_inner, s.conv_dim, s.ngroups * s.dstate, s.nheads
    states = nseq * 2 * s.nheads * s.headdim * s.dstate * 4
    conv_state = nseq * 2 * 3 * cd * 4
    norm = T * (di * 4 + di * act + di * 4)
    if w.act != "bf16":
        return {"conv": T * (cd * 4 + cd * 8), "conv_state": conv_state,
                "scan_pass": T * (cd * 8 + H * 4 + di * 4) + states, "scan_out": 0, "norm": norm}
    if raw and fused:
        return {"conv": 0, "conv_state": conv_state,
                "scan_pass": T * ((di + gn) * act + H * 4) + states,
                "scan_out": T * (cd * act + H * 4 + di * act + di * 4), "norm": 0}
    if raw:
        return {"conv": 0, "conv_state": conv_state,
                "scan_pass": T * ((di + gn) * act + H * 4) + states,
                "scan_out": T * (cd * act + H * 4 + di * 4), "norm": norm}
    return {"conv": T * (cd * act + cd * 4), "conv_state": conv_state,
            "scan_pass": T * ((di + gn) * 4 + H * 4) + states,
            "scan_out": T * (cd * 4 + H * 4 + di * 4), "norm": norm}


def design_extra_bytes(w, T, nseq, q16=False):
    """Bytes a kernel moves beyond its method bytes because of this design's
    decomposition: the state entering every chunk slot, written by the state
    pass and read by the chunk output (the staged carry).  fp32, or with q16
    (the raw-row kernels at dstate 128 when no sequence is split) 16-bit
    values plus one fp32 scale per row of 32 values."""
    s = w.shape
    if w.act != "bf16":
        return {}
    per_state = s.headdim * s.dstate * (2 + 4 / 32) if q16 else s.headdim * s.dstate * 4
    entry = int((T // w.chunk_size + nseq) * s.nheads * per_state)
    return {"scan_pass": entry, "scan_out": entry}


# The device sources each measured kernel set is built from: a traffic record holds
# their sha1 and counts only while the sources are unchanged.
CHAIN_SOURCES = ("conv_rows.hip", "ssd_chunked.hip", "ssd_scan.hip", "gated_norm.hip", "norm_row.h",
                 "device_common.h")
DECODE_SOURCES = ("decode_step.hip", "step_size.h", "device_common.h")


def kernel_sources_sha1(files=CHAIN_SOURCES):
    """sha1 over the named kernel sources (name + bytes, sorted): ties a traffic record to a build."""
    import hashlib
    h = hashlib.sha1()
    for name in sorted(files):
        h.update(name.encode())
        with open(os.path.join(ROOT, "mamba_ssd_selective_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel, files=CHAIN_SOURCES):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE / WRITE_SIZE record in
    profiles/, scaled by the copy calibration stored with it; None when no record matches
    the workload and the current kernel sources."""
    import glob
    for f in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.md")):
        with open(f) as fh:
            for line in fh:
                if not line.startswith("traffic-record:"):
                    continue
                rec = json.loads(line.split(":", 1)[1])
                k = rec["kernels"].get(kernel)
                if rec["workload"] == workload and k and rec["sources_sha1"] == kernel_sources_sha1(files):
                    return int((k["fetch_kib"] * rec["fetch_scale"] + k["write_kib"] * rec["write_scale"]) * 1024)
    return None


def fused_bytes(w, T, nseq):
    """Algorithmic bytes of the whole step: read x|B|C, z, dt, states; write y (fp32), states."""
    s = w.shape
    act = 2 if w.act == "bf16" else 4
    state = s.nheads * s.headdim * s.dstate * 4 + 3 * s.conv_dim * 4
    return T * (s.conv_dim * act + s.d_inner * act + s.nheads * 4 + s.d_inner * 4) + nseq * 2 * state


def scan_flops(w, T):
    """Algorithmic flops of the chunk contractions (causal intra, C B^T per group, state, inter)."""
    s = w.shape
    Q, P, N = w.chunk_size, s.headdim, s.dstate
    per_chunk = s.nheads * (P * Q * (Q + 1) + 2 * Q * P * N * 2) + s.ngroups * N * Q * (Q + 1)
    return per_chunk * T / Q


def scan_mfma_flops(w, lens):
    """Executed matrix-core flops of the two scan kernels on the chunk-parallel path
    when every sequence is a whole number of 128-row chunks (None otherwise), with
    fp32 post-conv operands split in (hi, lo) bf16 pairs, 3 products each:
      state pass   per (chunk, head): 4 waves x (dstate / 64) 32x32 tiles x 8 K
                   blocks x 3 products of 32x32x16 (32,768 flop each)
      chunk output per (chunk, group): C B^T over the causal 16x16 tiles, 36 tile
                   columns x (dstate / 32) K blocks x 3, and per head 8 waves x
                   (dstate / 32 x 4 p tiles x 3) for h_in C^T plus 12 x 20 for the
                   causal X^T M^T, all 16x16x32 (16,384 flop each)
    The counts match SQ_INSTS_MFMA on the 8 x 4096 workload."""
    s = w.shape
    if w.act != "bf16" or any(L % 128 for L in lens) or s.headdim != 64 or s.dstate != 128:
        return None
    chunks = sum(L // 128 for L in lens)
    hpg = s.nheads // s.ngroups
    kb = s.dstate // 32
    state = chunks * s.nheads * 4 * (s.dstate // 64) * 8 * 3 * 32768
    out = chunks * s.ngroups * (36 * kb * 3 + hpg * (8 * kb * 4 * 3 + 12 * 20)) * 16384
    return state, out


def mfma_line(w, lens, kms):
    """Matrix-core utilisation of the scan kernels: executed bf16 MFMA flops over
    kernel time and the 2.5 PFLOP/s dense bf16 peak (and algorithmic flops)."""
    ex = scan_mfma_flops(w, lens)
    if ex is None:
        return None
    sp, so = ex
    t_sp, t_so = kms["scan_pass"] * 1e-3, kms["scan_out"] * 1e-3
    return {"peak_tflops": MFMA_PEAK_TFLOPS,
            "state_pass_exec_frac": round(sp / t_sp / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "chunk_out_exec_frac": round(so / t_so / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "scan_alg_frac": round(scan_flops(w, sum(lens)) / (t_sp + t_so) / 1e12 / MFMA_PEAK_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU takes ~20 steps (~25 ms of this load) to reach its steady clocks
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=("prefill", "prefill_inproj", "decode", "mixed"),
                    default="prefill")
    ap.add_argument("--workload", type=int, choices=(1, 2, 3, 4), default=WORKLOAD_ID,
                    help="prefill workload: 2 = 8 x 4096 nano (the headline), 1 = one 137-token "
                         "nano prompt (a latency), 3 = 2 x 2048 fp32 decay stress (the fp64 "
                         "path), 4 = 16 packed sequences of U[1, 8192] tokens at the 8B shape "
                         "with states from a 64-slot pool")
    ap.add_argument("--print-sources-sha1", action="store_true",
                    help="print the sha1 of the prefill-chain and decode kernel sources and exit")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many MiB "
                         "(a reference kernel of known traffic for hardware byte counters)")
    args = ap.parse_args()
    if args.print_sources_sha1:
        print(json.dumps({"chain": kernel_sources_sha1(CHAIN_SOURCES),
                          "decode": kernel_sources_sha1(DECODE_SOURCES)}))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.mode != "prefill":
        return run_other_mode(args)

    import numpy as np
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS[args.workload]
    s = w.shape
    t0 = time.time()
    inp = make_inputs(w, args.workload)
    T = int(inp["cu_seqlens"][-1])
    nseq = len(inp["cu_seqlens"]) - 1
    lens = [int(v) for v in np.diff(inp["cu_seqlens"])]
    log(f"inputs: {w.name} T={T} generated in {time.time() - t0:.1f}s")

    cpu = None
    if not args.no_cpu_baseline:   # before the GPU is touched: the pool spawns processes
        t0 = time.time()
        cpu = cpu_baseline(inp, w, seqs=tuple(range(min(8, nseq))),
                           tokens=1536 if s.nheads <= 64 else 768)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores ({time.time() - t0:.1f}s)")

    import torch
    import mamba_ssd_selective_amd as m2
    m2.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    at = torch.bfloat16 if w.act == "bf16" else torch.float32
    g = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, t)
    xbc = g(inp["xbc"], at)
    z = g(inp["z"], at)
    dt, A, D = g(inp["dt"]), g(inp["A"]), g(inp["D"])
    conv_w, conv_b, norm_w = g(inp["conv_w"]), g(inp["conv_b"]), g(inp["norm_w"])
    conv_state, ssm_state = g(inp["conv_state"]), g(inp["ssm_state"])
    cu = g(inp["cu_seqlens"], torch.int32)
    sidx, hinit = g(inp["state_idx"], torch.int32), g(inp["has_init"], torch.uint8)
    del inp
    di, gn = s.d_inner, s.ngroups * s.dstate
    x, B, C = xbc[:, :di], xbc[:, di:di + gn], xbc[:, di + gn:]
    maxlen = max(lens)
    ws = torch.empty(m2.mamba2_prefill_workspace_size(T, nseq, maxlen, s.nheads, s.headdim, s.dstate,
                                                      s.ngroups, w.chunk_size, at),
                     dtype=torch.uint8, device=dev)
    y = torch.empty((T, di), dtype=torch.float32, device=dev)

    def step():
        m2.mamba2_prefill(x, B, C, z, dt, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state, cu,
                          maxlen, s.nheads, s.headdim, s.dstate, s.ngroups, w.chunk_size, sidx,
                          hinit, w.eps, True, y=y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    m2.timing_enable(args.steps)
    m2.reset_counters()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    kt = m2.timing_read()
    m2.timing_enable(0)
    assert kt["calls"] == args.steps, kt
    assert torch.isfinite(y).all().item(), "non-finite output"
    stages = ("conv", "conv_state", "scan_pass", "scan_out", "norm")
    kms = {k: kt[k + "_ms"] / args.steps for k in stages}
    log(f"timed {args.steps} steps: {ms:.3f} ms/step; kernel ms/step: " +
        ", ".join(f"{k} {v:.3f}" for k, v in kms.items()))

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calib_mib} MiB read + {args.copy_calib_mib} MiB written")
        del src, dst

    cnt = m2.get_counters()
    raw = cnt["conv_launches"] == 0      # the scan kernels convolved the raw rows
    fused = cnt["norm_launches"] == 0    # the chunk output applied the norm
    kb = kernel_bytes(w, T, nseq, raw, fused)
    q16 = False
    if raw and w.act == "bf16" and w.shape.dstate == 128:
        # 16-bit entry states unless the plan splits sequences into segments
        _, seg, _ = m2.ssd_chunk_scan_plan(T, nseq, maxlen, w.shape.nheads, w.shape.headdim,
                                           w.shape.dstate, w.shape.ngroups, w.chunk_size)
        q16 = seg == 0
    extra = design_extra_bytes(w, T, nseq, q16)
    dom = max(kms, key=kms.get)
    step_b = fused_bytes(w, T, nseq)
    step_frac = round(step_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if w.act == "bf16":
        achieved = kb[dom] / (kms[dom] * 1e-3) / 1e9
        roof = {"step_frac": step_frac, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(w.name, dom), "design_extra_bytes": extra.get(dom, 0)}
    else:
        # fp32 inputs: the one-pass scan on fp64 matrix instructions dominates,
        # against the fp64 peak (algorithmic flops over its time)
        achieved = scan_flops(w, T) / (kms["scan_pass"] * 1e-3) / 1e12
        roof = {"step_frac": step_frac, "bound": "fp64", "achieved": round(achieved, 2),
                "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP64_PEAK_TFLOPS, 4),
                "traffic": None}
        dom = "scan_pass"
    path = ("four-kernel chain" if not raw else
            "raw rows convolved in the scan, norm in the chunk output" if fused else "raw rows convolved in the scan")
    roof.update({"kernel": dom, "path": path,
            "kernel_ms": round(kms[dom], 4), "kernel_bytes": kb[dom],
            "step_bytes": step_b,
            "scan_tflops_alg": round(scan_flops(w, T) / ((kms["scan_pass"] + kms["scan_out"]) * 1e-3) / 1e12, 2),
            "mfma": mfma_line(w, lens, kms),
            "kernel_ms_all": {k: round(v, 4) for k, v in kms.items()}})
    out = {"metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if w.act == "bf16" else "f64",
           "data": "synthetic",
           "config": {"workload": w.name, "batch": nseq,
                      "seq_len": lens[0] if len(set(lens)) == 1 else f"varlen {min(lens)}..{max(lens)}",
                      "total_tokens": T,
                      "nheads": s.nheads, "headdim": s.headdim, "dstate": s.dstate,
                      "ngroups": s.ngroups, "conv_width": s.width, "chunk": w.chunk_size,
                      "activations": w.act, "output": "f32", "parallelism": "single-gpu"},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- other steps of the layer

DECODE_BATCH = 256        # decode rows per step (one per sequence), at the nano shape
MIXED_PREFILL = (4096, 4096)


def decode_bytes(s, batch, act, dt_bytes=4):
    """Algorithmic bytes of one decode launch: per sequence the SSM state and conv
    state read and written (fp32), the new x|B|C and z row, the step size, y (fp32);
    per launch the conv and norm weights and A, D."""
    per_seq = (2 * s.nheads * s.headdim * s.dstate * 4 + 2 * 3 * s.conv_dim * 4 +
               s.conv_dim * act + s.d_inner * act + s.nheads * dt_bytes + s.d_inner * 4)
    return batch * per_seq + s.conv_dim * 5 * 4 + s.d_inner * 4 + 2 * s.nheads * 4


def _oracle_rows(args):
    inp, H, P, N, G = args
    from oracle import inproj as IP
    t = time.perf_counter()
    IP.prefill_inproj(inp, H, P, N, G)
    return time.perf_counter() - t


def cpu_baseline_rows(inp, s, seqs, tokens, label):
    """The oracle on the first `tokens` rows of each sequence in `seqs` (packed-row
    inputs), one task per sequence, in a process pool on the host cores."""
    import multiprocessing as mp
    import concurrent.futures as cf
    import numpy as np
    cu = inp["cu_seqlens"]
    items, ntok = [], 0
    for b in seqs:
        lo = int(cu[b])
        n = min(tokens, int(cu[b + 1]) - lo)
        slot = int(inp["state_idx"][b])
        one = dict(inp, row=inp["row"][lo:lo + n], cu_seqlens=np.array([0, n], np.int32),
                   conv_state=inp["conv_state"][slot:slot + 1],
                   ssm_state=inp["ssm_state"][slot:slot + 1],
                   state_idx=np.zeros(1, np.int32), has_init=inp["has_init"][b:b + 1])
        items.append((one, s.nheads, s.headdim, s.dstate, s.ngroups))
        ntok += n
    cores = max(1, min(16, len(os.sched_getaffinity(0)), len(items)))
    os.environ["OMP_NUM_THREADS"] = "1"
    t = time.perf_counter()
    with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as ex:
        busy = sum(ex.map(_oracle_rows, items))
    wall = time.perf_counter() - t
    return {"value": ntok / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{label}: {ntok} tokens in {len(items)} per-sequence tasks; fp64 oracle "
                      f"(row split, softplus step size, token recurrence, gated norm); "
                      f"wall {wall:.2f} s, summed task time {busy:.1f} s"}


def run_other_mode(args):
    import numpy as np
    from workloads import NANO, WORKLOADS, inproj_inputs
    s = NANO
    mode = args.mode
    if mode == "decode":
        lens = [1] * DECODE_BATCH
        nd = DECODE_BATCH
    elif mode == "mixed":
        lens = [1] * DECODE_BATCH + list(MIXED_PREFILL)
        nd = DECODE_BATCH
    else:
        lens = list(WORKLOADS[WORKLOAD_ID].seqlens)
        nd = 0
    t0 = time.time()
    inp = inproj_inputs(s, lens, seed=20 + ["prefill_inproj", "decode", "mixed"].index(mode),
                        act="bf16", init="pool", n_slots=len(lens))
    T, nseq = sum(lens), len(lens)
    log(f"inputs: {mode} T={T} sequences={nseq} generated in {time.time() - t0:.1f}s")
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        if mode == "decode":
            cpu = cpu_baseline_rows(inp, s, range(DECODE_BATCH), 1, "all 256 decode rows")
        else:
            pre = list(range(nd, nseq))
            cpu = cpu_baseline_rows(inp, s, pre, 768,
                                    f"first 768 tokens of the {len(pre)} prefill sequences")
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores ({time.time() - t0:.1f}s)")

    import torch
    import mamba_ssd_selective_amd as m2
    m2.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    g = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev, t)
    row = g(inp["row"], torch.bfloat16)
    dt_bias, A, D = g(inp["dt_bias"]), g(inp["A"]), g(inp["D"])
    conv_w, conv_b, norm_w = g(inp["conv_w"]), g(inp["conv_b"]), g(inp["norm_w"])
    conv_state, ssm_state = g(inp["conv_state"]), g(inp["ssm_state"])
    cu = g(inp["cu_seqlens"], torch.int32)
    sidx, hinit = g(inp["state_idx"], torch.int32), g(inp["has_init"], torch.uint8)
    del inp
    di = s.d_inner
    y = torch.empty((T, di), dtype=torch.float32, device=dev)
    maxlen = max(lens)
    H, P, N, G = s.nheads, s.headdim, s.dstate, s.ngroups
    if mode == "decode":
        def step():
            m2.mamba2_decode_inproj(row, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state,
                                    ssm_state, H, P, N, G, sidx, hinit, 1e-5, True, y=y)
    elif mode == "mixed":
        ws = torch.empty(m2.mamba2_mixed_inproj_workspace_size(T, nseq, maxlen, H, P, N, G, 128, torch.bfloat16),
                         dtype=torch.uint8, device=dev)
        def step():
            m2.mamba2_mixed_inproj(row, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                                   cu, nd, maxlen, H, P, N, G, 128, sidx, hinit, y=y, workspace=ws)
    else:
        ws = torch.empty(m2.mamba2_prefill_inproj_workspace_size(T, nseq, maxlen, H, P, N, G, 128, torch.bfloat16),
                         dtype=torch.uint8, device=dev)
        def step():
            m2.mamba2_prefill_inproj(row, dt_bias, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state,
                                     cu, maxlen, H, P, N, G, 128, sidx, hinit, y=y, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    stream = torch.cuda.current_stream()
    chain = mode != "decode"
    if chain:
        m2.timing_enable(args.steps)
    m2.reset_counters()
    # one event pair per step on the launch stream: for decode that brackets the one kernel
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
    assert torch.isfinite(y).all().item(), "non-finite output"
    log(f"timed {args.steps} steps: {ms:.4f} ms/step")
    if args.copy_calib_mib > 0:
        src = torch.ones(args.copy_calib_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calib_mib} MiB read + {args.copy_calib_mib} MiB written")
        del src, dst
    cfg = {"workload": {"decode": "nano_decode_256", "mixed": "nano_mixed_256dec_2x4096",
                        "prefill_inproj": "nano_8x4096_bf16_inproj"}[mode],
           "decode_rows": nd, "prefill_lens": lens[nd:] if len(lens) - nd <= 8 else f"{len(lens) - nd} x 4096",
           "total_tokens": T, "nheads": H, "headdim": P, "dstate": N, "ngroups": G,
           "conv_width": 4, "chunk": 128, "activations": "bf16", "output": "f32",
           "state_pool_slots": nseq, "parallelism": "single-gpu"}
    if chain:
        kt = m2.timing_read()
        m2.timing_enable(0)
        stages = ("conv", "conv_state", "scan_pass", "scan_out", "norm")
        kms = {k: kt[k + "_ms"] / max(1, kt["calls"]) for k in stages}
        from workloads import Workload
        wl = Workload("x", s, tuple(lens[nd:]), "bf16", "pool")
        cnt = m2.get_counters()
        kb = kernel_bytes(wl, T - nd, nseq - nd, raw=cnt["conv_launches"] == 0, fused=cnt["norm_launches"] == 0)
        if mode == "mixed":
            # the decode rows run on a second stream beside the prefill chain, so
            # the chain's kernel times overlap them: the whole step is the unit
            step_b = decode_bytes(s, nd, 2, dt_bytes=2) + sum(kb.values())
            achieved = step_b / (ms * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": "whole step (decode rows and prefill chain, overlapped)",
                    "kernel_ms": round(ms, 4), "kernel_bytes": step_b,
                    "kernel_ms_all": {k: round(v, 4) for k, v in kms.items()}}
        else:
            dom = max(kms, key=kms.get)
            achieved = kb[dom] / (kms[dom] * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
                    "kernel_ms": round(kms[dom], 4), "kernel_bytes": kb[dom],
                    "kernel_ms_all": {k: round(v, 4) for k, v in kms.items()}}
        log("kernel ms/step (prefill chain): " + ", ".join(f"{k} {v:.3f}" for k, v in kms.items()))
        metric = "SSD prefill tokens/s per Mamba-2 layer @chunk128" if mode == "prefill_inproj" else \
            "Mixed decode+prefill step tokens/s per Mamba-2 layer @chunk128"
    else:
        kb = decode_bytes(s, T, 2, dt_bytes=2)
        achieved = kb / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(cfg["workload"], "decode_step", DECODE_SOURCES),
                "kernel": "decode_step",
                "kernel_ms": round(ms, 4), "kernel_bytes": kb}
        metric = "Decode tokens/s per Mamba-2 layer (one token per sequence at cache slots)"
    out = {"metric": metric, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": cfg, "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
