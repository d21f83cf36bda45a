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
  roofline     the dominant kernel's algorithmic bytes per launch over its
               average launch time (HIP events recorded by the library on the
               launch stream during the timed steps), against 8 TB/s HBM
  cpu_baseline the fp64 oracle on a bounded sample of the same input, on the
               host cores, in a process pool over (sequence, group) slices
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
    for b in seqs:
        lo = int(cu[b])
        one = dict(inp)
        for k in ("xbc", "z", "dt"):
            one[k] = inp[k][lo:lo + tokens]
        one["cu_seqlens"] = np.array([0, tokens], dtype=np.int32)
        one["state_idx"] = inp["state_idx"][b:b + 1]
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
    ntok = tokens * len(seqs)
    return {"value": ntok / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {tokens} tokens of sequences {list(seqs)} ({ntok} tokens, all "
                      f"{s.ngroups} groups / {s.nheads} heads) of the same input; fp64 "
                      f"token-by-token oracle, {len(items)} (sequence, group) tasks; "
                      f"wall {wall:.2f} s, summed task time {busy:.1f} s"}


# ---------------------------------------------------------------- algorithmic work per kernel

def kernel_bytes(w, T, nseq):
    """Algorithmic HBM bytes of one launch of each kernel of the prefill chain (bf16 inputs).

    conv         read x|B|C, write the post-conv activations (fp32)
    conv_state   read the old and write the new conv state of each sequence
    scan_pass    read post-conv x, B and dt; write the state entering every
                 chunk; read the initial and write the final SSM state
    scan_out     read post-conv x, B, C, dt and the entry state of every chunk;
                 write y before the norm (fp32)
    norm         read y (fp32) and z, write the output (fp32)
    """
    s = w.shape
    act = 2 if w.act == "bf16" else 4
    di, cd, gn = s.d_inner, s.conv_dim, s.ngroups * s.dstate
    state = s.nheads * s.headdim * s.dstate * 4
    slots = T // w.chunk_size + nseq
    return {
        "conv": T * (cd * act + cd * 4),
        "conv_state": nseq * 2 * 3 * cd * 4,
        "scan_pass": T * (di * 4 + gn * 4 + s.nheads * 4) + slots * state + nseq * 2 * state,
        "scan_out": T * (di * 4 + 2 * gn * 4 + s.nheads * 4 + di * 4) + slots * state,
        "norm": T * (di * 4 + di * act + di * 4),
    }


def kernel_sources_sha1():
    """sha1 over the kernel sources (name + bytes, sorted): ties a traffic record to a build."""
    import glob
    import hashlib
    h = hashlib.sha1()
    for f in sorted(glob.glob(os.path.join(ROOT, "mamba_ssd_selective_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
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
                if rec["workload"] == workload and k and rec["sources_sha1"] == kernel_sources_sha1():
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU takes ~20 steps (~25 ms of this load) to reach its steady clocks
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many MiB "
                         "(a reference kernel of known traffic for hardware byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS[WORKLOAD_ID]
    s = w.shape
    t0 = time.time()
    inp = make_inputs(w, WORKLOAD_ID)
    T = int(inp["cu_seqlens"][-1])
    nseq = len(inp["cu_seqlens"]) - 1
    log(f"inputs: {w.name} T={T} generated in {time.time() - t0:.1f}s")

    cpu = None
    if not args.no_cpu_baseline:   # before the GPU is touched: the pool spawns processes
        t0 = time.time()
        cpu = cpu_baseline(inp, w)
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
    maxlen = 4096
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

    kb = kernel_bytes(w, T, nseq)
    dom = max(kms, key=kms.get)
    achieved = kb[dom] / (kms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(w.name, dom),
            "kernel": dom,
            "kernel_ms": round(kms[dom], 4), "kernel_bytes": kb[dom],
            "step_bytes": fused_bytes(w, T, nseq),
            "step_frac": round(fused_bytes(w, T, nseq) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "scan_tflops_alg": round(scan_flops(w, T) / ((kms["scan_pass"] + kms["scan_out"]) * 1e-3) / 1e12, 2),
            "kernel_ms_all": {k: round(v, 4) for k, v in kms.items()}}
    out = {"metric": METRIC, "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": w.name, "batch": nseq, "seq_len": 4096, "total_tokens": T,
                      "nheads": s.nheads, "headdim": s.headdim, "dstate": s.dstate,
                      "ngroups": s.ngroups, "conv_width": s.width, "chunk": w.chunk_size,
                      "activations": w.act, "output": "f32", "parallelism": "single-gpu"},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
