"""Full-size parity checks against the fp64 oracle, one (sequence, group) pair
per task, in a pool of host processes.

Groups never interact in the mixer core (each owns its heads, its B/C, x, z
and conv channels and its norm group), so the oracle run on one sequence's
rows and one group's channels is an exact sub-problem.  A worker regenerates
its sequence from the workload's seed (every sequence draws from its own
substream), runs the oracle on the pair, reads the device results for that
pair from memory-mapped .npy files the test process wrote, and returns
max|gpu - oracle| and RMS(oracle) per tensor.  Workers start as fresh
interpreters (spawn): they import numpy, the oracle and the generators only,
never the GPU stack.  Test infrastructure only.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

from oracle import recurrence as R
from workloads import group_channels, make_inputs, seqlens_of, slice_group


def _metrics(g: np.ndarray, r: np.ndarray):
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    finite = bool(np.all(np.isfinite(g)))
    err = float(np.max(np.abs(g - r))) if r.size else 0.0
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return dict(n=int(r.size), err=err, rms=rms, finite=finite)


def pair_task(args):
    w, seed, b, g, outdir, nbg = args
    s = w.shape
    inp = make_inputs(w, seed, only_seq=b)
    cu = inp["cu_seqlens"]
    lo, hi = int(cu[b]), int(cu[b + 1])
    heads, xch, ch = group_channels(s, g)
    one = dict(inp)
    for k in ("xbc", "z", "dt"):
        one[k] = inp[k][lo:hi]
    one["cu_seqlens"] = np.array([0, hi - lo], dtype=np.int32)
    one["state_idx"] = inp["state_idx"][b:b + 1]
    one["has_init"] = inp["has_init"][b:b + 1]
    sub_inp, sub = slice_group(one, s, g)
    ref = R.prefill(sub_inp, sub.nheads, sub.headdim, sub.dstate, 1, eps=w.eps, norm_before_gate=nbg)
    slot = int(inp["state_idx"][b])
    y = np.load(os.path.join(outdir, "y.npy"), mmap_mode="r")
    ss = np.load(os.path.join(outdir, "ssm_state.npy"), mmap_mode="r")
    cs = np.load(os.path.join(outdir, "conv_state.npy"), mmap_mode="r")
    return dict(seq=b, group=g, len=hi - lo, slot=slot,
                y=_metrics(y[lo:hi][:, xch], ref["y"]),
                ssm_state=_metrics(ss[slot][heads], ref["ssm_state"][slot]),
                conv_state=_metrics(cs[slot][:, ch], ref["conv_state"][slot]))


def all_pairs(w, seed, outdir, nbg=True, workers=None):
    """Every (sequence, group) pair of workload w (longest sequences first)."""
    lens = seqlens_of(w, seed)
    order = sorted(range(len(lens)), key=lambda b: -lens[b])
    tasks = [(w, seed, b, g, outdir, nbg) for b in order for g in range(w.shape.ngroups)]
    n = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    with ctx.Pool(n) as pool:
        return pool.map(pair_task, tasks, chunksize=1)
