"""The chunk-parallel scan's split into segments, checked on the host.

`ssd_chunk_scan_plan` reports the plan `ssd_chunk_scan` and `mamba2_prefill`
make for a batch (chunk-output workgroups per (chunk, group), chunks per
segment, segment levels).  Three kernels read the segment plan, and they must
agree on which segment a chunk of a sequence belongs to.  Their rules, as
ssd_chunked.hip states them:

  state pass   level k walks chunks [k seg, cend), cend = min((k + 1) seg, nch)
               below the last level and nch on the last level; a level k >= 1
               whose first chunk lies past the sequence's end does nothing
  carry        joins min(ceil(nch / seg), levels) segments
  chunk output a chunk c takes segment min(c // seg, levels - 1)

For sequences up to four times max_seqlen (longer than the plan was made for)
every chunk must be walked by exactly one level, that level must be the
segment the chunk output takes, and the carry must join exactly the levels
that walked.  The GPU side of a longer-than-planned sequence is
tests/test_gpu_raw_conv.py::test_sequence_longer_than_planned_levels.
"""
import math

import pytest
import torch

import mamba_ssd_selective_amd as m2

Q = 128

# (nheads, ngroups, dstate, batch, max_seqlen): shapes whose walks fill fewer
# than 256 workgroups, so long sequences are split
SPLIT_SHAPES = [
    (8, 2, 128, 1, 65536),
    (16, 2, 128, 4, 1024),
    (64, 8, 128, 1, 8192),
    (12, 4, 64, 2, 20000),
    (4, 4, 64, 1, 3000),
    (32, 1, 64, 3, 4000),
]


def walks(nch, seg, levels):
    """Chunks each state-pass level walks for a sequence of nch chunks."""
    out = []
    for k in range(levels):
        first = k * seg
        if k > 0 and first >= nch:
            out.append([])
            continue
        end = min(first + seg, nch) if k < levels - 1 else nch
        out.append(list(range(first, end)))
    return out


@pytest.mark.parametrize("shape", SPLIT_SHAPES)
def test_every_chunk_is_walked_once_and_found_by_the_chunk_output(shape):
    H, G, N, batch, max_seqlen = shape
    split, seg, levels = m2.ssd_chunk_scan_plan(batch * max_seqlen, batch, max_seqlen, H, 64, N, G)
    nplan = math.ceil(max_seqlen / Q)
    assert seg > 0, "these shapes are split"
    assert seg >= 4 and levels >= 2
    assert seg * levels >= nplan and seg * (levels - 1) < nplan
    hpg = H // G
    assert split >= 1 and hpg % split == 0 and (split & (split - 1)) == 0
    for L in sorted({1, Q - 1, Q, Q + 1, max_seqlen - 1, max_seqlen, max_seqlen + 1, 2 * max_seqlen,
                     4 * max_seqlen + 3} - {0}):
        nch = math.ceil(L / Q)
        w = walks(nch, seg, levels)
        seen = [c for lv in w for c in lv]
        assert sorted(seen) == list(range(nch)), (L, seg, levels)
        for k, lv in enumerate(w):
            for c in lv:
                assert min(c // seg, levels - 1) == k, (L, c, k)
        joined = min(math.ceil(nch / seg), levels)
        assert joined == sum(1 for lv in w if lv), (L, joined)


def test_plans_of_the_measured_workloads():
    # 8 x 4096 nano: 256 state-pass workgroups already, so no split, and 2112
    # (chunk, group) items, so whole groups per chunk-output workgroup
    assert m2.ssd_chunk_scan_plan(8 * 4096, 8, 4096, 64, 64, 128, 8) == (1, 0, 1)
    # one 137-token nano prompt: 16 (chunk, group) items, each group's 8 heads
    # over 8 workgroups
    assert m2.ssd_chunk_scan_plan(137, 1, 137, 64, 64, 128, 8) == (8, 0, 1)


def test_one_pass_sizes_have_no_chunk_plan():
    # fp32 inputs take the one-pass fp64 scan
    with pytest.raises(m2.M2Error):
        m2.ssd_chunk_scan_plan(4096, 2, 2048, 64, 64, 128, 8, act_dtype=torch.float32)
    # total_tokens above batch * max_seqlen is refused
    with pytest.raises(m2.M2Error):
        m2.ssd_chunk_scan_plan(5000, 2, 2048, 64, 64, 128, 8)
