"""The 16-bit entry-state layout of the chunk-parallel scan, checked on the host.

At dstate 128 the raw-row state pass hands each chunk's entry state to the
chunk output as 16-bit rows with a scale each (ssd_chunked.hip,
store_entry_q16 and the chunk output's decode).  Their index rules, restated:

  fp32 order   float4 f = (tile * 4 + m) * 64 + lane holds p = 32 (tile & 1) +
               lane % 32, n = 32 (tile >> 1) + 8 m + 4 (lane / 32) + 0..3
  writer       consumer cw holds tiles 2 cw + pt; its lane stores uint4
               u = (tile * 2 + m2) * 64 + lane with the values of float4s
               (tile * 4 + 2 m2) * 64 + lane and the one 64 after, and lanes
               l < 32 store the scales of row (p % 32 = l) for tiles 2 cw,
               2 cw + 1 at float P * N / 2 + l * 8 + 2 cw
  reader       producer thread t < 256 loads uint4 t + 256 k (k < 4), decodes
               float4s f = ((2 k + t / 128) * 4 + 2 ((t / 64) % 2)) * 64 + t % 64
               and f + 64, and takes their scale from the two float4s at
               P * N / 2 + (t % 32) * 8, element 2 k + t / 128

The reader must find, for every (p, n) of the P x N state, the value and the
scale the writer stored for it, and every byte the reader touches must lie
in the block's first 17 KB.
"""
import numpy as np

P, N = 64, 128
NTQ = (P // 32) * (N // 32)


def fp32_pn(f):
    lane, m, tile = f & 63, (f >> 6) & 3, f >> 8
    return 32 * (tile & 1) + (lane & 31), 32 * (tile >> 1) + 8 * m + 4 * (lane >> 5)


def writer():
    """uint4 index -> the 8 (p, n) it holds; scale float index -> (row p, n tile)."""
    values, scales = {}, {}
    for cw in range(4):
        for pt in range(2):
            tile = 2 * cw + pt
            for lane in range(64):
                for m2 in range(2):
                    u = (tile * 2 + m2) * 64 + lane
                    pn = []
                    for half in range(2):
                        p, n = fp32_pn((tile * 4 + 2 * m2 + half) * 64 + lane)
                        pn += [(p, n + e) for e in range(4)]
                    assert u not in values
                    values[u] = pn
                if lane < 32:
                    idx = P * N // 2 + lane * NTQ + tile
                    assert idx not in scales
                    scales[idx] = (32 * (tile & 1) + lane, tile >> 1)
    return values, scales


def test_writer_covers_the_state_once():
    values, scales = writer()
    allpn = [pn for v in values.values() for pn in v]
    assert len(allpn) == P * N and len(set(allpn)) == P * N
    assert sorted(values) == list(range(P * N // 8))          # 16 KB of uint4s
    # one scale per (p, n tile), right after the values, within 17 KB
    assert sorted(scales.values()) == sorted((p, t) for p in range(P) for t in range(N // 32))
    assert min(scales) == P * N // 2 and max(scales) < P * N // 2 + 32 * NTQ
    # every value's scale is the one of its own row of 32
    for u, pns in values.items():
        for p, n in pns:
            assert (p, n // 32) in scales.values()


def test_reader_decodes_what_the_writer_stored():
    values, scales = writer()
    inv_scale = {v: k for k, v in scales.items()}
    seen = set()
    for t in range(256):
        for k in range(4):
            u = t + 256 * k
            f = ((2 * k + t // 128) * 4 + 2 * ((t // 64) % 2)) * 64 + t % 64
            pn = []
            for ff in (f, f + 64):
                p, n = fp32_pn(ff)
                pn += [(p, n + e) for e in range(4)]
            assert pn == values[u], (t, k)
            # the scale the reader picks: float4 (t % 32) * 8 / 4 + j // 4, element j % 4,
            # j = 2 k + t / 128, i.e. float P N / 2 + (t % 32) * 8 + j
            j = 2 * k + t // 128
            sidx = P * N // 2 + (t % 32) * NTQ + j
            for p, n in pn:
                assert inv_scale[(p, n // 32)] == sidx, (t, k, p, n)
            seen.update(pn)
    assert len(seen) == P * N
