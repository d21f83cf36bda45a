"""Host-side checks of the C ABI (CPU only, no kernel runs): the library loads,
exports every function include/m2ssd.h declares, and rejects bad arguments
with the documented status before touching the device."""
import ctypes
import os
import re

import pytest

import mamba_ssd_selective_amd as m2

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "m2ssd.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mamba2_conv_rows", "ssd_chunk_scan", "ssd_chunk_scan_workspace_size",
              "gated_rmsnorm_group", "mamba2_prefill", "mamba2_prefill_workspace_size",
              "mamba2_decode", "mamba2_prefill_inproj", "mamba2_prefill_inproj_workspace_size",
              "mamba2_decode_inproj", "mamba2_mixed_inproj", "mamba2_mixed_inproj_workspace_size",
              "m2_last_error", "m2_get_counters"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = m2.load()
    for n in declared_functions():
        assert hasattr(lib, n), f"libm2ssd.so does not export {n}"


def test_version_and_counters():
    assert "gfx950" in m2.version()
    m2.reset_counters()
    assert all(v == 0 for v in m2.get_counters().values())


def _scan(lib, **kw):
    a = dict(x=16, ld_x=64, B=32, ld_B=32, C=48, ld_C=32, act=0, dt=64, ld_dt=4, A=80, D=None,
             ss=96, n_slots=1, cu=112, batch=1, T=8, maxlen=8, idx=None, init=None,
             H=4, P=16, N=16, G=2, chunk=16, y=128, ld_y=64, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.ssd_chunk_scan(a["x"], a["ld_x"], a["B"], a["ld_B"], a["C"], a["ld_C"], a["act"],
                              a["dt"], a["ld_dt"], a["A"], a["D"], a["ss"], a["n_slots"], a["cu"],
                              a["batch"], a["T"], a["maxlen"], a["idx"], a["init"], a["H"],
                              a["P"], a["N"], a["G"], a["chunk"], a["y"], a["ld_y"], a["ws"],
                              a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(act=7), -3), (dict(chunk=144), -4), (dict(chunk=24), -4),
    (dict(chunk=0), -4), (dict(P=24), -7), (dict(G=3), -2), (dict(ld_x=10), -5),
    (dict(ld_y=60), -5), (dict(B=40), -6), (dict(ld_B=34), -6), (dict(batch=0), -2),
    (dict(T=100, maxlen=8), -2), (dict(n_slots=0), -2), (dict(x=24), -6), (dict(ld_x=66), -6),
    # bf16, headdim 64, dstate 128, chunk 128 takes the chunk-parallel path, which needs a workspace
    (dict(act=1, H=4, P=64, N=128, G=1, ld_x=256, ld_B=128, ld_C=128, ld_y=256, chunk=128), -8),
    (dict(act=1, H=4, P=64, N=128, G=1, ld_x=256, ld_B=128, ld_C=128, ld_y=256, chunk=128,
          ws=4096, ws_bytes=64), -8),
    (dict(act=1, H=4, P=64, N=128, G=1, ld_x=256, ld_B=128, ld_C=128, ld_y=256, chunk=128,
          ws=4104, ws_bytes=1 << 30), -6),
])
def test_scan_rejects_bad_arguments(kw, code):
    """Validation happens on the host: the fake (aligned, never dereferenced) pointers are not touched."""
    lib = m2.load()
    assert _scan(lib, **kw) == code
    assert lib.m2_last_error().decode() != ""


def test_conv_and_norm_reject_bad_arguments():
    lib = m2.load()
    # width 5 is unsupported
    assert lib.mamba2_conv_rows(16, 8, 32, 8, 48, 8, 8, 8, 0, 64, None, 5, 128, 1, 256, 1, 0, 0,
                                None, None, 1, 512, 24, 0, None) == -7
    # d_x not a multiple of 8
    assert lib.mamba2_conv_rows(16, 12, 32, 8, 48, 8, 12, 8, 0, 64, None, 4, 128, 1, 256, 1, 0, 0,
                                None, None, 1, 512, 28, 0, None) == -2
    # norm: group width above 2048
    assert lib.gated_rmsnorm_group(16, 4096, 32, 4096, 0, 64, 1e-5, 1, 1, 4, 4096, 128, 4096, 0,
                                   None) == -7
    # norm: in place with a different stride
    assert lib.gated_rmsnorm_group(16, 64, 32, 64, 0, 64, 1e-5, 2, 1, 4, 64, 16, 128, 0, None) == -5


def test_workspace_query_and_prefill_workspace_error(monkeypatch):
    lib = m2.load()
    r = lambda v: (v + 255) // 256 * 256
    scan = lib.ssd_chunk_scan_workspace_size(1000, 1, 64, 64, 128, 8, 128, 1)
    # bf16 rows at a shape whose scan convolves the raw rows itself: the pre-norm
    # output and the scan's own buffers, no post-conv activations
    n = lib.mamba2_prefill_workspace_size(1000, 1, 1000, 64, 64, 128, 8, 128, 1)
    assert scan > 0 and n == r(1000 * 4096 * 4) + scan
    # the four-kernel chain keeps the fp32 post-conv activations as well
    monkeypatch.setenv("M2SSD_PREFILL_CHAIN", "1")
    n_chain = lib.mamba2_prefill_workspace_size(1000, 1, 1000, 64, 64, 128, 8, 128, 1)
    assert n_chain == r(1000 * 6144 * 4) + r(1000 * 4096 * 4) + scan
    monkeypatch.delenv("M2SSD_PREFILL_CHAIN")
    # an odd number of heads per group at dstate 128 takes the chain
    n_odd = lib.mamba2_prefill_workspace_size(1000, 1, 1000, 56, 64, 128, 8, 128, 1)
    assert n_odd >= 1000 * (3584 + 2048) * 4 + 1000 * 3584 * 4
    n32 = lib.mamba2_prefill_workspace_size(1000, 1, 1000, 64, 64, 128, 8, 128, 0)
    assert n32 >= 1000 * (4096 + 2048) * 8 + 1000 * 4096 * 4
    assert lib.mamba2_prefill_workspace_size(-1, 1, 1, 64, 64, 128, 8, 128, 1) == 0
    assert lib.mamba2_prefill_workspace_size(10, 1, 10, 64, 64, 128, 8, 128, 5) == 0


def test_scan_workspace_query():
    """Chunk-parallel path: one fp32 state per chunk slot (slots = T // 128 + batch), the
    int32 dispatch order of the sequences, the end states of split sequences' last
    segments (at most 512 states) and two fp64 log decays per (chunk slot, head); each
    part rounded up to 256 bytes."""
    lib = m2.load()
    per_slot = 64 * 64 * 128 * 4
    r = lambda v: (v + 255) // 256 * 256

    def expect(T, b, H=64):
        slots = T // 128 + b
        return slots * per_slot + r(4 * b) + min(b * H, 512) * 64 * 128 * 4 + 2 * r(8 * slots * H)
    assert lib.ssd_chunk_scan_workspace_size(1000, 3, 64, 64, 128, 8, 128, 1) == expect(1000, 3)
    assert lib.ssd_chunk_scan_workspace_size(4096 * 8, 8, 64, 64, 128, 8, 128, 1) == expect(4096 * 8, 8)
    assert lib.ssd_chunk_scan_workspace_size(1000, 100, 64, 64, 128, 8, 128, 1) == expect(1000, 100)
    # bf16 paths without workspace: other chunk sizes, other shapes
    assert lib.ssd_chunk_scan_workspace_size(1000, 3, 64, 64, 128, 8, 64, 1) == 0
    assert lib.ssd_chunk_scan_workspace_size(1000, 3, 8, 32, 64, 2, 128, 1) == 0
    # fp32 inputs (the one-pass fp64 path): with fewer than 256 (sequence, head)
    # items, room for ceil(256 / items) segments per item, an fp64 P x N state
    # and an fp64 log decay each; none from 256 items on
    def expect_f64(b, H, P, N):
        items = b * H
        nseg = -(-256 // items)
        return r(nseg * items * P * N * 8) + r(nseg * items * 8)
    assert lib.ssd_chunk_scan_workspace_size(1000, 3, 64, 64, 128, 8, 128, 0) == expect_f64(3, 64, 64, 128)
    assert lib.ssd_chunk_scan_workspace_size(11, 1, 4, 16, 16, 2, 16, 0) == expect_f64(1, 4, 16, 16)
    assert lib.ssd_chunk_scan_workspace_size(1000, 4, 64, 64, 128, 8, 128, 0) == 0
    # the prefill workspace includes it, plus the fp32 pre-norm output (the scan
    # convolves the raw bf16 rows itself at this shape)
    n = lib.mamba2_prefill_workspace_size(1000, 3, 1000, 64, 64, 128, 8, 128, 1)
    assert n == r(1000 * 4096 * 4) + expect(1000, 3)


def _decode(lib, **kw):
    a = dict(x=16, ld_x=64, B=32, ld_B=32, C=48, ld_C=32, z=64, ld_z=64, act=0, dt=80, ld_dt=4,
             A=96, D=None, cw=112, cb=None, nw=128, cs=144, ss=160, n_slots=2, batch=2, idx=None,
             init=None, H=4, P=16, N=16, G=2, y=176, ld_y=64, ydt=0)
    a.update(kw)
    return lib.mamba2_decode(a["x"], a["ld_x"], a["B"], a["ld_B"], a["C"], a["ld_C"], a["z"],
                             a["ld_z"], a["act"], a["dt"], a["ld_dt"], a["A"], a["D"], a["cw"],
                             a["cb"], a["nw"], 1e-5, 1, a["cs"], a["ss"], a["n_slots"], a["batch"],
                             a["idx"], a["init"], a["H"], a["P"], a["N"], a["G"], a["y"],
                             a["ld_y"], a["ydt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), -1), (dict(ss=None), -1), (dict(act=2), -3), (dict(ydt=5), -3),
    (dict(batch=-1), -2), (dict(G=3), -2), (dict(n_slots=1), -2), (dict(n_slots=0), -2),
    (dict(P=24), -7), (dict(N=32), -7), (dict(H=64, G=1, ld_x=4096, ld_z=4096, ld_y=4096, ld_dt=64,
                                              P=64, N=128, ld_B=128, ld_C=128), -7),
    (dict(ld_x=60), -5), (dict(ld_B=31), -5), (dict(ld_dt=3), -5), (dict(ld_y=10), -5),
    (dict(ss=168), -6), (dict(cw=120), -6),
])
def test_decode_rejects_bad_arguments(kw, code):
    """Host validation of mamba2_decode (fake, never dereferenced pointers)."""
    lib = m2.load()
    assert _decode(lib, **kw) == code
    assert lib.m2_last_error().decode() != ""


def test_decode_empty_batch_is_a_no_op():
    """batch 0 returns M2_OK after the shape checks, without touching any pointer."""
    lib = m2.load()
    assert _decode(lib, batch=0, x=None, B=None, C=None, z=None, y=None, ss=None, cs=None) == 0
    assert _decode(lib, batch=0, G=3) == -2


# ---- packed in-projection rows and mixed batches (fake, never dereferenced pointers)

_TINY_ROW = 2 * 64 + 2 * 2 * 16 + 4  # z | x | B | C | dt of H=4, P=16, N=16, G=2


def test_inproj_workspace_queries():
    lib = m2.load()
    T, b = 1000, 3
    pre = lib.mamba2_prefill_workspace_size(T, b, T, 64, 64, 128, 8, 128, 1)
    n = lib.mamba2_prefill_inproj_workspace_size(T, b, T, 64, 64, 128, 8, 128, 1)
    assert n == pre + (T * 64 * 4 + 255) // 256 * 256
    # always nonzero for valid arguments (the step sizes need room even when the chain does not)
    assert lib.mamba2_prefill_inproj_workspace_size(0, 1, 0, 4, 16, 16, 2, 16, 0) >= 256
    assert lib.mamba2_prefill_inproj_workspace_size(10, 1, 10, 4, 16, 16, 2, 16, 7) == 0
    mixed = lib.mamba2_mixed_inproj_workspace_size(T, b, T, 64, 64, 128, 8, 128, 1)
    assert mixed == n + 256 + 256
    assert lib.mamba2_mixed_inproj_workspace_size(T, 0, T, 64, 64, 128, 8, 128, 1) == 0


def _prefill_inproj(lib, **kw):
    a = dict(row=4096, ld=_TINY_ROW, act=0, bias=None, A=96, D=None, cw=112, cb=None, nw=128,
             cs=144, ss=160, n_slots=2, cu=176, batch=2, T=10, maxlen=10, idx=None, init=None,
             H=4, P=16, N=16, G=2, chunk=16, y=8192, ld_y=64, ydt=0, ws=16384, ws_bytes=1 << 30)
    a.update(kw)
    return lib.mamba2_prefill_inproj(a["row"], a["ld"], a["act"], a["bias"], a["A"], a["D"], a["cw"],
                                     a["cb"], a["nw"], 1e-5, 1, a["cs"], a["ss"], a["n_slots"], a["cu"],
                                     a["batch"], a["T"], a["maxlen"], a["idx"], a["init"], a["H"],
                                     a["P"], a["N"], a["G"], a["chunk"], a["y"], a["ld_y"], a["ydt"],
                                     a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(row=None), -1), (dict(A=None), -1), (dict(y=None), -1), (dict(cu=None), -1),
    (dict(act=3), -3), (dict(ydt=9), -3),
    (dict(ld=_TINY_ROW - 1), -5), (dict(ld_y=32), -5),
    (dict(ws=None), -8), (dict(ws_bytes=100), -8), (dict(ws=16388), -6),
    (dict(row=4100), -6), (dict(ld=_TINY_ROW + 1), -6),
    (dict(chunk=24), -4), (dict(P=24, ld=264, ld_y=96), -7), (dict(G=3, ld=228), -2), (dict(batch=0), -2),
])
def test_prefill_inproj_rejects_bad_arguments(kw, code):
    lib = m2.load()
    assert _prefill_inproj(lib, **kw) == code
    assert lib.m2_last_error().decode() != ""


def _decode_inproj(lib, **kw):
    a = dict(row=4096, ld=_TINY_ROW, act=0, bias=None, A=96, D=None, cw=112, cb=None, nw=128,
             cs=144, ss=160, n_slots=2, batch=2, idx=None, init=None, H=4, P=16, N=16, G=2,
             y=8192, ld_y=64, ydt=0)
    a.update(kw)
    return lib.mamba2_decode_inproj(a["row"], a["ld"], a["act"], a["bias"], a["A"], a["D"], a["cw"],
                                    a["cb"], a["nw"], 1e-5, 1, a["cs"], a["ss"], a["n_slots"],
                                    a["batch"], a["idx"], a["init"], a["H"], a["P"], a["N"], a["G"],
                                    a["y"], a["ld_y"], a["ydt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(row=None), -1), (dict(ss=None), -1), (dict(act=2), -3), (dict(ld=_TINY_ROW - 1), -5),
    (dict(n_slots=1), -2), (dict(G=3, ld=228), -2), (dict(P=24, ld=264, ld_y=96), -7), (dict(ss=168), -6),
])
def test_decode_inproj_rejects_bad_arguments(kw, code):
    lib = m2.load()
    assert _decode_inproj(lib, **kw) == code


def test_decode_inproj_empty_batch_is_a_no_op():
    lib = m2.load()
    assert _decode_inproj(lib, batch=0, row=None, y=None, ss=None, cs=None) == 0


def _mixed(lib, **kw):
    a = dict(row=4096, ld=_TINY_ROW, act=0, bias=None, A=96, D=None, cw=112, cb=None, nw=128,
             cs=144, ss=160, n_slots=4, cu=176, batch=4, nd=2, T=12, maxlen=10, idx=None, init=None,
             H=4, P=16, N=16, G=2, chunk=16, y=8192, ld_y=64, ydt=0, ws=16384, ws_bytes=1 << 30)
    a.update(kw)
    return lib.mamba2_mixed_inproj(a["row"], a["ld"], a["act"], a["bias"], a["A"], a["D"], a["cw"],
                                   a["cb"], a["nw"], 1e-5, 1, a["cs"], a["ss"], a["n_slots"], a["cu"],
                                   a["batch"], a["nd"], a["T"], a["maxlen"], a["idx"], a["init"],
                                   a["H"], a["P"], a["N"], a["G"], a["chunk"], a["y"], a["ld_y"],
                                   a["ydt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(nd=-1), -2), (dict(nd=5), -2), (dict(batch=0), -2), (dict(T=1), -2),
    (dict(cu=None), -1), (dict(row=None), -1), (dict(n_slots=3), -2),
    (dict(ws=None), -8), (dict(ws_bytes=1000), -8), (dict(ws=16392), -6),
    (dict(act=4), -3), (dict(ld=_TINY_ROW - 2), -5), (dict(chunk=200), -4),
    # a bad prefill-part argument is found before the decode part launches
    (dict(P=24, ld=264, ld_y=96), -7), (dict(nd=4, T=4, P=24, ld=264, ld_y=96), -7),
])
def test_mixed_inproj_rejects_bad_arguments(kw, code):
    lib = m2.load()
    assert _mixed(lib, **kw) == code
    assert lib.m2_last_error().decode() != ""


def test_mixed_workspace_covers_every_prefill_part():
    """The mixed entry hands its prefill part (batch - num_decodes sequences)
    the rest of its workspace; for fp32 inputs the one-pass path's segment
    buffers do not grow with the batch (a smaller batch can be split where a
    larger one is not), so the mixed size must cover every sub-batch."""
    lib = m2.load()
    for (H, P, N, G) in ((64, 64, 128, 8), (4, 16, 16, 2), (24, 32, 64, 2)):
        for batch in (1, 3, 5, 8, 40):
            T = 64 * batch + 4000
            mixed = lib.mamba2_mixed_inproj_workspace_size(T, batch, 4000, H, P, N, G, 128, 0)
            for nd in range(batch):
                part = lib.mamba2_prefill_inproj_workspace_size(T - nd, batch - nd, 4000, H, P, N, G, 128, 0)
                assert mixed - 2 * ((4 * (batch + 1) + 255) // 256 * 256) >= part, (H, batch, nd)
