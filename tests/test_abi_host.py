"""Host-only checks of the C ABI (no GPU needed).

The library must load, export every entry point that include/lattice_osr.h
declares, and reject bad arguments with the documented status codes before
any HIP call is made (so these run on a machine without a GPU).
"""
import ctypes
import os
import re

import pytest

from compressed_memory_linear_amd import osr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lattice_osr.h")

# Fake device addresses: only compared and range-checked on the host, never
# dereferenced, because every case below fails validation first.
BASE = 1 << 40


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LATTICE_OSR_API\s+[\w\s\*]+?\b(lattice_osr_\w+)\s*\(", text)))


def test_header_declarations_are_exported():
    declared = _declared_functions()
    assert set(declared) == set(osr.EXPORTED)
    lib = osr.load_library()
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings():
    assert osr.lattice_osr_abi_version() == 6
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = osr.status_string(code)
        assert s and s != "unknown status"
    assert osr.status_string(-99) == "unknown status"


def _ptrs(desc, gap=1 << 32):
    """Disjoint fake buffers for q, k, v, gamma, mu, state_in, state_out, y."""
    return [BASE + i * gap for i in range(8)]


def _call(fn, desc, ptrs, chunk=None, ws=None, ws_bytes=0):
    lib = osr.load_library()
    args = [ctypes.byref(desc)]
    if chunk is not None:
        args.append(chunk)
    args += ptrs + [ws, ws_bytes, None]
    return getattr(lib, fn)(*args)


FWD = ["lattice_osr_fwd_recurrent", "lattice_osr_decode_step"]


@pytest.mark.parametrize("fn", FWD + ["lattice_osr_fwd_chunked"])
def test_null_pointers(fn):
    d = osr.make_desc(1, 1, 1, 16, 16)
    chunk = 1 if fn == "lattice_osr_fwd_chunked" else None
    lib = osr.load_library()
    assert getattr(lib, fn)(None, *([chunk] if chunk else []), *_ptrs(d), None, 0, None) == osr.ERR_NULL
    for i in range(8):
        p = _ptrs(d)
        p[i] = None
        assert _call(fn, d, p, chunk) == osr.ERR_NULL, i


@pytest.mark.parametrize("field,value,status", [
    ("B", 0, osr.ERR_SHAPE), ("T", 0, osr.ERR_SHAPE), ("H", -1, osr.ERR_SHAPE),
    ("m", 0, osr.ERR_SHAPE), ("m", 48, osr.ERR_UNSUPPORTED), ("d", 256, osr.ERR_UNSUPPORTED),
    ("in_dtype", 2, osr.ERR_UNSUPPORTED), ("y_dtype", 7, osr.ERR_UNSUPPORTED),
    ("mode", 3, osr.ERR_UNSUPPORTED), ("mode", -1, osr.ERR_UNSUPPORTED), ("gamma_per_slot", 2, osr.ERR_UNSUPPORTED),
    ("linearisation", 2, osr.ERR_UNSUPPORTED), ("linearisation", -1, osr.ERR_UNSUPPORTED),
    ("schedule", 3, osr.ERR_UNSUPPORTED), ("schedule", -1, osr.ERR_UNSUPPORTED),
    ("chain_pairs", 2, osr.ERR_UNSUPPORTED), ("chain_pairs", -1, osr.ERR_UNSUPPORTED),
    ("chain_wgs", 2, osr.ERR_UNSUPPORTED), ("chain_wgs", -1, osr.ERR_UNSUPPORTED),
    ("readout_overlap", 2, osr.ERR_UNSUPPORTED), ("readout_overlap", -1, osr.ERR_UNSUPPORTED),
    ("bwd_form", 3, osr.ERR_UNSUPPORTED), ("bwd_form", -1, osr.ERR_UNSUPPORTED),
])
def test_bad_descriptor(field, value, status):
    d = osr.make_desc(2, 8, 2, 32, 32)
    setattr(d, field, value)
    for fn in FWD:
        if fn == "lattice_osr_decode_step" and field != "T":
            d.T = 1
        assert _call(fn, d, _ptrs(d)) == status, fn
        d.T = 8 if field != "T" else value
    assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), 4) == status


def test_first_linearisation_workspace():
    """bf16 inputs with C >= 16 run both linearisations on the split MFMA
    schedule; the first keeps one more per-chunk array (e, m x C fp32).  The
    token loop (fp32 inputs or C < 16) needs none."""
    B, T, H, m, d = 2, 256, 4, 64, 64
    d2 = osr.make_desc(B, T, H, m, d)
    d1 = osr.make_desc(B, T, H, m, d, linearisation=osr.LIN1)
    for C in (16, 64):
        extra = B * H * (T // C) * m * C * 4
        assert osr.lattice_osr_workspace_bytes(d1, C) == osr.lattice_osr_workspace_bytes(d2, C) + extra
    for C in (1, 4):
        assert osr.lattice_osr_workspace_bytes(d1, C) == 0
    f1 = osr.make_desc(B, T, H, m, d, in_dtype=osr.F32, linearisation=osr.LIN1)
    assert osr.lattice_osr_workspace_bytes(f1, 64) == 0
    # many sequences: the default switches to the fused kernel (no workspace), the first stays split
    big2 = osr.make_desc(64, 256, 8, m, d)
    big1 = osr.make_desc(64, 256, 8, m, d, linearisation=osr.LIN1)
    assert osr.lattice_osr_workspace_bytes(big2, 64) == 0
    assert osr.lattice_osr_workspace_bytes(big1, 64) > 0


def test_schedule_field_sets_the_workspace():
    """The workspace query follows the descriptor's schedule, so the query and
    the launch it sizes always agree: the split schedule needs the per-chunk
    arrays, the fused kernel none; the first linearisation has no fused form."""
    B, T, H, m, d, C = 2, 256, 4, 64, 64, 64
    per_chunk = (m * d + 2 * m * C + d * C) * 4
    auto = osr.make_desc(B, T, H, m, d)
    split = osr.make_desc(B, T, H, m, d, schedule=osr.SCHED_SPLIT)
    fused = osr.make_desc(B, T, H, m, d, schedule=osr.SCHED_FUSED)
    assert osr.lattice_osr_workspace_bytes(auto, C) == B * H * (T // C) * per_chunk  # few sequences: split
    assert osr.lattice_osr_workspace_bytes(split, C) == B * H * (T // C) * per_chunk
    assert osr.lattice_osr_workspace_bytes(fused, C) == 0
    fused1 = osr.make_desc(B, T, H, m, d, schedule=osr.SCHED_FUSED, linearisation=osr.LIN1)
    assert osr.lattice_osr_workspace_bytes(fused1, C) > 0
    big_split = osr.make_desc(64, 256, 8, m, d, schedule=osr.SCHED_SPLIT)
    assert osr.lattice_osr_workspace_bytes(big_split, C) == 64 * 8 * (256 // C) * per_chunk
    # the pair switch changes no buffer
    nopair = osr.make_desc(B, T, H, m, d, chain_pairs=osr.PAIRS_OFF)
    assert osr.lattice_osr_workspace_bytes(nopair, C) == osr.lattice_osr_workspace_bytes(auto, C)


def test_workgroup_split_workspace():
    """The state passing split over P workgroups per sequence (a chunk of P
    sub-blocks, few sequences) adds its hand-off buffers to the workspace: per
    (b,h), two chunk parities x P parts of (m d + 4 m) floats, and P m/16
    counters of 128 bytes.  chain_wgs ONE, or more than 32 sequences, adds none."""
    m = d = C = 128
    T = 1024
    per_chunk = (m * d + 2 * m * C + d * C) * 4
    for BH, P in ((16, 4), (32, 4), (33, 1), (200, 1)):
        auto = osr.make_desc(1, T, BH, m, d)
        one = osr.make_desc(1, T, BH, m, d, chain_wgs=osr.WGS_ONE)
        base = BH * (T // C) * per_chunk
        xchg = BH * (2 * P * (m * d + 4 * m) * 4 + P * (m // 16) * 128) if P > 1 else 0
        assert osr.lattice_osr_workspace_bytes(auto, C) == base + xchg, (BH, P)
        assert osr.lattice_osr_workspace_bytes(one, C) == base
    # a chunk of two sub-blocks (m = d = 128, C = 64: 32-token sub-blocks)
    two = osr.make_desc(1, 256, 16, 128, 128)
    assert osr.lattice_osr_workspace_bytes(two, 64) == 16 * 4 * (m * d + 2 * m * 64 + d * 64) * 4 + \
        16 * (2 * 2 * (m * d + 4 * m) * 4 + 2 * 8 * 128)


def test_overlapped_readout_workspace():
    """The read-out overlapped by chunk ranges (at most 128 state-passing
    workgroups, a multiple of 64 chunks) hands the state from range to range
    through one more array of B H m d floats; OVERLAP_OFF, too few or ragged
    chunk counts, or more workgroups add none."""
    m = d = C = 128
    per_chunk = (m * d + 2 * m * C + d * C) * 4
    for BH, P, NC, carry in ((16, 4, 64, True), (16, 4, 512, True), (33, 1, 64, True), (64, 1, 128, True),
                             (65, 1, 64, True), (128, 1, 64, True), (129, 1, 64, False), (16, 4, 32, False),
                             (16, 4, 96, False)):
        T = NC * C
        auto = osr.make_desc(1, T, BH, m, d)
        off = osr.make_desc(1, T, BH, m, d, readout_overlap=osr.OVERLAP_OFF)
        base = BH * NC * per_chunk
        base += BH * (2 * P * (m * d + 4 * m) * 4 + P * (m // 16) * 128) if P > 1 else 0
        assert osr.lattice_osr_workspace_bytes(off, C) == base, (BH, NC)
        assert osr.lattice_osr_workspace_bytes(auto, C) == base + (BH * m * d * 4 if carry else 0), (BH, NC)


def test_library_reads_no_environment():
    """Every knob is a descriptor field: no source of the library reads the
    process environment."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "compressed_memory_linear_amd", "csrc", "*")):
        assert "getenv" not in open(path).read(), path


def test_chunk_size_rules():
    d = osr.make_desc(1, 48, 1, 32, 32)
    assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), 32) == osr.ERR_SHAPE      # ragged tail
    assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), 0) == osr.ERR_SHAPE
    assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), 3) == osr.ERR_UNSUPPORTED  # 48 % 3 == 0
    assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), 6) == osr.ERR_UNSUPPORTED
    d2 = osr.make_desc(1, 512, 1, 32, 32)
    assert _call("lattice_osr_fwd_chunked", d2, _ptrs(d2), 256) == osr.ERR_UNSUPPORTED
    with pytest.raises(osr.OSRError):
        osr.lattice_osr_workspace_bytes(d, 32)


def test_gated_forward_rejects_bad_gate():
    """The gate of the fused post-gate is an input: null, misaligned or
    overlapping an output is rejected before any HIP call."""
    lib = osr.load_library()
    d = osr.make_desc(1, 8, 1, 16, 16, in_dtype=osr.F32)
    p = _ptrs(d)
    gate = BASE + 20 * (1 << 32)

    def call(g, ptrs=p):
        return lib.lattice_osr_fwd_chunked_gated(ctypes.byref(d), 4, *ptrs[:5], g, *ptrs[5:], None, 0, None)

    assert call(None) == osr.ERR_NULL
    assert call(gate + 4) == osr.ERR_ALIGN
    assert call(p[7]) == osr.ERR_ALIAS      # the gate is y
    assert call(p[6]) == osr.ERR_ALIAS      # the gate is state_out
    bad = list(p)
    bad[0] = None
    assert call(gate, bad) == osr.ERR_NULL  # the other rules are the forward's


def test_decode_requires_single_token():
    d = osr.make_desc(4, 2, 2, 32, 32)
    assert _call("lattice_osr_decode_step", d, _ptrs(d)) == osr.ERR_SHAPE


def test_aliasing_rules():
    d = osr.make_desc(1, 1, 1, 16, 16, in_dtype=osr.F32)
    state_bytes = 16 * 16 * 4
    p = _ptrs(d)
    # partial overlap of state_out with state_in
    p[6] = p[5] + 64
    assert _call("lattice_osr_decode_step", d, p) == osr.ERR_ALIAS
    # y overlapping an input
    p = _ptrs(d)
    p[7] = p[2]
    assert _call("lattice_osr_decode_step", d, p) == osr.ERR_ALIAS
    # y overlapping the state
    p = _ptrs(d)
    p[7] = p[5] + state_bytes - 16
    assert _call("lattice_osr_decode_step", d, p) == osr.ERR_ALIAS
    # state_out overlapping an input
    p = _ptrs(d)
    p[6] = p[0]
    assert _call("lattice_osr_fwd_recurrent", d, p) == osr.ERR_ALIAS


@pytest.mark.parametrize("fn", FWD + ["lattice_osr_fwd_chunked"])
def test_misaligned_pointers_are_rejected(fn):
    """q, k, v, per-slot gamma, the states and y need 16-byte alignment; mu
    and a per-token gamma only element alignment."""
    chunk = 1 if fn == "lattice_osr_fwd_chunked" else None
    for gps in (1, 0):
        d = osr.make_desc(1, 1, 1, 16, 16, gamma_per_slot=gps)
        for i in range(8):
            if i == 4 or (i == 3 and not gps):
                continue  # element-aligned offsets are accepted (never launched here)
            for off in (2, 4, 8):
                p = _ptrs(d)
                p[i] += off
                assert _call(fn, d, p, chunk) == osr.ERR_ALIGN, (gps, i, off)
        # mu / per-token gamma at an odd byte offset are rejected
        for i in ([4] if gps else [3, 4]):
            p = _ptrs(d)
            p[i] += 1
            assert _call(fn, d, p, chunk) == osr.ERR_ALIGN, (gps, i)


def test_misaligned_workspace_is_rejected():
    d = osr.make_desc(2, 256, 2, 64, 64)
    need = osr.lattice_osr_workspace_bytes(d, 64)
    if need:
        assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), 64, BASE * 4 + 8, need) == osr.ERR_ALIGN


def test_workspace_too_small_is_rejected():
    for (m, dd, C) in ((64, 64, 64), (32, 32, 16), (64, 128, 64), (128, 128, 128)):
        d = osr.make_desc(2, 4 * C, 2, m, dd)
        need = osr.lattice_osr_workspace_bytes(d, C)
        if need == 0:
            continue
        assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), C, None, 0) == osr.ERR_NULL
        assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), C, BASE * 4, need - 1) == osr.ERR_WORKSPACE
        # workspace overlapping an input
        assert _call("lattice_osr_fwd_chunked", d, _ptrs(d), C, _ptrs(d)[0], need) == osr.ERR_ALIAS


# ---------------------------------------------------------------- backward --
# Argument order after (desc, chunk): q, k, v, gamma, mu, state_in, dy,
# dstate_out (inputs 0..7), dq, dk, dv, dgamma, dmu, dstate_in (outputs 8..13).
def _bwd_ptrs(gap=1 << 32):
    return [BASE + i * gap for i in range(14)]


def _bwd_call(d, ptrs, chunk, ws=None, ws_bytes=None):
    lib = osr.load_library()
    if ws_bytes is None:
        need = lib.lattice_osr_bwd_workspace_bytes(ctypes.byref(d), chunk)
        ws_bytes = need if need != ctypes.c_size_t(-1).value else 0
    if ws is None:
        ws = BASE + 14 * (1 << 32)
    return lib.lattice_osr_bwd_chunked(ctypes.byref(d), chunk, *ptrs, ws, ws_bytes, None)


def test_bwd_workspace_formula():
    """Per (b,h): 4 (T/C + 1 + C) m d bytes of states and 4 C (2m + 4)
    bytes of per-token values; at C <= 8 with the decoding objective every
    token's h (4 T d bytes, the small-chunk form); with bf16 inputs and C >= 16 (not the encoding
    layer) also the state-passing kernel's per-chunk arrays, 4 (m d + 2 m C +
    d C) bytes per chunk (one more m C with the first linearisation), and the
    c, beta and |h|^2 it keeps for the backward, 4 (2 m C + C) per chunk."""
    for (B, T, H, m, dd, C) in ((4, 2048, 8, 64, 64, 64), (1, 64, 1, 16, 32, 1), (2, 512, 3, 128, 128, 128)):
        for in_dtype in (osr.BF16, osr.F32):
            for mode in (osr.MODE_DEC, osr.MODE_ENC):
                for lin in (osr.LIN2, osr.LIN1):
                    d = osr.make_desc(B, T, H, m, dd, in_dtype=in_dtype, mode=mode, linearisation=lin)
                    per = 4 * ((T // C + 1 + C) * m * dd + C * (2 * m + 4))
                    want = B * H * per
                    if C <= 8 and mode == osr.MODE_DEC:
                        want += B * H * T * dd * 4  # every token's h (the small-chunk form)
                    if in_dtype == osr.BF16 and C >= 16 and mode != osr.MODE_ENC:
                        per_chunk = m * dd + (3 if lin == osr.LIN1 else 2) * m * C + dd * C
                        per_chunk += 2 * m * C + C  # c, beta and |h|^2 kept for the backward
                        want += B * H * (T // C) * per_chunk * 4
                        want += _bwd_xchg(B * H, m, dd)
                    assert osr.lattice_osr_bwd_workspace_bytes(d, C) == want, (B, T, H, m, dd, C, in_dtype, mode, lin)


def _bwd_xchg(bh, m, d):
    """Hand-off buffers of the backward split over P workgroups per sequence
    (the largest P in 1, 2, 4, 8 with m / P >= 16 and B H P <= 256): per (b,h)
    2 P parts of 8 (d + 4) floats and P counters of 128 bytes."""
    P = 1
    while P < 8 and m // (2 * P) >= 16 and bh * 2 * P <= 256:
        P *= 2
    return 0 if P == 1 else bh * (2 * P * 8 * (d + 4) * 4 + P * 128)


def test_bwd_split_workspace():
    """The split's hand-off buffers follow the descriptor's chain_wgs: ONE,
    or a layout without the state-passing kernel's arrays, adds none."""
    for (B, H, m, dd, P) in ((1, 16, 128, 128, 8), (4, 8, 64, 64, 4), (8, 16, 64, 128, 2), (16, 16, 64, 64, 1),
                             (1, 4, 16, 32, 1), (2, 2, 32, 16, 2)):
        T, C = 256, 64
        auto = osr.make_desc(B, T, H, m, dd)
        one = osr.make_desc(B, T, H, m, dd, chain_wgs=osr.WGS_ONE)
        extra = 0 if P == 1 else B * H * (2 * P * 8 * (dd + 4) * 4 + P * 128)
        assert extra == _bwd_xchg(B * H, m, dd)
        assert osr.lattice_osr_bwd_workspace_bytes(auto, C) - osr.lattice_osr_bwd_workspace_bytes(one, C) == extra
        f32 = osr.make_desc(B, T, H, m, dd, in_dtype=osr.F32)
        assert osr.lattice_osr_bwd_workspace_bytes(f32, C) == B * H * 4 * ((T // C + 1 + C) * m * dd + C * (2 * m + 4))


def test_bwd_null_pointers_and_shapes():
    d = osr.make_desc(1, 8, 1, 16, 16)
    lib = osr.load_library()
    assert lib.lattice_osr_bwd_chunked(None, 4, *_bwd_ptrs(), None, 0, None) == osr.ERR_NULL
    for i in range(14):
        p = _bwd_ptrs()
        p[i] = None
        assert _bwd_call(d, p, 4) == osr.ERR_NULL, i
    assert _bwd_call(d, _bwd_ptrs(), 4, ws=None, ws_bytes=0) in (osr.ERR_WORKSPACE,)
    lib2 = osr.load_library()
    assert lib2.lattice_osr_bwd_chunked(ctypes.byref(d), 4, *_bwd_ptrs(), None, 1 << 30, None) == osr.ERR_NULL
    assert _bwd_call(d, _bwd_ptrs(), 3) == osr.ERR_SHAPE          # ragged tail
    assert _bwd_call(d, _bwd_ptrs(), 0) == osr.ERR_SHAPE
    d2 = osr.make_desc(1, 8, 1, 16, 48)
    assert _bwd_call(d2, _bwd_ptrs(), 4) == osr.ERR_UNSUPPORTED
    # (the linearisation does not change the workspace)
    d3 = osr.make_desc(1, 8, 1, 16, 16, linearisation=osr.LIN1)
    assert osr.lattice_osr_bwd_workspace_bytes(d3, 4) == osr.lattice_osr_bwd_workspace_bytes(d, 4)
    d4 = osr.make_desc(1, 8, 1, 16, 16, linearisation=2)
    assert _bwd_call(d4, _bwd_ptrs(), 4) == osr.ERR_UNSUPPORTED
    with pytest.raises(osr.OSRError):
        osr.lattice_osr_bwd_workspace_bytes(d4, 4)


def test_bwd_form_choice():
    """The chunk-parallel backward is built for m = d = C = 64 with bf16 inputs,
    the default linearisation and the decoding or similarity objective: asking
    for it elsewhere is ERR_UNSUPPORTED; the walk and the automatic choice take
    every configuration, and the workspace does not depend on the form."""
    ok = dict(B=1, T=128, H=2, m=64, d=64)
    for form in (osr.BWD_AUTO, osr.BWD_WALK, osr.BWD_CHUNK):
        d = osr.make_desc(**ok, bwd_form=form)
        assert osr.lattice_osr_bwd_workspace_bytes(d, 64) == \
            osr.lattice_osr_bwd_workspace_bytes(osr.make_desc(**ok), 64)
    bad = [dict(C=32), dict(C=64, in_dtype=osr.F32), dict(C=64, linearisation=osr.LIN1),
           dict(C=64, mode=osr.MODE_ENC), dict(C=64, m=32), dict(C=64, d=128)]
    for b in bad:
        kw = dict(ok)
        C = b.pop("C")
        kw.update(b)
        chunk = osr.make_desc(**kw, bwd_form=osr.BWD_CHUNK)
        assert _bwd_call(chunk, _bwd_ptrs(), C) == osr.ERR_UNSUPPORTED, b
        with pytest.raises(osr.OSRError):
            osr.lattice_osr_bwd_workspace_bytes(chunk, C)
        for form in (osr.BWD_AUTO, osr.BWD_WALK):
            assert osr.lattice_osr_bwd_workspace_bytes(osr.make_desc(**kw, bwd_form=form), C) > 0


def test_bwd_small_chunk_form_workspace():
    """The small-chunk reverse walk (automatic form, C in {2, 4, 8}, either
    linearisation, at most 2 slot rows per thread of the token loop, C within
    its exchange batch) adds every token's h (fp32 [B*H][T][d]) to the
    workspace for the decoding objective, and, where the rows of a sequence
    split over two workgroups, their hand-off buffers; nothing where the
    general walk runs."""
    def ws(C, form=osr.BWD_AUTO, **kw):
        return osr.lattice_osr_bwd_workspace_bytes(osr.make_desc(**kw, bwd_form=form), C)

    applies = [(2, 16, 16), (4, 64, 64), (8, 64, 64), (4, 32, 128), (8, 128, 16), (2, 128, 32), (1, 64, 64)]
    for C, m, d in applies:
        kw = dict(B=2, T=64, H=3, m=m, d=d)
        # from m = 32 and C = 4 the rows of a sequence split over P workgroups (B*H*P <= 256):
        # 4 at C = 8 where each keeps 16 rows and the threads to stage a chunk (m = d = 64
        # here; not m128 d16, where a quarter of the rows has 128 threads for 256 staged
        # units), else 2; their hand-off buffers, 2 parities x P parts x 8 tokens x (d + 4)
        # (value, tag) pairs
        P = 1 if m < 32 or C < 4 else (4 if (C, m, d) == (8, 64, 64) else 2)
        xchg = 2 * 3 * (2 * P * 8 * (d + 4) * 8) if P > 1 else 0
        one = dict(kw, chain_wgs=osr.WGS_ONE)
        assert ws(C, **kw) - ws(C, osr.BWD_WALK, **kw) == 2 * 3 * 64 * d * 4 + xchg, (C, m, d)
        assert ws(C, **one) - ws(C, osr.BWD_WALK, **one) == 2 * 3 * 64 * d * 4, (C, m, d)
        for mode in (osr.MODE_SIM, osr.MODE_ENC):
            assert ws(C, mode=mode, **kw) - ws(C, osr.BWD_WALK, mode=mode, **kw) == xchg, (C, m, d, mode)
            assert ws(C, mode=mode, **one) == ws(C, osr.BWD_WALK, mode=mode, **one), (C, m, d, mode)
    # no split once B*H*2 exceeds 256 compute units
    big = dict(B=8, T=64, H=17, m=64, d=64)
    assert ws(4, **big) - ws(4, osr.BWD_WALK, **big) == 8 * 17 * 64 * 64 * 4
    # m d = 8192 (C <= 4) and m = d = 128 (C = 2): only with the rows over 2 or 4 workgroups, which
    # B*H*P <= 256 must allow; WGS_ONE then gives the fewest, not one
    for C, m, d, pmin in ((4, 64, 128, 2), (2, 128, 64, 2), (4, 128, 64, 2), (2, 128, 128, 4)):
        kw = dict(B=2, T=64, H=3, m=m, d=d)
        xchg = 2 * 3 * (2 * pmin * 8 * (d + 4) * 8)
        for wgs in (osr.WGS_AUTO, osr.WGS_ONE):
            assert ws(C, chain_wgs=wgs, **kw) - ws(C, osr.BWD_WALK, chain_wgs=wgs, **kw) == \
                2 * 3 * 64 * d * 4 + xchg, (C, m, d, wgs)
        many = dict(B=8, T=64, H=129 // pmin, m=m, d=d)  # B*H*pmin > 256: the general walk
        assert ws(C, **many) == ws(C, osr.BWD_WALK, **many), (C, m, d)
    # C = 16 with bf16 inputs (not the encoding layer): after the state-passing kernel, which
    # supplies h, on at least 2 workgroups (one slot row per thread) with parts of 16 tokens
    # (m64 d64: two workgroups, the fewest with one row per thread; m32 d32 and m64 d16: one,
    # as two would lack the threads to stage a chunk of 16 tokens)
    for m, d, P in ((64, 64, 2), (32, 32, 1), (64, 16, 1)):
        kw = dict(B=2, T=64, H=3, m=m, d=d)
        xchg = 2 * 3 * (2 * P * 16 * (d + 4) * 8) if P > 1 else 0
        assert ws(16, **kw) - ws(16, osr.BWD_WALK, chain_wgs=osr.WGS_ONE, **kw) == xchg, (m, d)
    for kw16 in (dict(in_dtype=osr.F32), dict(mode=osr.MODE_ENC)):
        kw = dict(B=2, T=64, H=3, m=64, d=64, **kw16)
        assert ws(16, **kw) == ws(16, osr.BWD_WALK, **kw), kw16
    # the first linearisation takes the same form below C = 16 (not at 16)
    for C in (2, 4, 8):
        kw = dict(B=2, T=64, H=3, m=64, d=64)
        assert ws(C, linearisation=osr.LIN1, **kw) == ws(C, **kw), C
    general = [dict(C=8, m=64, d=128), dict(C=4, m=128, d=128), dict(C=8, m=32, d=128), dict(C=32, m=64, d=64),
               dict(C=16, m=64, d=64, linearisation=osr.LIN1)]
    for g in general:
        kw = dict(B=2, T=64, H=3)
        kw.update(g)
        C = kw.pop("C")
        assert ws(C, **kw) == ws(C, osr.BWD_WALK, **kw), g


def _fwd_save_call(d, chunk, ptrs=None, saved=None, saved_bytes=None):
    lib = osr.load_library()
    if saved_bytes is None:
        need = lib.lattice_osr_bwd_workspace_bytes(ctypes.byref(d), chunk)
        saved_bytes = need if need != ctypes.c_size_t(-1).value else 0
    if saved is None:
        saved = BASE + 8 * (1 << 32)
    return lib.lattice_osr_fwd_chunked_save(ctypes.byref(d), chunk, *(ptrs or _ptrs(d)), saved, saved_bytes, None)


def _bwd_saved_call(d, ptrs, chunk, ws=None, ws_bytes=None):
    lib = osr.load_library()
    if ws_bytes is None:
        need = lib.lattice_osr_bwd_workspace_bytes(ctypes.byref(d), chunk)
        ws_bytes = need if need != ctypes.c_size_t(-1).value else 0
    if ws is None:
        ws = BASE + 14 * (1 << 32)
    return lib.lattice_osr_bwd_chunked_saved(ctypes.byref(d), chunk, *ptrs, ws, ws_bytes, None)


def test_saved_training_pair_rules():
    """lattice_osr_fwd_chunked_save and lattice_osr_bwd_chunked_saved exist only
    where the backward takes its small-chunk form at C in 1, 2, 4, 8 (BWD_AUTO, C
    within the token loop's batch, at most 2 slot rows per thread on 1, 2 or 4
    workgroups; either linearisation): UNSUPPORTED elsewhere; null pointers, a
    short saved buffer and misalignment are refused before anything runs."""
    ok = dict(B=1, T=64, H=2, m=64, d=64)
    for C, kw in ((16, {}), (16, dict(linearisation=osr.LIN1)), (4, dict(bwd_form=osr.BWD_WALK)),
                  (4, dict(m=128, d=128)), (8, dict(m=32, d=128))):
        d = osr.make_desc(**dict(ok, **{k: v for k, v in kw.items() if k in ("m", "d")}),
                          **{k: v for k, v in kw.items() if k not in ("m", "d")})
        assert _fwd_save_call(d, C) == osr.ERR_UNSUPPORTED, (C, kw)
        assert _bwd_saved_call(d, _bwd_ptrs(), C) == osr.ERR_UNSUPPORTED, (C, kw)
    d = osr.make_desc(**ok)
    for i in range(8):
        p = _ptrs(d)
        p[i] = None
        assert _fwd_save_call(d, 4, ptrs=p) == osr.ERR_NULL, i
    lib = osr.load_library()
    assert lib.lattice_osr_fwd_chunked_save(ctypes.byref(d), 4, *_ptrs(d), None, 1 << 20, None) == osr.ERR_NULL
    need = lib.lattice_osr_bwd_workspace_bytes(ctypes.byref(d), 4)
    assert _fwd_save_call(d, 4, saved_bytes=need - 1) == osr.ERR_WORKSPACE
    assert _fwd_save_call(d, 4, saved=BASE + 8 * (1 << 32) + 4) == osr.ERR_ALIGN
    assert _fwd_save_call(d, 3) == osr.ERR_SHAPE
    for i in range(14):
        p = _bwd_ptrs()
        p[i] = None
        assert _bwd_saved_call(d, p, 4) == osr.ERR_NULL, i
    assert _bwd_saved_call(d, _bwd_ptrs(), 4, ws_bytes=need - 1) == osr.ERR_WORKSPACE
    # the saved buffer is an output of the forward: it may overlap no argument
    assert _fwd_save_call(d, 4, saved=_ptrs(d)[7]) == osr.ERR_ALIAS


def test_bwd_workspace_too_small():
    d = osr.make_desc(2, 64, 2, 32, 32)
    need = osr.lattice_osr_bwd_workspace_bytes(d, 16)
    assert _bwd_call(d, _bwd_ptrs(), 16, ws_bytes=need - 1) == osr.ERR_WORKSPACE


def test_bwd_aliasing_rules():
    d = osr.make_desc(1, 8, 1, 16, 16, in_dtype=osr.F32)
    for out in range(8, 14):
        for other in list(range(0, 8)) + [o for o in range(8, 14) if o != out]:
            p = _bwd_ptrs()
            p[out] = p[other]
            assert _bwd_call(d, p, 4) == osr.ERR_ALIAS, (out, other)
    # workspace overlapping an input or an output
    for other in (0, 5, 9, 13):
        assert _bwd_call(d, _bwd_ptrs(), 4, ws=_bwd_ptrs()[other]) == osr.ERR_ALIAS, other


def test_bwd_alignment_rules():
    d = osr.make_desc(1, 8, 1, 16, 16, in_dtype=osr.F32)
    sixteen = [0, 1, 2, 3, 5, 6, 7, 10, 13]     # vector-accessed buffers
    for i in sixteen:
        p = _bwd_ptrs()
        p[i] += 8
        assert _bwd_call(d, p, 4) == osr.ERR_ALIGN, i
    for i in (8, 9, 11, 12):                    # scalar fp32 outputs
        p = _bwd_ptrs()
        p[i] += 2
        assert _bwd_call(d, p, 4) == osr.ERR_ALIGN, i
    assert _bwd_call(d, _bwd_ptrs(), 4, ws=BASE + 14 * (1 << 32) + 8) == osr.ERR_ALIGN


# ------------------------------------------------------------ layer glue --
# lattice_osr_glue_pre pointers: xq, xk, gamma_logit, conv_wq, conv_wk, conv_bq, conv_bk,
# hist_q_in, hist_k_in, q, k, gamma, hist_q_out, hist_k_out
def _glue_ptrs(gap=1 << 32):
    return [BASE + i * gap for i in range(14)]


def _glue_pre(d, ptrs):
    return osr.load_library().lattice_osr_glue_pre(ctypes.byref(d) if d is not None else None, *ptrs, None)


def test_glue_pre_null_pointers():
    d = osr.make_desc(1, 8, 2, 16, 16)
    assert _glue_pre(None, _glue_ptrs()) == osr.ERR_NULL
    for i in (0, 1, 2, 3, 4, 9, 10, 11):
        p = _glue_ptrs()
        p[i] = None
        assert _glue_pre(d, p) == osr.ERR_NULL, i
    # the histories come in pairs; an unpaired one is a null-pointer error
    for i in (7, 8, 12, 13):
        p = _glue_ptrs()
        p[i] = None
        assert _glue_pre(d, p) == osr.ERR_NULL, i


def test_glue_pre_alignment_and_descriptor():
    d = osr.make_desc(1, 8, 2, 16, 16)
    for i in (0, 1, 3, 4, 7, 8, 9, 10, 11, 12, 13):  # moved in 16-byte pieces
        q = _glue_ptrs()
        q[i] += 8
        assert _glue_pre(d, q) == osr.ERR_ALIGN, i
    for i in (5, 6):  # biases: 4-byte alignment
        q = _glue_ptrs()
        q[i] += 2
        assert _glue_pre(d, q) == osr.ERR_ALIGN, i
    # per-slot gamma moves in 16-byte pieces; per-token gamma element by element
    q = _glue_ptrs()
    q[2] += 8
    assert _glue_pre(d, q) == osr.ERR_ALIGN
    dt = osr.make_desc(1, 8, 2, 16, 16, gamma_per_slot=0)
    q = _glue_ptrs()
    q[2] += 1
    assert _glue_pre(dt, q) == osr.ERR_ALIGN
    assert _glue_pre(osr.make_desc(1, 8, 2, 24, 16), _glue_ptrs()) == osr.ERR_UNSUPPORTED
    assert _glue_pre(osr.make_desc(1, 0, 2, 16, 16), _glue_ptrs()) == osr.ERR_SHAPE
    assert _glue_pre(osr.make_desc(1, 8, 2, 16, 16, in_dtype=7), _glue_ptrs()) == osr.ERR_UNSUPPORTED


def test_glue_pre_aliasing_rules():
    d = osr.make_desc(1, 8, 2, 16, 16)
    for out in (9, 10, 11, 12, 13):
        for other in [o for o in range(14) if o != out]:
            p = _glue_ptrs()
            p[out] = p[other]
            assert _glue_pre(d, p) == osr.ERR_ALIAS, (out, other)


def test_glue_post_argument_checks():
    lib = osr.load_library()
    d = osr.make_desc(1, 8, 2, 16, 16)
    y, g, o = BASE, BASE + (1 << 32), BASE + (2 << 32)
    assert lib.lattice_osr_glue_post(None, y, g, o, None) == osr.ERR_NULL
    for args in ((None, g, o), (y, None, o), (y, g, None)):
        assert lib.lattice_osr_glue_post(ctypes.byref(d), *args, None) == osr.ERR_NULL
    for args in ((y + 8, g, o), (y, g + 8, o), (y, g, o + 8)):
        assert lib.lattice_osr_glue_post(ctypes.byref(d), *args, None) == osr.ERR_ALIGN
    assert lib.lattice_osr_glue_post(ctypes.byref(d), y, g, g, None) == osr.ERR_ALIAS
    assert lib.lattice_osr_glue_post(ctypes.byref(d), y, g, y + 16, None) == osr.ERR_ALIAS
    assert lib.lattice_osr_glue_post(ctypes.byref(osr.make_desc(1, 8, 2, 16, 20)), y, g, o, None) == \
        osr.ERR_UNSUPPORTED
