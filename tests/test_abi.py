"""The C ABI of libgdn.so on the CPU: it loads, exports every function that
include/gdn.h declares, and its host-side validation refuses bad arguments with
the documented status before anything is launched (no GPU needed: every call
here fails validation, so no kernel is enqueued).
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_recurrent_decode_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, NULL, SHAPE, UNSUPPORTED, REFUSED, HIP, SCRATCH = range(7)
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(gdn.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = gdn.lib()
    for name in _declared():
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in nm.stdout.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name


def test_status_strings():
    for s in range(7):
        assert gdn.status_string(s)
    assert gdn.status_string(0) == "ok"
    assert "unknown" in gdn.status_string(99)


def _dims(**kw):
    base = dict(B=4, T=1, H_k=4, H_v=4, d_k=64, d_v=64, W=4, N=9)
    base.update(kw)
    return gdn.Dims(*[base[k] for k in ("B", "T", "H_k", "H_v", "d_k", "d_v", "W", "N")])


def _step(d, *, x=FAKE, stride=None, conv_w=FAKE, state=FAKE, out=FAKE, write_slot=FAKE, eps=1e-6, qs=1.0,
          dims_ptr=True):
    C = 2 * d.H_k * d.d_k + d.H_v * d.d_v
    st = d.T * C if stride is None else stride
    return gdn.lib().gdn_decode_step(ctypes.byref(d) if dims_ptr else None, x, st, conv_w, None, FAKE, state,
                                     FAKE, FAKE, FAKE, write_slot, out, qs, eps, None)


def test_step_validation():
    assert _step(_dims(), dims_ptr=False) == NULL
    assert _step(_dims(), x=None) == NULL
    assert _step(_dims(), out=None) == NULL
    assert _step(_dims(B=-1)) == SHAPE
    assert _step(_dims(T=0)) == SHAPE
    assert _step(_dims(H_k=3, H_v=4)) == SHAPE
    assert _step(_dims(N=0)) == SHAPE
    assert _step(_dims(d_k=96)) == UNSUPPORTED
    assert _step(_dims(d_v=256)) == UNSUPPORTED
    assert _step(_dims(W=3)) == UNSUPPORTED
    d = _dims()
    assert _step(d, stride=2 * 4 * 64 + 4 * 64 - 1) == SHAPE
    assert _step(_dims(), eps=-1.0) == SHAPE
    assert _step(_dims(), qs=float("nan")) == SHAPE
    # twin writes take one token a row; multi-token walks stay in place
    assert _step(_dims(T=4)) == REFUSED
    # in place needs H_v / H_k in {1, 2, 4}
    assert _step(_dims(H_k=1, H_v=8), write_slot=None) == UNSUPPORTED
    # alignment
    assert _step(_dims(), state=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    assert _step(_dims(), out=ctypes.c_void_p(0x10002)) == UNSUPPORTED
    assert _step(_dims(), conv_w=ctypes.c_void_p(0x10004)) == UNSUPPORTED
    # a row's x (with eight tokens of overrun), out and gates stay under 2 GiB:
    # C = 2*16*128 + 16*128 = 6144 channels, 2^31 / (2 C) = 174762.67 tokens,
    # so T + 8 <= 174762.  The largest legal T passes the size checks and is
    # stopped by the alignment check after them (nothing is launched).
    big = dict(H_k=16, H_v=16, d_k=128, d_v=128)
    assert _step(_dims(T=174755, **big), write_slot=None) == SHAPE
    assert _step(_dims(T=174754, **big), write_slot=None, state=ctypes.c_void_p(0x10008)) == UNSUPPORTED


def test_step_commit_validation():
    f = gdn.lib().gdn_decode_step_commit
    d = _dims()
    C = 2 * 4 * 64 + 4 * 64
    other = ctypes.c_void_p(0x20000)
    other2 = ctypes.c_void_p(0x30000)

    def call(rd=FAKE, wr=FAKE, nrd=other, nwr=other2):
        return f(ctypes.byref(d), FAKE, C, FAKE, None, FAKE, FAKE, FAKE, FAKE, rd, wr, nrd, nwr, FAKE, 1.0, 1e-6,
                 None)
    assert call(wr=None) == NULL
    assert call(nrd=None) == NULL
    assert call(nwr=None) == NULL
    assert call(rd=ctypes.c_void_p(0x40000), wr=ctypes.c_void_p(0x50000), nrd=ctypes.c_void_p(0x40000)) == SHAPE
    assert call(nrd=other, nwr=other) == SHAPE
    empty = gdn.Dims(0, 1, 4, 4, 64, 64, 4, 9)
    assert f(ctypes.byref(empty), None, 0, None, None, None, None, None, None, None, None, None, None, None, 1.0,
             1e-6, None) == OK


def test_step_tokens_validation():
    f = gdn.lib().gdn_decode_step_tokens

    def call(d, tok=FAKE, x=FAKE):
        C = 2 * d.H_k * d.d_k + d.H_v * d.d_v
        return f(ctypes.byref(d), x, d.T * C, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, tok, FAKE, 1.0, 1e-6, None)
    assert call(_dims(T=3), tok=None) == NULL
    assert call(_dims(T=3), x=None) == NULL
    assert call(_dims(T=0)) == SHAPE
    assert call(_dims(T=3, H_k=1, H_v=8)) == UNSUPPORTED       # in-place kernel: H_v / H_k in {1, 2, 4}
    assert call(_dims(T=3, d_k=96)) == UNSUPPORTED
    empty = gdn.Dims(0, 3, 4, 4, 64, 64, 4, 9)
    assert f(ctypes.byref(empty), None, 0, None, None, None, None, None, None, None, None, None, 1.0, 1e-6,
             None) == OK


def test_prefill_validation():
    f = gdn.lib().gdn_prefill

    def call(d, stride=None, x=FAKE, cu=FAKE, state=FAKE, cs=FAKE, eps=1e-6):
        C = 2 * d.H_k * d.d_k + d.H_v * d.d_v
        return f(ctypes.byref(d), x, C if stride is None else stride, cu, FAKE, None, cs, state, FAKE, FAKE, FAKE,
                 FAKE, 1.0, eps, None)
    assert f(None, FAKE, 0, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1e-6, None) == NULL
    assert call(_dims(T=40), cu=None) == NULL
    assert call(_dims(T=40), x=None) == NULL
    assert call(_dims(T=-1)) == SHAPE
    assert call(_dims(T=40, H_k=3, H_v=4)) == SHAPE
    assert call(_dims(T=40), stride=10) == SHAPE
    assert call(_dims(T=40), eps=-1.0) == SHAPE
    assert call(_dims(T=40, d_k=96)) == UNSUPPORTED
    assert call(_dims(T=40, W=3)) == UNSUPPORTED
    assert call(_dims(T=40), state=ctypes.c_void_p(0x10008)) == UNSUPPORTED
    assert call(_dims(T=40), cs=ctypes.c_void_p(0x10002)) == UNSUPPORTED
    assert call(_dims(T=40), stride=2 * 4 * 64 + 4 * 64 + 1) == UNSUPPORTED
    assert call(_dims(T=0)) == OK      # every sequence empty: nothing enqueued
    empty = gdn.Dims(0, 0, 4, 4, 64, 64, 4, 9)
    assert f(ctypes.byref(empty), None, 0, None, None, None, None, None, None, None, None, None, 1.0, 1e-6,
             None) == OK


def test_prefill_two_pass_validation():
    L = gdn.lib()
    f = L.gdn_prefill_two_pass
    d = _dims(T=40)
    need = L.gdn_prefill_two_pass_workspace_bytes(ctypes.byref(d))
    # per value head room for ceil(T / 32) + B chunks of (3 d_k + d_v + 32) * 32 + 1 floats, plus B + 1
    # ints and a 4-int record per chunk, each region rounded to 256 bytes
    nchunk = (d.T + 31) // 32 + d.B
    blocks = d.H_v * nchunk
    parts = [4 * (d.B + 1), 16 * nchunk, 4 * blocks * 32 * d.d_k, 4 * blocks * 32 * d.d_k, 4 * blocks * 32 * d.d_k,
             4 * blocks * 32 * 32, 4 * blocks * 32 * d.d_v, 4 * blocks]
    assert need == sum((x + 255) // 256 * 256 for x in parts)
    # from 256 prompt-head pairs (B H_v), with the last round of 256 at least three
    # quarters full, the slim layout: T' and P (32 x 32 floats each) and 128 floats
    # of row factors a chunk and value head, and each prompt's [3][C] bf16 window
    for B, T, H_k, H_v, dk, dv, slim in ((16, 8192, 16, 16, 128, 128, True), (16, 300, 8, 16, 128, 128, True),
                                         (8, 300, 8, 16, 128, 128, False),
                                         (16, 900, 16, 16, 64, 64, True), (7, 900, 16, 16, 128, 128, False),
                                         (15, 900, 16, 16, 64, 64, False), (1, 4096, 16, 16, 128, 128, False),
                                         (20, 900, 16, 16, 128, 128, False), (24, 900, 16, 16, 128, 128, True),
                                         (40, 900, 16, 16, 128, 128, True)):
        dd = gdn.Dims(B, T, H_k, H_v, dk, dv, 4, 9)
        nchunk = (T + 31) // 32 + B
        blocks = H_v * nchunk
        C = 2 * H_k * dk + H_v * dv
        if slim:
            parts = [4 * (B + 1), 16 * nchunk, 4 * blocks * 32 * 32, 4 * blocks * 128, 2 * B * 3 * C,
                     4 * blocks * 32 * 32]
        else:
            parts = [4 * (B + 1), 16 * nchunk, 4 * blocks * 32 * dk, 4 * blocks * 32 * dk, 4 * blocks * 32 * dk,
                     4 * blocks * 32 * dv, 4 * blocks, 4 * blocks * 32 * 32]
        assert L.gdn_prefill_two_pass_workspace_bytes(ctypes.byref(dd)) == sum((x + 255) // 256 * 256 for x in parts)
    assert L.gdn_prefill_two_pass_workspace_bytes(None) == 0
    assert L.gdn_prefill_two_pass_workspace_bytes(ctypes.byref(_dims(T=40, d_k=96))) == 0
    ws = ctypes.c_void_p(0x100000)

    def call(dd, workspace=ws, nbytes=need, cu=FAKE):
        C = 2 * dd.H_k * dd.d_k + dd.H_v * dd.d_v
        return f(ctypes.byref(dd), FAKE, C, cu, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1e-6,
                 workspace, nbytes, None)
    assert call(d, workspace=None) == NULL
    assert call(d, cu=None) == NULL
    assert call(d, workspace=ctypes.c_void_p(0x100080)) == UNSUPPORTED   # not 256-byte aligned
    assert call(d, nbytes=need - 1) == SHAPE
    assert call(_dims(T=40, H_k=3, H_v=4)) == SHAPE
    assert call(_dims(T=40, d_k=96)) == UNSUPPORTED
    assert call(_dims(T=0), workspace=None) == OK                        # nothing to do, no workspace needed
    empty = gdn.Dims(0, 0, 4, 4, 64, 64, 4, 9)
    assert f(ctypes.byref(empty), None, 0, None, None, None, None, None, None, None, None, None, 1.0, 1e-6, None, 0,
             None) == OK


def test_slot_ops_validation():
    L = gdn.lib()
    d = _dims()
    assert L.gdn_slot_reset(None, FAKE, FAKE, FAKE, 4, None) == NULL
    assert L.gdn_slot_reset(ctypes.byref(d), FAKE, FAKE, None, 4, None) == NULL
    assert L.gdn_slot_reset(ctypes.byref(d), FAKE, FAKE, FAKE, -1, None) == SHAPE
    assert L.gdn_slot_reset(ctypes.byref(d), FAKE, FAKE, FAKE, 70000, None) == SHAPE
    assert L.gdn_slot_reset(ctypes.byref(d), ctypes.c_void_p(0x10008), FAKE, FAKE, 4, None) == UNSUPPORTED
    assert L.gdn_slot_reset(ctypes.byref(d), None, None, None, 0, None) == OK
    assert L.gdn_slot_copy(ctypes.byref(d), FAKE, FAKE, None, FAKE, 4, None) == NULL
    assert L.gdn_slot_copy(ctypes.byref(d), FAKE, FAKE, FAKE, None, 4, None) == NULL
    assert L.gdn_slot_copy(ctypes.byref(_dims(H_k=3, H_v=4)), FAKE, FAKE, FAKE, FAKE, 4, None) == SHAPE


def test_conv_decode_validation():
    f = gdn.lib().conv_decode
    assert f(4, 16, 4, 9, None, 16, FAKE, None, FAKE, FAKE, None, FAKE, 16, 1, None) == NULL
    assert f(-1, 16, 4, 9, FAKE, 16, FAKE, None, FAKE, FAKE, None, FAKE, 16, 1, None) == SHAPE
    assert f(4, 16, 4, 9, FAKE, 15, FAKE, None, FAKE, FAKE, None, FAKE, 16, 1, None) == SHAPE
    assert f(4, 16, 4, 9, FAKE, 16, FAKE, None, FAKE, FAKE, None, FAKE, 15, 1, None) == SHAPE
    assert f(4, 16, 4, 9, FAKE, 16, FAKE, None, FAKE, FAKE, None, FAKE, 16, 2, None) == SHAPE
    assert f(4, 16, 3, 9, FAKE, 16, FAKE, None, FAKE, FAKE, None, FAKE, 16, 1, None) == UNSUPPORTED


def test_slot_commit_and_probe_validation():
    L = gdn.lib()
    assert L.slot_commit(None, FAKE, 4, None) == NULL
    assert L.slot_commit(FAKE, FAKE, -1, None) == SHAPE
    def pr(traffic=2, layout=0, shape=0, hold=0, order=0, threads=256, loads=8, persistent=0, policy=0):
        return ctypes.byref(gdn.Probe(traffic, layout, shape, hold, order, threads, loads, persistent, policy))
    assert L.gdn_traffic_probe(None, 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == NULL
    assert L.gdn_traffic_probe(pr(2), 4, 4, 64, 64, 9, FAKE, FAKE, None, FAKE, None) == NULL      # copy needs writes
    assert L.gdn_traffic_probe(pr(1), 4, 4, 64, 64, 9, FAKE, FAKE, None, FAKE, None) == NULL
    assert L.gdn_traffic_probe(pr(4), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE     # no such traffic
    assert L.gdn_traffic_probe(pr(layout=2), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(shape=6), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(order=3), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(policy=3), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(shape=3, persistent=9), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(shape=3, persistent=1, hold=100), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE,
                               None) == SHAPE  # holds are for one-shot grids
    assert L.gdn_traffic_probe(pr(shape=3, threads=384), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(shape=3, loads=2), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(shape=3, threads=512, loads=16), 4, 4, 128, 128, 9, FAKE, FAKE, FAKE, FAKE,
                               None) == SHAPE  # 128 KiB chunks: over 64 KiB
    assert L.gdn_traffic_probe(pr(hold=-1), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(hold=2000000), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE
    assert L.gdn_traffic_probe(pr(layout=1), 40000, 4, 128, 128, 9, FAKE, FAKE, FAKE, FAKE, None) == SHAPE  # > 2 GiB
    assert L.gdn_traffic_probe(pr(0), 4, 4, 96, 64, 9, FAKE, FAKE, None, FAKE, None) == UNSUPPORTED
    assert L.gdn_traffic_probe(pr(shape=1), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE, None) == UNSUPPORTED  # 128 only
    assert L.gdn_traffic_probe(pr(shape=3, loads=16), 4, 4, 64, 64, 9, FAKE, FAKE, FAKE, FAKE,
                               None) == UNSUPPORTED  # a 64 KiB chunk over a 16 KiB tile
    assert L.gdn_traffic_probe(pr(), 4, 4, 64, 64, 9, ctypes.c_void_p(0x10008), FAKE, FAKE, FAKE, None) == UNSUPPORTED


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdn, "_lib", None)
    with pytest.raises(ImportError):
        gdn.lib()


def test_prefill_noalloc_validation():
    """The allocation-free prefill refuses, before touching the GPU, a call
    whose workspace would not fit its static scratch, and validates like the
    two-pass prefill otherwise."""
    f = gdn.lib().gdn_prefill_two_pass_noalloc

    def call(d, x=FAKE):
        C = 2 * d.H_k * d.d_k + d.H_v * d.d_v
        return f(ctypes.byref(d), x, C, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 1e-6, None)
    big = gdn.Dims(1, 4096, 16, 16, 128, 128, 4, 9)
    need = gdn.gdn_prefill_two_pass_workspace_bytes(1, 4096, 16, 16, 128, 128)
    assert need > gdn.NOALLOC_SCRATCH_BYTES
    assert call(big) == SCRATCH
    assert call(gdn.Dims(1, 64, 16, 16, 128, 128, 4, 9), x=None) == NULL
    assert call(gdn.Dims(1, 64, 16, 16, 96, 128, 4, 9)) == UNSUPPORTED
    empty = gdn.Dims(0, 0, 16, 16, 128, 128, 4, 9)
    assert f(ctypes.byref(empty), None, 0, None, None, None, None, None, None, None, None, None, 1.0, 1e-6,
             None) == OK


def test_check_slots_validation():
    L = gdn.lib()
    f = L.gdn_check_slots
    d = gdn.Dims(8, 1, 1, 1, 64, 64, 4, 17)
    assert f(None, FAKE, None, FAKE, None) == NULL
    assert f(ctypes.byref(gdn.Dims(0, 1, 1, 1, 64, 64, 4, 17)), None, None, None, None) == OK  # nothing to check
    assert f(ctypes.byref(d), None, None, FAKE, None) == NULL
    assert f(ctypes.byref(d), FAKE, None, None, None) == NULL
    assert f(ctypes.byref(gdn.Dims(-1, 1, 1, 1, 64, 64, 4, 17)), FAKE, None, FAKE, None) == SHAPE
    assert f(ctypes.byref(gdn.Dims(8, 1, 1, 1, 64, 64, 4, 0)), FAKE, None, FAKE, None) == SHAPE
    odd = ctypes.c_void_p(0x100002)
    assert f(ctypes.byref(d), odd, None, FAKE, None) == UNSUPPORTED
    assert f(ctypes.byref(d), FAKE, odd, FAKE, None) == UNSUPPORTED
    assert f(ctypes.byref(d), FAKE, None, odd, None) == UNSUPPORTED
