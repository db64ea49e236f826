"""Python binding of libgdn.so, the MI355X (gfx950) Gated DeltaNet decode step.

Argument marshalling only: every function here checks dtypes, devices and
layouts of torch tensors, turns them into device pointers and calls the C ABI
declared in ``include/gdn.h`` on the current torch stream (or the stream
given).  All arithmetic runs in the HIP kernels.  There is no fallback: if
libgdn.so is missing or a call fails, this raises.

Build the library with ``python -m gated_deltanet_recurrent_decode_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["GdnError", "lib", "gdn_decode_step", "gdn_decode_step_commit", "gdn_decode_step_tokens", "gdn_prefill",
           "gdn_prefill_two_pass", "gdn_prefill_two_pass_workspace_bytes", "gdn_prefill_two_pass_noalloc",
           "NOALLOC_SCRATCH_BYTES", "conv_decode",
           "slot_commit",
           "slot_reset", "slot_copy", "check_slots", "traffic_probe", "status_string", "LIB_PATH", "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")
EXPORTS = ("gdn_decode_step", "gdn_decode_step_commit", "gdn_decode_step_tokens", "gdn_prefill",
           "gdn_prefill_two_pass", "gdn_prefill_two_pass_workspace_bytes", "gdn_prefill_two_pass_noalloc",
           "conv_decode",
           "slot_commit", "gdn_check_slots",
           "gdn_slot_reset",
           "gdn_slot_copy", "gdn_status_string", "gdn_traffic_probe")

GDN_OK = 0
NOALLOC_SCRATCH_BYTES = 64 << 20  # GDN_NOALLOC_SCRATCH_BYTES in include/gdn.h


class GdnError(RuntimeError):
    """A non-OK status from libgdn."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status}: {status_string(status)}")


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("B", "T", "H_k", "H_v", "d_k", "d_v", "W", "N")]


class Probe(ctypes.Structure):
    """gdn_probe: a calibration design (see gdn_traffic_probe in include/gdn.h)."""
    _fields_ = [(n, ctypes.c_int32) for n in ("traffic", "layout", "shape", "hold_ns", "order", "threads", "loads",
                                               "persistent", "policy")]


# gdn_probe fields, by name
PROBE_TRAFFIC = {"read": 0, "write": 1, "copy": 2, "inplace": 3}
PROBE_SHAPES = {"tile1": 0, "tile2": 1, "tile4": 2, "chunk": 3, "empty": 4, "slot_load": 5}
PROBE_ORDERS = {"stream": 0, "lane": 1, "workgroup": 2}
PROBE_POLICIES = {"nt": 0, "plain": 1, "sc0sc1": 2}


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdn.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run: python -m gated_deltanet_recurrent_decode_amd.build")
    try:
        # load torch's HIP runtime first, so libgdn binds to the same runtime
        # instance that owns the caller's streams and memory
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.gdn_decode_step.restype = i32
    L.gdn_decode_step.argtypes = [ctypes.POINTER(Dims), P, i64, P, P, P, P, P, P, P, P, P, f32, f32, P]
    L.gdn_decode_step_commit.restype = i32
    L.gdn_decode_step_commit.argtypes = [ctypes.POINTER(Dims), P, i64, P, P, P, P, P, P, P, P, P, P, P, f32, f32, P]
    L.gdn_decode_step_tokens.restype = i32
    L.gdn_decode_step_tokens.argtypes = [ctypes.POINTER(Dims), P, i64, P, P, P, P, P, P, P, P, P, f32, f32, P]
    L.gdn_prefill.restype = i32
    L.gdn_prefill.argtypes = [ctypes.POINTER(Dims), P, i64, P, P, P, P, P, P, P, P, P, f32, f32, P]
    L.gdn_prefill_two_pass.restype = i32
    L.gdn_prefill_two_pass.argtypes = [ctypes.POINTER(Dims), P, i64, P, P, P, P, P, P, P, P, P, f32, f32, P,
                                       ctypes.c_size_t, P]
    L.gdn_prefill_two_pass_noalloc.restype = i32
    L.gdn_prefill_two_pass_noalloc.argtypes = [ctypes.POINTER(Dims), P, i64, P, P, P, P, P, P, P, P, P, f32, f32, P]
    L.gdn_prefill_two_pass_workspace_bytes.restype = ctypes.c_size_t
    L.gdn_prefill_two_pass_workspace_bytes.argtypes = [ctypes.POINTER(Dims)]
    L.conv_decode.restype = i32
    L.conv_decode.argtypes = [i32, i32, i32, i32, P, i64, P, P, P, P, P, P, i64, i32, P]
    L.slot_commit.restype = i32
    L.slot_commit.argtypes = [P, P, i32, P]
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_status_string.argtypes = [i32]
    L.gdn_check_slots.restype = i32
    L.gdn_check_slots.argtypes = [ctypes.POINTER(Dims), P, P, P, P]
    L.gdn_slot_reset.restype = i32
    L.gdn_slot_reset.argtypes = [ctypes.POINTER(Dims), P, P, P, i32, P]
    L.gdn_slot_copy.restype = i32
    L.gdn_slot_copy.argtypes = [ctypes.POINTER(Dims), P, P, P, P, i32, P]
    L.gdn_traffic_probe.restype = i32
    L.gdn_traffic_probe.argtypes = [ctypes.POINTER(Probe), i32, i32, i32, i32, i32, P, P, P, P, P]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != GDN_OK:
        raise GdnError(fn, status)


# ------------------------------------------------------------------ marshalling helpers

def _torch():
    import torch
    return torch


def _dev(t, name, dtype, *, allow_none=False):
    torch = _torch()
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: expected dtype {dtype}, got {t.dtype}")
    return t


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device(*tensors):
    """The one GPU every given tensor lives on (None entries skipped)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(str(d) for d in devs)}")
    return devs.pop()


def _stream(stream, device):
    """The stream to launch on: the given one, which must belong to the tensors'
    GPU, or that GPU's current torch stream."""
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    if s.device != device:
        raise ValueError(f"stream is on {s.device}, the tensors on {device}")
    return ctypes.c_void_p(s.cuda_stream)


class _on:
    """Make the tensors' GPU the current HIP device for the call (a no-op when it already is)."""

    def __init__(self, device):
        self.device, self.prev = device, None

    def __enter__(self):
        torch = _torch()
        cur = torch.cuda.current_device()
        if cur != self.device.index:
            self.prev = cur
            torch.cuda.set_device(self.device)
        return self

    def __exit__(self, *exc):
        if self.prev is not None:
            _torch().cuda.set_device(self.prev)
        return False


# ------------------------------------------------------------------ entry points

def _channels(H_k, H_v, d_k, d_v):
    """The conv's channel count for these heads (q and k of every key head, v of
    every value head); the library derives every conv offset from it."""
    if H_k < 1 or H_v < 1 or H_v % H_k != 0:
        raise ValueError(f"H_v ({H_v}) must be a positive multiple of H_k ({H_k})")
    return 2 * H_k * d_k + H_v * d_v


def _step_layout(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out, H_k):
    """Shape and stride checks of a decode step (any device, meta tensors too);
    returns the Dims and x's row stride."""
    if x.dim() != 3 or x.stride(2) != 1 or x.stride(1) != x.shape[2]:
        raise ValueError("x: expected [B][T][C] with contiguous tokens and channels")
    if state.dim() != 4 or conv_state.dim() != 3 or conv_w.dim() != 2:
        raise ValueError("state must be [N][H_v][d_k][d_v], conv_state [N][W-1][C], conv_w [C][W]")
    B, T, C = x.shape
    N, H_v, d_k, d_v = state.shape
    W = conv_w.shape[1]
    if C != _channels(H_k, H_v, d_k, d_v):
        raise ValueError(f"x has {C} channels; H_k={H_k}, H_v={H_v}, d_k={d_k}, d_v={d_v} need 2*H_k*d_k + H_v*d_v")
    if tuple(conv_state.shape) != (N, W - 1, C) or conv_w.shape[0] != C:
        raise ValueError("conv_state / conv_w do not match x and state")
    if tuple(g.shape) != (B, T, H_v) or tuple(beta.shape) != (B, T, H_v) or tuple(out.shape) != (B, T, H_v, d_v):
        raise ValueError("g, beta, out do not match [B][T][H_v](, d_v)")
    if tuple(read_slot.shape) != (B,) or (write_slot is not None and tuple(write_slot.shape) != (B,)):
        raise ValueError("slot arrays must be [B]")
    if conv_b is not None and tuple(conv_b.shape) != (C,):
        raise ValueError("conv_b must be [C]")
    d = Dims(B, T, H_k, H_v, d_k, d_v, W, N)
    x_row_stride = x.stride(0) if B > 0 else T * C
    return d, x_row_stride


def _step_args(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out, H_k):
    torch = _torch()
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _dev(x, "x", bf)
    for t, n, dt in ((conv_w, "conv_w", bf), (conv_state, "conv_state", bf), (state, "state", f32),
                     (g, "g", f32), (beta, "beta", f32), (read_slot, "read_slot", i32), (out, "out", bf)):
        _contig(_dev(t, n, dt), n)
    _contig(_dev(conv_b, "conv_b", bf, allow_none=True), "conv_b")
    _contig(_dev(write_slot, "write_slot", i32, allow_none=True), "write_slot")
    return _step_layout(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out, H_k)


def gdn_decode_step(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out, *,
                    H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6, stream=None) -> None:
    """One fused decode step (see ``gdn_decode_step`` in include/gdn.h).

    x [B][T][C] bf16 (rows may be strided; the inner two dims contiguous),
    conv_w [C][4] bf16, conv_b [C] bf16 or None, conv_state [N][3][C] bf16,
    state [N][H_v][d_k][d_v] fp32, g/beta [B][T][H_v] fp32, read_slot/write_slot
    [B] int32 (write_slot None => in place), out [B][T][H_v][d_v] bf16."""
    d, xs = _step_args(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out, H_k)
    dev = _device(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out)
    with _on(dev):
        _check("gdn_decode_step", lib().gdn_decode_step(
            ctypes.byref(d), _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(state),
            _ptr(g), _ptr(beta), _ptr(read_slot), _ptr(write_slot), _ptr(out), float(q_scale), float(l2_eps),
            _stream(stream, dev)))


def gdn_decode_step_commit(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, next_read_slot,
                           next_write_slot, out, *, H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6,
                           stream=None) -> None:
    """A twin-slot decode step with the commit folded in (see ``gdn_decode_step_commit``
    in include/gdn.h): also writes next_read_slot = write_slot, next_write_slot = read_slot."""
    torch = _torch()
    if write_slot is None:
        raise ValueError("gdn_decode_step_commit writes twin slots: write_slot is required")
    for t, n in ((next_read_slot, "next_read_slot"), (next_write_slot, "next_write_slot")):
        _contig(_dev(t, n, torch.int32), n)
        if t.shape != read_slot.shape:
            raise ValueError(f"{n} must be [B]")
    d, xs = _step_args(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, out, H_k)
    dev = _device(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot, next_read_slot,
                  next_write_slot, out)
    with _on(dev):
        _check("gdn_decode_step_commit", lib().gdn_decode_step_commit(
            ctypes.byref(d), _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(state),
            _ptr(g), _ptr(beta), _ptr(read_slot), _ptr(write_slot), _ptr(next_read_slot), _ptr(next_write_slot),
            _ptr(out), float(q_scale), float(l2_eps), _stream(stream, dev)))


def gdn_decode_step_tokens(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, token_slots, out, *,
                           H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6, stream=None) -> None:
    """T tokens a row from the read slot, the state after token t kept in slot
    token_slots[r][t] (0: not kept); the read slot is not written (see
    ``gdn_decode_step_tokens`` in include/gdn.h).  token_slots is [B][T] int32."""
    torch = _torch()
    _contig(_dev(token_slots, "token_slots", torch.int32), "token_slots")
    if token_slots.shape != x.shape[:2]:
        raise ValueError("token_slots must be [B][T]")
    d, xs = _step_args(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, None, out, H_k)
    dev = _device(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, token_slots, out)
    with _on(dev):
        _check("gdn_decode_step_tokens", lib().gdn_decode_step_tokens(
            ctypes.byref(d), _ptr(x), xs, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state), _ptr(state),
            _ptr(g), _ptr(beta), _ptr(read_slot), _ptr(token_slots), _ptr(out), float(q_scale), float(l2_eps),
            _stream(stream, dev)))


def _prefill_layout(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, H_k):
    """Shape and stride checks of a prefill call (any device, meta tensors too);
    returns the Dims and x's row stride."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x: expected [T][C] with contiguous channels")
    if state.dim() != 4 or conv_state.dim() != 3 or conv_w.dim() != 2:
        raise ValueError("state must be [N][H_v][d_k][d_v], conv_state [N][W-1][C], conv_w [C][W]")
    T, C = x.shape
    N, H_v, d_k, d_v = state.shape
    W = conv_w.shape[1]
    if C != _channels(H_k, H_v, d_k, d_v):
        raise ValueError(f"x has {C} channels; H_k={H_k}, H_v={H_v}, d_k={d_k}, d_v={d_v} need 2*H_k*d_k + H_v*d_v")
    if slot.dim() != 1:
        raise ValueError("slot must be [B]")
    B = slot.shape[0]
    if (tuple(cu_seqlens.shape) != (B + 1,) or tuple(g.shape) != (T, H_v) or tuple(beta.shape) != (T, H_v)
            or tuple(out.shape) != (T, H_v, d_v)):
        raise ValueError("cu_seqlens [B+1], g/beta [T][H_v], out [T][H_v][d_v] expected")
    if tuple(conv_state.shape) != (N, W - 1, C) or conv_w.shape[0] != C:
        raise ValueError("conv_state / conv_w do not match x and state")
    if conv_b is not None and tuple(conv_b.shape) != (C,):
        raise ValueError("conv_b must be [C]")
    return Dims(B, T, H_k, H_v, d_k, d_v, W, N), (x.stride(0) if T > 0 else C)


def _prefill_dims(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, H_k):
    torch = _torch()
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    _dev(x, "x", bf)
    for t, n, dt in ((conv_w, "conv_w", bf), (conv_state, "conv_state", bf), (state, "state", f32),
                     (g, "g", f32), (beta, "beta", f32), (cu_seqlens, "cu_seqlens", i32), (slot, "slot", i32),
                     (out, "out", bf)):
        _contig(_dev(t, n, dt), n)
    _contig(_dev(conv_b, "conv_b", bf, allow_none=True), "conv_b")
    return _prefill_layout(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, H_k)


def gdn_prefill(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, *, H_k: int,
                q_scale: float = 1.0, l2_eps: float = 1e-6, stream=None) -> None:
    """Chunked prefill of packed sequences, in place (see ``gdn_prefill`` in include/gdn.h).

    x [T][C] bf16 (rows may be strided), g/beta [T][H_v] fp32, cu_seqlens [B+1] int32,
    slot [B] int32, out [T][H_v][d_v] bf16; the pool tensors as for gdn_decode_step."""
    d, xs = _prefill_dims(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, H_k)
    dev = _device(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out)
    with _on(dev):
        _check("gdn_prefill", lib().gdn_prefill(
            ctypes.byref(d), _ptr(x), xs, _ptr(cu_seqlens), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
            _ptr(state), _ptr(g), _ptr(beta), _ptr(slot), _ptr(out), float(q_scale), float(l2_eps),
            _stream(stream, dev)))


def gdn_prefill_two_pass_workspace_bytes(B: int, T: int, H_k: int, H_v: int, d_k: int, d_v: int) -> int:
    """Workspace bytes gdn_prefill_two_pass needs (see include/gdn.h); 0 for unusable sizes."""
    d = Dims(B, T, H_k, H_v, d_k, d_v, 4, 1)
    return int(lib().gdn_prefill_two_pass_workspace_bytes(ctypes.byref(d)))


def gdn_prefill_two_pass(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, workspace, *,
                         H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6, stream=None) -> None:
    """gdn_prefill in two passes with a caller-owned workspace (a device uint8 tensor of at
    least gdn_prefill_two_pass_workspace_bytes bytes); see include/gdn.h."""
    torch = _torch()
    d, xs = _prefill_dims(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, H_k)
    _contig(_dev(workspace, "workspace", torch.uint8), "workspace")
    dev = _device(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, workspace)
    with _on(dev):
        _check("gdn_prefill_two_pass", lib().gdn_prefill_two_pass(
            ctypes.byref(d), _ptr(x), xs, _ptr(cu_seqlens), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
            _ptr(state), _ptr(g), _ptr(beta), _ptr(slot), _ptr(out), float(q_scale), float(l2_eps), _ptr(workspace),
            workspace.numel(), _stream(stream, dev)))


def gdn_prefill_two_pass_noalloc(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, *,
                                 H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6, stream=None) -> None:
    """gdn_prefill_two_pass with its scratch in the library's static device buffer
    (NOALLOC_SCRATCH_BYTES a GPU) instead of a caller workspace: nothing is
    allocated.  Calls that overlap on one GPU race; see include/gdn.h."""
    d, xs = _prefill_dims(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out, H_k)
    dev = _device(x, conv_w, conv_b, conv_state, state, g, beta, cu_seqlens, slot, out)
    with _on(dev):
        _check("gdn_prefill_two_pass_noalloc", lib().gdn_prefill_two_pass_noalloc(
            ctypes.byref(d), _ptr(x), xs, _ptr(cu_seqlens), _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
            _ptr(state), _ptr(g), _ptr(beta), _ptr(slot), _ptr(out), float(q_scale), float(l2_eps),
            _stream(stream, dev)))


def _conv_layout(x, conv_w, conv_b, conv_state, read_slot, write_slot, out):
    """Shape and stride checks of conv_decode (any device, meta tensors too);
    returns B, C, W, N."""
    if conv_state.dim() != 3 or conv_w.dim() != 2 or read_slot.dim() != 1:
        raise ValueError("conv_state must be [N][W-1][C], conv_w [C][W], read_slot [B]")
    N, Wm1, C = conv_state.shape
    W = Wm1 + 1
    B = read_slot.shape[0]
    if tuple(conv_w.shape) != (C, W):
        raise ValueError(f"conv_w must be [C][W] = [{C}][{W}] to match conv_state")
    if conv_b is not None and tuple(conv_b.shape) != (C,):
        raise ValueError("conv_b must be [C]")
    if write_slot is not None and tuple(write_slot.shape) != (B,):
        raise ValueError("write_slot must be [B] like read_slot")
    if x.dim() != 2 or out.dim() != 2 or x.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("x and out must be [B][C] with contiguous channels")
    if x.shape[0] != B or out.shape[0] != B or x.shape[1] < C or out.shape[1] < C:
        raise ValueError("x / out do not match [B][C]")
    return B, C, W, N


def conv_decode(x, conv_w, conv_b, conv_state, read_slot, write_slot, out, *, activation: bool = True,
                stream=None) -> None:
    """Pooled conv decode for one token a row (see ``conv_decode`` in include/gdn.h).

    x [B][>=C] bf16 (row-strided), conv_w [C][4], conv_b [C] or None, conv_state [N][3][C],
    read_slot/write_slot [B] int32 (write_slot None => in place), out [B][>=C] bf16 (row-strided)."""
    torch = _torch()
    bf, i32 = torch.bfloat16, torch.int32
    _dev(x, "x", bf)
    _dev(out, "out", bf)
    for t, n, dt in ((conv_w, "conv_w", bf), (conv_state, "conv_state", bf), (read_slot, "read_slot", i32)):
        _contig(_dev(t, n, dt), n)
    _contig(_dev(conv_b, "conv_b", bf, allow_none=True), "conv_b")
    _contig(_dev(write_slot, "write_slot", i32, allow_none=True), "write_slot")
    B, C, W, N = _conv_layout(x, conv_w, conv_b, conv_state, read_slot, write_slot, out)
    dev = _device(x, conv_w, conv_b, conv_state, read_slot, write_slot, out)
    with _on(dev):
        _check("conv_decode", lib().conv_decode(
            B, C, W, N, _ptr(x), x.stride(0) if B > 0 else C, _ptr(conv_w), _ptr(conv_b), _ptr(conv_state),
            _ptr(read_slot), _ptr(write_slot), _ptr(out), out.stride(0) if B > 0 else C, int(bool(activation)),
            _stream(stream, dev)))


def slot_commit(read_slot, write_slot, *, stream=None) -> None:
    """Swap each row's read and write slot on the device (see ``slot_commit`` in include/gdn.h)."""
    torch = _torch()
    _contig(_dev(read_slot, "read_slot", torch.int32), "read_slot")
    _contig(_dev(write_slot, "write_slot", torch.int32), "write_slot")
    if read_slot.shape != write_slot.shape or read_slot.dim() != 1:
        raise ValueError("slot arrays must both be [B]")
    dev = _device(read_slot, write_slot)
    with _on(dev):
        _check("slot_commit", lib().slot_commit(_ptr(read_slot), _ptr(write_slot), read_slot.shape[0],
                                                _stream(stream, dev)))


def check_slots(read_slot, write_slot=None, *, N: int, stream=None):
    """The device-side debug check of a step's slot preconditions (see
    ``gdn_check_slots`` in include/gdn.h): returns a new int32 tensor [2] on the
    slots' device, filled in stream order with the number of rows that break a
    precondition and the first of them (-1 if none)."""
    torch = _torch()
    _contig(_dev(read_slot, "read_slot", torch.int32), "read_slot")
    if read_slot.dim() != 1:
        raise ValueError("read_slot must be [B]")
    if write_slot is not None:
        _contig(_dev(write_slot, "write_slot", torch.int32), "write_slot")
        if write_slot.shape != read_slot.shape:
            raise ValueError("write_slot must match read_slot")
    dev = _device(read_slot, write_slot) if write_slot is not None else _device(read_slot)
    result = torch.full((2,), -2, dtype=torch.int32, device=dev)
    B = read_slot.shape[0]
    with _on(dev):
        _check("gdn_check_slots", lib().gdn_check_slots(ctypes.byref(Dims(B, 1, 1, 1, 64, 64, 4, N)), _ptr(read_slot),
                                                          _ptr(write_slot), _ptr(result), _stream(stream, dev)))
    return result


def _pool_layout(state, conv_state, H_k):
    """Shape checks of a slot operation (any device, meta tensors too); returns the Dims."""
    if state.dim() != 4 or conv_state.dim() != 3 or state.shape[0] != conv_state.shape[0]:
        raise ValueError("state must be [N][H_v][d_k][d_v] and conv_state [N][W-1][C] over the same slots")
    N, H_v, d_k, d_v = state.shape
    if conv_state.shape[2] != _channels(H_k, H_v, d_k, d_v):
        raise ValueError(f"conv_state has {conv_state.shape[2]} channels; H_k={H_k}, H_v={H_v}, d_k={d_k}, "
                         f"d_v={d_v} need 2*H_k*d_k + H_v*d_v")
    return Dims(0, 1, H_k, H_v, d_k, d_v, conv_state.shape[1] + 1, N)


def _pool_dims(state, conv_state, H_k):
    torch = _torch()
    _contig(_dev(state, "state", torch.float32), "state")
    _contig(_dev(conv_state, "conv_state", torch.bfloat16), "conv_state")
    return _pool_layout(state, conv_state, H_k)


def slot_reset(state, conv_state, slots, *, H_k: int, stream=None) -> None:
    """Zero the state and conv window of every listed slot (see ``gdn_slot_reset`` in include/gdn.h)."""
    torch = _torch()
    _contig(_dev(slots, "slots", torch.int32), "slots")
    d = _pool_dims(state, conv_state, H_k)
    dev = _device(state, conv_state, slots)
    with _on(dev):
        _check("gdn_slot_reset", lib().gdn_slot_reset(ctypes.byref(d), _ptr(state), _ptr(conv_state), _ptr(slots),
                                                      slots.numel(), _stream(stream, dev)))


def slot_copy(state, conv_state, src_slots, dst_slots, *, H_k: int, stream=None) -> None:
    """Copy slot src[i] to slot dst[i], state and conv window (see ``gdn_slot_copy`` in include/gdn.h)."""
    torch = _torch()
    _contig(_dev(src_slots, "src_slots", torch.int32), "src_slots")
    _contig(_dev(dst_slots, "dst_slots", torch.int32), "dst_slots")
    if src_slots.shape != dst_slots.shape or src_slots.dim() != 1:
        raise ValueError("src_slots and dst_slots must both be [n]")
    d = _pool_dims(state, conv_state, H_k)
    dev = _device(state, conv_state, src_slots, dst_slots)
    with _on(dev):
        _check("gdn_slot_copy", lib().gdn_slot_copy(ctypes.byref(d), _ptr(state), _ptr(conv_state), _ptr(src_slots),
                                                    _ptr(dst_slots), src_slots.numel(), _stream(stream, dev)))


def traffic_probe(state, read_slot, write_slot, sink, *, traffic: str = "copy", layout: str = "slots",
                  shape: str = "tile1", hold_ns: int = 0, order: str = "stream", threads: int = 256, loads: int = 8,
                  persistent: int = 0, policy: str = "nt", rows: int | None = None, stream=None) -> None:
    """The step's state traffic with no arithmetic in one workgroup design (see
    ``gdn_traffic_probe`` in include/gdn.h).

    traffic: "read", "write", "copy" (read slot -> write slot) or "inplace";
    layout: "slots" (row r's tiles at read_slot[r] / write_slot[r]) or
    "contiguous" (`rows` consecutive slots from read_slot[0] to write_slot[0]);
    shape: one of PROBE_SHAPES; order: one of PROBE_ORDERS (when stores may
    go); policy: one of PROBE_POLICIES; threads, loads and persistent set the
    "chunk" shape; rows defaults to the length of read_slot."""
    torch = _torch()
    _contig(_dev(state, "state", torch.float32), "state")
    _contig(_dev(read_slot, "read_slot", torch.int32), "read_slot")
    _contig(_dev(write_slot, "write_slot", torch.int32, allow_none=True), "write_slot")
    _contig(_dev(sink, "sink", torch.float32), "sink")
    if (traffic not in PROBE_TRAFFIC or layout not in ("slots", "contiguous") or shape not in PROBE_SHAPES
            or order not in PROBE_ORDERS or policy not in PROBE_POLICIES):
        raise ValueError(f"unknown probe design {traffic!r}, {layout!r}, {shape!r}, {order!r}, {policy!r}")
    if state.dim() != 4 or read_slot.dim() != 1:
        raise ValueError("state must be [N][H][d_k][d_v] and read_slot [B]")
    N, H, d_k, d_v = state.shape
    n = read_slot.shape[0] if rows is None else int(rows)
    writes = traffic in ("write", "copy")
    if writes and write_slot is None:
        raise ValueError("write and copy traffic need write_slot")
    if layout == "slots" and (n > read_slot.shape[0] or (writes and write_slot.shape[0] < n)):
        raise ValueError("the slot arrays must hold an entry for every row")
    if layout == "contiguous" and (read_slot.shape[0] < 1 or (writes and write_slot.shape[0] < 1)):
        raise ValueError("the contiguous layout takes its first slots from read_slot[0] and write_slot[0]")
    pr = Probe(PROBE_TRAFFIC[traffic], 0 if layout == "slots" else 1, PROBE_SHAPES[shape], int(hold_ns),
               PROBE_ORDERS[order], int(threads), int(loads), int(persistent), PROBE_POLICIES[policy])
    dev = _device(state, read_slot, write_slot, sink)
    with _on(dev):
        _check("gdn_traffic_probe", lib().gdn_traffic_probe(
            ctypes.byref(pr), n, H, d_k, d_v, N, _ptr(state), _ptr(read_slot), _ptr(write_slot), _ptr(sink),
            _stream(stream, dev)))
