"""Plain fp64 CPU oracle for the Gated DeltaNet decode step (ctypes binding).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``gated_deltanet_recurrent_decode_amd``; both
sides only read the seeded arrays drawn by ``gdn_inputs``.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64 loops); this module
builds it with gcc, loads it and converts numpy arrays to pointers.  See the C
file's header for the sources on the mstar pages and for the readings taken
where they are silent.

Parity unpinned (nothing on the pages fixes these constants; oracle and kernel
follow the same written reading): the L2-norm epsilon, the q scale, the q|k|v
channel order, the value-head -> key-head grouping and the conv tap order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so with gcc (IEEE fp64, no contraction)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
           "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # GDN_ORACLE_LIB lets the mutation test load a copy of the oracle with a planted mistake.
    path = os.environ.get("GDN_ORACLE_LIB", _LIB)
    if path == _LIB and not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_silu.restype = dbl
    lib.oracle_silu.argtypes = [dbl]
    lib.oracle_l2norm.restype = None
    lib.oracle_l2norm.argtypes = [i32, P, dbl, dbl, P]
    lib.oracle_conv_token.restype = None
    lib.oracle_conv_token.argtypes = [i32, i32, P, P, P, P, i32, P]
    lib.oracle_conv_decode.restype = i32
    lib.oracle_conv_decode.argtypes = [i32, i32, i32, i32, P, i64, P, P, P, P, P, i32, P]
    lib.oracle_delta_rule.restype = None
    lib.oracle_delta_rule.argtypes = [i32, i32, P, P, P, P, dbl, dbl, P]
    lib.oracle_gdn_decode_step.restype = i32
    lib.oracle_gdn_decode_step.argtypes = [i32] * 8 + [P, i64, P, P, P, P, P, P, P, P, P, dbl, dbl]
    lib.oracle_slot_commit.restype = None
    lib.oracle_slot_commit.argtypes = [P, P, i32]
    lib.oracle_gdn_decode_step_tokens.restype = i32
    lib.oracle_gdn_decode_step_tokens.argtypes = [i32] * 8 + [P, i64, P, P, P, P, P, P, P, P, P, dbl, dbl]
    lib.oracle_slot_reset.restype = None
    lib.oracle_slot_reset.argtypes = [i32] * 6 + [P, P, P, i32]
    lib.oracle_slot_copy.restype = None
    lib.oracle_slot_copy.argtypes = [i32] * 6 + [P, P, P, P, i32]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if a is None:
        return None
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name}: expected a C-contiguous numpy array of {np.dtype(dtype)}")
    return a


# ---------------------------------------------------------------- pieces

def silu(y: float) -> float:
    """SiLU of one fp64 value."""
    return float(_load().oracle_silu(float(y)))


def l2norm(x: np.ndarray, eps: float, scale: float = 1.0) -> np.ndarray:
    """x / sqrt(sum x^2 + eps) * scale over a 1-D fp64 vector."""
    x = _check(np.ascontiguousarray(x, np.float64), np.float64, "x")
    out = np.empty_like(x)
    _load().oracle_l2norm(x.size, _ptr(x), float(eps), float(scale), _ptr(out))
    return out


def conv_token(conv_w: np.ndarray, conv_b, win: np.ndarray, x_t: np.ndarray, act: bool) -> np.ndarray:
    """One conv-decode token of one row.  ``win`` ([W-1][C] fp64) is shifted in place.

    conv_w [C][W] and conv_b [C] / x_t [C] are bf16 bit patterns (uint16)."""
    C, W = conv_w.shape
    _check(conv_w, np.uint16, "conv_w")
    _check(conv_b, np.uint16, "conv_b")
    _check(win, np.float64, "win")
    _check(x_t, np.uint16, "x_t")
    assert win.shape == (W - 1, C) and x_t.shape == (C,)
    y = np.empty(C, np.float64)
    _load().oracle_conv_token(C, W, _ptr(conv_w), _ptr(conv_b), _ptr(win), _ptr(x_t), int(act), _ptr(y))
    return y


def conv_decode(x, conv_w, conv_b, conv_state, read_slot, write_slot, act: bool) -> np.ndarray:
    """Pooled conv decode over B rows; updates ``conv_state`` ([N][W-1][C] uint16) in place.

    x is [B][C] uint16 (or [B][>=C] with the row stride taken from its shape).
    Returns y [B][C] fp64."""
    B = read_slot.shape[0]
    N, Wm1, C = conv_state.shape
    _check(x, np.uint16, "x")
    _check(conv_w, np.uint16, "conv_w")
    _check(conv_b, np.uint16, "conv_b")
    _check(conv_state, np.uint16, "conv_state")
    _check(read_slot, np.int32, "read_slot")
    _check(write_slot, np.int32, "write_slot")
    out = np.empty((B, C), np.float64)
    rc = _load().oracle_conv_decode(B, C, Wm1 + 1, N, _ptr(x), x.shape[-1], _ptr(conv_w), _ptr(conv_b),
                                    _ptr(conv_state), _ptr(read_slot), _ptr(write_slot), int(act), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_conv_decode: invalid slot or non-bf16 window value")
    return out


def delta_rule(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: float, beta: float) -> np.ndarray:
    """Gated delta rule on one head and token; ``S`` ([d_k][d_v] fp64) is updated in place.

    q and k must already be normalised.  Returns o [d_v] fp64."""
    dk, dv = S.shape
    _check(S, np.float64, "S")
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    assert q.shape == (dk,) and k.shape == (dk,) and v.shape == (dv,)
    o = np.empty(dv, np.float64)
    _load().oracle_delta_rule(dk, dv, _ptr(S), _ptr(q), _ptr(k), _ptr(v), float(g), float(beta), _ptr(o))
    return o


def gdn_decode_step(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, write_slot,
                    *, H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6) -> np.ndarray:
    """The whole pooled decode step.  ``state`` and ``conv_state`` are updated in place.

    x [B][T][C] uint16 (row stride = T*C), conv_w [C][W] uint16, conv_b [C] uint16 or None,
    conv_state [N][W-1][C] uint16, state [N][H_v][d_k][d_v] fp32, g/beta [B][T][H_v] fp32,
    read_slot/write_slot [B] int32 (write_slot None => in place).
    Returns out [B][T][H_v][d_v] fp64 (unrounded)."""
    B, T, C = x.shape
    N, H_v, d_k, d_v = state.shape
    W = conv_state.shape[1] + 1
    for a, dt, n in ((x, np.uint16, "x"), (conv_w, np.uint16, "conv_w"), (conv_state, np.uint16, "conv_state"),
                     (state, np.float32, "state"), (g, np.float32, "g"), (beta, np.float32, "beta"),
                     (read_slot, np.int32, "read_slot")):
        _check(a, dt, n)
    _check(conv_b, np.uint16, "conv_b")
    _check(write_slot, np.int32, "write_slot")
    assert C == 2 * H_k * d_k + H_v * d_v, "channel count does not match the heads"
    assert g.shape == (B, T, H_v) and beta.shape == (B, T, H_v)
    out = np.empty((B, T, H_v, d_v), np.float64)
    rc = _load().oracle_gdn_decode_step(B, T, H_k, H_v, d_k, d_v, W, N, _ptr(x), T * C, _ptr(conv_w),
                                        _ptr(conv_b), _ptr(conv_state), _ptr(state), _ptr(g), _ptr(beta),
                                        _ptr(read_slot), _ptr(write_slot), _ptr(out), float(q_scale),
                                        float(l2_eps))
    if rc != 0:
        raise ValueError("oracle_gdn_decode_step: invalid slot, shape or window value")
    return out


def slot_commit(read_slot: np.ndarray, write_slot: np.ndarray) -> None:
    """Swap each row's read and write slot in place."""
    _check(read_slot, np.int32, "read_slot")
    _check(write_slot, np.int32, "write_slot")
    assert read_slot.shape == write_slot.shape
    _load().oracle_slot_commit(_ptr(read_slot), _ptr(write_slot), read_slot.shape[0])


def _pool_dims(state, conv_state):
    N, H_v, d_k, d_v = state.shape
    N2, Wm1, C = conv_state.shape
    assert N2 == N
    return H_v, d_k, d_v, Wm1 + 1, C, N


def slot_reset(state: np.ndarray, conv_state: np.ndarray, slots: np.ndarray) -> None:
    """Zero the state and conv window of every listed slot (slot 0 and out-of-range slots skipped)."""
    _check(state, np.float32, "state")
    _check(conv_state, np.uint16, "conv_state")
    _check(slots, np.int32, "slots")
    _load().oracle_slot_reset(*_pool_dims(state, conv_state), _ptr(state), _ptr(conv_state), _ptr(slots), slots.size)


def slot_copy(state: np.ndarray, conv_state: np.ndarray, src: np.ndarray, dst: np.ndarray) -> None:
    """Copy slot src[i] (state and conv window) to slot dst[i]; dst 0 and out-of-range pairs skipped."""
    _check(state, np.float32, "state")
    _check(conv_state, np.uint16, "conv_state")
    _check(src, np.int32, "src")
    _check(dst, np.int32, "dst")
    assert src.shape == dst.shape
    _load().oracle_slot_copy(*_pool_dims(state, conv_state), _ptr(state), _ptr(conv_state), _ptr(src), _ptr(dst),
                             src.size)


def gdn_decode_step_tokens(x, conv_w, conv_b, conv_state, state, g, beta, read_slot, token_slots,
                           *, H_k: int, q_scale: float = 1.0, l2_eps: float = 1e-6) -> np.ndarray:
    """T tokens a row from the read slot; after token t the state and window go to
    token_slots[r][t] (0: not kept).  Returns out [B][T][H_v][d_v] fp64."""
    B, T, C = x.shape
    N, H_v, d_k, d_v = state.shape
    W = conv_state.shape[1] + 1
    for a, dt, n in ((x, np.uint16, "x"), (conv_w, np.uint16, "conv_w"), (conv_state, np.uint16, "conv_state"),
                     (state, np.float32, "state"), (g, np.float32, "g"), (beta, np.float32, "beta"),
                     (read_slot, np.int32, "read_slot"), (token_slots, np.int32, "token_slots")):
        _check(a, dt, n)
    _check(conv_b, np.uint16, "conv_b")
    assert token_slots.shape == (B, T)
    out = np.empty((B, T, H_v, d_v), np.float64)
    rc = _load().oracle_gdn_decode_step_tokens(B, T, H_k, H_v, d_k, d_v, W, N, _ptr(x), T * C, _ptr(conv_w),
                                               _ptr(conv_b), _ptr(conv_state), _ptr(state), _ptr(g), _ptr(beta),
                                               _ptr(read_slot), _ptr(token_slots), _ptr(out), float(q_scale),
                                               float(l2_eps))
    if rc != 0:
        raise ValueError("oracle_gdn_decode_step_tokens: invalid slot or shape")
    return out
