"""Shared helpers for the GPU parity tests: moving the seeded host arrays to the
GPU, running the HIP path through the binding and the oracle on the same
inputs, and the tolerances of the comparison.

Tolerances (written here once, used by every parity test):
  fp32 state   |gpu - oracle| <= 1e-5 + 1e-5 * |oracle|  (oracle rounded to fp32 at storage)
  bf16 output  |gpu - oracle| <= 2e-2                      (oracle unrounded fp64)
  slots, conv windows, untouched pool memory: bit-exact
"""
from __future__ import annotations

import numpy as np

import gdn_inputs as gi

STATE_ABS = 1e-5
STATE_REL = 1e-5
OUT_ABS = 2e-2


def torch():
    import torch as _t
    return _t


def bf16_dev(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(t.bfloat16)


def bf16_host(t) -> np.ndarray:
    tt = torch()
    return t.contiguous().view(tt.int16).cpu().numpy().view(np.uint16)


def bf16_host_f64(t) -> np.ndarray:
    return gi.bf16_to_f32(bf16_host(t)).astype(np.float64)


class DevPool:
    """One pool on the GPU."""

    def __init__(self, pool: gi.Pool):
        t = torch()
        self.state = t.from_numpy(pool.state).cuda()
        self.conv_state = bf16_dev(pool.conv_state)
        self.conv_w = bf16_dev(pool.conv_w)
        self.rd = t.from_numpy(pool.read_slot).cuda()
        self.wr = t.from_numpy(pool.write_slot).cuda()


class HostPool:
    """A mutable host copy of one pool for the oracle."""

    def __init__(self, pool: gi.Pool):
        self.state = pool.state.copy()
        self.conv_state = pool.conv_state.copy()
        self.conv_w = pool.conv_w
        self.rd = pool.read_slot.copy()
        self.wr = pool.write_slot.copy()


def gpu_step(gdn, dp: DevPool, step: gi.StepInputs, shape: gi.Shape, *, twin=True, q_scale=1.0, l2_eps=1e-6,
             conv_b=None):
    t = torch()
    B, T = step.x.shape[0], step.x.shape[1]
    out = t.empty((B, T, shape.H_v, shape.d_v), dtype=t.bfloat16, device="cuda")
    gdn.gdn_decode_step(bf16_dev(step.x), dp.conv_w, conv_b, dp.conv_state, dp.state,
                        t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda(), dp.rd,
                        dp.wr if twin else None, out, H_k=shape.H_k, q_scale=q_scale, l2_eps=l2_eps)
    return out


def oracle_step(oracle, hp: HostPool, step: gi.StepInputs, shape: gi.Shape, *, twin=True, q_scale=1.0,
                l2_eps=1e-6, rows=None):
    x, g, beta, rd, wr = step.x, step.g, step.beta, hp.rd, hp.wr
    if rows is not None:
        x, g, beta = (np.ascontiguousarray(a[rows]) for a in (x, g, beta))
        rd, wr = np.ascontiguousarray(rd[rows]), np.ascontiguousarray(wr[rows])
    return oracle.gdn_decode_step(x, hp.conv_w, None, hp.conv_state, hp.state, g, beta, rd,
                                  wr if twin else None, H_k=shape.H_k, q_scale=q_scale, l2_eps=l2_eps)


def assert_state_close(got: np.ndarray, ref: np.ndarray, what: str = "state"):
    got = got.astype(np.float64)
    ref = ref.astype(np.float64)
    assert got.shape == ref.shape
    bad = ~(np.abs(got - ref) <= STATE_ABS + STATE_REL * np.abs(ref))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} elements out of tolerance; first at {tuple(i)}: "
                             f"gpu {got[tuple(i)]!r} oracle {ref[tuple(i)]!r}")


def assert_out_close(got_bf16, ref: np.ndarray, what: str = "out"):
    got = bf16_host_f64(got_bf16)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref)
    bad = ~(err <= OUT_ABS)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} out of tolerance (max err {np.nanmax(err):.3g}); "
                             f"first at {tuple(i)}: gpu {got[tuple(i)]!r} oracle {ref[tuple(i)]!r}")
