"""The Python binding's layout checks, on the CPU with meta tensors (shapes
and strides only, no memory, no launch).

The library derives every conv offset from the channel count it computes from
the head sizes (C = 2 H_k d_k + H_v d_v), so the binding must refuse tensors
whose shapes disagree with those sizes before it hands their pointers over:
otherwise a wrong H_k would address conv windows, weights and x rows past the
ends of the tensors.
"""
import pytest
import torch

import gated_deltanet_recurrent_decode_amd as gdn


def meta(*shape, dtype=torch.float32):
    return torch.empty(shape, dtype=dtype, device="meta")


def step_tensors(B=3, T=1, H_k=2, H_v=4, d_k=64, d_v=64, N=9, W=4, C=None):
    C = 2 * H_k * d_k + H_v * d_v if C is None else C
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    return dict(x=meta(B, T, C, dtype=bf), conv_w=meta(C, W, dtype=bf), conv_b=None,
                conv_state=meta(N, W - 1, C, dtype=bf), state=meta(N, H_v, d_k, d_v), g=meta(B, T, H_v),
                beta=meta(B, T, H_v), read_slot=meta(B, dtype=i32), write_slot=meta(B, dtype=i32),
                out=meta(B, T, H_v, d_v, dtype=bf))


def call_step(H_k=2, **kw):
    t = step_tensors(**kw)
    return gdn._step_layout(t["x"], t["conv_w"], t["conv_b"], t["conv_state"], t["state"], t["g"], t["beta"],
                            t["read_slot"], t["write_slot"], t["out"], H_k)


def test_step_layout_accepts_consistent_shapes():
    d, xs = call_step()
    assert (d.B, d.T, d.H_k, d.H_v, d.d_k, d.d_v, d.W, d.N) == (3, 1, 2, 4, 64, 64, 4, 9)
    assert xs == 2 * 2 * 64 + 4 * 64


def test_step_layout_refuses_head_counts_that_disagree_with_the_channels():
    with pytest.raises(ValueError, match="channels"):
        call_step(H_k=4)            # tensors built for H_k = 2: a larger H_k would address past them
    with pytest.raises(ValueError, match="channels"):
        call_step(H_k=1)
    with pytest.raises(ValueError, match="multiple"):
        call_step(H_k=3)            # H_v = 4 is not a multiple of 3
    with pytest.raises(ValueError, match="multiple"):
        call_step(H_k=0)


def test_step_layout_refuses_a_row_strided_x_with_too_many_heads():
    # a row-strided x (rows 2C apart) still has C channels: H_k = 4 would need more
    t = step_tensors()
    C = t["x"].shape[2]
    x = meta(3 * 2 * C, dtype=torch.bfloat16).as_strided((3, 1, C), (2 * C, C, 1))
    with pytest.raises(ValueError, match="channels"):
        gdn._step_layout(x, t["conv_w"], None, t["conv_state"], t["state"], t["g"], t["beta"], t["read_slot"],
                         t["write_slot"], t["out"], 4)
    d, xs = gdn._step_layout(x, t["conv_w"], None, t["conv_state"], t["state"], t["g"], t["beta"],
                             t["read_slot"], t["write_slot"], t["out"], 2)
    assert xs == 2 * C


def test_step_layout_refuses_mismatched_arrays():
    t = step_tensors()
    bad = dict(t)
    bad["conv_b"] = meta(7, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="conv_b"):
        gdn._step_layout(**{k: bad[k] for k in ("x", "conv_w", "conv_b", "conv_state", "state", "g", "beta",
                                                 "read_slot", "write_slot", "out")}, H_k=2)
    for name, shape, dt in (("write_slot", (2,), torch.int32), ("g", (3, 1, 3), torch.float32),
                            ("conv_state", (9, 3, 100), torch.bfloat16), ("out", (3, 1, 4, 32), torch.bfloat16)):
        bad = dict(t)
        bad[name] = meta(*shape, dtype=dt)
        with pytest.raises(ValueError):
            gdn._step_layout(**{k: bad[k] for k in ("x", "conv_w", "conv_b", "conv_state", "state", "g", "beta",
                                                     "read_slot", "write_slot", "out")}, H_k=2)


def prefill_tensors(B=2, T=40, H_k=2, H_v=2, d=64, N=5, C=None):
    C = 2 * H_k * d + H_v * d if C is None else C
    bf, i32 = torch.bfloat16, torch.int32
    return (meta(T, C, dtype=bf), meta(C, 4, dtype=bf), None, meta(N, 3, C, dtype=bf), meta(N, H_v, d, d),
            meta(T, H_v), meta(T, H_v), meta(B + 1, dtype=i32), meta(B, dtype=i32), meta(T, H_v, d, dtype=bf))


def test_prefill_layout_checks_channels_and_bias():
    a = prefill_tensors()
    d, xs = gdn._prefill_layout(*a, 2)
    assert (d.B, d.T, d.H_k, d.H_v) == (2, 40, 2, 2) and xs == 2 * 2 * 64 + 2 * 64
    with pytest.raises(ValueError, match="channels"):
        gdn._prefill_layout(*a, 1)
    with pytest.raises(ValueError, match="multiple"):
        gdn._prefill_layout(*prefill_tensors(H_v=3, C=2 * 2 * 64 + 3 * 64), 2)
    b = list(a)
    b[2] = meta(5, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="conv_b"):
        gdn._prefill_layout(*b, 2)


def test_pool_layout_checks_channels():
    state = meta(9, 4, 64, 64)
    cs = meta(9, 3, 2 * 2 * 64 + 4 * 64, dtype=torch.bfloat16)
    d = gdn._pool_layout(state, cs, 2)
    assert (d.H_k, d.H_v, d.W, d.N) == (2, 4, 4, 9)
    with pytest.raises(ValueError, match="channels"):
        gdn._pool_layout(state, cs, 4)   # would write (W-1) * C_wrong values past each window
    with pytest.raises(ValueError, match="multiple"):
        gdn._pool_layout(state, cs, 3)
    with pytest.raises(ValueError, match="same slots"):
        gdn._pool_layout(meta(8, 4, 64, 64), cs, 2)


def test_conv_layout_checks_weights_bias_and_write_slots():
    bf, i32 = torch.bfloat16, torch.int32
    B, C, N = 5, 96, 7
    x, out = meta(B, C, dtype=bf), meta(B, C, dtype=bf)
    cs, w = meta(N, 3, C, dtype=bf), meta(C, 4, dtype=bf)
    rd, wr = meta(B, dtype=i32), meta(B, dtype=i32)
    assert gdn._conv_layout(x, w, None, cs, rd, wr, out) == (B, C, 4, N)
    assert gdn._conv_layout(x, w, meta(C, dtype=bf), cs, rd, None, out) == (B, C, 4, N)
    with pytest.raises(ValueError, match="conv_w"):
        gdn._conv_layout(x, meta(C, 3, dtype=bf), None, cs, rd, wr, out)
    with pytest.raises(ValueError, match="conv_w"):
        gdn._conv_layout(x, meta(C - 4, 4, dtype=bf), None, cs, rd, wr, out)
    with pytest.raises(ValueError, match="conv_b"):
        gdn._conv_layout(x, w, meta(C - 1, dtype=bf), cs, rd, wr, out)
    with pytest.raises(ValueError, match="write_slot"):
        gdn._conv_layout(x, w, None, cs, rd, meta(B - 1, dtype=i32), out)
    with pytest.raises(ValueError):
        gdn._conv_layout(meta(B, C - 2, dtype=bf), w, None, cs, rd, wr, out)
