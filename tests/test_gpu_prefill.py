"""GPU parity of the chunked prefill (gdn_prefill, through the C ABI) against the
fp64 oracle.  A prompt's prefill is, by definition, the in-place decode step run
over its tokens in order, so the oracle for each sequence is
oracle.gdn_decode_step in place with T = that sequence's length.  The kernel's
chunked arithmetic differs from the token-by-token order only by rounding, so
the state and read-out bars are those of the decode step (tests/helpers.py).
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_recurrent_decode_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _oracle_prefill(case, hp, conv_b=None, q_scale=1.0):
    """Each sequence through the oracle's in-place step with T = its length."""
    s = case.shape
    out = np.zeros((s.T, s.H_v, s.d_v), np.float64)
    for b in range(s.B):
        a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        if e == a:
            continue
        o = oracle.gdn_decode_step(np.ascontiguousarray(case.x[None, a:e]), hp.conv_w, conv_b, hp.conv_state, hp.state,
                                   np.ascontiguousarray(case.g[None, a:e]), np.ascontiguousarray(case.beta[None, a:e]),
                                   np.array([case.pool.read_slot[b]], np.int32), None, H_k=s.H_k, q_scale=q_scale)
        out[a:e] = o[0]
    return out


def _run(gdn, t, case, dp, conv_b=None, q_scale=1.0, cu=None):
    s = case.shape
    out = t.full((s.T, s.H_v, s.d_v), 7.0, dtype=t.bfloat16, device="cuda")  # any unwritten row shows
    cu_dev = t.from_numpy(case.cu_seqlens if cu is None else cu).cuda()
    gdn.gdn_prefill(H.bf16_dev(case.x), dp.conv_w, conv_b, dp.conv_state, dp.state, t.from_numpy(case.g).cuda(),
                    t.from_numpy(case.beta).cuda(), cu_dev, dp.rd, out, H_k=s.H_k, q_scale=q_scale)
    return out


def _check(gdn, t, case, conv_b=None, q_scale=1.0):
    s, pool = case.shape, case.pool
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    before_state, before_conv = dp.state.clone(), dp.conv_state.clone()
    bias_dev = None if conv_b is None else H.bf16_dev(conv_b)
    out = _run(gdn, t, case, dp, conv_b=bias_dev, q_scale=q_scale)
    ref = _oracle_prefill(case, hp, conv_b=conv_b, q_scale=q_scale)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    lens = np.diff(case.cu_seqlens)
    written = sorted(int(pool.read_slot[b]) for b in range(s.B) if pool.read_slot[b] != 0 and lens[b] > 0)
    if written:
        idx = t.tensor(written, dtype=t.int64, device="cuda")
        H.assert_state_close(dp.state[idx].cpu().numpy(), hp.state[written])
        np.testing.assert_array_equal(H.bf16_host(dp.conv_state[idx]), hp.conv_state[written])
    mask = t.ones(s.N, dtype=t.bool, device="cuda")
    if written:
        mask[t.tensor(written, dtype=t.int64, device="cuda")] = False
    assert t.equal(dp.state[mask].view(t.int32), before_state[mask].view(t.int32)), "a slot outside the prompts changed"
    assert t.equal(dp.conv_state[mask].view(t.int16), before_conv[mask].view(t.int16))
    return dp, out


CASES = [
    # lengths, H_k, H_v, d, d_v, padding sequences
    ((1, 5, 32, 33, 70, 0, 100, 7), 2, 4, 128, 128, (7,)),   # chunk edges, an empty and a padding sequence, G = 2
    ((64, 3, 200), 2, 2, 64, 64, ()),                        # d = 64
    ((40, 17), 1, 4, 128, 64, ()),                           # G = 4, d_k != d_v
    ((31, 65, 2), 2, 2, 64, 128, (1,)),                      # d_k < d_v, a long padding sequence
]


@pytest.mark.parametrize("lengths,hk,hv,d,dv,pad", CASES,
                         ids=[f"{len(c[0])}seq-{c[1]}x{c[2]}-d{c[3]}x{c[4]}" for c in CASES])
def test_prefill_matches_oracle(gdn, torch, lengths, hk, hv, d, dv, pad):
    case = gi.prefill(list(lengths), H_k=hk, H_v=hv, d=d, d_v=dv, pad=pad, seed=len(lengths) + d)
    _, out = _check(gdn, torch, case)
    for b in pad:
        a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        assert torch.count_nonzero(out[a:e].view(torch.int16)) == 0, "padding sequences read out +0.0"


def test_prefill_bias_and_q_scale(gdn, torch):
    case = gi.prefill([45, 12], H_k=2, H_v=2, d=128, seed=11)
    bias = gi.bf16_bits(np.random.Generator(np.random.PCG64(4)).standard_normal(case.shape.C).astype(np.float32))
    _check(gdn, torch, case, conv_b=bias, q_scale=128 ** -0.5)


def test_prefill_08b_shapes(gdn, torch):
    """The 0.8B-like layer's shapes: 16+16 heads of 128, 6144 channels."""
    case = gi.prefill([300, 45, 1], H_k=16, H_v=16, d=128, seed=2)
    _check(gdn, torch, case)


def test_prefill_in_two_calls_equals_one(gdn, torch):
    """A prompt prefilled in two calls (the first 40 tokens, then the other 30)
    leaves the slot where one 70-token prefill does, within rounding, and the
    windows bit for bit (the conv window carries exactly the last inputs)."""
    t = torch
    case = gi.prefill([70], H_k=2, H_v=2, d=64, seed=5)
    dp1, dp2 = H.DevPool(case.pool), H.DevPool(case.pool)
    _run(gdn, t, case, dp1)
    for a, e in ((0, 40), (40, 70)):
        sub = gi.PrefillCase(gi.Shape(B=1, T=e - a, H_k=2, H_v=2, d_k=64, d_v=64, W=4, N=case.shape.N), case.pool,
                             np.ascontiguousarray(case.x[a:e]), np.ascontiguousarray(case.g[a:e]),
                             np.ascontiguousarray(case.beta[a:e]), np.array([0, e - a], np.int32))
        _run(gdn, t, sub, dp2)
    t.cuda.synchronize()
    sl = int(case.pool.read_slot[0])
    H.assert_state_close(dp2.state[sl].cpu().numpy(), dp1.state[sl].cpu().numpy().astype(np.float64), "split prefill")
    assert t.equal(dp1.conv_state[sl].view(t.int16), dp2.conv_state[sl].view(t.int16))


def test_prefill_unusable_ranges_touch_nothing(gdn, torch):
    t = torch
    case = gi.prefill([10, 20, 5], H_k=1, H_v=1, d=64, seed=8)
    dp = H.DevPool(case.pool)
    before = dp.state.clone()
    bad = np.array([0, 10, 5, 99], np.int32)   # sequence 1 runs backwards, sequence 2 past T
    out = _run(gdn, t, case, dp, cu=bad)
    t.cuda.synchronize()
    for b in (1, 2):
        sl = int(case.pool.read_slot[b])
        assert t.equal(dp.state[sl].view(t.int32), before[sl].view(t.int32))
    assert bool((out[10:].float() == 7.0).all()), "rows of unusable sequences stay as they were"
