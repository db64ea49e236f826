"""GPU: the allocation-free prefill (gdn_prefill_two_pass_noalloc, through the
C ABI) against the two-pass prefill with a caller workspace, bit for bit, on
two calls in a row, the second with a smaller input (the static scratch keeps
the first call's contents; they must not matter).  Both start from copies of
the same pool, and each call's outputs, final states and windows are compared
element by element; the first call is also checked against the oracle.
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


def _call(gdn, t, case, dp, noalloc):
    s = case.shape
    out = t.full((s.T, s.H_v, s.d_v), 7.0, dtype=t.bfloat16, device="cuda")  # any unwritten row shows
    args = (H.bf16_dev(case.x), dp.conv_w, None, dp.conv_state, dp.state, t.from_numpy(case.g).cuda(),
            t.from_numpy(case.beta).cuda(), t.from_numpy(case.cu_seqlens).cuda(), dp.rd, out)
    if noalloc:
        gdn.gdn_prefill_two_pass_noalloc(*args, H_k=s.H_k)
    else:
        nbytes = gdn.gdn_prefill_two_pass_workspace_bytes(s.B, s.T, s.H_k, s.H_v, s.d_k, s.d_v)
        ws = t.full((nbytes,), 0xFF, dtype=t.uint8, device="cuda")
        gdn.gdn_prefill_two_pass(*args, ws, H_k=s.H_k)
    return out


def test_noalloc_prefill_matches_the_workspace_prefill_on_two_calls(gdn, torch):
    t = torch
    # first call: 1800 tokens over three prompts at the 0.8B-like heads (the
    # workspace then fills most of the 64 MiB scratch); second: two short prompts
    big = gi.prefill([1000, 700, 100], H_k=16, H_v=16, d=128, N=9, seed=3)
    small = gi.prefill([40, 9], H_k=16, H_v=16, d=128, N=9, seed=4)
    need = gdn.gdn_prefill_two_pass_workspace_bytes(3, 1800, 16, 16, 128, 128)
    assert gdn.NOALLOC_SCRATCH_BYTES // 2 < need <= gdn.NOALLOC_SCRATCH_BYTES
    for k, case in enumerate((big, small)):
        s, pool = case.shape, case.pool
        dp_n, dp_w = H.DevPool(pool), H.DevPool(pool)
        out_n = _call(gdn, t, case, dp_n, noalloc=True)
        out_w = _call(gdn, t, case, dp_w, noalloc=False)
        t.cuda.synchronize()
        assert t.equal(out_n.view(t.int16), out_w.view(t.int16)), f"call {k}: outputs differ"
        assert t.equal(dp_n.state.view(t.int32), dp_w.state.view(t.int32)), f"call {k}: states differ"
        assert t.equal(dp_n.conv_state.view(t.int16), dp_w.conv_state.view(t.int16)), f"call {k}: windows differ"
        if k == 0:
            hp = H.HostPool(pool)
            ref = np.zeros((s.T, s.H_v, s.d_v), np.float64)
            for b in range(s.B):
                a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
                o = oracle.gdn_decode_step(np.ascontiguousarray(case.x[None, a:e]), hp.conv_w, None, hp.conv_state,
                                           hp.state, np.ascontiguousarray(case.g[None, a:e]),
                                           np.ascontiguousarray(case.beta[None, a:e]),
                                           np.array([pool.read_slot[b]], np.int32), None, H_k=s.H_k)
                ref[a:e] = o[0]
            H.assert_out_close(out_n, ref, "noalloc out")
            slots = [int(x) for x in pool.read_slot]
            H.assert_state_close(dp_n.state[slots].cpu().numpy(), hp.state[slots], "noalloc state")


def test_noalloc_prefill_refuses_more_than_its_scratch(gdn, torch):
    t = torch
    case = gi.prefill([2100], H_k=16, H_v=16, d=128, N=3, seed=5)
    s = case.shape
    assert gdn.gdn_prefill_two_pass_workspace_bytes(1, 2100, 16, 16, 128, 128) > gdn.NOALLOC_SCRATCH_BYTES
    dp = H.DevPool(case.pool)
    before = dp.state.clone()
    with pytest.raises(gdn.GdnError) as e:
        _call(gdn, t, case, dp, noalloc=True)
    assert e.value.status == 6
    t.cuda.synchronize()
    assert t.equal(dp.state.view(t.int32), before.view(t.int32))
