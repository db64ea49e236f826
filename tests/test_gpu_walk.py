"""The in-place token walk (T tokens a row, all of a key head's value heads in
one workgroup, tokens in blocks of eight) against the single-token kernels, bit
for bit: a walk of T tokens gives the same outputs, states and conv windows as
T in-place steps of one token, and an in-place step with grouped value heads
the same as a twin-slot step (PR #1139, "Tests": twin and in place give the
same values; "What changed": split walks).  Every path sums in the same order,
so equality is exact, not within a tolerance; the oracle comparisons of the
same walks are in test_gpu_parity.py.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gdn():
    import gated_deltanet_recurrent_decode_amd as m
    m.lib()
    return m


def _bits_equal(a, b, what):
    t = H.torch()
    view = t.int16 if a.dtype == t.bfloat16 else t.int32
    assert t.equal(a.view(view), b.view(view)), f"{what} differs"


WALKS = [(1, 4), (2, 4), (4, 4), (1, 11), (2, 17), (4, 9)]


@pytest.mark.parametrize("G,T", WALKS, ids=[f"G{g}-T{t}" for g, t in WALKS])
def test_walk_equals_single_token_steps(gdn, G, T):
    """T tokens in one launch == T launches of one token, in place, on the
    same pool (with padding rows).  G = 1 single steps run in the one-tile
    kernel, so that case also pins the walk kernel to it."""
    t = H.torch()
    H_k = 4 // G if G < 4 else 1
    case = gi.small(B=6, T=T, H_k=H_k, H_v=H_k * G, d=128, twin=False, real_rows=4, seed=31 * G + T)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    walk = H.DevPool(pool)
    out_walk = H.gpu_step(gdn, walk, step, s, twin=False)
    single = H.DevPool(pool)
    outs = []
    for k in range(T):
        one = gi.StepInputs(x=np.ascontiguousarray(step.x[:, k:k + 1]), g=np.ascontiguousarray(step.g[:, k:k + 1]),
                            beta=np.ascontiguousarray(step.beta[:, k:k + 1]))
        outs.append(H.gpu_step(gdn, single, one, s, twin=False))
    t.cuda.synchronize()
    _bits_equal(out_walk, t.cat(outs, dim=1), "out")
    _bits_equal(walk.state, single.state, "state pool")
    _bits_equal(walk.conv_state, single.conv_state, "conv pool")
    assert not t.isnan(out_walk.float()).any()


@pytest.mark.parametrize("G", [2, 4])
def test_grouped_in_place_equals_twin(gdn, G):
    """In place with G value heads a key head (the walk kernel) == a twin-slot
    step (one head tile a workgroup), at d = 128 and 24 rows with padding."""
    t = H.torch()
    H_k = 8 // G
    case = gi.small(B=24, T=1, H_k=H_k, H_v=8, d=128, twin=True, real_rows=20, seed=5 + G)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    tw = H.DevPool(pool)
    out_t = H.gpu_step(gdn, tw, step, s, twin=True)
    ip = H.DevPool(pool)
    out_i = H.gpu_step(gdn, ip, step, s, twin=False)
    t.cuda.synchronize()
    _bits_equal(out_t, out_i, "out")
    real = pool.read_slot != 0
    wr = t.from_numpy(pool.write_slot[real].astype(np.int64)).cuda()
    rd = t.from_numpy(pool.read_slot[real].astype(np.int64)).cuda()
    _bits_equal(tw.state[wr], ip.state[rd], "state")
    _bits_equal(tw.conv_state[wr], ip.conv_state[rd], "conv window")


@pytest.mark.parametrize("B,G", [(48, 1), (64, 1), (64, 2), (44, 2)], ids=["48rows-G1", "64rows-G1", "64rows-G2",
                                                                          "44rows-G2"])
def test_grouped_key_heads_in_place(gdn, B, G):
    """Single-token in-place steps of 128 x 128 tiles with 2.5-4 tiles a CU run
    four value heads a workgroup (four key heads of one value head, or two of
    two).  With padding rows spread over the bucket: the oracle's values, the
    twin step's bits, zero outputs for padding, and nothing else in the pool
    touched."""
    import oracle
    t = H.torch()
    H_v = 16
    case = gi.small(B=B, T=1, H_k=H_v // G, H_v=H_v, d=128, twin=True, seed=B + G)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    pad = np.arange(B) % 7 == 3
    rd = pool.read_slot.copy()
    rd[pad] = 0
    wr = pool.write_slot.copy()
    wr[pad] = 0
    p2 = gi.Pool(pool.state, pool.conv_state, pool.conv_w, rd, wr)
    tw = H.DevPool(p2)
    out_t = H.gpu_step(gdn, tw, step, s, twin=True)
    ip = H.DevPool(p2)
    before = ip.state.clone()
    before_cs = ip.conv_state.clone()
    out_i = H.gpu_step(gdn, ip, step, s, twin=False)
    hp = H.HostPool(gi.Pool(pool.state, pool.conv_state, pool.conv_w, rd, rd.copy()))
    ref = H.oracle_step(oracle, hp, step, s, twin=False)
    t.cuda.synchronize()
    H.assert_out_close(out_i, ref)
    real = ~pad
    idx = t.from_numpy(rd[real].astype(np.int64)).cuda()
    H.assert_state_close(ip.state[idx].cpu().numpy(), hp.state[rd[real]])
    np.testing.assert_array_equal(H.bf16_host(ip.conv_state[idx]), hp.conv_state[rd[real]])
    _bits_equal(out_t, out_i, "out")
    widx = t.from_numpy(wr[real].astype(np.int64)).cuda()
    _bits_equal(tw.state[widx], ip.state[idx], "state")
    _bits_equal(tw.conv_state[widx], ip.conv_state[idx], "conv window")
    assert not bool(out_i[t.from_numpy(np.nonzero(pad)[0]).cuda()].float().abs().sum())
    mask = t.ones(s.N, dtype=t.bool, device="cuda")
    mask[idx] = False
    _bits_equal(ip.state[mask], before[mask], "untouched slots")
    _bits_equal(ip.conv_state[mask], before_cs[mask], "untouched windows")
