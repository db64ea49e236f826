"""GPU parity with slot addresses past 4 GiB: a pool of 4609 slots at the
0.8B-like layer's shapes (16 value heads of 128 x 128 fp32, 1 MiB a slot, so
4.5 GiB of state), whose rows use the highest slots, for every entry point that
addresses the pool (the twin step with its fused commit, in-place token walks,
per-token states, prefill, slot reset and copy).  A 32-bit byte offset anywhere
in the slot addressing would land these rows in the wrong place.

The device pool is zero except for the slots in use.  The oracle runs on the
small drawn pool: its slot s is device slot s + OFF (slot 0 stays the null
slot on both sides), so only the slot numbers differ between the two runs.
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from tests import helpers as H
from tests.test_gpu_prefill import _oracle_prefill

pytestmark = pytest.mark.gpu

N_BIG = 4609
H_K = H_V = 16
D = 128
C = 2 * H_K * D + H_V * D


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


@pytest.fixture(scope="module")
def big(torch):
    t = torch
    state = t.zeros((N_BIG, H_V, D, D), dtype=t.float32, device="cuda")
    conv = t.zeros((N_BIG, 3, C), dtype=t.bfloat16, device="cuda")
    yield state, conv
    del state, conv
    t.cuda.empty_cache()


class BigPool:
    """The drawn pool's slots 1..n-1 placed at the top of the big device pool."""

    def __init__(self, t, big, pool: gi.Pool):
        self.t = t
        self.state, self.conv = big
        self.n = pool.state.shape[0]
        self.off = N_BIG - self.n
        assert (self.off + 1) * H_V * D * D * 4 > 1 << 32, "the rows must sit past 4 GiB"
        self.state.zero_()
        self.conv.zero_()
        self.state[self.off + 1:] = t.from_numpy(pool.state[1:]).cuda()
        self.conv[self.off + 1:] = H.bf16_dev(pool.conv_state[1:])
        self.conv_w = H.bf16_dev(pool.conv_w)

    def dev_slots(self, slots: np.ndarray):
        s = np.asarray(slots, np.int64)
        return self.t.from_numpy(np.where(s > 0, s + self.off, s).astype(np.int32)).cuda()

    def check(self, hp_state: np.ndarray, hp_conv: np.ndarray, written):
        """Every used slot against the oracle's pool (written ones to the state
        bar, the rest bit for bit), and nothing written below them."""
        t = self.t
        written = sorted(set(int(s) for s in written if s > 0))
        got = self.state[self.off + 1:].cpu().numpy()
        for s in range(1, self.n):
            if s in written:
                H.assert_state_close(got[s - 1], hp_state[s], f"slot {s + self.off}")
            else:
                np.testing.assert_array_equal(got[s - 1].view(np.uint32), hp_state[s].view(np.uint32))
        np.testing.assert_array_equal(H.bf16_host(self.conv[self.off + 1:]), hp_conv[1:])
        assert not bool(t.any(self.state[:self.off + 1] != 0)), "a slot below the rows was written"
        assert not bool(t.any(self.conv[:self.off + 1].view(t.int16) != 0))


def test_twin_step_with_fused_commit_past_4gib(gdn, torch, big):
    t = torch
    case = gi.small(B=4, T=1, H_k=H_K, H_v=H_V, d=D, real_rows=3, N=9, seed=61)
    pool, step, s = case.pools[0], case.steps[0][0], case.shape
    bp = BigPool(t, big, pool)
    hp = H.HostPool(pool)
    out = t.empty((4, 1, H_V, D), dtype=t.bfloat16, device="cuda")
    nrd, nwr = t.empty(4, dtype=t.int32, device="cuda"), t.empty(4, dtype=t.int32, device="cuda")
    gdn.gdn_decode_step_commit(H.bf16_dev(step.x), bp.conv_w, None, bp.conv, bp.state, t.from_numpy(step.g).cuda(),
                               t.from_numpy(step.beta).cuda(), bp.dev_slots(pool.read_slot),
                               bp.dev_slots(pool.write_slot), nrd, nwr, out, H_k=H_K)
    ref = H.oracle_step(oracle, hp, step, s)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    bp.check(hp.state, hp.conv_state, pool.write_slot)
    np.testing.assert_array_equal(nrd.cpu().numpy(), bp.dev_slots(pool.write_slot).cpu().numpy())
    np.testing.assert_array_equal(nwr.cpu().numpy(), bp.dev_slots(pool.read_slot).cpu().numpy())


def test_in_place_token_walk_past_4gib(gdn, torch, big):
    t = torch
    case = gi.small(B=3, T=3, H_k=H_K, H_v=H_V, d=D, N=9, twin=False, seed=62)
    pool, step, s = case.pools[0], case.steps[0][0], case.shape
    bp = BigPool(t, big, pool)
    hp = H.HostPool(pool)
    out = t.empty((3, 3, H_V, D), dtype=t.bfloat16, device="cuda")
    gdn.gdn_decode_step(H.bf16_dev(step.x), bp.conv_w, None, bp.conv, bp.state, t.from_numpy(step.g).cuda(),
                        t.from_numpy(step.beta).cuda(), bp.dev_slots(pool.read_slot), None, out, H_k=H_K)
    ref = H.oracle_step(oracle, hp, step, s, twin=False)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    bp.check(hp.state, hp.conv_state, pool.read_slot)


def test_per_token_states_past_4gib(gdn, torch, big):
    t = torch
    B, T = 2, 3
    case = gi.small(B=B, T=T, H_k=H_K, H_v=H_V, d=D, N=1 + 2 * B + 2 * B * T, twin=False, seed=63)
    pool, step = case.pools[0], case.steps[0][0]
    used = set(pool.read_slot.tolist())
    free = [sl for sl in range(1, case.shape.N) if sl not in used]
    tok = np.array(free[:B * T], np.int32).reshape(B, T)
    tok[1, 1] = 0                                   # a token whose state is not kept
    bp = BigPool(t, big, pool)
    hp = H.HostPool(pool)
    out = t.empty((B, T, H_V, D), dtype=t.bfloat16, device="cuda")
    gdn.gdn_decode_step_tokens(H.bf16_dev(step.x), bp.conv_w, None, bp.conv, bp.state, t.from_numpy(step.g).cuda(),
                               t.from_numpy(step.beta).cuda(), bp.dev_slots(pool.read_slot),
                               bp.dev_slots(tok.ravel()).view(B, T), out, H_k=H_K)
    ref = oracle.gdn_decode_step_tokens(step.x, hp.conv_w, None, hp.conv_state, hp.state, step.g, step.beta, hp.rd,
                                        tok, H_k=H_K)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    bp.check(hp.state, hp.conv_state, tok.ravel())


@pytest.mark.parametrize("two_pass,lengths", [(False, [45, 3, 70]), (True, [45, 3, 70]),
                                              (True, [45, 3, 70, 12, 33, 1, 64, 20] * 2)],
                         ids=["one-kernel", "two-pass", "two-pass-slim"])
def test_prefill_past_4gib(gdn, torch, big, two_pass, lengths):
    t = torch
    case = gi.prefill(lengths, H_k=H_K, H_v=H_V, d=D, seed=64)
    s, pool = case.shape, case.pool
    bp = BigPool(t, big, pool)
    hp = H.HostPool(pool)
    out = t.full((s.T, H_V, D), 7.0, dtype=t.bfloat16, device="cuda")
    args = (H.bf16_dev(case.x), bp.conv_w, None, bp.conv, bp.state, t.from_numpy(case.g).cuda(),
            t.from_numpy(case.beta).cuda(), t.from_numpy(case.cu_seqlens).cuda(), bp.dev_slots(pool.read_slot), out)
    if two_pass:
        ws = t.empty((gdn.gdn_prefill_two_pass_workspace_bytes(s.B, s.T, H_K, H_V, D, D),), dtype=t.uint8,
                     device="cuda")
        gdn.gdn_prefill_two_pass(*args, ws, H_k=H_K)
    else:
        gdn.gdn_prefill(*args, H_k=H_K)
    ref = _oracle_prefill(case, hp)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    bp.check(hp.state, hp.conv_state, pool.read_slot)


def test_slot_reset_and_copy_past_4gib(gdn, torch, big):
    t = torch
    case = gi.small(B=4, T=1, H_k=H_K, H_v=H_V, d=D, N=9, seed=65)
    pool = case.pools[0]
    bp = BigPool(t, big, pool)
    hp = H.HostPool(pool)
    reset = np.array([2, 0, 7], np.int32)
    src, dst = np.array([1, 5, 8], np.int32), np.array([3, 6, 4], np.int32)
    gdn.slot_reset(bp.state, bp.conv, bp.dev_slots(reset), H_k=H_K)
    oracle.slot_reset(hp.state, hp.conv_state, reset)
    gdn.slot_copy(bp.state, bp.conv, bp.dev_slots(src), bp.dev_slots(dst), H_k=H_K)
    oracle.slot_copy(hp.state, hp.conv_state, src, dst)
    t.cuda.synchronize()
    bp.check(hp.state, hp.conv_state, [])   # copies and zeros are bit-exact
