"""Invariances of the HIP path that hold bit for bit at any size, checked at the
0.8B-like layer's shapes (16 + 16 heads of 128, 6144 conv channels) without the
oracle:

  - rows are independent: a decode step over the rows in another order gives the
    same outputs in that order and leaves every slot with the same bits;
  - prompts are independent: a prefill over the same prompts packed in another
    order gives each prompt the same outputs and the same final slot;
  - a call is deterministic: the same call on the same pool gives the same bits.

A kernel that lets one row or prompt read another's data, or whose sums depend
on which workgroup ran first, fails one of them.  Parity with the oracle is
tested elsewhere; here the GPU is compared with itself.
"""
import dataclasses

import numpy as np
import pytest

import gdn_inputs as gi
from tests import helpers as H
from tests.test_gpu_prefill import _run as _prefill_run

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


def _bits_equal(t, a, b):
    return t.equal(a.contiguous().view(t.int32 if a.dtype == t.float32 else t.int16),
                   b.contiguous().view(t.int32 if b.dtype == t.float32 else t.int16))


def _step(gdn, t, pool, step, s, twin, order):
    """One decode step with the rows taken in `order`; returns (out, pool on device)."""
    dp = H.DevPool(pool)
    o = t.from_numpy(np.asarray(order, np.int64))
    dp.rd, dp.wr = dp.rd[o.cuda()].contiguous(), dp.wr[o.cuda()].contiguous()
    permuted = gi.StepInputs(*(np.ascontiguousarray(a[order]) for a in (step.x, step.g, step.beta)))
    return H.gpu_step(gdn, dp, permuted, s, twin=twin), dp


@pytest.mark.parametrize("twin,T", [(True, 1), (False, 1), (False, 4)], ids=["twin", "inplace", "inplace-4-tokens"])
def test_decode_rows_in_another_order(gdn, torch, twin, T):
    case = gi.qwen08b(seed=41, B=64, twin=twin, T=T)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    order = np.random.Generator(np.random.PCG64(42)).permutation(s.B)
    out_a, dp_a = _step(gdn, torch, pool, step, s, twin, np.arange(s.B))
    out_b, dp_b = _step(gdn, torch, pool, step, s, twin, order)
    torch.cuda.synchronize()
    assert _bits_equal(torch, out_b, out_a[torch.from_numpy(order).cuda()]), "a row's output depends on the row order"
    assert _bits_equal(torch, dp_b.state, dp_a.state), "a slot's state depends on the row order"
    assert _bits_equal(torch, dp_b.conv_state, dp_a.conv_state)


@pytest.mark.parametrize("B,H_v", [(192, 16), (64, 32)], ids=["192rows-16heads", "64rows-32heads"])
def test_twin_step_in_row_parts_equals_one_round_calls(gdn, torch, B, H_v):
    """A twin step of 128 x 128 heads past one round of four-tile workgroups
    goes as consecutive row parts (here three of 64 rows, or two of 32 rows of
    32 value heads); the same rows stepped as separate calls, each one round,
    give the same bits: every output row and every slot."""
    t = torch
    case = gi.make_case(f"parts-B{B}-{H_v}", gi.Shape(B=B, T=1, H_k=16, H_v=H_v, d_k=128, d_v=128, W=4, N=2 * B + 1),
                        seed=B + H_v)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp_a = H.DevPool(pool)
    out_a = H.gpu_step(gdn, dp_a, step, s, twin=True)
    dp_b = H.DevPool(pool)
    out_b = t.empty_like(out_a)
    x, g, beta = H.bf16_dev(step.x), t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda()
    part = 1024 // H_v  # rows of one round of four-tile workgroups on 256 CUs
    for r0 in range(0, B, part):
        r1 = min(B, r0 + part)
        gdn.gdn_decode_step(x[r0:r1], dp_b.conv_w, None, dp_b.conv_state, dp_b.state, g[r0:r1], beta[r0:r1],
                            dp_b.rd[r0:r1], dp_b.wr[r0:r1], out_b[r0:r1], H_k=s.H_k)
    t.cuda.synchronize()
    assert _bits_equal(t, out_a, out_b), "a row's output depends on how the rows were split into launches"
    assert _bits_equal(t, dp_a.state, dp_b.state)
    assert _bits_equal(t, dp_a.conv_state, dp_b.conv_state)


def _reordered(case, order):
    """The same prompts packed in `order` (each keeps its slot and its tokens)."""
    cu = case.cu_seqlens
    spans = [(int(cu[b]), int(cu[b + 1])) for b in order]
    take = np.concatenate([np.arange(a, e) for a, e in spans] + [np.zeros(0, np.int64)]).astype(np.int64)
    lengths = [e - a for a, e in spans]
    new_cu = np.zeros(len(order) + 1, np.int32)
    new_cu[1:] = np.cumsum(lengths)
    pool = dataclasses.replace(case.pool, read_slot=np.ascontiguousarray(case.pool.read_slot[order]),
                               write_slot=np.ascontiguousarray(case.pool.write_slot[order]))
    return gi.PrefillCase(case.shape, pool, np.ascontiguousarray(case.x[take]), np.ascontiguousarray(case.g[take]),
                          np.ascontiguousarray(case.beta[take]), new_cu)


# ragged prompts over chunk edges, an empty one and a padding one; eight of
# them (the two-pass prefill's full layout) or sixteen (its slim layout)
ORDERS = {"8": ([700, 33, 1, 0, 1500, 64, 95, 320], (5,), [4, 7, 0, 3, 6, 2, 5, 1]),
          "16": ([700, 33, 1, 0, 150, 64, 95, 320, 31, 7, 256, 2, 96, 45, 1, 190], (5, 12),
                 [4, 15, 7, 0, 11, 3, 9, 6, 13, 2, 5, 10, 1, 14, 8, 12])}


@pytest.mark.parametrize("prompts", ["8", "16"], ids=["8prompts", "16prompts"])
@pytest.mark.parametrize("two_pass", [False, True], ids=["one-kernel", "two-pass"])
def test_prefill_prompts_in_another_order(gdn, torch, two_pass, prompts):
    lengths, pad, order = ORDERS[prompts]
    case = gi.prefill(lengths, H_k=16, H_v=16, d=128, pad=pad, seed=43)
    moved = _reordered(case, order)
    dp_a, dp_b = H.DevPool(case.pool), H.DevPool(moved.pool)
    out_a = _prefill_run(gdn, torch, case, dp_a, two_pass=two_pass)
    out_b = _prefill_run(gdn, torch, moved, dp_b, two_pass=two_pass)
    torch.cuda.synchronize()
    cu_a, cu_b = case.cu_seqlens, moved.cu_seqlens
    for j, b in enumerate(order):
        a0, a1, b0, b1 = int(cu_a[b]), int(cu_a[b + 1]), int(cu_b[j]), int(cu_b[j + 1])
        assert _bits_equal(torch, out_b[b0:b1], out_a[a0:a1]), f"prompt {b}'s output depends on its place in the pack"
    assert _bits_equal(torch, dp_b.state, dp_a.state), "a slot's state depends on the prompt order"
    assert _bits_equal(torch, dp_b.conv_state, dp_a.conv_state)


@pytest.mark.parametrize("lengths", [(4096,), (512,) * 16], ids=["1x4096", "16x512"])
@pytest.mark.parametrize("two_pass", [False, True], ids=["one-kernel", "two-pass"])
def test_prefill_is_deterministic(gdn, torch, lengths, two_pass):
    case = gi.prefill(list(lengths), H_k=16, H_v=16, d=128, seed=44)
    runs = []
    for _ in range(2):
        dp = H.DevPool(case.pool)
        runs.append((_prefill_run(gdn, torch, case, dp, two_pass=two_pass), dp))
    torch.cuda.synchronize()
    (out_a, dp_a), (out_b, dp_b) = runs
    assert _bits_equal(torch, out_a, out_b)
    assert _bits_equal(torch, dp_a.state, dp_b.state)
    assert _bits_equal(torch, dp_a.conv_state, dp_b.conv_state)


def test_decode_step_is_deterministic(gdn, torch):
    case = gi.qwen08b(seed=45, B=64)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    (out_a, dp_a), (out_b, dp_b) = (_step(gdn, torch, pool, step, s, True, np.arange(s.B)) for _ in range(2))
    torch.cuda.synchronize()
    assert _bits_equal(torch, out_a, out_b)
    assert _bits_equal(torch, dp_a.state, dp_b.state)
