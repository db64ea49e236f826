"""GPU parity of the chunked prefill (gdn_prefill and gdn_prefill_two_pass,
through the C ABI) against the fp64 oracle.  A prompt's prefill is, by definition, the in-place decode step run
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


def _run(gdn, t, case, dp, conv_b=None, q_scale=1.0, cu=None, two_pass=False):
    s = case.shape
    out = t.full((s.T, s.H_v, s.d_v), 7.0, dtype=t.bfloat16, device="cuda")  # any unwritten row shows
    cu_dev = t.from_numpy(case.cu_seqlens if cu is None else cu).cuda()
    args = (H.bf16_dev(case.x), dp.conv_w, conv_b, dp.conv_state, dp.state, t.from_numpy(case.g).cuda(),
            t.from_numpy(case.beta).cuda(), cu_dev, dp.rd, out)
    if two_pass:
        nbytes = gdn.gdn_prefill_two_pass_workspace_bytes(s.B, s.T, s.H_k, s.H_v, s.d_k, s.d_v)
        # stale contents must not matter: fill the workspace with NaN bits
        ws = t.full((nbytes,), 0xFF, dtype=t.uint8, device="cuda")
        gdn.gdn_prefill_two_pass(*args, ws, H_k=s.H_k, q_scale=q_scale)
    else:
        gdn.gdn_prefill(*args, H_k=s.H_k, q_scale=q_scale)
    return out


def _check(gdn, t, case, conv_b=None, q_scale=1.0, two_pass=False):
    s, pool = case.shape, case.pool
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    before_state, before_conv = dp.state.clone(), dp.conv_state.clone()
    bias_dev = None if conv_b is None else H.bf16_dev(conv_b)
    out = _run(gdn, t, case, dp, conv_b=bias_dev, q_scale=q_scale, two_pass=two_pass)
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


PATHS = pytest.mark.parametrize("two_pass", [False, True], ids=["one-kernel", "two-pass"])


@PATHS
@pytest.mark.parametrize("lengths,hk,hv,d,dv,pad", CASES,
                         ids=[f"{len(c[0])}seq-{c[1]}x{c[2]}-d{c[3]}x{c[4]}" for c in CASES])
def test_prefill_matches_oracle(gdn, torch, lengths, hk, hv, d, dv, pad, two_pass):
    case = gi.prefill(list(lengths), H_k=hk, H_v=hv, d=d, d_v=dv, pad=pad, seed=len(lengths) + d)
    _, out = _check(gdn, torch, case, two_pass=two_pass)
    for b in pad:
        a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        assert torch.count_nonzero(out[a:e].view(torch.int16)) == 0, "padding sequences read out +0.0"


@PATHS
def test_prefill_bias_and_q_scale(gdn, torch, two_pass):
    case = gi.prefill([45, 12], H_k=2, H_v=2, d=128, seed=11)
    bias = gi.bf16_bits(np.random.Generator(np.random.PCG64(4)).standard_normal(case.shape.C).astype(np.float32))
    _check(gdn, torch, case, conv_b=bias, q_scale=128 ** -0.5, two_pass=two_pass)


@PATHS
def test_prefill_08b_shapes(gdn, torch, two_pass):
    """The 0.8B-like layer's shapes: 16+16 heads of 128, 6144 channels."""
    case = gi.prefill([300, 45, 1], H_k=16, H_v=16, d=128, seed=2)
    _check(gdn, torch, case, two_pass=two_pass)


def test_two_pass_long_prompt_and_slices(gdn, torch):
    """One long prompt (16-column slices, the state in registers; every chunk in
    flight in pass 1), then many short ones (the slim layout: the conv run again
    in the walk), at the 0.8B shapes."""
    _check(gdn, torch, gi.prefill([1000], H_k=16, H_v=16, d=128, seed=21), two_pass=True)
    _check(gdn, torch, gi.prefill([3, 40, 1, 33] * 4 + [2] * 8, H_k=16, H_v=16, d=128, N=97, seed=22),
           two_pass=True)


@PATHS
@pytest.mark.parametrize("g_scale", [0.01, 0.0], ids=["weak-decay", "no-decay"])
def test_prefill_long_prompt_with_weak_or_no_decay(gdn, torch, two_pass, g_scale):
    """2048 tokens at the 0.8B shapes with the log decay scaled by 0.01 (a state
    that remembers for hundreds of tokens), and with g = 0 exactly (every decay
    factor 1): errors of the chunked form would accumulate here if anywhere,
    yet the bars are the decode step's."""
    case = gi.prefill([2048], H_k=16, H_v=16, d=128, seed=33)
    case.g[:] = (case.g * np.float32(g_scale)).astype(np.float32)
    _check(gdn, torch, case, two_pass=two_pass)


def test_two_pass_bench_workload_one_long_prompt(gdn, torch):
    """The prefill bench's single-prompt workload as it times it: one prompt of
    4096 tokens at the 0.8B-like shapes (128 chunks, 16-column slices), every
    output row and the final state against the oracle."""
    _check(gdn, torch, gi.prefill([4096], H_k=16, H_v=16, d=128, seed=31), two_pass=True)


@pytest.mark.parametrize("lengths,hk,hv", [
    ([100, 33, 64, 5], 16, 16),                                     # 64 heads: 32-column slices
    ([40, 1, 70, 32, 31, 65, 2], 16, 16),                           # 112 heads: 64-column slices
    ([9, 40, 1, 33, 64, 2, 17, 30, 5, 71, 3, 32, 8, 45, 1, 20, 6], 2, 4),  # 68 heads: 16-column, 4 past the last group of 8
    ([9, 40, 1, 33, 64, 2, 17, 30, 5], 2, 4),                       # 36 heads: 32-column, 4 past the last group of 8
    ([40, 1, 70, 32, 31, 65, 2, 50], 16, 16),                       # 128 heads: 64-column slices
    ([30, 7, 61, 2, 33, 12, 40, 1, 64, 25, 3, 50], 16, 16),         # 192 heads: 32-column slices
    ([40, 3, 65, 32, 1, 70], 16, 16),                               # 96 heads: 16-column slices
], ids=["4seq-slices32", "7seq-slices64", "17seq-slices16-tail", "9seq-slices32-tail", "8seq-slices64",
        "12seq-slices32", "6seq-slices16"])
def test_two_pass_wide_slices(gdn, torch, lengths, hk, hv):
    """The walk over column slices of each width the call's head count picks
    under 256 heads (16 wide: the state in registers; 32 and 64: state and U
    in LDS), and prompt-head pairs past the last whole group of eight placed in
    order."""
    _check(gdn, torch, gi.prefill(lengths, H_k=hk, H_v=hv, d=128, seed=len(lengths) + 90), two_pass=True)


SLIM_CASES = [
    # lengths, H_k, H_v, d_k, d_v, padding prompts; B * H_v in 256, 512
    ((1, 5, 32, 33, 70, 0, 100, 7, 64, 31, 2, 40, 9, 16, 65, 3), 8, 16, 128, 128, (7,)),  # G = 2, chunk edges, an empty
                                                                                           # and a padding prompt
    ((40, 17, 3, 65, 96, 2, 33, 12) * 2, 4, 16, 128, 128, ()),       # G = 4
    ((64, 3, 200, 1, 31, 9, 9, 9, 9, 9, 9, 9, 9, 9, 9, 9), 16, 16, 64, 64, (2,)),  # d = 64, a long padding prompt
    ((31, 65, 2, 40) * 4, 16, 16, 128, 64, ()),                      # d_k > d_v
    ((31, 65, 2, 40, 7, 33, 64, 1) * 2, 16, 16, 64, 128, (1,)),      # d_k < d_v
    ((9, 40, 1, 33, 64, 2, 17, 30, 5, 71, 3, 32, 8, 45, 1, 20) * 2, 16, 16, 128, 128, ()),  # 512 pairs: two rounds
]


@pytest.mark.parametrize("lengths,hk,hv,d,dv,pad", SLIM_CASES,
                         ids=[f"{len(c[0])}seq-{c[1]}x{c[2]}-d{c[3]}x{c[4]}" for c in SLIM_CASES])
def test_two_pass_slim_layout(gdn, torch, lengths, hk, hv, d, dv, pad):
    """The slim layout (calls whose walk, a workgroup a prompt and value head,
    fills the compute units): pass 1 keeps T', P and the row factors only, and
    the walk runs the conv again from x, with a prompt's first inputs from the
    window copy; GQA groups of 2 and 4, d = 64, d_k != d_v, padding and empty
    prompts, more workgroups than compute units."""
    case = gi.prefill(list(lengths), H_k=hk, H_v=hv, d=d, d_v=dv, pad=pad, seed=len(lengths) + d + 400)
    _, out = _check(gdn, torch, case, two_pass=True)
    for b in pad:
        a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        assert torch.count_nonzero(out[a:e].view(torch.int16)) == 0, "padding sequences read out +0.0"


def test_two_pass_slim_bias_and_q_scale(gdn, torch):
    """A conv bias and q_scale through the slim walk's own conv and row factors."""
    case = gi.prefill([45, 12, 33, 64, 1, 80, 31, 2] * 2, H_k=16, H_v=16, d=128, seed=12)
    bias = gi.bf16_bits(np.random.Generator(np.random.PCG64(5)).standard_normal(case.shape.C).astype(np.float32))
    _check(gdn, torch, case, conv_b=bias, q_scale=128 ** -0.5, two_pass=True)


@pytest.mark.parametrize("g_scale", [0.01, 0.0], ids=["weak-decay", "no-decay"])
def test_two_pass_slim_long_prompts_weak_or_no_decay(gdn, torch, g_scale):
    """Sixteen prompts of 384 tokens (the slim layout) with the log decay scaled
    by 0.01 and with g = 0: the chunked form's rounding would build up here."""
    case = gi.prefill([384] * 16, H_k=16, H_v=16, d=128, seed=34)
    case.g[:] = (case.g * np.float32(g_scale)).astype(np.float32)
    _check(gdn, torch, case, two_pass=True)


def test_two_pass_bench_workload_many_prompts(gdn, torch):
    """The prefill bench's many-prompt workload as it times it: 16 prompts of 512
    tokens at the 0.8B-like shapes (the slim layout), every output row and every
    final state against the oracle."""
    _check(gdn, torch, gi.prefill([512] * 16, H_k=16, H_v=16, d=128, seed=32), two_pass=True)


@PATHS
def test_prefill_many_ragged_sequences(gdn, torch, two_pass):
    """300 sequences (more than one 256-wide tile of the two-pass chunk map,
    whose scan carries across tiles): lengths 0-70 drawn at random, some on the
    null slot."""
    rng = np.random.Generator(np.random.PCG64(77))
    lengths = [int(v) for v in rng.integers(0, 71, size=300)]
    lengths[5] = lengths[256] = 0          # empty sequences on each side of the tile edge
    lengths[255], lengths[257] = 33, 64     # chunk edges next to it
    pad = tuple(int(b) for b in rng.choice(300, size=12, replace=False))
    case = gi.prefill(lengths, H_k=1, H_v=2, d=64, pad=pad, seed=78)
    _, out = _check(gdn, torch, case, two_pass=two_pass)
    for b in pad:
        a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        assert torch.count_nonzero(out[a:e].view(torch.int16)) == 0, "padding sequences read out +0.0"


def test_two_pass_agrees_with_one_kernel(gdn, torch):
    """The two paths on the same inputs: within the state bar of each other."""
    t = torch
    case = gi.prefill([200, 7, 64], H_k=2, H_v=4, d=128, seed=23)
    dp1, dp2 = H.DevPool(case.pool), H.DevPool(case.pool)
    o1 = _run(gdn, t, case, dp1)
    o2 = _run(gdn, t, case, dp2, two_pass=True)
    t.cuda.synchronize()
    H.assert_state_close(dp2.state.cpu().numpy(), dp1.state.cpu().numpy().astype(np.float64), "two-pass vs one-kernel")
    assert t.equal(dp1.conv_state.view(t.int16), dp2.conv_state.view(t.int16))
    H.assert_out_close(o2, H.bf16_host_f64(o1), "two-pass vs one-kernel out")


@PATHS
def test_prefill_in_two_calls_equals_one(gdn, torch, two_pass):
    """A prompt prefilled in two calls (the first 40 tokens, then the other 30)
    leaves the slot where one 70-token prefill does, within rounding, and the
    windows bit for bit (the conv window carries exactly the last inputs)."""
    t = torch
    case = gi.prefill([70], H_k=2, H_v=2, d=64, seed=5)
    dp1, dp2 = H.DevPool(case.pool), H.DevPool(case.pool)
    _run(gdn, t, case, dp1, two_pass=two_pass)
    for a, e in ((0, 40), (40, 41), (41, 70)):   # a one-token call in the middle: the window shifts by one
        sub = gi.PrefillCase(gi.Shape(B=1, T=e - a, H_k=2, H_v=2, d_k=64, d_v=64, W=4, N=case.shape.N), case.pool,
                             np.ascontiguousarray(case.x[a:e]), np.ascontiguousarray(case.g[a:e]),
                             np.ascontiguousarray(case.beta[a:e]), np.array([0, e - a], np.int32))
        _run(gdn, t, sub, dp2, two_pass=two_pass)
    t.cuda.synchronize()
    sl = int(case.pool.read_slot[0])
    H.assert_state_close(dp2.state[sl].cpu().numpy(), dp1.state[sl].cpu().numpy().astype(np.float64), "split prefill")
    assert t.equal(dp1.conv_state[sl].view(t.int16), dp2.conv_state[sl].view(t.int16))


@PATHS
@pytest.mark.parametrize("lengths,hk,hv", [([70, 5, 33], 2, 4), ([70, 5, 33, 12, 40, 1, 64, 9] * 2, 16, 16)],
                         ids=["full-layout", "slim-layout"])
def test_prefill_strided_x(gdn, torch, lengths, hk, hv, two_pass):
    """x rows 72 channels apart past C (a column slice of a wider buffer) give
    the bits of packed x: outputs, states and windows."""
    t = torch
    case = gi.prefill(lengths, H_k=hk, H_v=hv, d=128, seed=51)
    s = case.shape
    dp1, dp2 = H.DevPool(case.pool), H.DevPool(case.pool)
    o1 = _run(gdn, t, case, dp1, two_pass=two_pass)
    wide = t.full((s.T, s.C + 72), 3.0, dtype=t.bfloat16, device="cuda")
    wide[:, :s.C] = H.bf16_dev(case.x)
    x = wide[:, :s.C]
    assert x.stride(0) == s.C + 72
    o2 = t.full((s.T, s.H_v, s.d_v), 7.0, dtype=t.bfloat16, device="cuda")
    args = (x, dp2.conv_w, None, dp2.conv_state, dp2.state, t.from_numpy(case.g).cuda(),
            t.from_numpy(case.beta).cuda(), t.from_numpy(case.cu_seqlens).cuda(), dp2.rd, o2)
    if two_pass:
        nbytes = gdn.gdn_prefill_two_pass_workspace_bytes(s.B, s.T, s.H_k, s.H_v, s.d_k, s.d_v)
        gdn.gdn_prefill_two_pass(*args, t.full((nbytes,), 0xFF, dtype=t.uint8, device="cuda"), H_k=s.H_k)
    else:
        gdn.gdn_prefill(*args, H_k=s.H_k)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16))
    assert t.equal(dp1.state.view(t.int32), dp2.state.view(t.int32))
    assert t.equal(dp1.conv_state.view(t.int16), dp2.conv_state.view(t.int16))


@PATHS
def test_prefill_unusable_ranges_touch_nothing(gdn, torch, two_pass):
    t = torch
    case = gi.prefill([10, 20, 5], H_k=1, H_v=1, d=64, seed=8)
    dp = H.DevPool(case.pool)
    before = dp.state.clone()
    bad = np.array([0, 10, 5, 99], np.int32)   # sequence 1 runs backwards, sequence 2 past T
    out = _run(gdn, t, case, dp, cu=bad, two_pass=two_pass)
    t.cuda.synchronize()
    for b in (1, 2):
        sl = int(case.pool.read_slot[b])
        assert t.equal(dp.state[sl].view(t.int32), before[sl].view(t.int32))
    assert bool((out[10:].float() == 7.0).all()), "rows of unusable sequences stay as they were"


def test_two_pass_slim_unusable_ranges(gdn, torch):
    """256 prompts (the slim layout), the last two unusable (one running
    backwards, one past T): their slots and rows stay as they were, and every
    other prompt matches the oracle."""
    t = torch
    case = gi.prefill([10] * 256, H_k=1, H_v=1, d=64, seed=9)
    dp, hp = H.DevPool(case.pool), H.HostPool(case.pool)
    before = dp.state.clone()
    bad = case.cu_seqlens.copy()
    bad[255] = bad[254] - 5          # prompt 254 runs backwards
    bad[256] = case.shape.T + 50     # prompt 255 ends past T
    out = _run(gdn, t, case, dp, cu=bad, two_pass=True)
    ref = _oracle_prefill(case, hp)
    t.cuda.synchronize()
    for b in (254, 255):
        sl = int(case.pool.read_slot[b])
        assert t.equal(dp.state[sl].view(t.int32), before[sl].view(t.int32))
    end = int(case.cu_seqlens[254])
    assert bool((out[end:].float() == 7.0).all()), "rows of unusable prompts stay as they were"
    H.assert_out_close(out[:end], ref[:end])


@pytest.mark.parametrize("lengths,hk,hv,d,pad", [
    ([1200, 37, 0, 900, 1, 333, 50], 1, 2, 128, (6,)),   # G = 2, an empty and a padding prompt, 3 chunk ranges
    ([2500, 40, 700], 2, 2, 64, ()),                    # d = 64 (four 16-column slices a head), 3 ranges
    ([3000], 4, 4, 128, ()),                            # one prompt, 4 heads, 3 ranges
], ids=["ragged-G2", "d64", "one-prompt-4-heads"])
def test_two_pass_pipelined_ranges(gdn, torch, lengths, hk, hv, d, pad):
    """Calls whose 16-column walk leaves compute units idle go in chunk ranges
    of about 32: pass 1 of a range runs beside the walk of the one before.
    Ranges cut through prompts here (and pass an empty and a padding prompt):
    every output row, the final states and windows against the oracle, and
    every other slot untouched."""
    case = gi.prefill(lengths, H_k=hk, H_v=hv, d=d, pad=pad, seed=sum(lengths) % 97)
    _, out = _check(gdn, torch, case, two_pass=True)
    for b in pad:
        a, e = int(case.cu_seqlens[b]), int(case.cu_seqlens[b + 1])
        assert torch.count_nonzero(out[a:e].view(torch.int16)) == 0, "padding prompts read out +0.0"


def test_two_pass_ranges_give_the_bits_of_one_walk(gdn, torch):
    """One prompt of 2048 tokens at 16 heads runs in two chunk ranges; the same
    prompt beside an empty padding prompt (32 prompt-head pairs: a walk that
    fills the chip) runs in one walk.  The prompt's output rows, state and
    window are the same bits either way."""
    t = torch
    case = gi.prefill([2048], H_k=16, H_v=16, d=128, seed=44)
    s = case.shape
    x, g, beta = H.bf16_dev(case.x), t.from_numpy(case.g).cuda(), t.from_numpy(case.beta).cuda()
    res = []
    for pad in (False, True):
        dp = H.DevPool(case.pool)
        cu = t.tensor([0, 2048, 2048] if pad else [0, 2048], dtype=t.int32, device="cuda")
        slots = t.cat([dp.rd, t.zeros(1, dtype=t.int32, device="cuda")]) if pad else dp.rd
        B = 2 if pad else 1
        ws = t.empty((gdn.gdn_prefill_two_pass_workspace_bytes(B, s.T, s.H_k, s.H_v, s.d_k, s.d_v),),
                     dtype=t.uint8, device="cuda")
        out = t.empty((s.T, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
        gdn.gdn_prefill_two_pass(x, dp.conv_w, None, dp.conv_state, dp.state, g, beta, cu, slots, out, ws, H_k=s.H_k)
        t.cuda.synchronize()
        sl = int(case.pool.read_slot[0])
        res.append((out, dp.state[sl].clone(), dp.conv_state[sl].clone()))
    (o1, s1, c1), (o2, s2, c2) = res
    assert t.equal(o1.view(t.int16), o2.view(t.int16))
    assert t.equal(s1.view(t.int32), s2.view(t.int32))
    assert t.equal(c1.view(t.int16), c2.view(t.int16))


def test_two_pass_slim_long_prompts(gdn, torch):
    """Sixteen prompts of 1024 tokens (the slim layout, 32 chunks a walk), every
    output row and final state against the oracle."""
    _check(gdn, torch, gi.prefill([1024] * 16, H_k=16, H_v=16, d=128, seed=35), two_pass=True)


@pytest.mark.parametrize("lengths,hk,hv", [([70, 5, 33], 2, 4), ([70, 5, 33, 12, 40, 1, 64, 9] * 2, 16, 16),
                                            ([1500, 70, 600], 1, 2)],
                         ids=["full-layout", "slim-layout", "pipelined-ranges"])
def test_two_pass_graph_replay_matches_eager(gdn, torch, lengths, hk, hv):
    """The two-pass prefill (three launches, a caller workspace, no allocation)
    captured once and replayed several times, with eager work between replays,
    gives the bits of the same calls run eagerly (each replay continues the
    prompts from where the previous one left the slots), in both layouts."""
    t = torch
    case = gi.prefill(lengths, H_k=hk, H_v=hv, d=128, seed=31)
    s = case.shape
    dp_e, dp_g = H.DevPool(case.pool), H.DevPool(case.pool)
    x, g, beta = H.bf16_dev(case.x), t.from_numpy(case.g).cuda(), t.from_numpy(case.beta).cuda()
    cu = t.from_numpy(case.cu_seqlens).cuda()
    nbytes = gdn.gdn_prefill_two_pass_workspace_bytes(s.B, s.T, s.H_k, s.H_v, s.d_k, s.d_v)
    ws_e = t.empty((nbytes,), dtype=t.uint8, device="cuda")
    ws_g = t.empty_like(ws_e)
    out_e = t.empty((s.T, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    out_g = t.empty_like(out_e)

    def run(dp, out, ws):
        gdn.gdn_prefill_two_pass(x, dp.conv_w, None, dp.conv_state, dp.state, g, beta, cu, dp.rd, out, ws, H_k=s.H_k)

    stream = t.cuda.Stream()
    graph = t.cuda.CUDAGraph()
    with t.cuda.stream(stream):
        run(dp_g, out_g, ws_g)  # warm-up outside capture
    t.cuda.synchronize()
    dp_g.state.copy_(t.from_numpy(case.pool.state).cuda())
    dp_g.conv_state.copy_(H.bf16_dev(case.pool.conv_state))
    t.cuda.synchronize()
    with t.cuda.graph(graph, stream=stream):
        run(dp_g, out_g, ws_g)
    t.cuda.synchronize()
    assert t.equal(dp_g.state, t.from_numpy(case.pool.state).cuda()), "capture must not execute"
    for k in range(4):
        run(dp_e, out_e, ws_e)
        graph.replay()
        t.cuda.synchronize()
        _ = (dp_e.state.sum() + 1).item()  # eager work between replays
        assert t.equal(out_g.view(t.int16), out_e.view(t.int16)), f"replay {k}"
        assert t.equal(dp_g.state.view(t.int32), dp_e.state.view(t.int32)), f"replay {k}"
        assert t.equal(dp_g.conv_state.view(t.int16), dp_e.conv_state.view(t.int16)), f"replay {k}"
