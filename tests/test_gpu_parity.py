"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, at small shapes that span several tiles and ragged rows and
at the full workload sizes, plus the relational invariants the mstar pages
test for this path (PR #1139 "Tests": twin == in place, a twin step touches no
other slot, conv decode with null slots / strided rows / write slots; PR #965
"What changed": padding width changes no real row).

Tolerances are the ones in tests/helpers.py.
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


def _check_step(gdn, case, *, twin=True, q_scale=1.0, layer=0, step_i=0, poison=True):
    """One step on GPU and oracle; compare out, every written slot, and that
    nothing else in the pool changed."""
    t = H.torch()
    s = case.shape
    pool = case.pools[layer]
    step = case.steps[step_i][layer]
    hp = H.HostPool(pool)
    dp = H.DevPool(pool)
    real = pool.read_slot != 0
    if twin and poison:
        # NaN-poison the write slots: every element must be written by the step
        wr_real = t.from_numpy(pool.write_slot[real].astype(np.int64)).cuda()
        dp.state[wr_real] = float("nan")
    before_state = dp.state.clone()
    before_conv = dp.conv_state.clone()
    out = H.gpu_step(gdn, dp, step, s, twin=twin, q_scale=q_scale)
    ref = H.oracle_step(oracle, hp, step, s, twin=twin, q_scale=q_scale)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    written = sorted({int(x) for x in (pool.write_slot if twin else pool.read_slot)[real]})
    idx = t.tensor(written, dtype=t.int64, device="cuda")
    H.assert_state_close(dp.state[idx].cpu().numpy(), hp.state[written])
    np.testing.assert_array_equal(H.bf16_host(dp.conv_state[idx]), hp.conv_state[written])
    # nothing but the written slots changed (bitwise, NaN-aware)
    mask = t.ones(s.N, dtype=t.bool, device="cuda")
    mask[idx] = False
    assert t.equal(dp.state[mask].view(t.int32), before_state[mask].view(t.int32)), "a slot outside the write set changed"
    assert t.equal(dp.conv_state[mask].view(t.int16), before_conv[mask].view(t.int16))
    return dp, out


# ------------------------------------------------------------------ small shapes

SMALL = [
    # B, T, H_k, H_v, d, d_v, twin, real_rows
    (4, 1, 4, 4, 64, 64, True, None),      # the tiny workload's shapes
    (5, 1, 2, 2, 128, 128, True, None),    # ragged rows, column-split tiles (4 slices)
    (3, 1, 2, 4, 128, 128, True, None),    # GQA, G = 2
    (2, 1, 1, 4, 64, 64, True, None),      # GQA, G = 4
    (7, 1, 2, 2, 128, 64, True, None),     # d_k != d_v
    (6, 1, 2, 2, 64, 128, True, 4),        # padding rows on slot 0
    (32, 1, 4, 4, 128, 128, True, None),   # 128 heads: 2 slices (128 mod 256 is in 1..128)
    (150, 1, 2, 4, 64, 64, True, None),    # 600 heads: whole tiles
    (5, 1, 2, 2, 128, 128, False, None),   # in place
    (3, 3, 2, 4, 128, 128, False, None),   # in place, 3 tokens, G = 2
    (4, 2, 1, 4, 64, 64, False, 3),        # in place, G = 4, padding
    (9, 4, 2, 2, 64, 128, False, None),    # in place, 4 tokens
    (3, 11, 2, 2, 128, 128, False, None),  # in place, 11 tokens: a full block of 8, then 3
    (4, 17, 1, 4, 64, 64, False, 3),       # in place, G = 4, 17 tokens (blocks of 8, 8, 1), padding
    (2, 9, 2, 4, 128, 64, False, None),    # in place, G = 2, d_k != d_v, 9 tokens
]


@pytest.mark.parametrize("B,T,hk,hv,d,dv,twin,real", SMALL,
                         ids=[f"B{c[0]}-T{c[1]}-{c[2]}x{c[3]}-d{c[4]}x{c[5]}-{'twin' if c[6] else 'inplace'}"
                              f"{'' if c[7] is None else '-pad'}" for c in SMALL])
def test_small_shapes_match_oracle(gdn, torch, B, T, hk, hv, d, dv, twin, real):
    case = gi.small(B=B, T=T, H_k=hk, H_v=hv, d=d, d_v=dv, twin=twin, real_rows=real, seed=B * 7 + T)
    _check_step(gdn, case, twin=twin)


def test_q_scale(gdn, torch):
    case = gi.small(B=3, T=1, H_k=2, H_v=2, d=128, seed=5)
    _check_step(gdn, case, q_scale=128 ** -0.5)


def test_conv_bias(gdn, torch):
    t = torch
    case = gi.small(B=3, T=1, H_k=2, H_v=2, d=64, seed=6)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    bias = gi.bf16_bits(np.random.Generator(np.random.PCG64(9)).standard_normal(s.C).astype(np.float32))
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    out = H.gpu_step(gdn, dp, step, s, conv_b=H.bf16_dev(bias))
    ref = oracle.gdn_decode_step(step.x, hp.conv_w, bias, hp.conv_state, hp.state, step.g, step.beta, hp.rd, hp.wr,
                                 H_k=s.H_k)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    wr = [int(x) for x in pool.write_slot]
    H.assert_state_close(dp.state[wr].cpu().numpy(), hp.state[wr])


# ------------------------------------------------------------------ workload: tiny, 8 chained steps

def test_tiny_eight_chained_steps_with_commit(gdn, torch):
    t = torch
    case = gi.tiny()
    s, pool = case.shape, case.pools[0]
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    for k in range(8):
        step = case.steps[k][0]
        out = H.gpu_step(gdn, dp, step, s)
        ref = H.oracle_step(oracle, hp, step, s)
        gdn.slot_commit(dp.rd, dp.wr)
        oracle.slot_commit(hp.rd, hp.wr)
        t.cuda.synchronize()
        H.assert_out_close(out, ref, f"out step {k}")
        H.assert_state_close(dp.state.cpu().numpy(), hp.state, f"pool after step {k}")
        np.testing.assert_array_equal(H.bf16_host(dp.conv_state), hp.conv_state)
        np.testing.assert_array_equal(dp.rd.cpu().numpy(), hp.rd)
        np.testing.assert_array_equal(dp.wr.cpu().numpy(), hp.wr)


@pytest.mark.parametrize("twin", [True, False], ids=["twin", "inplace"])
def test_256_chained_steps_without_decay(gdn, torch, twin):
    """256 steps of 4 rows (2 + 2 heads of 128) with g = 0: nothing decays, so the
    state remembers every step and rounding differences would pile up; each
    side chains through its own fp32 slots, twin slots committed between steps.
    The last step's output and the whole pool against the oracle."""
    t = torch
    case = gi.small(4, 1, 2, 2, 128, twin=twin, steps=256, seed=7)
    s, pool = case.shape, case.pools[0]
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    for k in range(256):
        step = case.steps[k][0]
        step.g[:] = 0.0
        out = H.gpu_step(gdn, dp, step, s, twin=twin)
        ref = H.oracle_step(oracle, hp, step, s, twin=twin)
        if twin:
            gdn.slot_commit(dp.rd, dp.wr)
            oracle.slot_commit(hp.rd, hp.wr)
    t.cuda.synchronize()
    H.assert_out_close(out, ref, "out of the last step")
    H.assert_state_close(dp.state.cpu().numpy(), hp.state, "pool after 256 steps")
    np.testing.assert_array_equal(H.bf16_host(dp.conv_state), hp.conv_state)


# ------------------------------------------------------------------ workload: 0.8B layer, 64 rows

def test_08b_layer_64_rows_twin(gdn, torch):
    case = gi.qwen08b()
    _check_step(gdn, case)


# ------------------------------------------------------------------ workload: row sweep, twin and in place

@pytest.mark.parametrize("B", gi.SWEEP_ROWS)
def test_sweep_twin_and_in_place(gdn, torch, B):
    t = torch
    case = gi.qwen08b(B=B)
    dp_t, out_t = _check_step(gdn, case, twin=True, poison=False)
    dp_i, out_i = _check_step(gdn, case, twin=False)
    # same values from both write modes, bit for bit (PR #1139: same kernel, same values)
    assert t.equal(out_t.view(t.int16), out_i.view(t.int16))
    pool = case.pools[0]
    wr = t.from_numpy(pool.write_slot.astype(np.int64)).cuda()
    rd = t.from_numpy(pool.read_slot.astype(np.int64)).cuda()
    assert t.equal(dp_t.state[wr].view(t.int32), dp_i.state[rd].view(t.int32))
    assert t.equal(dp_t.conv_state[wr].view(t.int16), dp_i.conv_state[rd].view(t.int16))


@pytest.mark.parametrize("B", [8, 24, 40, 44, 48, 56])
def test_twin_launch_shapes_equal_whole_tile_in_place(gdn, torch, B):
    """Row counts at which the twin step changes its launch shape while the
    in-place step keeps one whole tile a workgroup: 8, 24 and 40 rows of 16
    heads leave a remainder of 1..128 tiles over the 256 CUs, so the twin step
    splits each head into two column slices; 44 and 48 rows put three whole
    tiles in a workgroup (44: the last workgroup holds two tiles and an empty
    one), 56 rows two.  Both match the oracle and each other bit for bit
    (every tile sums over d_k in the same order whatever the launch shape)."""
    t = torch
    case = gi.qwen08b(B=B, seed=B)
    dp_t, out_t = _check_step(gdn, case, twin=True, poison=True)
    dp_i, out_i = _check_step(gdn, case, twin=False)
    assert t.equal(out_t.view(t.int16), out_i.view(t.int16))
    pool = case.pools[0]
    wr = t.from_numpy(pool.write_slot.astype(np.int64)).cuda()
    rd = t.from_numpy(pool.read_slot.astype(np.int64)).cuda()
    assert t.equal(dp_t.state[wr].view(t.int32), dp_i.state[rd].view(t.int32))
    assert t.equal(dp_t.conv_state[wr].view(t.int16), dp_i.conv_state[rd].view(t.int16))


def test_four_tile_workgroups_with_a_partial_last_group(gdn, torch):
    """45 rows of 15 heads (675 tiles of 128 x 128) take four tiles a
    workgroup; the last workgroup holds three tiles and one past the end.
    Twin against the oracle (with padding rows) and bit for bit against the
    same step in place, which takes one tile a workgroup."""
    t = torch
    case = gi.small(B=45, T=1, H_k=15, H_v=15, d=128, twin=True, real_rows=41, seed=45)
    dp_t, out_t = _check_step(gdn, case, twin=True, poison=True)
    pool = case.pools[0]
    ip = gi.Case(case.name, case.shape, [gi.Pool(pool.state, pool.conv_state, pool.conv_w, pool.read_slot,
                                                 pool.read_slot.copy())], case.steps, case.real_rows, False)
    dp_i, out_i = _check_step(gdn, ip, twin=False)
    assert t.equal(out_t.view(t.int16), out_i.view(t.int16))
    real = pool.read_slot != 0
    wr = t.from_numpy(pool.write_slot[real].astype(np.int64)).cuda()
    rd = t.from_numpy(pool.read_slot[real].astype(np.int64)).cuda()
    assert t.equal(dp_t.state[wr].view(t.int32), dp_i.state[rd].view(t.int32))
    assert t.equal(dp_t.conv_state[wr].view(t.int16), dp_i.conv_state[rd].view(t.int16))


@pytest.mark.parametrize("B,pad_rows", [(48, (5, 17, 30, 47)), (64, (0, 3, 31, 32, 63))], ids=["48rows", "64rows"])
def test_multi_tile_workgroups_with_padding_rows(gdn, torch, B, pad_rows):
    """Twin steps whose workgroups hold several head tiles (three at 48 rows,
    two at 64), with padding rows scattered among the real ones so that some
    workgroups hold tiles of a real and of a padding row.  Real rows match the
    oracle, padding rows read out +0.0, slot 0 stays zero, nothing else in the
    pool changes, and every real row's bits equal those of the same rows
    stepped without the padding (a launch of another shape)."""
    t = torch
    case = gi.qwen08b(B=B, seed=100 + B)
    pool, step, s = case.pools[0], case.steps[0][0], case.shape
    for r in pad_rows:
        pool.read_slot[r] = 0
        pool.write_slot[r] = 0
    dp, out = _check_step(gdn, case, twin=True)
    pad = list(pad_rows)
    assert t.count_nonzero(out[pad].view(t.int16)) == 0, "padding rows must read out +0.0"
    assert t.count_nonzero(dp.state[0].view(t.int32)) == 0 and t.count_nonzero(dp.conv_state[0].view(t.int16)) == 0
    real = [r for r in range(B) if r not in pad_rows]
    dp2 = H.DevPool(pool)
    idx = t.tensor(real, dtype=t.int64, device="cuda")
    dp2.rd, dp2.wr = dp2.rd[idx].contiguous(), dp2.wr[idx].contiguous()
    sub = gi.StepInputs(np.ascontiguousarray(step.x[real]), np.ascontiguousarray(step.g[real]),
                        np.ascontiguousarray(step.beta[real]))
    out2 = H.gpu_step(gdn, dp2, sub, s, twin=True)
    t.cuda.synchronize()
    assert t.equal(out[idx].view(t.int16), out2.view(t.int16))
    wr = t.from_numpy(pool.write_slot[real].astype(np.int64)).cuda()
    assert t.equal(dp.state[wr].view(t.int32), dp2.state[wr].view(t.int32))
    assert t.equal(dp.conv_state[wr].view(t.int16), dp2.conv_state[wr].view(t.int16))


# ------------------------------------------------------------------ workload: 9B-like, 24 layers

def test_9b_24_layers_back_to_back_every_row(gdn, torch):
    """The 9B-like stack: 24 layers (16 key heads shared by 32 value heads, so
    only the first value head of a key head writes back its q/k windows) run
    back to back on their own pools, then every row of every layer is compared
    with the oracle (outputs, written states and windows), with the write slots
    NaN-poisoned beforehand and every other slot of each pool unchanged."""
    t = torch
    case = gi.qwen9b()
    s = case.shape
    dps, befores = [], []
    for L in range(24):
        pool = case.pools[L]
        dp = H.DevPool(pool)
        dp.state[t.from_numpy(pool.write_slot.astype(np.int64)).cuda()] = float("nan")
        dps.append(dp)
        befores.append((dp.state.clone(), dp.conv_state.clone()))
    outs = [H.gpu_step(gdn, dps[L], case.steps[0][L], s) for L in range(24)]
    t.cuda.synchronize()
    for L in range(24):
        pool, dp = case.pools[L], dps[L]
        hp = H.HostPool(pool)
        ref = H.oracle_step(oracle, hp, case.steps[0][L], s)
        H.assert_out_close(outs[L], ref, f"layer {L} out")
        wr = [int(x) for x in pool.write_slot]
        idx = t.tensor(wr, dtype=t.int64, device="cuda")
        H.assert_state_close(dp.state[idx].cpu().numpy(), hp.state[wr], f"layer {L} state")
        np.testing.assert_array_equal(H.bf16_host(dp.conv_state[idx]), hp.conv_state[wr])
        mask = t.ones(s.N, dtype=t.bool, device="cuda")
        mask[idx] = False
        bs, bc = befores[L]
        assert t.equal(dp.state[mask].view(t.int32), bs[mask].view(t.int32)), f"layer {L}: a slot outside the write set changed"
        assert t.equal(dp.conv_state[mask].view(t.int16), bc[mask].view(t.int16))


# ------------------------------------------------------------------ workload: padded bucket

@pytest.mark.parametrize("twin", [True, False], ids=["twin", "inplace"])
def test_padded_bucket_real_rows_identical_to_unpadded(gdn, torch, twin):
    """The 128-row bucket with 46 real rows first and 82 on the null slot.  In
    place it is the mixed step's decode half (PR #965, "What changed": a run of
    one-token rows, width sized to the bucket, padding on slot 0; PR #1139,
    "What changed": that half updates in place)."""
    t = torch
    case = gi.padded(twin=twin)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp, out = _check_step(gdn, case, twin=twin)
    assert t.count_nonzero(out[gi.PADDED_REAL:].view(t.int16)) == 0, "padding rows must read out +0.0"
    assert t.count_nonzero(dp.state[0].view(t.int32)) == 0 and t.count_nonzero(dp.conv_state[0].view(t.int16)) == 0
    # the same 46 rows without the padding: bit-identical outputs and state
    n = gi.PADDED_REAL
    dp2 = H.DevPool(pool)
    dp2.rd, dp2.wr = dp2.rd[:n].contiguous(), dp2.wr[:n].contiguous()
    sub = gi.StepInputs(np.ascontiguousarray(step.x[:n]), np.ascontiguousarray(step.g[:n]),
                        np.ascontiguousarray(step.beta[:n]))
    out2 = H.gpu_step(gdn, dp2, sub, s, twin=twin)
    t.cuda.synchronize()
    assert t.equal(out[:n].view(t.int16), out2.view(t.int16))
    wr = t.from_numpy(pool.write_slot[:n].astype(np.int64)).cuda()
    assert t.equal(dp.state[wr].view(t.int32), dp2.state[wr].view(t.int32))
    assert t.equal(dp.conv_state[wr].view(t.int16), dp2.conv_state[wr].view(t.int16))


def test_padded_bucket_in_place_four_tokens(gdn, torch):
    t = torch
    case = gi.padded(T=4, twin=False)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp, out4 = _check_step(gdn, case, twin=False)
    # four single-token in-place calls give the same bits as one four-token call
    dp1 = H.DevPool(pool)
    for k in range(4):
        sub = gi.StepInputs(np.ascontiguousarray(step.x[:, k:k + 1]), np.ascontiguousarray(step.g[:, k:k + 1]),
                            np.ascontiguousarray(step.beta[:, k:k + 1]))
        o = H.gpu_step(gdn, dp1, sub, s, twin=False)
        assert t.equal(o[:, 0].view(t.int16), out4[:, k].view(t.int16)), f"token {k}"
    assert t.equal(dp1.state.view(t.int32), dp.state.view(t.int32))
    assert t.equal(dp1.conv_state.view(t.int16), dp.conv_state.view(t.int16))


# ------------------------------------------------------------------ a state per token (speculative verify)

def _token_slots(pool, B, T, keep, rng_seed):
    """Distinct slots, none a read slot, for the kept tokens (keep[r][t]); 0 elsewhere."""
    used = set(int(x) for x in pool.read_slot)
    free = [sl for sl in range(1, pool.state.shape[0]) if sl not in used]
    rng = np.random.Generator(np.random.PCG64(rng_seed))
    rng.shuffle(free)
    tok = np.zeros((B, T), np.int32)
    k = 0
    for r in range(B):
        for t in range(T):
            if keep[r][t]:
                tok[r, t] = free[k]
                k += 1
    return tok


@pytest.mark.parametrize("B,T,hk,hv,d,real", [(5, 3, 2, 4, 128, 4), (6, 4, 2, 2, 64, None), (3, 2, 1, 4, 64, None)],
                         ids=["B5-T3-G2-pad", "B6-T4-d64", "B3-T2-G4"])
def test_per_token_states_match_oracle(gdn, torch, B, T, hk, hv, d, real):
    t = torch
    case = gi.small(B=B, T=T, H_k=hk, H_v=hv, d=d, N=1 + 2 * B + 2 * B * T, twin=False, real_rows=real, seed=B + T)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    keep = [[(r + tt) % 3 != 2 for tt in range(T)] for r in range(B)]   # some tokens not kept
    tok = _token_slots(pool, B, T, keep, 7)
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    before_state, before_conv = dp.state.clone(), dp.conv_state.clone()
    out = t.empty((B, T, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    gdn.gdn_decode_step_tokens(H.bf16_dev(step.x), dp.conv_w, None, dp.conv_state, dp.state,
                               t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda(), dp.rd,
                               t.from_numpy(tok).cuda(), out, H_k=s.H_k)
    ref = oracle.gdn_decode_step_tokens(step.x, hp.conv_w, None, hp.conv_state, hp.state, step.g, step.beta, hp.rd,
                                        tok, H_k=s.H_k)
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    real_rows = pool.read_slot != 0
    kept = sorted(int(x) for x in tok[real_rows].ravel() if x != 0)
    idx = t.tensor(kept, dtype=t.int64, device="cuda")
    H.assert_state_close(dp.state[idx].cpu().numpy(), hp.state[kept], "kept states")
    np.testing.assert_array_equal(H.bf16_host(dp.conv_state[idx]), hp.conv_state[kept])
    mask = t.ones(s.N, dtype=t.bool, device="cuda")
    mask[idx] = False   # every other slot, the read slots included, is untouched
    assert t.equal(dp.state[mask].view(t.int32), before_state[mask].view(t.int32))
    assert t.equal(dp.conv_state[mask].view(t.int16), before_conv[mask].view(t.int16))
    # the state kept after token k is, bit for bit, an in-place call over the first k+1 tokens
    for k in range(T):
        dpk = H.DevPool(pool)
        sub = gi.StepInputs(np.ascontiguousarray(step.x[:, :k + 1]), np.ascontiguousarray(step.g[:, :k + 1]),
                            np.ascontiguousarray(step.beta[:, :k + 1]))
        ok = H.gpu_step(gdn, dpk, sub, s, twin=False)
        t.cuda.synchronize()
        assert t.equal(ok.view(t.int16), out[:, :k + 1].view(t.int16)), f"outputs through token {k}"
        for r in range(B):
            if real_rows[r] and tok[r, k]:
                rs = int(pool.read_slot[r])
                assert t.equal(dp.state[int(tok[r, k])].view(t.int32), dpk.state[rs].view(t.int32)), (r, k)
                assert t.equal(dp.conv_state[int(tok[r, k])].view(t.int16), dpk.conv_state[rs].view(t.int16))


@pytest.mark.parametrize("path", ["twin", "inplace-tokens", "inplace-G2", "per-token-states"])
def test_conv_bias_and_q_scale_on_every_step_kernel(gdn, torch, path):
    """A conv bias and q_scale = d_k^-1/2 through each step kernel: the single-token
    tile (twin), the in-place token walk (3 tokens; G = 1, and G = 2 with its
    key-head groups), and the per-token-state walk."""
    t = torch
    T = 1 if path == "twin" else 3
    hv = 4 if path == "inplace-G2" else 2
    B = 4
    case = gi.small(B=B, T=T, H_k=2, H_v=hv, d=128, N=1 + 2 * B + 2 * B * T, twin=path == "twin", seed=17)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    bias = gi.bf16_bits(np.random.Generator(np.random.PCG64(18)).standard_normal(s.C).astype(np.float32))
    qs = 128 ** -0.5
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    a = (H.bf16_dev(step.x), dp.conv_w, H.bf16_dev(bias), dp.conv_state, dp.state, t.from_numpy(step.g).cuda(),
         t.from_numpy(step.beta).cuda(), dp.rd)
    out = t.empty((B, T, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    if path == "per-token-states":
        tok = _token_slots(pool, B, T, [[True] * T] * B, 19)
        gdn.gdn_decode_step_tokens(*a, t.from_numpy(tok).cuda(), out, H_k=s.H_k, q_scale=qs)
        ref = oracle.gdn_decode_step_tokens(step.x, hp.conv_w, bias, hp.conv_state, hp.state, step.g, step.beta,
                                            hp.rd, tok, H_k=s.H_k, q_scale=qs)
        written = sorted(int(x) for x in tok.ravel())
    else:
        twin = path == "twin"
        gdn.gdn_decode_step(*a, dp.wr if twin else None, out, H_k=s.H_k, q_scale=qs)
        ref = oracle.gdn_decode_step(step.x, hp.conv_w, bias, hp.conv_state, hp.state, step.g, step.beta, hp.rd,
                                     hp.wr if twin else None, H_k=s.H_k, q_scale=qs)
        written = sorted(int(x) for x in (pool.write_slot if twin else pool.read_slot))
    t.cuda.synchronize()
    H.assert_out_close(out, ref)
    H.assert_state_close(dp.state[written].cpu().numpy(), hp.state[written])
    np.testing.assert_array_equal(H.bf16_host(dp.conv_state[written]), hp.conv_state[written])


def test_per_token_states_unusable_slot(gdn, torch):
    """A token slot outside the pool, or equal to the row's read slot, makes the
    row NaN and touches nothing; the other rows are unaffected."""
    t = torch
    B, T = 3, 2
    case = gi.small(B=B, T=T, H_k=2, H_v=2, d=64, N=1 + 2 * B + 2 * B * T, twin=False, seed=3)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    tok = _token_slots(pool, B, T, [[True] * T] * B, 5)
    tok[1, 1] = s.N            # outside the pool
    tok[2, 0] = pool.read_slot[2]  # the row's own read slot
    dp = H.DevPool(pool)
    before = dp.state.clone()
    out = t.empty((B, T, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    gdn.gdn_decode_step_tokens(H.bf16_dev(step.x), dp.conv_w, None, dp.conv_state, dp.state,
                               t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda(), dp.rd,
                               t.from_numpy(tok).cuda(), out, H_k=s.H_k)
    t.cuda.synchronize()
    assert bool(t.isnan(out[1:].float()).all()) and not bool(t.isnan(out[0].float()).any())
    for r in (1, 2):
        for sl in [int(x) for x in tok[r] if 0 < x < s.N]:
            assert t.equal(dp.state[sl].view(t.int32), before[sl].view(t.int32))


# ------------------------------------------------------------------ fused commit

def test_step_commit_equals_step_then_commit(gdn, torch):
    t = torch
    case = gi.small(B=12, T=1, H_k=4, H_v=8, d=128, real_rows=10, N=25, seed=31)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp1, dp2 = H.DevPool(pool), H.DevPool(pool)
    out1 = H.gpu_step(gdn, dp1, step, s)
    gdn.slot_commit(dp1.rd, dp1.wr)
    out2 = t.empty_like(out1)
    nrd = t.full_like(dp2.rd, -7)
    nwr = t.full_like(dp2.wr, -7)
    gdn.gdn_decode_step_commit(H.bf16_dev(step.x), dp2.conv_w, None, dp2.conv_state, dp2.state,
                               t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda(), dp2.rd, dp2.wr, nrd, nwr,
                               out2, H_k=s.H_k)
    t.cuda.synchronize()
    assert t.equal(out1.view(t.int16), out2.view(t.int16))
    assert t.equal(dp1.state.view(t.int32), dp2.state.view(t.int32))
    assert t.equal(dp1.conv_state.view(t.int16), dp2.conv_state.view(t.int16))
    assert t.equal(nrd, dp1.rd) and t.equal(nwr, dp1.wr)
    # the arrays the step read are left as they were
    assert t.equal(dp2.rd, t.from_numpy(pool.read_slot).cuda()) and t.equal(dp2.wr, t.from_numpy(pool.write_slot).cuda())


def test_tiny_chain_with_fused_commit_matches_oracle(gdn, torch):
    """The tiny workload's 8 chained steps, with the commit folded into each step
    through two alternating pairs of slot arrays."""
    t = torch
    case = gi.tiny()
    s, pool = case.shape, case.pools[0]
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    pairs = [(dp.rd, dp.wr), (t.empty_like(dp.rd), t.empty_like(dp.wr))]
    for k in range(8):
        step = case.steps[k][0]
        (rd, wr), (nrd, nwr) = pairs[k % 2], pairs[(k + 1) % 2]
        out = t.empty((s.B, 1, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
        gdn.gdn_decode_step_commit(H.bf16_dev(step.x), dp.conv_w, None, dp.conv_state, dp.state,
                                   t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda(), rd, wr, nrd, nwr, out,
                                   H_k=s.H_k)
        ref = H.oracle_step(oracle, hp, step, s)
        oracle.slot_commit(hp.rd, hp.wr)
        t.cuda.synchronize()
        H.assert_out_close(out, ref, f"out step {k}")
        H.assert_state_close(dp.state.cpu().numpy(), hp.state, f"pool after step {k}")
        np.testing.assert_array_equal(H.bf16_host(dp.conv_state), hp.conv_state)
        np.testing.assert_array_equal(nrd.cpu().numpy(), hp.rd)
        np.testing.assert_array_equal(nwr.cpu().numpy(), hp.wr)


# ------------------------------------------------------------------ standalone conv decode

@pytest.mark.parametrize("bias,act,twin", [(False, True, True), (True, True, True), (False, False, True),
                                           (True, False, False)])
def test_conv_decode_matches_oracle(gdn, torch, bias, act, twin):
    t = torch
    rng = np.random.Generator(np.random.PCG64(11))
    B, C, N = 7, 6144 + 40, 17
    w = gi.bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(np.float32))
    b = gi.bf16_bits(rng.standard_normal(C).astype(np.float32)) if bias else None
    cs = np.zeros((N, 3, C), np.uint16)
    cs[1:] = gi.bf16_bits(rng.standard_normal((N - 1, 3, C)).astype(np.float32))
    # strided rows: x and out rows padded past C
    xs = gi.bf16_bits(rng.standard_normal((B, C + 24)).astype(np.float32))
    rd = np.array([3, 0, 5, 7, 9, 0, 1], np.int32)
    wr = np.array([4, 0, 6, 8, 10, 0, 2], np.int32) if twin else rd.copy()
    cs_dev = H.bf16_dev(cs)
    out = t.zeros((B, C + 8), dtype=t.bfloat16, device="cuda")
    before = cs_dev.clone()
    gdn.conv_decode(H.bf16_dev(xs)[:, :], H.bf16_dev(w), None if b is None else H.bf16_dev(b), cs_dev,
                    t.from_numpy(rd).cuda(), t.from_numpy(wr).cuda() if twin else None, out, activation=act)
    cs_ref = cs.copy()
    ref = oracle.conv_decode(np.ascontiguousarray(xs), w, b, cs_ref, rd, wr if twin else None, act=act)
    t.cuda.synchronize()
    got = H.bf16_host_f64(out[:, :C])
    # output: fp32 arithmetic rounded once to bf16 -> within one bf16 ulp of the fp64 value
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(got - ref) <= ulp + 1e-30), np.max(np.abs(got - ref) / ulp)
    np.testing.assert_array_equal(H.bf16_host(cs_dev), cs_ref)
    # padding rows zero; the read slot stays as it was in twin mode
    assert np.all(got[[1, 5]] == 0)
    if twin:
        for r in rd[rd != 0]:
            assert t.equal(cs_dev[int(r)].view(t.int16), before[int(r)].view(t.int16))


# ------------------------------------------------------------------ slot lifecycle

def test_slot_reset_and_copy_match_oracle(gdn, torch):
    t = torch
    case = gi.small(B=8, T=1, H_k=2, H_v=4, d=128, N=21, seed=41)
    s, pool = case.shape, case.pools[0]
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    reset = np.array([3, 0, 17, 25, -2, 8], np.int32)         # 0, 25 and -2 are skipped
    src = np.array([1, 2, 0, 9, 30], np.int32)
    dst = np.array([11, 12, 13, 0, 14], np.int32)             # dst 0 and src 30 are skipped
    gdn.slot_reset(dp.state, dp.conv_state, t.from_numpy(reset).cuda(), H_k=s.H_k)
    oracle.slot_reset(hp.state, hp.conv_state, reset)
    gdn.slot_copy(dp.state, dp.conv_state, t.from_numpy(src).cuda(), t.from_numpy(dst).cuda(), H_k=s.H_k)
    oracle.slot_copy(hp.state, hp.conv_state, src, dst)
    t.cuda.synchronize()
    np.testing.assert_array_equal(dp.state.cpu().numpy().view(np.uint32), hp.state.view(np.uint32))
    np.testing.assert_array_equal(H.bf16_host(dp.conv_state), hp.conv_state)
    assert t.count_nonzero(dp.state[0].view(t.int32)) == 0


@pytest.mark.parametrize("H_k,H_v,d,d_v,pairs", [
    (3, 3, 64, 64, 9),      # 48 KiB of state a slot
    (5, 5, 128, 128, 7),    # 320 KiB
    (2, 6, 128, 64, 13),    # 192 KiB, two value heads a key head
    (1, 3, 64, 128, 40),    # 96 KiB, 40 pairs
])
def test_slot_copy_shapes_match_oracle(gdn, torch, H_k, H_v, d, d_v, pairs):
    """Slot copies over several slot sizes and pair counts, with skipped pairs
    among them: the whole pool bit for bit against the oracle."""
    t = torch
    N = 2 * pairs + 3
    case = gi.small(B=2, T=1, H_k=H_k, H_v=H_v, d=d, d_v=d_v, N=N, seed=97 + pairs)
    s, pool = case.shape, case.pools[0]
    dp, hp = H.DevPool(pool), H.HostPool(pool)
    rng = np.random.default_rng(pairs)
    perm = rng.permutation(np.arange(1, N)).astype(np.int32)
    src, dst = perm[:pairs].copy(), perm[pairs:2 * pairs].copy()
    # a copy from the null slot; skipped: dst 0, src out of range, dst negative
    src[1], dst[2], src[3], dst[4] = 0, 0, N + 4, -1
    gdn.slot_copy(dp.state, dp.conv_state, t.from_numpy(src).cuda(), t.from_numpy(dst).cuda(), H_k=s.H_k)
    oracle.slot_copy(hp.state, hp.conv_state, src, dst)
    t.cuda.synchronize()
    np.testing.assert_array_equal(dp.state.cpu().numpy().view(np.uint32), hp.state.view(np.uint32))
    np.testing.assert_array_equal(H.bf16_host(dp.conv_state), hp.conv_state)
    assert t.count_nonzero(dp.state[0].view(t.int32)) == 0


def test_forked_slot_steps_like_its_source(gdn, torch):
    """A snapshot made with slot_copy steps bit-identically to the slot it was
    copied from (PR #1139 "Tests": forks read the right slot)."""
    t = torch
    case = gi.qwen08b(B=4, seed=3)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp = H.DevPool(pool)
    src = t.from_numpy(pool.read_slot.copy()).cuda()
    free = [sl for sl in range(s.N - 1, 0, -1) if sl not in set(pool.read_slot.tolist())][:4]
    forks = t.from_numpy(np.array(free, np.int32)).cuda()
    gdn.slot_copy(dp.state, dp.conv_state, src, forks, H_k=s.H_k)
    o1 = t.empty((4, 1, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    o2 = t.empty_like(o1)
    x, g, beta = H.bf16_dev(step.x), t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda()
    gdn.gdn_decode_step(x, dp.conv_w, None, dp.conv_state, dp.state, g, beta, src, None, o1, H_k=s.H_k)
    gdn.gdn_decode_step(x, dp.conv_w, None, dp.conv_state, dp.state, g, beta, forks, None, o2, H_k=s.H_k)
    t.cuda.synchronize()
    assert t.equal(o1.view(t.int16), o2.view(t.int16))
    assert t.equal(dp.state[src.long()].view(t.int32), dp.state[forks.long()].view(t.int32))
    assert t.equal(dp.conv_state[src.long()].view(t.int16), dp.conv_state[forks.long()].view(t.int16))


# ------------------------------------------------------------------ slot commit

def test_slot_commit(gdn, torch):
    t = torch
    rd0 = np.array([1, 0, 5, 7, 9], np.int32)
    wr0 = np.array([2, 0, 6, 7, 10], np.int32)
    rd, wr = t.from_numpy(rd0).cuda(), t.from_numpy(wr0).cuda()
    gdn.slot_commit(rd, wr)
    t.cuda.synchronize()
    np.testing.assert_array_equal(rd.cpu().numpy(), wr0)
    np.testing.assert_array_equal(wr.cpu().numpy(), rd0)
    gdn.slot_commit(rd, wr)
    t.cuda.synchronize()
    np.testing.assert_array_equal(rd.cpu().numpy(), rd0)
    np.testing.assert_array_equal(wr.cpu().numpy(), wr0)
    # more rows than one launch's threads: the grid-stride loop covers them all
    ar = t.arange(1, 300001, dtype=t.int32, device="cuda")
    big, big2 = ar.clone(), ar + 7
    gdn.slot_commit(big, big2)
    t.cuda.synchronize()
    assert t.equal(big, ar + 7)
    assert t.equal(big2, ar)


# ------------------------------------------------------------------ edge cases

def test_empty_step_is_a_no_op(gdn, torch):
    t = torch
    case = gi.small(B=2, T=1, H_k=2, H_v=2, d=64)
    s, pool = case.shape, case.pools[0]
    dp = H.DevPool(pool)
    before = dp.state.clone()
    out = t.empty((0, 1, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    gdn.gdn_decode_step(t.empty((0, 1, s.C), dtype=t.bfloat16, device="cuda"), dp.conv_w, None, dp.conv_state,
                        dp.state, t.empty((0, 1, s.H_v), device="cuda"), t.empty((0, 1, s.H_v), device="cuda"),
                        dp.rd[:0], dp.wr[:0], out, H_k=s.H_k)
    gdn.slot_commit(dp.rd[:0], dp.wr[:0])
    t.cuda.synchronize()
    assert t.equal(before, dp.state)


def test_unusable_slots_give_nan_and_touch_nothing(gdn, torch):
    """Rows with an unusable slot read out NaN and touch no pool memory: a read
    slot out of range, a twin row writing over its own read slot, and a real
    twin row whose write slot is the null slot (slot 0 holds no row)."""
    t = torch
    case = gi.small(B=4, T=1, H_k=2, H_v=2, d=64, N=11)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp = H.DevPool(pool)
    rd = pool.read_slot.copy()
    wr = pool.write_slot.copy()
    rd[1] = s.N + 5      # out of range
    wr[2] = rd[2]        # twin row writing over its own read slot
    wr[3] = 0            # real twin row writing into the null slot
    dp.rd, dp.wr = t.from_numpy(rd).cuda(), t.from_numpy(wr).cuda()
    before_s, before_c = dp.state.clone(), dp.conv_state.clone()
    out = H.gpu_step(gdn, dp, step, s)
    t.cuda.synchronize()
    o = H.bf16_host_f64(out)
    assert np.isnan(o[1:]).all() and not np.isnan(o[0]).any()
    mask = t.ones(s.N, dtype=t.bool, device="cuda")
    mask[int(wr[0])] = False
    assert t.equal(dp.state[mask], before_s[mask])
    assert t.equal(dp.conv_state[mask].view(t.int16), before_c[mask].view(t.int16))
    assert t.count_nonzero(dp.state[0].view(t.int32)) == 0 and t.count_nonzero(dp.conv_state[0].view(t.int16)) == 0


def test_conv_decode_never_writes_the_null_slot(gdn, torch):
    """conv_decode with a real row whose write slot is 0: NaN outputs, no slot
    touched; the other rows match the oracle and slot 0 stays zero."""
    t = torch
    case = gi.small(B=3, T=1, H_k=2, H_v=2, d=64, N=9, seed=4)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    rd = pool.read_slot.copy()
    wr = pool.write_slot.copy()
    wr[1] = 0
    cs = H.bf16_dev(pool.conv_state)
    before = cs.clone()
    x = H.bf16_dev(np.ascontiguousarray(step.x[:, 0]))
    out = t.empty((s.B, s.C), dtype=t.bfloat16, device="cuda")
    gdn.conv_decode(x, H.bf16_dev(pool.conv_w), None, cs, t.from_numpy(rd).cuda(), t.from_numpy(wr).cuda(), out)
    t.cuda.synchronize()
    o = H.bf16_host_f64(out)
    assert np.isnan(o[1]).all() and not np.isnan(o[[0, 2]]).any()
    keep = [0, 2]
    hcs = pool.conv_state.copy()
    ref = oracle.conv_decode(np.ascontiguousarray(step.x[keep, 0]), pool.conv_w, None, hcs,
                             np.ascontiguousarray(rd[keep]), np.ascontiguousarray(wr[keep]), act=True)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    assert np.all(np.abs(o[keep] - ref) <= ulp + 1e-30)
    mask = t.ones(s.N, dtype=t.bool, device="cuda")
    mask[[int(wr[0]), int(wr[2])]] = False
    assert t.equal(cs[mask].view(t.int16), before[mask].view(t.int16))
    np.testing.assert_array_equal(H.bf16_host(cs[[int(wr[0]), int(wr[2])]]), hcs[[int(wr[0]), int(wr[2])]])


def test_refusals_through_the_binding(gdn, torch):
    t = torch
    case = gi.small(B=2, T=2, H_k=2, H_v=2, d=64)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp = H.DevPool(pool)
    with pytest.raises(gdn.GdnError) as e:
        H.gpu_step(gdn, dp, step, s, twin=True)
    assert e.value.status == 4


# ------------------------------------------------------------------ graph capture

def test_graph_replay_of_step_and_commit_matches_eager(gdn, torch):
    """Step + commit captured once and replayed several times, with eager work
    between replays, gives the bits of the same steps run eagerly."""
    t = torch
    case = gi.small(B=16, T=1, H_k=4, H_v=4, d=128, steps=1, seed=21)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    dp_e, dp_g = H.DevPool(pool), H.DevPool(pool)
    x, g, beta = H.bf16_dev(step.x), t.from_numpy(step.g).cuda(), t.from_numpy(step.beta).cuda()
    out_e = t.empty((s.B, 1, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")
    out_g = t.empty_like(out_e)

    def run(dp, out):
        gdn.gdn_decode_step(x, dp.conv_w, None, dp.conv_state, dp.state, g, beta, dp.rd, dp.wr, out, H_k=s.H_k)
        gdn.slot_commit(dp.rd, dp.wr)

    stream = t.cuda.Stream()
    graph = t.cuda.CUDAGraph()
    # capture on a copy of the pool that is then reset, so the first replay starts from the initial state
    with t.cuda.stream(stream):
        run(dp_g, out_g)  # warm-up outside capture
    t.cuda.synchronize()
    dp_g.state.copy_(t.from_numpy(pool.state).cuda())
    dp_g.conv_state.copy_(H.bf16_dev(pool.conv_state))
    dp_g.rd.copy_(t.from_numpy(pool.read_slot).cuda())
    dp_g.wr.copy_(t.from_numpy(pool.write_slot).cuda())
    t.cuda.synchronize()
    with t.cuda.graph(graph, stream=stream):
        run(dp_g, out_g)
    t.cuda.synchronize()
    # capture does not execute: the pool must still be the initial one
    assert t.equal(dp_g.state, t.from_numpy(pool.state).cuda())
    for k in range(4):
        run(dp_e, out_e)
        graph.replay()
        t.cuda.synchronize()
        _ = (dp_e.state.sum() + 1).item()  # eager work between replays
        assert t.equal(out_g.view(t.int16), out_e.view(t.int16)), f"replay {k}"
        assert t.equal(dp_g.state.view(t.int32), dp_e.state.view(t.int32)), f"replay {k}"
        assert t.equal(dp_g.rd, dp_e.rd) and t.equal(dp_g.wr, dp_e.wr)


# ------------------------------------------------------------------ calibration probe

PROBE_DESIGNS = {
    "tile1": dict(shape="tile1"),
    "tile1-workgroup-sc0sc1": dict(shape="tile1", order="workgroup", policy="sc0sc1"),
    "tile2-workgroup": dict(shape="tile2", order="workgroup"),
    "tile4": dict(shape="tile4"),
    "tile4-lane-plain": dict(shape="tile4", order="lane", policy="plain"),
    "chunk256x16": dict(shape="chunk", threads=256, loads=16),
    "chunk256x4-lane": dict(shape="chunk", threads=256, loads=4, order="lane"),
    "chunk256x1": dict(shape="chunk", threads=256, loads=1),
    "chunk512x8-workgroup": dict(shape="chunk", threads=512, loads=8, order="workgroup"),
    "chunk1024x4-plain": dict(shape="chunk", threads=1024, loads=4, policy="plain"),
    "chunk1024x1-sc0sc1": dict(shape="chunk", threads=1024, loads=1, policy="sc0sc1"),
    "chunk256x8-persistent2": dict(shape="chunk", threads=256, loads=8, persistent=2),
}


@pytest.mark.parametrize("design", list(PROBE_DESIGNS))
def test_traffic_probe_moves_the_tiles(gdn, torch, design):
    """Every calibration design moves exactly the step's tiles: a copy puts each
    read tile in its write slot, write-only fills the write slots, read-only and
    in-place traffic leave the pool as it was, and nothing else changes; the
    contiguous layout copies consecutive slots and is a no-op past the pool."""
    t = torch
    kw = PROBE_DESIGNS[design]
    hold = 0 if kw.get("persistent") else 2000
    case = gi.small(B=5, T=1, H_k=2, H_v=2, d=128, N=15)
    pool = case.pools[0]
    dp = H.DevPool(pool)
    sink = t.zeros(1, device="cuda")
    rd = [int(x) for x in pool.read_slot]
    wr = [int(x) for x in pool.write_slot]
    others = [sl for sl in range(15) if sl not in wr]
    before = dp.state.clone()
    gdn.traffic_probe(dp.state, dp.rd, dp.wr, sink, traffic="copy", **kw)
    t.cuda.synchronize()
    assert t.equal(dp.state[wr], before[rd])
    assert t.equal(dp.state[others], before[others])
    gdn.traffic_probe(dp.state, dp.rd, dp.wr, sink, traffic="write", hold_ns=hold, **kw)
    t.cuda.synchronize()
    assert bool((dp.state[wr] == 1.0).all())
    assert t.equal(dp.state[others], before[others])
    mid = dp.state.clone()
    gdn.traffic_probe(dp.state, dp.rd, None, sink, traffic="inplace", **kw)
    gdn.traffic_probe(dp.state, dp.rd, None, sink, traffic="read", **kw)
    t.cuda.synchronize()
    assert t.equal(mid, dp.state)
    assert float(sink[0]) == 0.0
    base = t.tensor([2, 7], dtype=t.int32, device="cuda")
    gdn.traffic_probe(dp.state, base[0:1], base[1:2], sink, traffic="copy", layout="contiguous", rows=3,
                      **kw)   # slots 2..4 -> 7..9
    t.cuda.synchronize()
    assert t.equal(dp.state[7:10], mid[2:5])
    assert t.equal(dp.state[:7], mid[:7]) and t.equal(dp.state[10:], mid[10:])
    gdn.traffic_probe(dp.state, base[1:2], base[0:1], sink, traffic="copy", layout="contiguous", rows=9,
                      **kw)   # 7..15 runs past N = 15: no-op
    t.cuda.synchronize()
    assert t.equal(dp.state[:7], mid[:7])


def test_persistent_probe_walks_every_chunk(gdn, torch):
    """A persistent grid smaller than the chunk count (one 256-thread
    workgroup a CU over 40 rows x 4 heads in 4 KiB chunks: 2560 chunks) still
    copies every tile once and touches nothing else."""
    t = torch
    case = gi.small(B=40, T=1, H_k=4, H_v=4, d=128)
    pool = case.pools[0]
    dp = H.DevPool(pool)
    sink = t.zeros(1, device="cuda")
    rd = [int(x) for x in pool.read_slot]
    wr = [int(x) for x in pool.write_slot]
    others = [sl for sl in range(pool.state.shape[0]) if sl not in wr]
    before = dp.state.clone()
    gdn.traffic_probe(dp.state, dp.rd, dp.wr, sink, traffic="copy", shape="chunk", threads=256, loads=1,
                      persistent=1)
    t.cuda.synchronize()
    assert t.equal(dp.state[wr], before[rd])
    assert t.equal(dp.state[others], before[others])


def test_launch_floor_probes_run(gdn, torch):
    t = torch
    state = t.zeros((3, 2, 128, 128), device="cuda")
    rd = t.tensor([1], dtype=t.int32, device="cuda")
    sink = t.zeros(1, device="cuda")
    gdn.traffic_probe(state, rd, None, sink, traffic="read", shape="empty")
    gdn.traffic_probe(state, rd, None, sink, traffic="read", shape="slot_load")
    t.cuda.synchronize()
    assert float(sink[0]) == 0.0
