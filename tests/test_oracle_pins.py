"""Pins of the fp64 CPU oracle to things other than itself (CPU only).

Each test ties one oracle function to a closed form, an invariant of the
mathematics, a library routine or a hand-worked example, so that a plausible
slip in the oracle (a dropped term, a wrong sign, a transposed operand, a wrong
head or slot index) fails at least one of them:

  SiLU          scipy.special.expit(y) * y, the odd-part identity, printed values
  L2 norm       hand-worked values, unit norm, parallel to the input
  conv          numpy.convolve over a whole sequence from zero history (tap
                order), window = last W-1 inputs, null slot, write slot
  delta rule    golden 2x2 worked example; beta = 0 (pure decay); unit key with
                g = 0, beta = 1 (S'^T k = v); alpha = 0 (S' = beta k v^T);
                beta = 2, v = 0 (Householder reflection); brute-force product
                form A_T...A_1 S_0 + sum ... over 8 tokens
  step          beta = 0 decays every head by its own gate; g = 0, beta = 1
                gives S'^T k = v with k, v taken from the pinned pieces (pins the
                q|k|v slicing and the value-head -> key-head grouping); o = S'^T q;
                q_scale scales o only; twin == in place; padding rows and slot 0;
                only real rows' write slots change; T tokens in place == T
                single-token steps (to fp32 rounding); commit swaps.
"""
import os

import numpy as np
import pytest
import scipy.special

import gdn_inputs as gi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=1):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(v):
    return v / np.linalg.norm(v)


# ------------------------------------------------------------------ SiLU

def test_silu_matches_library_logistic():
    ys = np.linspace(-30, 30, 241)
    got = np.array([oracle.silu(y) for y in ys])
    np.testing.assert_allclose(got, scipy.special.expit(ys) * ys, rtol=1e-15, atol=1e-300)


def test_silu_printed_values_and_identity():
    # sigmoid(1) = 0.7310585786300049, sigmoid(2) = 0.8807970779778823 (standard tables)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert oracle.silu(2.0) == pytest.approx(2 * 0.8807970779778823, rel=1e-15)
    for y in (0.3, 1.7, 5.0):
        # sigmoid(y) + sigmoid(-y) = 1  =>  silu(y) - silu(-y) = y
        assert oracle.silu(y) - oracle.silu(-y) == pytest.approx(y, rel=1e-14)


# ------------------------------------------------------------------ L2 norm

def test_l2norm_worked_values():
    np.testing.assert_array_equal(oracle.l2norm(np.array([3.0, 4.0]), 0.0), [0.6, 0.8])
    # sqrt(25 + 11) = 6
    np.testing.assert_allclose(oracle.l2norm(np.array([3.0, 4.0]), 11.0), [0.5, 4 / 6], rtol=1e-15)
    np.testing.assert_allclose(oracle.l2norm(np.array([3.0, 4.0]), 0.0, scale=0.5), [0.3, 0.4], rtol=1e-15)
    np.testing.assert_array_equal(oracle.l2norm(np.zeros(8), 1e-6), np.zeros(8))


def test_l2norm_unit_and_parallel():
    x = _rng().standard_normal(128)
    y = oracle.l2norm(x, 1e-12)
    assert np.linalg.norm(y) == pytest.approx(1.0, abs=1e-12)
    np.testing.assert_allclose(y * np.linalg.norm(x), x, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ conv decode

@pytest.mark.parametrize("with_bias", [False, True])
def test_conv_token_sequence_equals_library_convolution(with_bias):
    """Decoding T tokens one at a time from a zero window equals a causal
    depthwise convolution of the whole sequence (numpy.convolve per channel)."""
    rng = _rng(2)
    C, W, T = 24, 4, 11
    w = gi.bf16_bits(rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32))
    b = gi.bf16_bits(rng.standard_normal(C).astype(np.float32)) if with_bias else None
    xs = gi.bf16_bits(rng.standard_normal((T, C)).astype(np.float32))
    wf = gi.bf16_to_f32(w).astype(np.float64)
    xf = gi.bf16_to_f32(xs).astype(np.float64)
    bf = gi.bf16_to_f32(b).astype(np.float64) if with_bias else np.zeros(C)
    win = np.zeros((W - 1, C))
    for t in range(T):
        y = oracle.conv_token(w, b, win, np.ascontiguousarray(xs[t]), act=False)
        for c in range(C):
            ref = np.convolve(xf[:, c], wf[c, ::-1])[t] + bf[c]
            assert y[c] == pytest.approx(ref, rel=1e-13, abs=1e-13)
        # the window holds the last W-1 inputs, oldest first
        lo = max(0, t - (W - 2))
        hist = xf[lo:t + 1]
        np.testing.assert_array_equal(win[W - 1 - len(hist):], hist)
    # with activation, y is the SiLU of the same pre-activation
    win2 = np.zeros((W - 1, C))
    y2 = oracle.conv_token(w, b, win2, np.ascontiguousarray(xs[0]), act=True)
    pre = wf[:, W - 1] * xf[0] + bf
    np.testing.assert_allclose(y2, scipy.special.expit(pre) * pre, rtol=1e-13, atol=1e-15)


def test_pooled_conv_decode_slots():
    rng = _rng(3)
    C, W, N = 16, 4, 7
    w = gi.bf16_bits(rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32))
    cs = np.zeros((N, W - 1, C), np.uint16)
    cs[1:] = gi.bf16_bits(rng.standard_normal((N - 1, W - 1, C)).astype(np.float32))
    x = gi.bf16_bits(rng.standard_normal((3, C)).astype(np.float32))
    rd = np.array([1, 0, 3], np.int32)
    wr = np.array([2, 0, 4], np.int32)
    before = cs.copy()
    y = oracle.conv_decode(x, w, None, cs, rd, wr, act=True)
    # padding row: zero output; read slots and slot 0 untouched
    np.testing.assert_array_equal(y[1], 0.0)
    for s in (0, 1, 3, 5, 6):
        np.testing.assert_array_equal(cs[s], before[s])
    # write slot holds the read window shifted by one with x appended (bytes exact)
    np.testing.assert_array_equal(cs[2][:W - 2], before[1][1:])
    np.testing.assert_array_equal(cs[2][W - 2], x[0])
    np.testing.assert_array_equal(cs[4][W - 2], x[2])
    # in place gives the same values and the same window bytes
    cs2 = before.copy()
    y2 = oracle.conv_decode(x, w, None, cs2, rd, None, act=True)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(cs2[1], cs[2])
    np.testing.assert_array_equal(cs2[3], cs[4])


# ------------------------------------------------------------------ delta rule

def _golden_cases():
    rows = []
    with open(os.path.join(GOLDEN, "delta_rule_2x2.txt")) as f:
        for line in f:
            if not line.strip() or line.startswith("#"):
                continue
            head, k, v, q, S, S1, o = [p.split() for p in line.split("|")]
            rows.append(dict(name=head[0], g=float(head[1]), beta=float(head[2]),
                             k=np.array(k, float), v=np.array(v, float), q=np.array(q, float),
                             S=np.array(S, float).reshape(2, 2), S1=np.array(S1, float).reshape(2, 2),
                             o=np.array(o, float)))
    return rows


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_delta_rule_golden_worked_example(case):
    S = case["S"].copy()
    o = oracle.delta_rule(S, case["q"], case["k"], case["v"], case["g"], case["beta"])
    np.testing.assert_allclose(S, case["S1"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14)


def test_delta_rule_beta_zero_is_pure_decay():
    rng = _rng(4)
    S0 = rng.standard_normal((64, 48))
    q, k, v = _unit(rng.standard_normal(64)), _unit(rng.standard_normal(64)), rng.standard_normal(48)
    g = -0.37
    S = S0.copy()
    o = oracle.delta_rule(S, q, k, v, g, 0.0)
    np.testing.assert_array_equal(S, S0 * np.exp(g))
    np.testing.assert_allclose(o, np.exp(g) * (S0.T @ q), rtol=1e-12, atol=1e-12)
    S = S0.copy()
    oracle.delta_rule(S, q, k, v, 0.0, 0.0)
    np.testing.assert_array_equal(S, S0)


def test_delta_rule_unit_key_writes_v():
    """g = 0, beta = 1, |k| = 1: after the update S'^T k = v whatever S was."""
    rng = _rng(5)
    for dk, dv in ((64, 64), (128, 128), (32, 80)):
        S = rng.standard_normal((dk, dv))
        q, k, v = _unit(rng.standard_normal(dk)), _unit(rng.standard_normal(dk)), rng.standard_normal(dv)
        o = oracle.delta_rule(S, q, k, v, 0.0, 1.0)
        np.testing.assert_allclose(S.T @ k, v, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(o, S.T @ q, rtol=1e-12, atol=1e-12)


def test_delta_rule_zero_decay_forgets():
    """alpha = exp(-inf) = 0: S' = beta k v^T, and with q = k the read-out is beta v."""
    rng = _rng(6)
    S = rng.standard_normal((64, 64))
    k = _unit(rng.standard_normal(64))
    v = rng.standard_normal(64)
    o = oracle.delta_rule(S, k, k, v, -np.inf, 0.75)
    np.testing.assert_allclose(S, 0.75 * np.outer(k, v), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(o, 0.75 * v, rtol=1e-13, atol=1e-14)


def test_delta_rule_beta_two_is_householder():
    """beta = 2, g = 0, v = 0: S' = (I - 2 k k^T) S, a reflection: column norms are
    kept, S'^T k = -S^T k, and applying it twice gives S back."""
    rng = _rng(7)
    S0 = rng.standard_normal((128, 128))
    k = _unit(rng.standard_normal(128))
    q = _unit(rng.standard_normal(128))
    S = S0.copy()
    oracle.delta_rule(S, q, k, np.zeros(128), 0.0, 2.0)
    np.testing.assert_allclose(np.linalg.norm(S, axis=0), np.linalg.norm(S0, axis=0), rtol=1e-12)
    np.testing.assert_allclose(S.T @ k, -(S0.T @ k), rtol=1e-11, atol=1e-11)
    oracle.delta_rule(S, q, k, np.zeros(128), 0.0, 2.0)
    np.testing.assert_allclose(S, S0, rtol=1e-11, atol=1e-11)


def test_delta_rule_equals_unrolled_product_form():
    """8 chained tokens equal the brute-force unrolled recurrence
    S_T = A_T...A_1 S_0 + sum_t A_T...A_{t+1} beta_t k_t v_t^T,
    A_t = alpha_t (I - beta_t k_t k_t^T), o_t = S_t^T q_t (explicit d_k x d_k matrices)."""
    rng = _rng(8)
    dk, dv, T = 16, 12, 8
    S0 = rng.standard_normal((dk, dv)) * 0.1
    qs = [_unit(rng.standard_normal(dk)) for _ in range(T)]
    ks = [_unit(rng.standard_normal(dk)) for _ in range(T)]
    vs = [rng.standard_normal(dv) for _ in range(T)]
    gs = -np.logaddexp(0, rng.standard_normal(T))
    bs = scipy.special.expit(rng.standard_normal(T))
    S = S0.copy()
    outs = [oracle.delta_rule(S, qs[t], ks[t], vs[t], gs[t], bs[t]) for t in range(T)]
    A = [np.exp(gs[t]) * (np.eye(dk) - bs[t] * np.outer(ks[t], ks[t])) for t in range(T)]
    for tt in range(1, T + 1):
        P = np.eye(dk)
        for t in range(tt):
            P = A[t] @ P
        ref = P @ S0
        for t in range(tt):
            Q = np.eye(dk)
            for u in range(t + 1, tt):
                Q = A[u] @ Q
            ref = ref + Q @ (bs[t] * np.outer(ks[t], vs[t]))
        np.testing.assert_allclose(outs[tt - 1], ref.T @ qs[tt - 1], rtol=1e-12, atol=1e-12)
        if tt == T:
            np.testing.assert_allclose(S, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ the whole step

def _pieces(case, pool, step, r, t_tokens=1, q_scale=1.0, eps=1e-6):
    """Per-row q-hat, k-hat, v of every token, from the separately pinned conv and L2 pieces."""
    s = case.shape
    win = gi.bf16_to_f32(pool.conv_state[pool.read_slot[r]]).astype(np.float64).copy()
    res = []
    for t in range(t_tokens):
        y = oracle.conv_token(pool.conv_w, None, win, np.ascontiguousarray(step.x[r, t]), act=True)
        qs, ks, vs = [], [], []
        for hv in range(s.H_v):
            hk = hv // s.G
            qs.append(oracle.l2norm(y[hk * s.d_k:(hk + 1) * s.d_k], eps, q_scale))
            ks.append(oracle.l2norm(y[s.H_k * s.d_k + hk * s.d_k:s.H_k * s.d_k + (hk + 1) * s.d_k], eps))
            vs.append(y[2 * s.H_k * s.d_k + hv * s.d_v:2 * s.H_k * s.d_k + (hv + 1) * s.d_v])
        res.append((qs, ks, vs))
    return res


def _run(case, pool, step, twin=True, q_scale=1.0):
    st, cs = pool.state.copy(), pool.conv_state.copy()
    out = oracle.gdn_decode_step(step.x, pool.conv_w, None, cs, st, step.g, step.beta,
                                 pool.read_slot, pool.write_slot if twin else None,
                                 H_k=case.shape.H_k, q_scale=q_scale)
    return out, st, cs


@pytest.mark.parametrize("hk,hv", [(2, 2), (2, 4)])
def test_step_beta_zero_decays_each_head_by_its_gate(hk, hv):
    case = gi.small(B=3, T=1, H_k=hk, H_v=hv, d=64)
    pool, step = case.pools[0], case.steps[0][0]
    step.beta[:] = 0.0
    out, st, _ = _run(case, pool, step)
    for r in range(case.shape.B):
        rs, ws = pool.read_slot[r], pool.write_slot[r]
        for h in range(hv):
            alpha = np.exp(np.float64(step.g[r, 0, h]))
            ref = (alpha * pool.state[rs, h].astype(np.float64)).astype(np.float32)
            np.testing.assert_array_equal(st[ws, h], ref)


@pytest.mark.parametrize("hk,hv,d", [(2, 2, 64), (2, 4, 64), (1, 2, 128)])
def test_step_unit_key_writes_v_and_reads_out_with_q(hk, hv, d):
    """g = 0, beta = 1: each head's new state maps its own normalised key onto its own v;
    the read-out is the new state applied to its normalised query.  Fails on a wrong
    q|k|v slice, a wrong value-head -> key-head grouping or a transposed state."""
    case = gi.small(B=2, T=1, H_k=hk, H_v=hv, d=d)
    pool, step = case.pools[0], case.steps[0][0]
    step.g[:] = 0.0
    step.beta[:] = 1.0
    out, st, _ = _run(case, pool, step, q_scale=0.5)
    for r in range(case.shape.B):
        (qs, ks, vs), = _pieces(case, pool, step, r, q_scale=0.5)
        ws = pool.write_slot[r]
        for h in range(hv):
            S1 = st[ws, h].astype(np.float64)
            np.testing.assert_allclose(S1.T @ ks[h], vs[h], rtol=1e-5, atol=1e-5)
            np.testing.assert_allclose(out[r, 0, h], S1.T @ qs[h], rtol=1e-5, atol=1e-5)


def test_step_q_scale_scales_the_output_only():
    case = gi.small(B=2, T=1, H_k=2, H_v=2, d=64)
    pool, step = case.pools[0], case.steps[0][0]
    o1, s1, c1 = _run(case, pool, step, q_scale=1.0)
    o2, s2, c2 = _run(case, pool, step, q_scale=0.125)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-13, atol=1e-15)


def test_step_twin_equals_in_place_and_touches_no_other_slot():
    case = gi.small(B=4, T=1, H_k=2, H_v=4, d=64, N=13)
    pool, step = case.pools[0], case.steps[0][0]
    o_t, st_t, cs_t = _run(case, pool, step, twin=True)
    o_i, st_i, cs_i = _run(case, pool, step, twin=False)
    np.testing.assert_array_equal(o_t, o_i)
    for r in range(case.shape.B):
        np.testing.assert_array_equal(st_t[pool.write_slot[r]], st_i[pool.read_slot[r]])
        np.testing.assert_array_equal(cs_t[pool.write_slot[r]], cs_i[pool.read_slot[r]])
    changed = {int(s) for s in pool.write_slot}
    for sl in range(case.shape.N):
        if sl not in changed:
            np.testing.assert_array_equal(st_t[sl], pool.state[sl])
            np.testing.assert_array_equal(cs_t[sl], pool.conv_state[sl])


def test_step_padding_rows_sit_on_the_null_slot():
    """Padding rows (slot 0) give zero output, leave slot 0 zero, and the real rows'
    results equal an unpadded run of the same rows bit for bit."""
    case = gi.small(B=6, T=1, H_k=2, H_v=2, d=64, real_rows=3, N=9)
    pool, step = case.pools[0], case.steps[0][0]
    out, st, cs = _run(case, pool, step)
    np.testing.assert_array_equal(out[3:], 0.0)
    assert not np.signbit(out[3:]).any()
    np.testing.assert_array_equal(st[0], 0.0)
    np.testing.assert_array_equal(cs[0], 0)
    st2, cs2 = pool.state.copy(), pool.conv_state.copy()
    out2 = oracle.gdn_decode_step(np.ascontiguousarray(step.x[:3]), pool.conv_w, None, cs2, st2,
                                  np.ascontiguousarray(step.g[:3]), np.ascontiguousarray(step.beta[:3]),
                                  np.ascontiguousarray(pool.read_slot[:3]),
                                  np.ascontiguousarray(pool.write_slot[:3]), H_k=2)
    np.testing.assert_array_equal(out[:3], out2)
    np.testing.assert_array_equal(st, st2)
    np.testing.assert_array_equal(cs, cs2)


def test_real_rows_never_write_the_null_slot():
    """Slot 0 holds no row: the oracle refuses a real twin row whose write slot
    is 0 (or its own read slot), and a standalone conv decode whose real row
    would write slot 0, rather than putting a row's data into the null slot."""
    case = gi.small(B=2, T=1, H_k=2, H_v=2, d=64, N=9)
    pool, step = case.pools[0], case.steps[0][0]
    for bad in (0, int(pool.read_slot[1])):
        wr = pool.write_slot.copy()
        wr[1] = bad
        st, cs = pool.state.copy(), pool.conv_state.copy()
        with pytest.raises(ValueError):
            oracle.gdn_decode_step(step.x, pool.conv_w, None, cs, st, step.g, step.beta, pool.read_slot, wr, H_k=2)
    # padding rows may name slot 0 as their write slot: that is how they sit on it
    rd = pool.read_slot.copy()
    wr = pool.write_slot.copy()
    rd[1], wr[1] = 0, 0
    st, cs = pool.state.copy(), pool.conv_state.copy()
    oracle.gdn_decode_step(step.x, pool.conv_w, None, cs, st, step.g, step.beta, rd, wr, H_k=2)
    np.testing.assert_array_equal(st[0], 0.0)
    x2 = np.ascontiguousarray(step.x[:, 0])
    wr = pool.write_slot.copy()
    wr[0] = 0
    with pytest.raises(ValueError):
        oracle.conv_decode(x2, pool.conv_w, None, pool.conv_state.copy(), pool.read_slot, wr, act=True)


def test_step_multi_token_in_place_equals_chained_single_tokens():
    """T tokens in one in-place call equal T single-token in-place calls; the state
    only differs by the fp32 rounding the chained calls take between tokens."""
    case = gi.small(B=3, T=4, H_k=2, H_v=2, d=64, twin=False)
    pool, step = case.pools[0], case.steps[0][0]
    out4, st4, cs4 = _run(case, pool, step, twin=False)
    st1, cs1 = pool.state.copy(), pool.conv_state.copy()
    for t in range(4):
        o = oracle.gdn_decode_step(np.ascontiguousarray(step.x[:, t:t + 1]), pool.conv_w, None, cs1, st1,
                                   np.ascontiguousarray(step.g[:, t:t + 1]),
                                   np.ascontiguousarray(step.beta[:, t:t + 1]), pool.read_slot, None, H_k=2)
        np.testing.assert_allclose(o[:, 0], out4[:, t], rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(cs1, cs4)
    np.testing.assert_allclose(st1, st4, rtol=1e-6, atol=1e-7)


def test_step_chain_with_commit_matches_pieces():
    """8 twin steps with a commit between: every step reads what the previous wrote,
    checked with the pinned pieces (conv, L2, delta rule) chained by hand."""
    case = gi.tiny()
    s = case.shape
    pool = case.pools[0]
    st, cs = pool.state.copy(), pool.conv_state.copy()
    rd, wr = pool.read_slot.copy(), pool.write_slot.copy()
    # hand chain for row 0 in fp64, rounding the state to fp32 between steps as the pool does
    r = 0
    S = pool.state[rd[r]].astype(np.float64)
    win = gi.bf16_to_f32(pool.conv_state[rd[r]]).astype(np.float64).copy()
    for k in range(8):
        step = case.steps[k][0]
        out = oracle.gdn_decode_step(step.x, pool.conv_w, None, cs, st, step.g, step.beta, rd, wr, H_k=s.H_k)
        y = oracle.conv_token(pool.conv_w, None, win, np.ascontiguousarray(step.x[r, 0]), act=True)
        for h in range(s.H_v):
            q = oracle.l2norm(y[h * s.d_k:(h + 1) * s.d_k], 1e-6)
            kk = oracle.l2norm(y[s.H_k * s.d_k + h * s.d_k:s.H_k * s.d_k + (h + 1) * s.d_k], 1e-6)
            v = y[2 * s.H_k * s.d_k + h * s.d_v:2 * s.H_k * s.d_k + (h + 1) * s.d_v]
            Sh = S[h].copy()
            o = oracle.delta_rule(Sh, q, kk, v, float(step.g[r, 0, h]), float(step.beta[r, 0, h]))
            S[h] = Sh.astype(np.float32)
            np.testing.assert_allclose(out[r, 0, h], o, rtol=1e-6, atol=1e-6)
        np.testing.assert_array_equal(st[wr[r]], S.astype(np.float32))
        oracle.slot_commit(rd, wr)
    # after an even number of commits every pair is back in its first orientation
    np.testing.assert_array_equal(rd, pool.read_slot)
    np.testing.assert_array_equal(wr, pool.write_slot)


def test_slot_commit_swaps_and_is_an_involution():
    rd = np.array([1, 0, 5, 7], np.int32)
    wr = np.array([2, 0, 6, 7], np.int32)
    oracle.slot_commit(rd, wr)
    np.testing.assert_array_equal(rd, [2, 0, 6, 7])
    np.testing.assert_array_equal(wr, [1, 0, 5, 7])
    oracle.slot_commit(rd, wr)
    np.testing.assert_array_equal(rd, [1, 0, 5, 7])
    np.testing.assert_array_equal(wr, [2, 0, 6, 7])


def test_invalid_slot_is_refused():
    case = gi.small(B=2, T=1, H_k=1, H_v=1, d=64)
    pool, step = case.pools[0], case.steps[0][0]
    bad = pool.read_slot.copy()
    bad[1] = case.shape.N
    with pytest.raises(ValueError):
        oracle.gdn_decode_step(step.x, pool.conv_w, None, pool.conv_state.copy(), pool.state.copy(),
                               step.g, step.beta, bad, pool.write_slot, H_k=1)


# ------------------------------------------------------------------ slot lifecycle

def test_slot_reset_zeroes_listed_slots_only():
    case = gi.small(B=3, T=1, H_k=2, H_v=2, d=64, N=9)
    pool = case.pools[0]
    st, cs = pool.state.copy(), pool.conv_state.copy()
    oracle.slot_reset(st, cs, np.array([3, 0, 7, 99, -1], np.int32))
    for s_ in range(9):
        if s_ in (3, 7):
            assert not st[s_].any() and not cs[s_].any()
        else:
            np.testing.assert_array_equal(st[s_], pool.state[s_])
            np.testing.assert_array_equal(cs[s_], pool.conv_state[s_])


def test_slot_copy_then_step_equals_step_on_the_source():
    """A fork made by copying a slot steps exactly like the slot it came from."""
    case = gi.small(B=1, T=1, H_k=2, H_v=2, d=64, N=9)
    pool, step = case.pools[0], case.steps[0][0]
    st, cs = pool.state.copy(), pool.conv_state.copy()
    src, dst = int(pool.read_slot[0]), 5 if int(pool.read_slot[0]) != 5 else 6
    oracle.slot_copy(st, cs, np.array([src, 4], np.int32), np.array([dst, 0], np.int32))
    np.testing.assert_array_equal(st[dst], pool.state[src])
    np.testing.assert_array_equal(cs[dst], pool.conv_state[src])
    np.testing.assert_array_equal(st[0], 0.0)  # the null slot is never written
    o1 = oracle.gdn_decode_step(step.x, pool.conv_w, None, cs, st, step.g, step.beta,
                                np.array([src], np.int32), None, H_k=2)
    o2 = oracle.gdn_decode_step(step.x, pool.conv_w, None, cs, st, step.g, step.beta,
                                np.array([dst], np.int32), None, H_k=2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(st[src], st[dst])


# ------------------------------------------------------------------ a state per token

def test_per_token_states_equal_prefix_steps():
    """The state kept after token t equals an in-place call over the first t+1
    tokens (pins the per-token store: slot, token index, and that the kept
    state is the one after that token, not before it)."""
    case = gi.small(B=2, T=3, H_k=2, H_v=4, d=64, N=13, twin=False)
    pool, step = case.pools[0], case.steps[0][0]
    st, cs = pool.state.copy(), pool.conv_state.copy()
    free = [s_ for s_ in range(1, 13) if s_ not in set(pool.read_slot.tolist())]
    tok = np.array([[free[0], free[1], 0], [free[2], free[3], free[4]]], np.int32)  # row 0 keeps tokens 0, 1
    out = oracle.gdn_decode_step_tokens(step.x, pool.conv_w, None, cs, st, step.g, step.beta, pool.read_slot, tok,
                                        H_k=2)
    for t in range(3):
        st2, cs2 = pool.state.copy(), pool.conv_state.copy()
        o2 = oracle.gdn_decode_step(np.ascontiguousarray(step.x[:, :t + 1]), pool.conv_w, None, cs2, st2,
                                    np.ascontiguousarray(step.g[:, :t + 1]), np.ascontiguousarray(step.beta[:, :t + 1]),
                                    pool.read_slot, None, H_k=2)
        np.testing.assert_array_equal(out[:, :t + 1], o2)
        for r in range(2):
            if tok[r, t]:
                np.testing.assert_array_equal(st[tok[r, t]], st2[pool.read_slot[r]])
                np.testing.assert_array_equal(cs[tok[r, t]], cs2[pool.read_slot[r]])
    # the read slots are not written
    for r in range(2):
        np.testing.assert_array_equal(st[pool.read_slot[r]], pool.state[pool.read_slot[r]])
