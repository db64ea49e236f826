"""Properties of the oracle over drawn shapes and values (hypothesis), CPU only.

These pin the oracle's delta rule by the geometry of the update rather than by
its formula: with k^ a unit key, alpha = e^g and S' the updated state,
  - every direction w orthogonal to k^ only decays:  w^T S' = alpha w^T S;
  - along k^ the new value interpolates between the decayed prediction and the
    target:  S'^T k^ = (1 - beta) alpha S^T k^ + beta v;
  - the read-out uses the updated state:  o = S'^T q^.
Together they fix S' (the first two give S'^T on a basis), so a dropped decay,
a transposed outer product, a wrong sign or the read-out taken before the
update each fails one of them.  The L2 norm and the conv tap are pinned by
unit length and scaling, and by a direct convolution of the token sequence.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None)


def _unit(x):
    return x / np.linalg.norm(x)


def _orthonormal_complement(k):
    """An orthonormal basis of the complement of unit vector k (rows)."""
    q, _ = np.linalg.qr(np.column_stack([k, np.eye(k.size)[:, :k.size - 1]]))
    return q[:, 1:].T


@SETTINGS
@given(dk=st.integers(2, 12), dv=st.integers(1, 12), seed=st.integers(0, 2**32 - 1),
       g=st.floats(-6.0, 0.0), beta=st.floats(0.0, 2.0))
def test_update_decays_only_orthogonal_to_the_key(dk, dv, seed, g, beta):
    rng = np.random.Generator(np.random.PCG64(seed))
    S0 = rng.standard_normal((dk, dv))
    q, k, v = _unit(rng.standard_normal(dk)), _unit(rng.standard_normal(dk)), rng.standard_normal(dv)
    S = S0.copy()
    oracle.delta_rule(S, q, k, v, g, beta)
    W = _orthonormal_complement(k)
    np.testing.assert_allclose(W @ S, np.exp(g) * (W @ S0), rtol=1e-10, atol=1e-10)


@SETTINGS
@given(dk=st.integers(1, 12), dv=st.integers(1, 12), seed=st.integers(0, 2**32 - 1),
       g=st.floats(-6.0, 0.0), beta=st.floats(0.0, 2.0))
def test_update_along_the_key_interpolates_to_the_target(dk, dv, seed, g, beta):
    rng = np.random.Generator(np.random.PCG64(seed))
    S0 = rng.standard_normal((dk, dv))
    q, k, v = _unit(rng.standard_normal(dk)), _unit(rng.standard_normal(dk)), rng.standard_normal(dv)
    S = S0.copy()
    oracle.delta_rule(S, q, k, v, g, beta)
    alpha = np.exp(g)
    np.testing.assert_allclose(S.T @ k, (1 - beta) * alpha * (S0.T @ k) + beta * v, rtol=1e-10, atol=1e-10)


@SETTINGS
@given(dk=st.integers(1, 12), dv=st.integers(1, 12), seed=st.integers(0, 2**32 - 1),
       g=st.floats(-6.0, 0.0), beta=st.floats(0.0, 2.0))
def test_read_out_uses_the_updated_state(dk, dv, seed, g, beta):
    rng = np.random.Generator(np.random.PCG64(seed))
    S = rng.standard_normal((dk, dv))
    q, k, v = _unit(rng.standard_normal(dk)), _unit(rng.standard_normal(dk)), rng.standard_normal(dv)
    o = oracle.delta_rule(S, q, k, v, g, beta)
    np.testing.assert_allclose(o, S.T @ q, rtol=1e-10, atol=1e-10)


@SETTINGS
@given(n=st.integers(1, 64), seed=st.integers(0, 2**32 - 1), scale=st.floats(0.01, 100.0))
def test_l2norm_gives_unit_vectors_that_scale(n, seed, scale):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(n) * 10.0 + 0.1  # |x|^2 far above eps
    y = oracle.l2norm(x, 1e-12)
    np.testing.assert_allclose(np.linalg.norm(y), 1.0, rtol=1e-9)
    np.testing.assert_allclose(oracle.l2norm(x, 1e-12, scale), scale * y, rtol=1e-12)
    np.testing.assert_allclose(oracle.l2norm(3.0 * x, 1e-12), y, rtol=1e-9)  # direction only


def _bf16_bits(a):
    """fp32 values -> bf16 bit patterns, round to nearest even (inputs here are finite)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@SETTINGS
@given(C=st.integers(1, 24), T=st.integers(1, 9), seed=st.integers(0, 2**32 - 1))
def test_conv_tokens_equal_a_direct_convolution(C, T, seed):
    """T conv tokens from a zero window equal, per channel, the causal
    convolution of the token sequence with the taps (last tap on the current
    token), computed directly; SiLU off."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = 4
    w = _bf16_bits(rng.uniform(-0.5, 0.5, (C, W)).astype(np.float32))
    x = _bf16_bits(rng.standard_normal((T, C)).astype(np.float32))
    win = np.zeros((W - 1, C), np.float64)
    got = np.stack([oracle.conv_token(w, None, win, x[t], False) for t in range(T)])
    wf, xf = _bf16_value(w), _bf16_value(x)
    padded = np.vstack([np.zeros((W - 1, C)), xf])
    want = np.stack([sum(wf[:, j] * padded[t + j] for j in range(W)) for t in range(T)])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
