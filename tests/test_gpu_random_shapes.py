"""GPU parity over shapes drawn at random (a fixed seed, so the same cases every
run): key heads, grouping, head dims, rows, tokens, write mode and padding for
the decode step; heads, head dims and ragged prompt lengths (with empty and
padding prompts) for both prefill paths, and for the two-pass prefill's slim
layout (256 or 512 prompt-head pairs).  Each case is checked as the named
cases are: outputs, every written slot and the untouched rest of the pool
against the oracle, to the bars in tests/helpers.py.
"""
import numpy as np
import pytest

import gdn_inputs as gi
from tests.test_gpu_parity import _check_step
from tests.test_gpu_prefill import _check

pytestmark = pytest.mark.gpu


def _decode_cases(n=24, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        hk = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 4]))
        d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        twin = bool(rng.integers(0, 2))
        T = 1 if twin else int(rng.integers(1, 5))
        B = int(rng.integers(1, 41))
        real = int(rng.integers(0, B + 1)) if rng.random() < 0.3 else None  # some rows on slot 0
        cases.append((B, T, hk, hk * G, d, dv, twin, real, 100 + i))
    return cases


def _prefill_cases(n=12, seed=2025):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        hk = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4]))
        d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        B = int(rng.integers(1, 13))
        lengths = [int(v) for v in rng.integers(0, 101, size=B)]
        pad = tuple(int(b) for b in np.flatnonzero(rng.random(B) < 0.15))
        cases.append((tuple(lengths), hk, hk * G, d, dv, pad, 200 + i))
    return cases


def _slim_cases(n=8, seed=2026):
    """Prompt sets of 256 or 512 prompt-head pairs (B H_v), where the two-pass
    prefill takes its slim layout."""
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for i in range(n):
        hk = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4]))
        d, dv = int(rng.choice([64, 128])), int(rng.choice([64, 128]))
        B = 256 * int(rng.integers(1, 3)) // (hk * G)
        lengths = [int(v) for v in rng.integers(0, 71, size=B)]
        pad = tuple(int(b) for b in np.flatnonzero(rng.random(B) < 0.1))
        cases.append((tuple(lengths), hk, hk * G, d, dv, pad, 300 + i))
    return cases


DECODE = _decode_cases()
PREFILL = _prefill_cases()
SLIM = _slim_cases()


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


@pytest.mark.parametrize("B,T,hk,hv,d,dv,twin,real,seed", DECODE,
                         ids=[f"B{c[0]}-T{c[1]}-{c[2]}x{c[3]}-d{c[4]}x{c[5]}-{'twin' if c[6] else 'inplace'}"
                              f"{'' if c[7] is None else f'-real{c[7]}'}" for c in DECODE])
def test_decode_random_shape(gdn, torch, B, T, hk, hv, d, dv, twin, real, seed):
    case = gi.small(B, T, hk, hv, d, twin=twin, real_rows=real, seed=seed, d_v=dv)
    _check_step(gdn, case, twin=twin)


@pytest.mark.parametrize("two_pass", [False, True], ids=["one-kernel", "two-pass"])
@pytest.mark.parametrize("lengths,hk,hv,d,dv,pad,seed", PREFILL,
                         ids=[f"{len(c[0])}seq-{c[1]}x{c[2]}-d{c[3]}x{c[4]}" for c in PREFILL])
def test_prefill_random_shape(gdn, torch, lengths, hk, hv, d, dv, pad, seed, two_pass):
    case = gi.prefill(list(lengths), H_k=hk, H_v=hv, d=d, d_v=dv, pad=pad, seed=seed)
    _check(gdn, torch, case, two_pass=two_pass)


@pytest.mark.parametrize("lengths,hk,hv,d,dv,pad,seed", SLIM,
                         ids=[f"{len(c[0])}seq-{c[1]}x{c[2]}-d{c[3]}x{c[4]}" for c in SLIM])
def test_prefill_slim_random_shape(gdn, torch, lengths, hk, hv, d, dv, pad, seed):
    assert len(lengths) * hv in (256, 512)
    case = gi.prefill(list(lengths), H_k=hk, H_v=hv, d=d, d_v=dv, pad=pad, seed=seed)
    _check(gdn, torch, case, two_pass=True)
