"""The oracle's pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/gdn_oracle.c (never in the
real file), builds it, and runs tests/test_oracle_pins.py against it in a
subprocess: the run must fail.  A mistake the pins let through would mean the
oracle is not pinned where that line is.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTATIONS = {
    "delta_sign": ("+= beta * k[i] * (v[j] - pred[j]);", "+= beta * k[i] * (v[j] + pred[j]);"),
    "no_decay": ("S[(size_t)i * dv + j] *= alpha;", "S[(size_t)i * dv + j] *= 1.0;"),
    "pred_transposed": ("s += S[(size_t)i * dv + j] * k[i];", "s += S[(size_t)j * dv + i] * k[i];"),
    "readout_with_key": ("s += S[(size_t)i * dv + j] * q[i];", "s += S[(size_t)i * dv + j] * k[i];"),
    "gqa_modulo": ("int hk = hv / G;", "int hk = hv % H_k;"),
    "q_k_swapped": ("const double *q = y + (size_t)hk * d_k;",
                    "const double *q = y + (size_t)H_k * d_k + (size_t)hk * d_k;"),
    "conv_taps_reversed": ("acc += bf16_bits_to_double(conv_w[(size_t)c * W + w]) * win[(size_t)w * C + c];",
                           "acc += bf16_bits_to_double(conv_w[(size_t)c * W + (W - 2 - w)]) * win[(size_t)w * C + c];"),
    "l2_no_sqrt": ("double den = sqrt(ss + eps);", "double den = (ss + eps);"),
    "silu_sign": ("return y / (1.0 + exp(-y));", "return y / (1.0 + exp(y));"),
    "padding_not_skipped": ("double *out_r = out + (size_t)r * T * H_v * d_v;\n        if (rs == 0) {",
                            "double *out_r = out + (size_t)r * T * H_v * d_v;\n        if (rs == -7) {"),
    "commit_no_swap": ("write_slot[r] = t;", "write_slot[r] = write_slot[r] + 0 * t;"),
    "beta_dropped": ("S[(size_t)i * dv + j] += beta * k[i]", "S[(size_t)i * dv + j] += k[i]"),
    "store_to_read_slot": ("float *dst = state + (size_t)ws * slot_state;",
                           "float *dst = state + (size_t)rs * slot_state;"),
    "q_scale_on_k": ("oracle_l2norm(d_k, k, l2_eps, 1.0, kh);", "oracle_l2norm(d_k, k, l2_eps, q_scale, kh);"),
}


# the mistakes in the delta rule, the conv and the L2 norm, which the property
# tests (tests/test_oracle_properties.py) must catch on their own as well
PROPERTY_MUTATIONS = ("delta_sign", "no_decay", "pred_transposed", "readout_with_key", "beta_dropped",
                      "conv_taps_reversed", "l2_no_sqrt")


def _run_mutant(name, tmp, tests="test_oracle_pins.py"):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: pattern not found exactly once"
    path = os.path.join(tmp, f"{name}-{tests}.c")
    lib = os.path.join(tmp, f"lib_{name}-{tests}.so")
    open(path, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC", "-o", lib, path, "-lm"],
                   check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", tests)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            rcs = dict(zip(MUTATIONS, ex.map(lambda n: _run_mutant(n, tmp), MUTATIONS)))
    survivors = [n for n, rc in rcs.items() if rc == 0]
    assert not survivors, f"planted mistakes not caught by any pin: {survivors}"


def test_property_tests_alone_catch_the_delta_rule_conv_and_norm_mistakes():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            rcs = dict(zip(PROPERTY_MUTATIONS,
                           ex.map(lambda n: _run_mutant(n, tmp, "test_oracle_properties.py"), PROPERTY_MUTATIONS)))
    survivors = [n for n, rc in rcs.items() if rc == 0]
    assert not survivors, f"planted mistakes the property tests let through: {survivors}"
