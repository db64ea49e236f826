"""GPU: captured graphs replayed on other row layouts, and the conv decode as a
captured replay.

The mstar pages require that a graph captured on one layout of the decode
bucket and replayed on another gives the right rows (PR #965, "Correctness"),
and test the decode conv as a captured replay against eager steps (PR #1139,
"Tests").  Here one capture of a 128-row and a 64-row bucket (the mixed step's
decode half, in place, and the twin-slot step) is replayed after the device slot
arrays and inputs are rewritten to other real/padding splits; every replay is
compared with the oracle, padding rows must read out +0.0, slot 0 must stay
zero and no slot outside the real rows' write set may change.  Between replays
the program does eager work and synchronises (graphs are replayed several
times, as a capture can hide work that only the first replay gets right).
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


def _layouts(rows, captured):
    """(name, real row positions) of a bucket of `rows`, in replay order: the
    captured split first, then others, then the captured one again."""
    first = list(range(captured))
    half = rows // 2
    return [
        (f"{captured} real first (as captured)", first),
        (f"{half} real first", list(range(half))),
        ("10 real first", list(range(10))),
        ("no real row", []),
        (f"{half} real, every other row", list(range(0, rows, 2))),
        (f"{rows * 5 // 16} real scattered",
         sorted(np.random.Generator(np.random.PCG64(5)).choice(rows, rows * 5 // 16, replace=False).tolist())),
        (f"all {rows} rows real", list(range(rows))),
        (f"{captured} real first again", first),
    ]


# the 128-row bucket of the mixed step's decode half (46 real), and a 64-row
# bucket (30 real), whose single-token steps take four head tiles a workgroup
# (twin) and four value heads a workgroup (in place)
@pytest.mark.parametrize("mode", ["inplace-T1", "inplace-T4", "twin-T1", "inplace-T1-64rows", "twin-T1-64rows"])
def test_captured_bucket_replayed_on_other_layouts(gdn, torch, mode):
    t = torch
    twin = mode.startswith("twin")
    T = 4 if "-T4" in mode else 1
    if mode.endswith("64rows"):
        shape = gi.Shape(B=64, T=T, H_k=16, H_v=16, d_k=128, d_v=128, W=4, N=513)
        case = gi.make_case("bucket-64", shape, real_rows=30, twin=twin, seed=32)
        captured = 30
    else:
        case = gi.padded(T=T, twin=twin, seed=31)
        captured = gi.PADDED_REAL
    s, pool = case.shape, case.pools[0]
    hp = H.HostPool(pool)
    dp = H.DevPool(pool)
    # the pairs of the pool, in a fixed random order; real row i of a layout takes pair i
    pairs = np.random.Generator(np.random.PCG64(6)).permutation((s.N - 1) // 2).astype(np.int32) + 1
    rng = np.random.Generator(np.random.PCG64(7))

    # device buffers the graph reads: inputs, slot arrays, the read-out
    step0 = case.steps[0][0]
    x = H.bf16_dev(step0.x)
    g = t.from_numpy(step0.g).cuda()
    beta = t.from_numpy(step0.beta).cuda()
    out = t.empty((s.B, T, s.H_v, s.d_v), dtype=t.bfloat16, device="cuda")

    def set_layout(real):
        rd = np.zeros(s.B, np.int32)
        wr = np.zeros(s.B, np.int32)
        for i, r in enumerate(real):
            rd[r] = 2 * pairs[i] - 1
            wr[r] = 2 * pairs[i] if twin else rd[r]
        dp.rd.copy_(t.from_numpy(rd))
        dp.wr.copy_(t.from_numpy(wr))
        hp.rd, hp.wr = rd, wr
        st = gi.draw_step(rng, s)
        x.copy_(H.bf16_dev(st.x))
        g.copy_(t.from_numpy(st.g))
        beta.copy_(t.from_numpy(st.beta))
        return st

    def run():
        gdn.gdn_decode_step(x, dp.conv_w, None, dp.conv_state, dp.state, g, beta, dp.rd, dp.wr if twin else None,
                            out, H_k=s.H_k)

    layouts = _layouts(s.B, captured)
    set_layout(layouts[0][1])
    stream = t.cuda.Stream()
    graph = t.cuda.CUDAGraph()
    before_state = dp.state.clone()
    with t.cuda.graph(graph, stream=stream):
        run()
    t.cuda.synchronize()
    assert t.equal(dp.state.view(t.int32), before_state.view(t.int32)), "capture must not execute the step"
    del before_state

    for name, real in layouts:
        st = set_layout(real)
        t.cuda.synchronize()
        before_state = dp.state.clone()
        before_conv = dp.conv_state.clone()
        graph.replay()
        ref = oracle.gdn_decode_step(st.x, hp.conv_w, None, hp.conv_state, hp.state, st.g, st.beta, hp.rd,
                                     hp.wr if twin else None, H_k=s.H_k)
        t.cuda.synchronize()
        _ = float((dp.state[1:3].sum() + 1).item())  # eager work between replays
        pad = [r for r in range(s.B) if r not in set(real)]
        if real:
            H.assert_out_close(out[real], ref[real], f"{name}: out")
        assert t.count_nonzero(out[pad].view(t.int16)) == 0, f"{name}: padding rows must read out +0.0"
        written = sorted(int(v) for v in (hp.wr if twin else hp.rd)[real])
        if written:
            idx = t.tensor(written, dtype=t.int64, device="cuda")
            H.assert_state_close(dp.state[idx].cpu().numpy(), hp.state[written], f"{name}: state")
            np.testing.assert_array_equal(H.bf16_host(dp.conv_state[idx]), hp.conv_state[written])
        mask = t.ones(s.N, dtype=t.bool, device="cuda")
        if written:
            mask[t.tensor(written, dtype=t.int64, device="cuda")] = False
        assert t.equal(dp.state[mask].view(t.int32), before_state[mask].view(t.int32)), f"{name}: other slots changed"
        assert t.equal(dp.conv_state[mask].view(t.int16), before_conv[mask].view(t.int16))
        assert t.count_nonzero(dp.state[0].view(t.int32)) == 0 and t.count_nonzero(dp.conv_state[0].view(t.int16)) == 0
        del before_state, before_conv


@pytest.mark.parametrize("twin", [False, True], ids=["inplace", "twin"])
def test_conv_decode_captured_replay_matches_eager(gdn, torch, twin):
    """conv_decode captured once and replayed with new x each time (in place
    the window advances a token a replay) gives the bits of the same calls run
    eagerly on a copy of the pool, with padding rows among the real ones."""
    t = torch
    B, C, N = 24, 768, 49
    rng = np.random.Generator(np.random.PCG64(11))
    cs0 = np.zeros((N, 3, C), np.uint16)
    cs0[1:] = gi.bf16_bits(rng.standard_normal((N - 1, 3, C), dtype=np.float32))
    w = H.bf16_dev(gi.bf16_bits(rng.uniform(-0.5, 0.5, (C, 4)).astype(np.float32)))
    perm = rng.permutation(24).astype(np.int32) + 1
    rd = np.zeros(B, np.int32)
    wr = np.zeros(B, np.int32)
    for r in range(B):
        if r % 5 != 3:   # every fifth row (from row 3) is padding
            rd[r] = 2 * perm[r] - 1
            wr[r] = 2 * perm[r] if twin else rd[r]
    cs_g, cs_e = H.bf16_dev(cs0), H.bf16_dev(cs0)
    rd_d, wr_d = t.from_numpy(rd).cuda(), t.from_numpy(wr).cuda()
    x_g = t.empty((B, C), dtype=t.bfloat16, device="cuda")
    out_g, out_e = t.empty_like(x_g), t.empty_like(x_g)
    stream = t.cuda.Stream()
    graph = t.cuda.CUDAGraph()
    with t.cuda.graph(graph, stream=stream):
        gdn.conv_decode(x_g, w, None, cs_g, rd_d, wr_d if twin else None, out_g)
    t.cuda.synchronize()
    assert t.equal(cs_g.view(t.int16), cs_e.view(t.int16)), "capture must not execute the conv"
    for k in range(5):
        xk = H.bf16_dev(gi.bf16_bits(rng.standard_normal((B, C), dtype=np.float32)))
        x_g.copy_(xk)
        t.cuda.synchronize()
        graph.replay()
        gdn.conv_decode(xk, w, None, cs_e, rd_d, wr_d if twin else None, out_e)
        t.cuda.synchronize()
        _ = float((out_e.float().sum() + 1).item())  # eager work between replays
        assert t.equal(out_g.view(t.int16), out_e.view(t.int16)), f"replay {k}: out"
        assert t.equal(cs_g.view(t.int16), cs_e.view(t.int16)), f"replay {k}: conv state"
        pad = [r for r in range(B) if rd[r] == 0]
        assert t.count_nonzero(out_g[pad].view(t.int16)) == 0
        assert t.count_nonzero(cs_g[0].view(t.int16)) == 0
