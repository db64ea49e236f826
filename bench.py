"""Benchmark of the pooled GDN decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows B] [--mode twin|inplace]
                    [--hot] [--graph] [--no-cpu] [--no-calib]

Workload: one 0.8B-like GDN layer -- B = 64 rows, 16 key and 16 value heads,
d_k = d_v = 128 fp32 state (1 MiB a row), conv width 4 over 6144 channels with
bf16 conv windows, a pool of 257 slot pairs (N = 513), twin-slot writes.
A step is the whole path: the fused decode step (conv + SiLU, L2 norm, gates,
delta rule, read-out, twin write) and the slot commit, on synthetic seeded
inputs already resident in HBM.

Cold cache: MI355X's 256 MB Infinity Cache could hold one 64-row working set
(128 MiB), so consecutive steps rotate over four disjoint 64-row sets that use
all 256 slot pairs; a set's slots were last touched 384 MiB of traffic earlier.
--hot runs the same rows every step (reported as such).

Prints ONE JSON line on stdout.  value = rows/s over the timed steps
(step = decode kernel + commit kernel); roofline = the decode kernel's
algorithmic bytes / its mean duration (HIP events around every launch in the
timed region, on the launch stream) against 8 TB/s.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0


def algorithmic_bytes(B_real: int, B_pad: int, T: int, H_v: int, d_k: int, d_v: int, C: int, W: int,
                      twin: bool) -> int:
    """Bytes one decode launch must move.  Per real row: the state tile read and
    written (fp32), the conv window read and written (bf16), T tokens of x (bf16),
    the read-out (bf16), g and beta (fp32) and the two slot indices.  Per padding
    row: its slot indices and its zero read-out.  Once per launch: conv weights."""
    state = 2 * H_v * d_k * d_v * 4
    conv = 2 * (W - 1) * C * 2
    x = T * C * 2
    out = T * H_v * d_v * 2
    gates = 2 * T * H_v * 4
    slots = 8 if twin else 4
    per_real = state + conv + x + out + gates + slots
    per_pad = slots + out
    return B_real * per_real + B_pad * per_pad + C * W * 2


class HipTimer:
    """Timing events straight from the HIP runtime the process already uses,
    created with hipEventDisableSystemFence: recording them adds no system-scope
    release (no cache writeback), so the interval between two of them around a
    launch is the launch itself."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("no HIP runtime loaded")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        return ev

    def record(self, ev, stream_handle: int):
        rc = self.hip.hipEventRecord(ev, self.ct.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_ms(self, a, b) -> float:
        ms = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def _bf(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def cpu_baseline(seconds: float = 10.0) -> dict:
    """The fp64 oracle, as it stands, on 8-row slices of the same workload until
    about `seconds` of CPU time have passed (single thread)."""
    import gdn_inputs as gi
    import oracle

    case = gi.qwen08b(B=64)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    st, cs = pool.state.copy(), pool.conv_state.copy()
    rows = 0
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        sl = slice((8 * i) % 64, (8 * i) % 64 + 8)
        oracle.gdn_decode_step(np.ascontiguousarray(step.x[sl]), pool.conv_w, None, cs, st,
                               np.ascontiguousarray(step.g[sl]), np.ascontiguousarray(step.beta[sl]),
                               np.ascontiguousarray(pool.read_slot[sl]), np.ascontiguousarray(pool.write_slot[sl]),
                               H_k=s.H_k)
        rows += 8
        i += 1
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} rows of the 64-row workload (8-row slices, one step each), fp64 C loops, "
                      f"one thread, {dt:.1f} s", "us_per_64_row_step": 64 / (rows / dt) * 1e6}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--rows", type=int, default=64)
    ap.add_argument("--mode", choices=("twin", "inplace"), default="twin")
    ap.add_argument("--hot", action="store_true", help="same rows every step (cache-warm)")
    ap.add_argument("--graph", action="store_true", help="replay steps from a captured HIP graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-calib", action="store_true", help="skip the traffic calibration probes")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the decode step "
              "shards by rows or heads with no exchange inside the step, and no multi-GPU path is built.",
              file=sys.stderr)
        return 2

    import torch

    import gated_deltanet_recurrent_decode_amd as gdn
    import gdn_inputs as gi

    gdn.lib()
    torch.cuda.set_device(0)
    twin = args.mode == "twin"
    B = args.rows
    nsets = 1 if args.hot else max(1, min(4, 256 // B))
    # one pool of 257 slot pairs; the row sets take disjoint pairs
    case = gi.qwen08b(B=B * nsets, twin=twin)
    s, pool, step = case.shape, case.pools[0], case.steps[0][0]
    state = torch.from_numpy(pool.state).cuda()
    conv_state = _bf(torch, pool.conv_state)
    conv_w = _bf(torch, pool.conv_w)
    sets = []
    for k in range(nsets):
        sl = slice(k * B, (k + 1) * B)
        sets.append(dict(
            x=_bf(torch, step.x[sl]), g=torch.from_numpy(np.ascontiguousarray(step.g[sl])).cuda(),
            beta=torch.from_numpy(np.ascontiguousarray(step.beta[sl])).cuda(),
            rd=torch.from_numpy(np.ascontiguousarray(pool.read_slot[sl])).cuda(),
            wr=torch.from_numpy(np.ascontiguousarray(pool.write_slot[sl])).cuda(),
            out=torch.empty((B, 1, s.H_v, s.d_v), dtype=torch.bfloat16, device="cuda")))
    del case, pool, step
    torch.cuda.synchronize()

    def one_step(st):
        gdn.gdn_decode_step(st["x"], conv_w, None, conv_state, state, st["g"], st["beta"], st["rd"],
                            st["wr"] if twin else None, st["out"], H_k=s.H_k)
        if twin:
            gdn.slot_commit(st["rd"], st["wr"])

    stream = torch.cuda.current_stream()
    graph = None
    if args.graph:
        # one graph holding one step of every set, replayed as a unit
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for st in sets:
                one_step(st)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for st in sets:
                one_step(st)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        if graph is not None:
            graph.replay()
        else:
            one_step(sets[i % nsets])
    torch.cuda.synchronize()

    K = args.steps
    if graph is not None:
        K = max(nsets, (K // nsets) * nsets)
    timer = HipTimer()
    sh = stream.cuda_stream
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    kev = [(timer.event(), timer.event()) for _ in range(K)] if graph is None else []
    torch.cuda.synchronize()
    start.record(stream)
    if graph is not None:
        for _ in range(K // nsets):
            graph.replay()
    else:
        for i in range(K):
            st = sets[i % nsets]
            e0, e1 = kev[i]
            timer.record(e0, sh)
            gdn.gdn_decode_step(st["x"], conv_w, None, conv_state, state, st["g"], st["beta"], st["rd"],
                                st["wr"] if twin else None, st["out"], H_k=s.H_k)
            timer.record(e1, sh)
            if twin:
                gdn.slot_commit(st["rd"], st["wr"])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / K
    rows_per_s = B / (ms_per_step * 1e-3)

    step_bytes = algorithmic_bytes(B, 0, 1, s.H_v, s.d_k, s.d_v, s.C, s.W, twin)
    result = {
        "metric": "GDN decode rows/s and achieved HBM GB/s (% of peak) at 64 rows",
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_step": ms_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"0.8B-like GDN layer decode step: {B} rows x 16+16 heads x 128x128 fp32 state, "
                               f"conv width 4 over 6144 channels, bf16 conv windows and activations, "
                               f"257 slot pairs, {'twin-slot write + commit' if twin else 'in-place write'}, "
                               f"{'same rows every step (cache-warm)' if args.hot else f'{nsets} disjoint row sets rotated (cold cache)'}"
                               f"{', HIP graph replay' if graph is not None else ''}",
                   "B": B, "T": 1, "H_k": s.H_k, "H_v": s.H_v, "d_k": s.d_k, "d_v": s.d_v, "W": s.W, "N": s.N,
                   "write": args.mode, "row_sets": nsets, "graph": graph is not None},
        "step_GBps": step_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    if kev:
        kms = np.array([timer.elapsed_ms(a, b) for a, b in kev])
        for a, b in kev:
            timer.destroy(a)
            timer.destroy(b)
        k_us = float(kms.mean() * 1e3)
        achieved = step_bytes / (k_us * 1e-6) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                              "frac": achieved / PEAK_HBM_GBPS, "traffic": None,
                              "kernel": "gdn_step_kernel", "kernel_us_mean": k_us,
                              "kernel_us_p10": float(np.percentile(kms, 10) * 1e3),
                              "kernel_us_p50": float(np.percentile(kms, 50) * 1e3),
                              "kernel_us_p90": float(np.percentile(kms, 90) * 1e3),
                              "bytes_per_launch": step_bytes}

    if not args.no_calib:
        sink = torch.zeros(1, device="cuda")
        cal = {}
        for mode, name in ((0, "read_only"), (1, "write_only"), (2, "copy_twin"), (3, "read_write_in_place")):
            ts = []
            for i in range(max(8, args.warmup // 2) + 64):
                st = sets[i % nsets]
                e0, e1 = timer.event(), timer.event()
                timer.record(e0, sh)
                gdn.traffic_probe(mode, state, st["rd"], st["wr"], sink)
                timer.record(e1, sh)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            us = np.array([timer.elapsed_ms(a, b) for a, b in ts[-64:]]) * 1e3
            for a, b in ts:
                timer.destroy(a)
                timer.destroy(b)
            nbytes = (1 if mode in (0, 1) else 2) * B * s.H_v * s.d_k * s.d_v * 4
            cal[name] = {"us_mean": float(us.mean()), "GBps": nbytes / (us.mean() * 1e-6) / 1e9}
        result["calibration"] = cal

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
