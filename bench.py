"""Benchmark of the pooled GDN decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--rows B]
                    [--mode twin|inplace|tokens|prefill|stack|slotops] [--tokens T] [--prefill-len L]
                    [--layers L] [--commit fused|separate] [--hot] [--graph] [--no-cpu] [--no-calib]
                    [--no-sweep]

Workload: one 0.8B-like GDN layer -- B = 64 rows, 16 key and 16 value heads,
d_k = d_v = 128 fp32 state (1 MiB a row), conv width 4 over 6144 channels with
bf16 conv windows and activations, twin-slot writes.  A step is the whole path:
conv + SiLU, L2 norm, gates, delta rule, read-out, the twin write, and the slot
commit.  With --commit fused (default) the commit is folded into the step
kernel, which writes the swapped slot pair into a second pair of slot arrays
(the two pairs alternate); with --commit separate it is its own kernel after
the step.  Inputs are synthetic, seeded, and resident in HBM before the timed
region.

Cold cache: MI355X's 256 MB Infinity Cache takes in the lines a step writes
(streamed reads do not allocate there), so a slot read back within ~256 MB of
writes comes partly from that cache.  Consecutive steps rotate over enough
disjoint row sets that at least 768 MiB of state is written between two visits
of a set: 13 sets of 64 rows for twin writes, over a pool of 2049 slots (the
drawn 513-slot pool, its 512 non-null slots replicated four times on the
device), shared by every configuration the bench times.  --hot runs the same
rows every step (reported as such).

Timing: each timed loop is queued behind a GPU sleep long enough for the host
to enqueue the whole loop, so the GPU runs the steps back to back and the
Python launch cost never shows up as GPU idle time.  value = rows/s from the
loop without per-kernel events; roofline = the step kernel's algorithmic bytes
over its mean duration, from fence-free HIP events around every launch of a
second identical loop.

Beside the headline the default run adds (each labelled in the JSON line):
  calibration  the step's state traffic with no arithmetic in several workgroup
               designs over the same row sets (gdn_traffic_probe): read only,
               write only, copies in the step's own tile layout with one, two
               or four tiles a workgroup, plain chunk copies, copies whose
               stores are held until about the end of the read phase, and the
               same bytes between consecutive slots;
  roofline.ceiling  the best of those designs (GB/s), the step's time at that
               rate, and the step's fraction of it -- the practical ceiling of
               this traffic on this part, beside the 8 TB/s spec;
  sweep        twin and in place at 1, 4, 16, 64 and 128 rows (cold), and the
               64-row twin step hot;
  floor        an empty kernel, a kernel doing one slot-index load then one tile
               load, and the 1-row step: back to back, bracketed by events, and
               replayed from a captured HIP graph;
  cpu_baseline the fp64 oracle timed on the host on a bounded sample of the same
               workload (--no-cpu skips it).
Prints ONE JSON line on stdout.
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
METRIC = "GDN decode rows/s and achieved HBM GB/s (% of peak) at 64 rows"

# HBM bytes per launch of the step kernel on the default workload, from the two
# rocprofv3 counter passes summarised in profiles/ (FETCH_SIZE and WRITE_SIZE,
# each scaled by what it reads for a copy of known size).  Only valid for the
# machine code the counters were taken on: the gfx950 code of the kernels the
# launch runs is hashed from the built library, and traffic is reported as null
# when it differs.
STEP_KERNELS_64_TWIN = ("_ZN3gdn20gdn_step_tile_kernelILi128ELi128ELi128ELb0ELi4EEEvPKiS2_PKfS4_iiiiNS_10StepParamsE",)
MEASURED_TRAFFIC = {"kernel_code_sha256": "b4ee9a59f7b7983dca198b44b277973e94b5c1321fba97fde52640a699393df7",
                    "workload": (64, "twin", "fused", False, 16), "bytes_per_launch": 140_325_912}

# The same counters over one call of the two-pass prefill (chunk map, pass 1 and
# pass 2 summed), per (prompts, tokens a prompt) workload, scaled as above; the
# summary with its commands is in profiles/.  Valid only for this machine code.
PREFILL_KERNELS = ("_ZN3gdn12_GLOBAL__N_119tp_chunk_map_kernelENS_13TwoPassParamsE",
                   "_ZN3gdn12_GLOBAL__N_115tp_intra_kernelILi128ELi128ELb0EEEvNS_13TwoPassParamsEii",
                   "_ZN3gdn12_GLOBAL__N_115tp_intra_kernelILi128ELi128ELb1EEEvNS_13TwoPassParamsEii",
                   "_ZN3gdn12_GLOBAL__N_114tp_pipe_kernelILi128ELi128EEEvNS_13TwoPassParamsEiiiiii",
                   "_ZN3gdn12_GLOBAL__N_115tp_inter_kernelILi128ELi128ELi64EEEvNS_13TwoPassParamsE",
                   "_ZN3gdn12_GLOBAL__N_117tp_inter16_kernelILi128ELi128EEEvNS_13TwoPassParamsEii",
                   "_ZN3gdn12_GLOBAL__N_114tp_slim_kernelILi128ELi128EEEvNS_13TwoPassParamsE")
MEASURED_PREFILL_TRAFFIC = {"kernel_code_sha256": "c390195168709dbebe2d0634c405dbf14f767af16f4504880b67cc8c8337bf25",
                            "bytes_per_call": {(16, 512): 301_488_329, (1, 4096): 382_187_249}}


# The no-math copy designs the calibration sweeps (gdn_traffic_probe): the
# step's tile layout with one, two or four tiles a workgroup, and plain chunks
# varied one axis at a time around 256 threads x 8 loads: 16-byte loads in
# flight a lane, workgroup size, when stores may go (each after its own load,
# after all of the lane's loads, after all of the workgroup's loads), a
# persistent grid of k workgroups a CU, and the cache policy.
PROBE_SWEEP = {
    "tile1": dict(shape="tile1"),
    "tile1_wg": dict(shape="tile1", order="workgroup"),
    "tile2_wg": dict(shape="tile2", order="workgroup"),
    "tile2": dict(shape="tile2"),
    "tile4": dict(shape="tile4"),
    "tile4_wg": dict(shape="tile4", order="workgroup"),
    "tile4_plain": dict(shape="tile4", policy="plain"),
    "tile4_sc0sc1": dict(shape="tile4", policy="sc0sc1"),
    "chunk256x1": dict(shape="chunk", threads=256, loads=1),
    "chunk256x4": dict(shape="chunk", threads=256, loads=4),
    "chunk256x8": dict(shape="chunk", threads=256, loads=8),
    "chunk256x16": dict(shape="chunk", threads=256, loads=16),
    "chunk512x4": dict(shape="chunk", threads=512, loads=4),
    "chunk512x8": dict(shape="chunk", threads=512, loads=8),
    "chunk1024x1": dict(shape="chunk", threads=1024, loads=1),
    "chunk1024x4": dict(shape="chunk", threads=1024, loads=4),
    "chunk256x8_lane": dict(shape="chunk", threads=256, loads=8, order="lane"),
    "chunk256x8_wg": dict(shape="chunk", threads=256, loads=8, order="workgroup"),
    "chunk1024x4_wg": dict(shape="chunk", threads=1024, loads=4, order="workgroup"),
    "chunk256x8_persist1": dict(shape="chunk", threads=256, loads=8, persistent=1),
    "chunk256x8_persist2": dict(shape="chunk", threads=256, loads=8, persistent=2),
    "chunk256x8_persist4": dict(shape="chunk", threads=256, loads=8, persistent=4),
    "chunk1024x4_persist1": dict(shape="chunk", threads=1024, loads=4, persistent=1),
    "chunk256x8_plain": dict(shape="chunk", threads=256, loads=8, policy="plain"),
    "chunk256x8_sc0sc1": dict(shape="chunk", threads=256, loads=8, policy="sc0sc1"),
}
# designs also run over consecutive slots (the plain-copy pattern)
PROBE_CONTIGUOUS = ("tile1", "tile4", "chunk256x8", "chunk256x16", "chunk1024x4")


def _elf_sections(elf: bytes):
    """(name, type, addr, offset, size, link) of every section of a 64-bit ELF."""
    import struct
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    raw = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    strtab_off = raw[shstrndx][4]
    out = []
    for (name, typ, _flags, addr, off, size, link, _info, _align, _entsize) in raw:
        end = elf.index(b"\0", strtab_off + name)
        out.append((elf[strtab_off + name:end].decode(), typ, addr, off, size, link))
    return out


def device_code_objects(lib_path: str, arch: str = "gfx950") -> list:
    """The device code objects for `arch` in a HIP shared library's .hip_fatbin
    section (one offload bundle per translation unit, each 4 KiB aligned)."""
    import struct
    data = open(lib_path, "rb").read()
    sec = [x for x in _elf_sections(data) if x[0] == ".hip_fatbin"]
    if not sec:
        raise ValueError("no .hip_fatbin section")
    fat = data[sec[0][3]:sec[0][3] + sec[0][4]]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    out = []
    start = fat.find(magic)
    while start >= 0:
        n, = struct.unpack_from("<Q", fat, start + 24)
        pos = start + 32
        for _ in range(n):
            off, size, tlen = struct.unpack_from("<QQQ", fat, pos)
            triple = fat[pos + 24:pos + 24 + tlen]
            pos += 24 + tlen
            if arch.encode() in triple and size > 0:
                out.append(fat[start + off:start + off + size])
        start = fat.find(magic, pos)
    if not out:
        raise ValueError(f"no {arch} code object in the library")
    return out


def step_kernel_label(twin: bool, B: int, T: int, H_k: int, H_v: int, d_k: int, d_v: int, tokens_mode: bool,
                      cus: int = 256) -> str:
    """The kernel the library routes a decode step to (the same rule as its
    dispatch): twin writes take the tile kernel, in consecutive row parts when
    128 x 128 heads need more than one round of four-tile workgroups; in place,
    single tokens with one value head a key head take it too, unless 40-64
    rows' worth of 128 x 128 heads (2.5-4 a compute unit) group key heads in the
    walk kernel; token walks, per-token states and grouped value heads take the
    walk kernel."""
    if twin:
        heads = B * H_v
        parts = -(-heads // (4 * cus))
        if d_k == 128 and d_v == 128 and 1 < parts <= B and heads * 2 > 5 * cus * parts:
            return f"gdn_step_tile_kernel ({parts} launches over consecutive rows)"
        return "gdn_step_tile_kernel"
    G = H_v // H_k
    if T == 1 and not tokens_mode:
        heads = B * H_v
        kpw = 4 // G if G in (1, 2) else 1
        grouped = (d_k == 128 and d_v == 128 and G in (1, 2) and heads * 2 > 5 * cus and heads <= 4 * cus
                   and H_k % kpw == 0)
        if grouped:
            return f"gdn_step_kernel ({kpw} key heads a workgroup)"
        if G == 1:
            return "gdn_step_tile_kernel"
    return "gdn_step_kernel"


def kernel_code_sha256(symbols=STEP_KERNELS_64_TWIN, lib_path: str | None = None) -> str | None:
    """SHA-256 over the machine code of the named kernels in the built library's
    gfx950 code object (None if the library or a kernel is missing)."""
    import hashlib
    import struct
    if lib_path is None:
        lib_path = os.path.join(ROOT, "gated_deltanet_recurrent_decode_amd", "libgdn.so")
    try:
        objs = device_code_objects(lib_path)
    except (OSError, ValueError):
        return None
    found = {}
    for co in objs:
        secs = _elf_sections(co)
        symtab = [x for x in secs if x[0] == ".symtab"]
        if not symtab:
            continue
        _, _, _, st_off, st_size, link = symtab[0]
        str_off = secs[link][3]
        for i in range(st_size // 24):
            name_o, info, other, shndx, value, size = struct.unpack_from("<IBBHQQ", co, st_off + 24 * i)
            end = co.index(b"\0", str_off + name_o)
            name = co[str_off + name_o:end].decode()
            if name in symbols and size > 0 and shndx < len(secs):
                _, _, addr, off, _, _ = secs[shndx]
                found[name] = co[off + (value - addr):off + (value - addr) + size]
    if set(found) != set(symbols):
        return None
    h = hashlib.sha256()
    for name in symbols:
        h.update(found[name])
    return h.hexdigest()


def algorithmic_bytes(B_real: int, B_pad: int, T: int, H_v: int, d_k: int, d_v: int, C: int, W: int,
                      mode: str) -> int:
    """Bytes one decode launch must move.  Per real row: the state tile read (fp32)
    and written -- once (twin, in place) or once per kept token (tokens mode) --, the
    conv window read and written likewise (bf16), T tokens of x (bf16), of read-out
    (bf16) and of g and beta (fp32), and the slot indices (read and write slot, and
    two more written by a fused commit; the read slot in place; the read slot and
    T token slots in tokens mode).  Per padding row: its slot indices and its zero
    read-out.  Once per launch: the conv weights."""
    tile = H_v * d_k * d_v * 4
    win = (W - 1) * C * 2
    writes = T if mode == "tokens" else 1
    x = T * C * 2
    out = T * H_v * d_v * 2
    gates = 2 * T * H_v * 4
    slots = {"twin": 16, "inplace": 4, "tokens": 4 + 4 * T}[mode]
    per_real = (1 + writes) * (tile + win) + x + out + gates + slots
    per_pad = slots + out
    return B_real * per_real + B_pad * per_pad + C * W * 2


DRAWN_SLOTS = 512          # non-null slots of the drawn pool: 256 slot pairs
COLD_BYTES = 768 << 20     # state written between two visits of a row set


def row_sets(mode: str, B: int, T: int, slot_bytes: int, hot: bool) -> tuple[int, int]:
    """(row sets rotated, slots one set takes).  MI355X's 256 MB Infinity Cache
    takes in the lines a step writes (streamed reads do not allocate there), so
    a slot written and read back within ~256 MB of other writes is read partly
    from that cache.  Enough disjoint sets rotate that at least COLD_BYTES of
    state is written between two visits of one set: a twin set's write slots
    are its read slots the next time round, in place the same slots, in tokens
    mode the token slots."""
    per = {"twin": 2 * B, "inplace": B, "tokens": B * (T + 1)}[mode]
    if per > DRAWN_SLOTS:
        raise ValueError(f"a row set takes {per} slots; at most {DRAWN_SLOTS}")
    if hot:
        return 1, per
    written = B * slot_bytes * (T if mode == "tokens" else 1)
    return max(4, 1 + -(-COLD_BYTES // written)), per


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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_legs(call, seconds: float, threads: int):
    """Time `call(k, n)` -- thread k of n doing one piece of its own share of the
    sample and returning the units it did -- first on one host thread, then on
    `threads` threads (the oracle's ctypes calls release the GIL, so the threads
    run in parallel), each leg for about `seconds` / 2 of wall time."""
    import threading

    def leg(n, budget):
        done = [0] * n
        t0 = time.perf_counter()

        def work(k):
            while time.perf_counter() - t0 < budget:
                done[k] += call(k, n)

        ths = [threading.Thread(target=work, args=(k,)) for k in range(n)]
        for th in ths:
            th.start()
        for th in ths:
            th.join()
        dt = time.perf_counter() - t0
        return sum(done) / dt, sum(done), dt

    return leg(1, seconds / 2), leg(threads, seconds / 2)


def _host_threads(divides: int | None = None) -> int:
    n = max(1, min(16, os.cpu_count() or 1))
    while divides and divides % n:
        n -= 1
    return n


def cpu_baseline(args, seconds: float = 10.0) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the workload the
    bench line times (the same shapes, tokens a row and write mode), on one host
    thread and then on all of them (at most 16), each thread on its own rows,
    prompts or slots so that the shared pool arrays are written at disjoint
    places.  `value` is the all-threads rate in the bench line's unit."""
    import gdn_inputs as gi
    import oracle

    mode = args.mode
    if mode in ("twin", "inplace", "tokens", "stack"):
        if mode == "stack":
            shape = gi.Shape(B=64, T=1, H_k=16, H_v=32, d_k=128, d_v=128, W=4, N=129)
            case = gi.make_case("9b-oracle", shape, seed=0)
        else:
            T = args.tokens
            rows = 64 if mode != "tokens" else min(64, 512 // (1 + T))
            case = gi.qwen08b(B=rows, T=T, twin=mode == "twin")
        s, pool, step = case.shape, case.pools[0], case.steps[0][0]
        st, cs = pool.state.copy(), pool.conv_state.copy()
        n = _host_threads(s.B)
        if mode == "tokens":
            perm = np.random.Generator(np.random.PCG64(1)).permutation(DRAWN_SLOTS).astype(np.int32) + 1
            rd_all = perm[:s.B]
            tok_all = perm[s.B:s.B * (1 + s.T)].reshape(s.B, s.T)

        def call(k, nthreads):
            per = s.B // nthreads
            sl = slice(k * per, (k + 1) * per)
            a = (np.ascontiguousarray(step.x[sl]), pool.conv_w, None, cs, st, np.ascontiguousarray(step.g[sl]),
                 np.ascontiguousarray(step.beta[sl]))
            if mode == "tokens":
                oracle.gdn_decode_step_tokens(*a, np.ascontiguousarray(rd_all[sl]), np.ascontiguousarray(tok_all[sl]),
                                              H_k=s.H_k)
            else:
                oracle.gdn_decode_step(*a, np.ascontiguousarray(pool.read_slot[sl]),
                                       np.ascontiguousarray(pool.write_slot[sl]) if mode in ("twin", "stack") else None,
                                       H_k=s.H_k)
            return per

        (one, u1, dt1), (many, un, dtn) = _oracle_legs(call, seconds, n)
        if mode == "stack":
            # a row of the stack is a row through every layer; each layer is the same work
            one, many = one / args.layers, many / args.layers
            what = (f"one 9B-like layer's decode step (16 key / 32 value heads of 128, 8192 channels, twin): {un} "
                    f"row-layers in {dtn:.1f} s on {n} host threads, rates divided by the {args.layers} layers")
        else:
            what = (f"the 0.8B-like layer's decode step, {s.T} token{'s' if s.T > 1 else ''} a row, "
                    f"{ {'twin': 'twin-slot write', 'inplace': 'in place', 'tokens': 'a state kept per token'}[mode]}: "
                    f"{un} rows in {dtn:.1f} s on {n} host threads ({s.B // n} rows a call per thread)")
        unit = "rows/s"
    elif mode == "prefill":
        L = args.prefill_len
        piece = min(L, 128)
        n = _host_threads()
        case = gi.prefill([piece] * n, H_k=16, H_v=16, d=128, seed=0)
        s, pool = case.shape, case.pool
        st, cs = pool.state.copy(), pool.conv_state.copy()

        def call(k, nthreads):
            a, e = int(case.cu_seqlens[k]), int(case.cu_seqlens[k + 1])
            # prompt k continues on its own slot: each call is the next `piece` tokens of a prompt
            oracle.gdn_decode_step(np.ascontiguousarray(case.x[None, a:e]), pool.conv_w, None, cs, st,
                                   np.ascontiguousarray(case.g[None, a:e]), np.ascontiguousarray(case.beta[None, a:e]),
                                   np.ascontiguousarray(pool.read_slot[k:k + 1]), None, H_k=s.H_k)
            return e - a

        (one, u1, dt1), (many, un, dtn) = _oracle_legs(call, seconds, n)
        what = (f"prefill as its definition, the in-place recurrence token by token (0.8B-like heads), each host "
                f"thread on its own prompt in pieces of {piece} tokens: {un} tokens in {dtn:.1f} s on {n} threads")
        unit = "tokens/s"
    else:  # slot ops: the copy the bench line reports
        case = gi.qwen08b(B=256)
        pool = case.pools[0]
        st, cs = pool.state.copy(), pool.conv_state.copy()
        n = _host_threads(256)
        per_call = 8
        perm = np.random.Generator(np.random.PCG64(2)).permutation(DRAWN_SLOTS).astype(np.int32) + 1

        def call(k, nthreads):
            # thread k copies among its own 512/n slots: sources from its first half to its second
            own = perm[k * (DRAWN_SLOTS // nthreads):(k + 1) * (DRAWN_SLOTS // nthreads)]
            h = min(per_call, own.size // 2)
            oracle.slot_copy(st, cs, np.ascontiguousarray(own[:h]), np.ascontiguousarray(own[h:2 * h]))
            return h

        (one, u1, dt1), (many, un, dtn) = _oracle_legs(call, seconds, n)
        what = (f"slot copy (state and conv window of the 0.8B-like layer, 1 MiB + 36 KiB a slot), {per_call} slots a "
                f"call per thread: {un} slots in {dtn:.1f} s on {n} host threads")
        unit = "slots/s"
    return {"value": many, "unit": unit, "cores": n, "kind": "oracle",
            "sample": f"{what}; one thread: {u1} in {dt1:.1f} s",
            "single_thread_rate": one, "host_cpus": os.cpu_count(), "cpu_model": _cpu_model()}


POOL_SLOTS = 1 + 4 * DRAWN_SLOTS   # the drawn pool's 512 slots, four times over, after the null slot


class DevicePool:
    """The drawn pool of the 0.8B-like layer (the null slot and 256 slot pairs)
    with its 512 non-null slots replicated on the device to POOL_SLOTS slots
    (2 GiB of state), shared by every decode configuration the bench times, so
    each can rotate over disjoint row sets that are cold when visited.  With
    H_k below 16 the 16 value heads share H_k key heads (same state pool,
    fewer conv channels)."""

    def __init__(self, H_k: int = 16):
        import torch

        import gated_deltanet_recurrent_decode_amd as gdn
        import gdn_inputs as gi

        self.torch, self.gdn, self.gi = torch, gdn, gi
        gdn.lib()
        torch.cuda.set_device(0)
        if H_k == 16:
            case = gi.qwen08b(B=256, T=1)
        else:
            case = gi.make_case(f"0.8b-{H_k}x16", gi.Shape(B=256, T=1, H_k=H_k, H_v=16, d_k=128, d_v=128, W=4, N=513))
        s, pool = case.shape, case.pools[0]
        self.shape, self.case = s, case
        self.N = POOL_SLOTS
        copies = (POOL_SLOTS - 1) // DRAWN_SLOTS
        state0 = torch.from_numpy(pool.state).cuda()
        cs0 = _bf(torch, pool.conv_state)
        self.state = torch.empty((self.N,) + tuple(state0.shape[1:]), dtype=state0.dtype, device="cuda")
        self.conv_state = torch.empty((self.N,) + tuple(cs0.shape[1:]), dtype=cs0.dtype, device="cuda")
        self.state[0], self.conv_state[0] = state0[0], cs0[0]
        for c in range(copies):
            self.state[1 + DRAWN_SLOTS * c:1 + DRAWN_SLOTS * (c + 1)] = state0[1:]
            self.conv_state[1 + DRAWN_SLOTS * c:1 + DRAWN_SLOTS * (c + 1)] = cs0[1:]
        del state0, cs0
        self.conv_w = _bf(torch, pool.conv_w)
        self.read_slot, self.write_slot = pool.read_slot, pool.write_slot
        torch.cuda.synchronize()
        self.stream = torch.cuda.current_stream()
        self.timer = HipTimer()
        self.cycles_per_ms = None

    def inputs(self, T: int):
        """x, g, beta for 256 rows of T tokens: the drawn ones for one token,
        otherwise a seeded draw of the same distributions."""
        if T == 1:
            return self.case.steps[0][0]
        s = self.shape
        return self.gi.draw_step(np.random.Generator(np.random.PCG64(1000 + T)),
                                 self.gi.Shape(B=256, T=T, H_k=s.H_k, H_v=s.H_v, d_k=s.d_k, d_v=s.d_v, W=s.W, N=s.N))

    def sleep_for(self, ms: float):
        """Queue a GPU spin of about `ms` milliseconds on the current stream."""
        torch = self.torch
        if self.cycles_per_ms is None:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.cuda._sleep(2_000_000)
            b.record()
            torch.cuda.synchronize()
            self.cycles_per_ms = 2_000_000 / max(a.elapsed_time(b), 1e-3)
        torch.cuda._sleep(int(ms * self.cycles_per_ms))

    def time_launches(self, launch, K: int, per_launch_events: bool, host_ms_per_call: float | None = None):
        """K calls of launch(i) queued behind a GPU spin (so they run back to back);
        returns (ms per call from one event pair, per-call us from fence-free
        events around each call or None)."""
        torch, timer = self.torch, self.timer
        sh = self.stream.cuda_stream
        kev = [(timer.event(), timer.event()) for _ in range(K)] if per_launch_events else None
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # enough spin for the host to queue the whole loop (about 60 us a call from Python)
        if host_ms_per_call is None:
            host_ms_per_call = 0.12 if per_launch_events else 0.08
        self.sleep_for(max(5.0, K * host_ms_per_call))
        start.record()
        for i in range(K):
            if kev is not None:
                timer.record(kev[i][0], sh)
            launch(i)
            if kev is not None:
                timer.record(kev[i][1], sh)
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / K
        us = None
        if kev is not None:
            us = np.array([timer.elapsed_ms(a, b) for a, b in kev]) * 1e3
            for a, b in kev:
                timer.destroy(a)
                timer.destroy(b)
        return ms, us


class Bench:
    """One decode configuration over the shared pool: B rows (the first R real,
    the rest on the null slot), T tokens a row, a write mode, rotating over
    enough disjoint row sets to be cold (or the same rows every step when hot)."""

    def __init__(self, dp: DevicePool, mode: str = "twin", B: int = 64, T: int = 1, real=None, hot: bool = False,
                 commit: str = "fused"):
        torch = dp.torch
        self.dp, self.torch, self.gdn = dp, torch, dp.gdn
        self.mode, self.hot = mode, hot
        self.twin = mode == "twin"
        self.tokens_mode = mode == "tokens"
        self.fused = self.twin and commit == "fused"
        self.B, self.T = B, T
        R = self.R = B if real is None else real
        s = self.shape = dp.shape
        nsets, per = row_sets(mode, R, T, s.H_v * s.d_k * s.d_v * 4, hot)
        spc = DRAWN_SLOTS // per                  # disjoint row sets one copy of the drawn pool holds
        copies = -(-nsets // spc)
        if 1 + DRAWN_SLOTS * copies > dp.N:
            raise ValueError(f"{nsets} row sets of {per} slots do not fit the {dp.N}-slot pool")
        self.N = dp.N
        step = dp.inputs(T)
        perm = np.random.Generator(np.random.PCG64(1)).permutation(DRAWN_SLOTS).astype(np.int32) + 1
        slot_rows = []
        pad = np.zeros(B - R, np.int32)
        for k in range(nsets):
            j, off = k % spc, DRAWN_SLOTS * (k // spc)
            if self.twin:
                slot_rows.append((np.concatenate([dp.read_slot[j * R:(j + 1) * R] + off, pad]),
                                  np.concatenate([dp.write_slot[j * R:(j + 1) * R] + off, pad])))
            elif self.tokens_mode:
                # B read slots and B*T token slots, all distinct
                slot_rows.append((perm[j * per:j * per + B] + off, (perm[j * per + B:(j + 1) * per] + off).reshape(B, T)))
            else:
                slot_rows.append((np.concatenate([perm[j * R:(j + 1) * R] + off, pad]), None))
        self.nsets = nsets
        self.sets = []
        for k, (rd, wr) in enumerate(slot_rows):
            rows = np.arange(k * B, (k + 1) * B) % 256
            st = dict(x=_bf(torch, step.x[rows]), g=torch.from_numpy(np.ascontiguousarray(step.g[rows])).cuda(),
                      beta=torch.from_numpy(np.ascontiguousarray(step.beta[rows])).cuda(),
                      rd=torch.from_numpy(np.ascontiguousarray(rd)).cuda(),
                      wr=None if wr is None else torch.from_numpy(np.ascontiguousarray(wr)).cuda(),
                      out=torch.empty((B, T, s.H_v, s.d_v), dtype=torch.bfloat16, device="cuda"))
            # the second pair of slot arrays the fused commit alternates with
            st["pairs"] = [(st["rd"], st["wr"]), (torch.empty_like(st["rd"]), None if wr is None else
                                                  torch.empty_like(st["wr"]))]
            st["parity"] = 0
            self.sets.append(st)
        torch.cuda.synchronize()
        self.bytes = algorithmic_bytes(R, B - R, T, s.H_v, s.d_k, s.d_v, s.C, s.W, mode)

    def launch(self, st):
        g, s, dp = self.gdn, self.shape, self.dp
        if self.fused:
            (rd, wr), (nrd, nwr) = st["pairs"][st["parity"]], st["pairs"][1 - st["parity"]]
            g.gdn_decode_step_commit(st["x"], dp.conv_w, None, dp.conv_state, dp.state, st["g"], st["beta"],
                                     rd, wr, nrd, nwr, st["out"], H_k=s.H_k)
            st["parity"] ^= 1
        elif self.tokens_mode:
            g.gdn_decode_step_tokens(st["x"], dp.conv_w, None, dp.conv_state, dp.state, st["g"], st["beta"],
                                     st["rd"], st["wr"], st["out"], H_k=s.H_k)
        else:
            g.gdn_decode_step(st["x"], dp.conv_w, None, dp.conv_state, dp.state, st["g"], st["beta"],
                              st["rd"], st["wr"] if self.twin else None, st["out"], H_k=s.H_k)

    def commit(self, st):
        if self.twin and not self.fused:
            self.gdn.slot_commit(st["rd"], st["wr"])

    def step(self, i):
        st = self.sets[i % self.nsets]
        self.launch(st)
        self.commit(st)

    def warm(self, n: int):
        for i in range(n):
            self.step(i)
        self.torch.cuda.synchronize()

    def timed(self, K: int, per_kernel_events: bool, graph=None):
        """K steps queued behind a spin; returns (ms per step, per-kernel us or None).
        With per-kernel events only the step kernel is bracketed (a separate
        commit kernel runs outside the events)."""
        if graph is not None:
            reps = max(1, K // graph[1])
            ms, _ = self.dp.time_launches(lambda i: graph[0].replay(), reps, False)
            return ms / graph[1], None
        if not per_kernel_events:
            return self.dp.time_launches(self.step, K, False)
        torch, timer = self.torch, self.dp.timer
        sh = self.dp.stream.cuda_stream
        kev = [(timer.event(), timer.event()) for _ in range(K)]

        def one(i):
            st = self.sets[i % self.nsets]
            timer.record(kev[i][0], sh)
            self.launch(st)
            timer.record(kev[i][1], sh)
            self.commit(st)

        ms, _ = self.dp.time_launches(one, K, False, host_ms_per_call=0.14)
        us = np.array([timer.elapsed_ms(a, b) for a, b in kev]) * 1e3
        for a, b in kev:
            timer.destroy(a)
            timer.destroy(b)
        return ms, us

    def capture(self):
        """One graph holding two steps of every row set (both parities of the
        fused commit); returns (graph, steps per replay)."""
        torch = self.torch
        n = 2 * self.nsets
        side = torch.cuda.Stream()
        side.wait_stream(self.dp.stream)
        with torch.cuda.stream(side):
            for i in range(n):
                self.step(i)
        self.dp.stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                self.step(i)
        torch.cuda.synchronize()
        return g, n

    def calibration(self, laps: int = 10, only: tuple | None = None) -> dict:
        """The step's state traffic with no arithmetic, in several workgroup
        designs, over the same rotating row sets (the method of the PR #1139
        page, 'Numbers', widened to a sweep of designs; see gdn_traffic_probe).
        Twin visits swap a set's read and write slots every lap, as the commit
        does, so nothing is re-read warm.  The contiguous designs move the same
        bytes between consecutive slots (B read slots, then B write slots, a
        disjoint range each visit).  The hold designs keep every workgroup's
        stores until about the read phase's end (a fraction of the read bytes
        over 6.7 TB/s), which puts the whole launch's reads ahead of its writes.
        `only`: just these PROBE_SWEEP designs over the step's slots.
        Returns {design: {us_mean, GBps, frac, bytes}}."""
        torch, gdn, dp = self.torch, self.gdn, self.dp
        sink = torch.zeros(1, device="cuda")
        s = self.shape
        tile_bytes = s.d_k * s.d_v * 4
        read_bytes = self.R * s.H_v * tile_bytes
        inplace = not self.twin
        traffic = "inplace" if inplace else "copy"
        designs = [("read_only", "read", "slots", PROBE_SWEEP["tile1"], 0.0),
                   ("write_only", "write", "slots", PROBE_SWEEP["tile1"], 0.0)]
        for label, kw in PROBE_SWEEP.items():
            designs.append((f"{traffic}_slots_{label}", traffic, "slots", kw, 0.0))
        for f in (0.9, 1.0, 1.1):
            designs.append((f"{traffic}_slots_tile1_hold{f:.1f}", traffic, "slots", PROBE_SWEEP["tile1"], f))
        designs.append((f"{traffic}_slots_tile4_hold0.9", traffic, "slots", PROBE_SWEEP["tile4"], 0.9))
        for label in PROBE_CONTIGUOUS:
            designs.append((f"{traffic}_contiguous_{label}", traffic, "contiguous", PROBE_SWEEP[label], 0.0))
        if only is not None:
            designs = [(f"{traffic}_slots_{label}", traffic, "slots", PROBE_SWEEP[label], 0.0) for label in only]
        # consecutive-slot ranges, disjoint for every set: [1 + 2Rk, 1 + 2Rk + R) and the next R slots
        ranges = [(torch.tensor([1 + 2 * self.R * k], dtype=torch.int32, device="cuda"),
                   torch.tensor([1 + 2 * self.R * k + self.R], dtype=torch.int32, device="cuda"))
                  for k in range(self.nsets) if 1 + 2 * self.R * (k + 1) <= dp.N]
        out = {}
        for name, tr, layout, kw, hold in designs:
            if layout == "contiguous" and len(ranges) < min(self.nsets, 4):
                continue
            if kw["shape"] in ("tile2", "tile4") and (s.d_k, s.d_v) != (128, 128):
                continue
            if kw["shape"] == "chunk" and tile_bytes % (kw["threads"] * kw["loads"] * 16):
                continue
            nsets = self.nsets if layout == "slots" else len(ranges)
            hold_ns = int(hold * read_bytes / 6.7e12 * 1e9)

            def launch(i, tr=tr, layout=layout, kw=kw, hold_ns=hold_ns, nsets=nsets):
                if layout == "slots":
                    st = self.sets[i % nsets]
                    rd, wr = st["rd"], st["wr"]
                else:
                    rd, wr = ranges[i % nsets]
                if not inplace and (i // nsets) % 2:
                    rd, wr = wr, rd
                if wr is None:  # in place: the write-only half writes the rows' own slots
                    wr = rd
                gdn.traffic_probe(dp.state, rd, wr, sink, traffic=tr, layout=layout, hold_ns=hold_ns,
                                  rows=self.R if layout == "contiguous" else self.B, **kw)

            reps = laps * nsets if nsets < 64 else 2 * nsets
            for i in range(min(nsets, 16)):
                launch(i)
            torch.cuda.synchronize()
            _, us = dp.time_launches(launch, reps, True)
            nbytes = (1 if tr in ("read", "write") else 2) * read_bytes
            m = float(us.mean())
            out[name] = {"us_mean": m, "GBps": nbytes / (m * 1e-6) / 1e9,
                         "frac": nbytes / (m * 1e-6) / 1e9 / PEAK_HBM_GBPS, "bytes": nbytes}
        return out


def ceiling_of(cal: dict, step_bytes: int, achieved_GBps: float) -> dict | None:
    """The best no-math design of the calibration (the highest GB/s moving
    the step's traffic: copies for twin writes, read-and-write-back in place),
    and the best over the step's own slots; with the step's time at each rate."""
    best = {}
    for scope in ("any", "slots", "no_hold"):
        cands = [(v["GBps"], k) for k, v in cal.items()
                 if not k.startswith(("read_only", "write_only")) and (scope != "slots" or "_slots_" in k)
                 and (scope != "no_hold" or "_hold" not in k)]
        if not cands:
            return None
        g, k = max(cands)
        best[scope] = {"design": k, "us_mean": cal[k]["us_mean"], "GBps": g, "frac": g / PEAK_HBM_GBPS,
                       "us_at_step_bytes": step_bytes / (g * 1e9) * 1e6, "step_fraction": achieved_GBps / g}
    out = dict(best["any"])
    out["on_the_steps_slots"] = best["slots"]
    out["without_hold"] = best["no_hold"]
    out["note"] = ("best no-math copy design at the step's traffic (GB/s, so the step's own bytes can be priced at "
                   "it); step_fraction = the step's achieved GB/s over the design's; without_hold: the best design "
                   "whose stores are not held for a set time")
    return out


SWEEP = [(b, m) for b in (1, 4, 16, 64, 128) for m in ("twin", "inplace")]


# the no-math designs each sweep entry is held against (whole tiles for large
# batches, small chunks that spread a few rows over many CUs for small ones)
SWEEP_COPY = ("tile1", "tile4_wg", "chunk256x1", "chunk256x4", "chunk256x8")


def run_sweep(dp: DevicePool, K: int = 130) -> dict:
    """Twin and in-place steps at 1, 4, 16, 64 and 128 rows (cold row sets), plus
    the 64-row twin step hot (the same rows every step, labelled as such).
    Every cold entry carries the same run's fastest no-math copy of its state
    traffic over the same row sets (SWEEP_COPY designs), and the step's time
    over it."""
    out = {}
    for B, mode in SWEEP + [(64, "twin-hot")]:
        hot = mode.endswith("hot")
        b = Bench(dp, mode="twin" if hot else mode, B=B, hot=hot)
        b.warm(min(b.nsets, 20) + 4)
        ms, _ = b.timed(max(K, 2 * min(b.nsets, 13)), False)
        _, us = b.timed(K, True)
        k = float(us.mean())
        e = {"rows": B, "write": "twin" if hot else mode, "cold": not hot,
             "us_per_step": ms * 1e3, "kernel_us_mean": k, "rows_per_s": B / (ms * 1e-3),
             "GBps": b.bytes / (k * 1e-6) / 1e9, "frac": b.bytes / (k * 1e-6) / 1e9 / PEAK_HBM_GBPS,
             "bytes": b.bytes}
        if not hot:
            cal = b.calibration(laps=6, only=SWEEP_COPY)
            best = min(cal, key=lambda d: cal[d]["us_mean"])
            e["copy"] = {"design": best, "us_mean": cal[best]["us_mean"], "bytes": cal[best]["bytes"],
                         "step_over_copy": k / cal[best]["us_mean"]}
        out[f"{B}_{mode}"] = e
        del b
    return out


def run_floors(dp: DevicePool, K: int = 64) -> dict:
    """The launch floor of small batches: an empty kernel, and a kernel that
    loads one slot index and then that slot's first tile (a step's first two
    dependent loads; the index and the tile cold: each launch takes the first
    row of the next of the 1-row sets the 1-row step rotates over), back to
    back from the stream and from a captured graph, beside the 1-row fused
    twin step the same two ways (the PR #1139 page, 'Numbers', measured ~1.8
    us a kernel inside a captured graph on MI325X)."""
    torch, gdn = dp.torch, dp.gdn
    sink = torch.zeros(1, device="cuda")
    one = Bench(dp, mode="twin", B=1)
    rds = [st["rd"] for st in one.sets]
    out = {}
    for shape in ("empty", "slot_load"):
        def launch(i, shape=shape):
            gdn.traffic_probe(dp.state, rds[i % len(rds)], None, sink, traffic="read", shape=shape, rows=1)
        for i in range(8):
            launch(i)
        torch.cuda.synchronize()
        ms, _ = dp.time_launches(launch, K, False)
        _, us = dp.time_launches(launch, K, True)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(K):
                launch(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        gms, _ = dp.time_launches(lambda i: g.replay(), 8, False)
        out[shape] = {"us_back_to_back": ms * 1e3, "us_events_mean": float(us.mean()), "us_graph": gms * 1e3 / K}
        del g
    del one
    b = Bench(dp, mode="twin", B=1)
    b.warm(24)
    ms, _ = b.timed(max(K, 130), False)
    _, us = b.timed(max(K, 130), True)
    graph = b.capture()
    graph[0].replay()
    torch.cuda.synchronize()
    gms, _ = b.timed(graph[1] * 2, False, graph=graph)
    out["step_1_row_twin"] = {"us_back_to_back": ms * 1e3, "us_events_mean": float(us.mean()), "us_graph": gms * 1e3}
    return out


STACK_METRIC = "GDN decode rows/s and achieved HBM GB/s (% of peak), 24-layer 9B-like stack"


def run_stack(args) -> dict:
    """The 9B-like decode: B rows, 16 key heads shared by 32 value heads (d = 128),
    8192 conv channels, one pool of 1 + 2B slots per layer, --layers layers stepped
    back to back (twin slots, fused commit) -- one step is every layer's launch.
    Layers share one drawn pool (copied per layer) and one set of inputs; the
    layer pools together (6.3 GB at 24 layers) keep every layer's state cold."""
    import torch

    import gated_deltanet_recurrent_decode_amd as gdn
    import gdn_inputs as gi

    gdn.lib()
    torch.cuda.set_device(0)
    B, layers = args.rows, args.layers
    shape = gi.Shape(B=B, T=1, H_k=16, H_v=32, d_k=128, d_v=128, W=4, N=1 + 2 * B)
    case = gi.make_case("9b-bench", shape, seed=0)
    pool, step = case.pools[0], case.steps[0][0]
    s = case.shape
    state0 = torch.from_numpy(pool.state).cuda()
    cs0 = _bf(torch, pool.conv_state)
    L = []
    for _ in range(layers):
        rd = torch.from_numpy(pool.read_slot.copy()).cuda()
        wr = torch.from_numpy(pool.write_slot.copy()).cuda()
        L.append(dict(state=state0.clone(), cs=cs0.clone(), pairs=[(rd, wr), (torch.empty_like(rd), torch.empty_like(wr))],
                      parity=0))
    del state0, cs0
    conv_w = _bf(torch, pool.conv_w)
    x, g, beta = _bf(torch, step.x), torch.from_numpy(step.g).cuda(), torch.from_numpy(step.beta).cuda()
    out = torch.empty((B, 1, s.H_v, s.d_v), dtype=torch.bfloat16, device="cuda")

    def one_step():
        for lay in L:
            (rd, wr), (nrd, nwr) = lay["pairs"][lay["parity"]], lay["pairs"][1 - lay["parity"]]
            gdn.gdn_decode_step_commit(x, conv_w, None, lay["cs"], lay["state"], g, beta, rd, wr, nrd, nwr, out,
                                       H_k=s.H_k)
            lay["parity"] ^= 1

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    K = args.steps
    # queue the timed loop behind a GPU spin long enough for the host to enqueue
    # all of it (the launches are issued from Python), so the layers run back to
    # back and host launch cost never shows as GPU idle time
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(2_000_000)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 2_000_000 / max(c0.elapsed_time(c1), 1e-3)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int((5.0 + K * layers * 0.04) * cycles_per_ms))
    a.record()
    for _ in range(K):
        one_step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    per_layer = algorithmic_bytes(B, 0, 1, s.H_v, s.d_k, s.d_v, s.C, s.W, "twin")
    total = per_layer * layers
    achieved = total / (ms * 1e-3) / 1e9
    return {
        "metric": STACK_METRIC, "value": B / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"9B-like GDN decode: {B} rows x 16 key / 32 value heads x 128x128 fp32 state, conv "
                               f"width 4 over 8192 channels, {layers} layers back to back on separate {s.N}-slot "
                               f"pools, twin-slot write with the commit folded in, stream launches",
                   "B": B, "layers": layers, "H_k": s.H_k, "H_v": s.H_v, "d_k": s.d_k, "d_v": s.d_v, "N": s.N},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None, "kernel": "gdn_step_tile_kernel",
                     "note": "whole-step time: every layer's launch queued back to back on one stream",
                     "bytes_per_step": total, "us_per_layer": ms * 1e3 / layers},
    }


SLOTOPS_METRIC = "GDN slot copy slots/s and achieved HBM GB/s (% of peak)"


def run_slotops(args) -> dict:
    """Slot lifecycle ops at the 0.8B-like layer's shapes: gdn_slot_copy of --rows
    slots (state and conv window, e.g. forking requests) and gdn_slot_reset of
    --rows slots (releasing them), each timed with fence-free HIP events around
    every launch.  Calls rotate over disjoint slot sets so that at least 768 MiB
    is written between two visits of a set (cold cache, as for the step)."""
    import torch

    import gated_deltanet_recurrent_decode_amd as gdn
    import gdn_inputs as gi

    gdn.lib()
    torch.cuda.set_device(0)
    B = args.rows
    case = gi.qwen08b(B=256)
    s, pool = case.shape, case.pools[0]
    slot_bytes = s.H_v * s.d_k * s.d_v * 4 + (s.W - 1) * s.C * 2
    nsets, per = row_sets("twin", B, 1, slot_bytes, args.hot)   # a copy set: B sources and B destinations
    spc = DRAWN_SLOTS // per
    copies = -(-nsets // spc)
    N = 1 + DRAWN_SLOTS * copies
    state0 = torch.from_numpy(pool.state).cuda()
    cs0 = _bf(torch, pool.conv_state)
    state = torch.zeros((N,) + tuple(state0.shape[1:]), dtype=state0.dtype, device="cuda")
    conv_state = torch.zeros((N,) + tuple(cs0.shape[1:]), dtype=cs0.dtype, device="cuda")
    for c in range(copies):
        state[1 + DRAWN_SLOTS * c:1 + DRAWN_SLOTS * (c + 1)] = state0[1:]
        conv_state[1 + DRAWN_SLOTS * c:1 + DRAWN_SLOTS * (c + 1)] = cs0[1:]
    del state0, cs0
    perm = np.random.Generator(np.random.PCG64(2)).permutation(DRAWN_SLOTS).astype(np.int32) + 1
    sets = []
    for k in range(nsets):
        j, off = k % spc, DRAWN_SLOTS * (k // spc)
        sets.append((torch.from_numpy(perm[j * per:j * per + B] + off).cuda(),
                     torch.from_numpy(perm[j * per + B:(j + 1) * per] + off).cuda()))
    timer = HipTimer()
    sh = torch.cuda.current_stream().cuda_stream
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    torch.cuda._sleep(2_000_000)
    c1.record()
    torch.cuda.synchronize()
    cycles_per_ms = 2_000_000 / max(c0.elapsed_time(c1), 1e-3)

    def timed(op):
        for i in range(args.warmup):
            op(sets[i % nsets])
        torch.cuda.synchronize()
        K = args.steps
        evs = [(timer.event(), timer.event()) for _ in range(K)]
        torch.cuda._sleep(int((5.0 + K * 0.12) * cycles_per_ms))
        for i in range(K):
            timer.record(evs[i][0], sh)
            op(sets[i % nsets])
            timer.record(evs[i][1], sh)
        torch.cuda.synchronize()
        us = np.array([timer.elapsed_ms(a, b) for a, b in evs]) * 1e3
        for a, b in evs:
            timer.destroy(a)
            timer.destroy(b)
        return us

    # a copy reads the source slot and writes the destination; a reset writes zeros
    copy_us = timed(lambda st: gdn.slot_copy(state, conv_state, st[0], st[1], H_k=s.H_k))
    reset_us = timed(lambda st: gdn.slot_reset(state, conv_state, st[1], H_k=s.H_k))
    copy_bytes = B * (2 * slot_bytes + 8)
    reset_bytes = B * (slot_bytes + 4)
    k_us = float(copy_us.mean())
    achieved = copy_bytes / (k_us * 1e-6) / 1e9
    r_us = float(reset_us.mean())
    return {
        "metric": SLOTOPS_METRIC, "value": B / (k_us * 1e-6), "unit": "slots/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": k_us * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"slot copy and slot reset of {B} slots a call (0.8B-like layer: 16 heads x 128x128 "
                               f"fp32 state and a bf16 conv window of 3 x 6144 a slot), {nsets} disjoint slot sets "
                               f"rotated over a {N}-slot pool (cold cache)",
                   "slots": B, "H_v": s.H_v, "d_k": s.d_k, "d_v": s.d_v, "C": s.C, "N": N, "row_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": None, "kernel": "slot_ops_kernel (copy)",
                     "kernel_us_mean": k_us, "kernel_us_p10": float(np.percentile(copy_us, 10)),
                     "kernel_us_p50": float(np.percentile(copy_us, 50)),
                     "kernel_us_p90": float(np.percentile(copy_us, 90)), "bytes_per_launch": copy_bytes},
        "reset": {"kernel_us_mean": r_us, "kernel_us_p50": float(np.percentile(reset_us, 50)),
                  "bytes_per_launch": reset_bytes, "GBps": reset_bytes / (r_us * 1e-6) / 1e9,
                  "frac": reset_bytes / (r_us * 1e-6) / 1e9 / PEAK_HBM_GBPS},
    }


PEAK_FP32_MFMA_TFLOPS = 157.3
PREFILL_METRIC = "GDN chunked prefill tokens/s and achieved fp32 matrix TFLOP/s (% of peak)"


def prefill_flops_per_token(H_v: int, d_k: int, d_v: int, chunk: int = 32) -> float:
    """Matrix-core flops the chunked prefill executes per token: per chunk and value
    head K S0 and Q S0 (2 * chunk * d_k * d_v each), K K^T and Q K^T (2 * chunk^2 * d_k
    each), P U (2 * chunk^2 * d_v) and K^T U (2 * d_k * chunk * d_v)."""
    per_chunk = 3 * 2 * chunk * d_k * d_v + 2 * 2 * chunk * chunk * d_k + 2 * chunk * chunk * d_v
    return H_v * per_chunk / chunk


def run_prefill(args) -> dict:
    """Packed prompts of --prefill-len tokens, --rows of them per call, at the 0.8B-like
    layer's shapes, in place; two sets of slots alternate.  Times each call (the two-pass
    form's three launches, or with --one-kernel the single prefill kernel) with fence-free
    HIP events around it; the workspace is allocated before the timed region."""
    import torch

    import gated_deltanet_recurrent_decode_amd as gdn
    import gdn_inputs as gi

    gdn.lib()
    torch.cuda.set_device(0)
    nseq, L = args.rows, args.prefill_len
    case = gi.prefill([L] * (2 * nseq), H_k=16, H_v=16, d=128, N=513, seed=0)
    s = case.shape
    state = torch.from_numpy(case.pool.state).cuda()
    conv_state = _bf(torch, case.pool.conv_state)
    conv_w = _bf(torch, case.pool.conv_w)
    sets = []
    for k in range(2):
        rows = slice(k * nseq * L, (k + 1) * nseq * L)
        sets.append(dict(x=_bf(torch, case.x[rows]), g=torch.from_numpy(np.ascontiguousarray(case.g[rows])).cuda(),
                         beta=torch.from_numpy(np.ascontiguousarray(case.beta[rows])).cuda(),
                         cu=torch.arange(0, (nseq + 1) * L, L, dtype=torch.int32, device="cuda"),
                         slot=torch.from_numpy(np.ascontiguousarray(case.pool.read_slot[k * nseq:(k + 1) * nseq])).cuda(),
                         out=torch.empty((nseq * L, s.H_v, s.d_v), dtype=torch.bfloat16, device="cuda")))

    ws = None
    if not args.one_kernel:
        ws = torch.empty((gdn.gdn_prefill_two_pass_workspace_bytes(nseq, nseq * L, s.H_k, s.H_v, s.d_k, s.d_v),),
                         dtype=torch.uint8, device="cuda")

    def launch(i):
        st = sets[i % 2]
        a = (st["x"], conv_w, None, conv_state, state, st["g"], st["beta"], st["cu"], st["slot"], st["out"])
        if ws is not None:
            gdn.gdn_prefill_two_pass(*a, ws, H_k=s.H_k)
        else:
            gdn.gdn_prefill(*a, H_k=s.H_k)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    timer = HipTimer()
    sh = torch.cuda.current_stream().cuda_stream
    K = args.steps
    evs = [(timer.event(), timer.event()) for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        timer.record(evs[i][0], sh)
        launch(i)
        timer.record(evs[i][1], sh)
    end.record()
    torch.cuda.synchronize()
    us = np.array([timer.elapsed_ms(a, b) for a, b in evs]) * 1e3
    for a, b in evs:
        timer.destroy(a)
        timer.destroy(b)
    ms_per_call = start.elapsed_time(end) / K
    tokens = nseq * L
    flops = prefill_flops_per_token(s.H_v, s.d_k, s.d_v) * tokens
    k_us = float(us.mean())
    achieved = flops / (k_us * 1e-6) / 1e12
    hbm = tokens * (s.C * 2 + s.H_v * s.d_v * 2 + 2 * s.H_v * 4) + nseq * 2 * (s.H_v * s.d_k * s.d_v * 4 + 3 * s.C * 2)
    traffic = None
    if ws is not None and kernel_code_sha256(PREFILL_KERNELS) == MEASURED_PREFILL_TRAFFIC["kernel_code_sha256"]:
        traffic = MEASURED_PREFILL_TRAFFIC["bytes_per_call"].get((nseq, L))
    return {
        "metric": PREFILL_METRIC, "value": tokens / (k_us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms_per_call, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"chunked prefill, {nseq} prompts of {L} tokens a call, 0.8B-like layer (16+16 heads "
                               f"of 128, 6144 conv channels, fp32 state), in place, two slot sets alternating, "
                               + ("two passes (chunk-parallel, then a column-sliced walk)" if ws is not None else
                                  "one kernel (a workgroup per prompt and key head)"),
                   "prompts": nseq, "prompt_len": L, "H_k": s.H_k, "H_v": s.H_v, "d_k": s.d_k, "d_v": s.d_v,
                   "path": "two-pass" if ws is not None else "one-kernel",
                   "workspace_bytes": 0 if ws is None else int(ws.numel())},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_MFMA_TFLOPS, "traffic": traffic,
                     "traffic_unit": "HBM bytes per call, its three kernels (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                     "copy-calibrated)",
                     "kernel": ("tp_chunk_map + tp_intra + tp_inter (one call)" if ws is not None else
                                "gdn_prefill_kernel"),
                     "kernel_us_mean": k_us, "kernel_us_p50": float(np.percentile(us, 50)),
                     "flops_per_launch": flops, "hbm_bytes_per_launch": hbm,
                     "hbm_GBps": hbm / (k_us * 1e-6) / 1e9},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--rows", type=int, default=64)
    ap.add_argument("--mode", choices=("twin", "inplace", "tokens", "prefill", "stack", "slotops"), default="twin",
                    help="twin-slot write, in-place write, a kept state per token (speculative verify), the "
                         "chunked prefill of --rows prompts of --prefill-len tokens, the 9B-like stack of "
                         "--layers layers (twin), or slot copy and reset of --rows slots a call")
    ap.add_argument("--layers", type=int, default=24)
    ap.add_argument("--key-heads", type=int, default=16,
                    help="decode modes: key heads shared by the 16 value heads (16, 8 or 4; in place G = 16 / H_k)")
    ap.add_argument("--prefill-len", type=int, default=512)
    ap.add_argument("--one-kernel", action="store_true",
                    help="prefill through gdn_prefill (one kernel, no workspace) instead of gdn_prefill_two_pass")
    ap.add_argument("--tokens", type=int, default=1, help="tokens a row (in place and tokens mode)")
    ap.add_argument("--real", type=int, default=None,
                    help="a padded bucket: only the first REAL of the --rows rows are real, the rest point at the "
                         "null slot (twin and in place)")
    ap.add_argument("--commit", choices=("fused", "separate"), default="fused")
    ap.add_argument("--hot", action="store_true", help="same rows every step (cache-warm)")
    ap.add_argument("--graph", action="store_true", help="time steps replayed from a captured HIP graph")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-calib", action="store_true", help="skip the traffic calibration probes")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the row sweep (1-128 rows, twin and in place, and a hot 64-row step) and the "
                         "launch-floor figures")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the decode step runs on one GPU (asked for --gpus {args.gpus}); it "
              "shards by rows or by heads with no exchange inside the step, and no multi-GPU path is built.",
              file=sys.stderr)
        return 2

    if args.mode == "stack":
        if args.rows < 1 or args.layers < 1:
            print("bench.py: the stack needs --rows >= 1 and --layers >= 1", file=sys.stderr)
            return 2
        result = run_stack(args)
        if not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(args, args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return 0
    if args.mode == "prefill":
        if args.rows < 1 or args.prefill_len < 1 or 4 * args.rows > 512:
            print("bench.py: prefill needs 1 <= --rows <= 128 and --prefill-len >= 1", file=sys.stderr)
            return 2
        result = run_prefill(args)
        if not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(args, args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return 0
    if args.mode == "slotops":
        if not 1 <= args.rows <= 256:
            print("bench.py: slot ops take 1 <= --rows <= 256", file=sys.stderr)
            return 2
        result = run_slotops(args)
        if not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(args, args.cpu_seconds)
        print(json.dumps(result), flush=True)
        return 0
    if args.real is not None and (args.mode == "tokens" or not 1 <= args.real <= args.rows):
        print("bench.py: --real takes 1 <= REAL <= --rows, twin or in place", file=sys.stderr)
        return 2
    if args.tokens < 1 or (args.mode == "twin" and args.tokens != 1):
        print("bench.py: --tokens must be >= 1, and twin-slot writes take one token a row", file=sys.stderr)
        return 2

    if args.key_heads not in (4, 8, 16):
        print("bench.py: --key-heads takes 16, 8 or 4 (the in-place kernel groups 1, 2 or 4 value heads)",
              file=sys.stderr)
        return 2
    dp = DevicePool(args.key_heads)
    try:
        b = Bench(dp, mode=args.mode, B=args.rows, T=args.tokens, real=args.real, hot=args.hot, commit=args.commit)
    except ValueError as e:
        print(f"bench.py: {e}", file=sys.stderr)
        return 2
    s = b.shape
    b.warm(args.warmup)

    K = args.steps
    graph = None
    if args.graph:
        graph = b.capture()
        K = max(graph[1], (K // graph[1]) * graph[1])
        for _ in range(2):
            graph[0].replay()
        b.torch.cuda.synchronize()
    ms_per_step, _ = b.timed(K, per_kernel_events=False, graph=graph)
    _, kus = b.timed(K, per_kernel_events=True)

    rows_per_s = b.R / (ms_per_step * 1e-3)
    twin = b.twin
    commit = ("folded into the step kernel (next slot pair written by the step)" if b.fused else
              "separate slot_commit kernel" if twin else
              "none (states kept per token)" if b.tokens_mode else "none (in place)")
    result = {
        "metric": METRIC,
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
        "config": {"workload": f"0.8B-like GDN layer decode step: {b.B} rows"
                               + (f" ({b.R} real, {b.B - b.R} on the null slot)" if b.R < b.B else "")
                               + f" x {s.H_k}+{s.H_v} heads x 128x128 fp32 state, "
                               f"conv width 4 over {s.C} channels, bf16 conv windows and activations, "
                               f"{b.N}-slot pool, {b.T} token{'s' if b.T > 1 else ''} a row, "
                               f"{ {'twin': 'twin-slot write', 'inplace': 'in-place write', 'tokens': 'state kept per token (speculative verify)'}[args.mode]}, commit "
                               f"{commit}, "
                               + ("same rows every step (cache-warm)" if args.hot else
                                  f"{b.nsets} disjoint row sets rotated (cold cache)")
                               + (", HIP graph replay" if graph is not None else ", stream launches"),
                   "B": b.B, "real_rows": b.R, "T": b.T, "H_k": s.H_k, "H_v": s.H_v, "d_k": s.d_k, "d_v": s.d_v, "W": s.W, "N": b.N,
                   "write": args.mode, "commit": "fused" if b.fused else ("separate" if twin else "none"),
                   "row_sets": b.nsets, "graph": graph is not None},
        "step_GBps": b.bytes / (ms_per_step * 1e-3) / 1e9,
    }
    k_us = float(kus.mean())
    achieved = b.bytes / (k_us * 1e-6) / 1e9
    traffic = None
    workload_key = (b.B, args.mode, "fused" if b.fused else "separate", bool(args.hot), s.H_k)
    if (MEASURED_TRAFFIC["kernel_code_sha256"] is not None
            and kernel_code_sha256() == MEASURED_TRAFFIC["kernel_code_sha256"]
            and workload_key == MEASURED_TRAFFIC["workload"]):
        traffic = MEASURED_TRAFFIC["bytes_per_launch"]
    result["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                          "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                          "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                          "kernel": step_kernel_label(twin, b.B, b.T, s.H_k, s.H_v, s.d_k, s.d_v, b.tokens_mode,
                                                      b.torch.cuda.get_device_properties(0).multi_processor_count),
                          "kernel_us_mean": k_us,
                          "kernel_us_p10": float(np.percentile(kus, 10)),
                          "kernel_us_p50": float(np.percentile(kus, 50)),
                          "kernel_us_p90": float(np.percentile(kus, 90)),
                          "bytes_per_launch": b.bytes,
                          # the counted bytes over the same kernel mean (null without counters)
                          "achieved_counted": traffic / (k_us * 1e-6) / 1e9 if traffic is not None else None}
    if not args.no_calib and not b.tokens_mode and b.T == 1:
        cal = b.calibration()
        result["calibration"] = cal
        ceiling = ceiling_of(cal, b.bytes, achieved)
        if ceiling is not None:
            result["roofline"]["ceiling"] = ceiling
    del b
    if not args.no_sweep:
        result["sweep"] = run_sweep(dp)
        result["floor"] = run_floors(dp)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(args, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
