"""The built library's gfx950 machine code, checked for three things.

No kernel uses scratch memory: each kernel's metadata (llvm-readelf --notes
on the code objects of the offload bundle) states a private segment of 0
bytes and no spilled vector register, so no launch shape of any entry point
spills its registers to memory.

And one hazard: a vector instruction that writes a register holding the data
of a 16- or 12-byte store issued by the instruction right before it.

A store with more than 8 bytes of data reads part of its data registers one
cycle late, so a vector write to them must wait at least one instruction.  The
compiler inserts that wait for most stores but not for buffer stores whose
offset sits in a scalar register, and on MI355X that case is real: a copy
kernel whose stores were staged through shared registers (a 64-bit register
move straight behind each buffer store) wrote, now and then, the next row's
values into half of a 16-byte store.  This test disassembles every kernel of
libgdn.so (llvm-objdump on the code objects of the offload bundle) and fails
on any vector write to a wide store's data registers by the next instruction,
so a recompile cannot bring the pattern back unnoticed.  Loads (LDS included)
into those registers are not counted: their data arrives long after the store
has read its registers.

And the step kernels' argument preloading: the build has the hardware load
their leading arguments (what the first round of scalar loads needs) into
scalar registers, which each kernel descriptor states (its 16-bit kernarg
preload field at byte 58: bits 0-6 the length in dwords, bits 7-15 the offset).
Losing the build flag would bring back a round trip before every step's first
load without failing any parity test, so the lengths are checked here.
"""
import os
import re
import subprocess
import tempfile

import pytest

import bench

LIB = os.path.join(bench.ROOT, "gated_deltanet_recurrent_decode_amd", "libgdn.so")
OBJDUMP = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-objdump")
READELF = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-readelf")

STORE = re.compile(r"^\s*(buffer_store_dwordx[34]|global_store_dwordx[34]|flat_store_dwordx[34]|"
                   r"scratch_store_dwordx[34])\s+(.*)$")
VREG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)")


def _regs(tok):
    m = VREG.fullmatch(tok.strip())
    if not m:
        return set()
    if m.group(3) is not None:
        return {int(m.group(3))}
    return set(range(int(m.group(1)), int(m.group(2)) + 1))


def _store_data(op, args):
    ops = [a.strip() for a in args.split(",")]
    # buffer stores: data first; global / flat / scratch stores: address, then data
    return _regs(ops[0]) if op.startswith("buffer") else (_regs(ops[1]) if len(ops) > 1 else set())


def _written(line):
    m = re.match(r"^\s*([a-z_0-9]+)\s+(.*)$", line)
    if not m:
        return "", set()
    op, args = m.group(1), m.group(2)
    if op.startswith(("s_", "buffer_store", "global_store", "flat_store", "scratch_store", "ds_", "buffer_load",
                      "global_load", "flat_load", "scratch_load", "exp")):
        return op, set()
    return op, _regs(args.split(",")[0])


def _disassembly():
    if not os.path.exists(LIB):
        pytest.skip("libgdn.so is not built")
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump is not available")
    out = []
    with tempfile.TemporaryDirectory() as d:
        for i, co in enumerate(bench.device_code_objects(LIB)):
            path = os.path.join(d, f"co{i}.elf")
            with open(path, "wb") as f:
                f.write(co)
            r = subprocess.run([OBJDUMP, "-d", "--no-show-raw-insn", path], capture_output=True, text=True,
                               check=True)
            out.append(r.stdout)
    return "\n".join(out)


def test_no_write_into_store_data_right_behind_a_wide_store():
    text = _disassembly()
    func = None
    bad = []
    insts = []
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            func = m.group(1)
            continue
        s = line.split("//")[0].strip()
        if not s or s.endswith(":"):
            continue
        insts.append((func, s))
    n = len(insts)
    stores = 0
    for i, (f, s) in enumerate(insts):
        m = STORE.match(s)
        if not m:
            continue
        stores += 1
        data = _store_data(m.group(1), m.group(2))
        for j in range(i + 1, min(n, i + 2)):
            if insts[j][0] != f:
                break
            op, w = _written(insts[j][1])
            if w & data:
                bad.append(f"{f}: '{s}' then '{insts[j][1]}' ({j - i} later)")
                break
    assert stores > 100, "expected the library's wide stores in the disassembly"
    assert not bad, "store data overwritten right behind the store:\n" + "\n".join(bad[:20])


def test_no_kernel_uses_scratch():
    if not os.path.exists(LIB):
        pytest.skip("libgdn.so is not built")
    if not os.path.exists(READELF):
        pytest.skip("llvm-readelf is not available")
    kernels = {}
    with tempfile.TemporaryDirectory() as d:
        for i, co in enumerate(bench.device_code_objects(LIB)):
            path = os.path.join(d, f"co{i}.elf")
            with open(path, "wb") as f:
                f.write(co)
            notes = subprocess.run([READELF, "--notes", path], capture_output=True, text=True, check=True).stdout
            name = None
            for line in notes.splitlines():
                m = re.match(r"^\s*\.name:\s+(\S+)", line)
                if m:
                    name = m.group(1)
                    kernels.setdefault(name, {})
                    continue
                m = re.match(r"^\s*\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)", line)
                if m and name is not None:
                    kernels[name][m.group(1)] = int(m.group(2))
    steps = [k for k in kernels if "gdn_step" in k]
    assert len(kernels) > 60 and len(steps) >= 40, "expected every kernel's metadata"
    scratch = {k: v for k, v in kernels.items() if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)}
    assert not scratch, f"kernels using scratch: {scratch}"


def _kernel_descriptors(co: bytes) -> dict:
    """name -> the 64-byte kernel descriptor (symbol `name.kd`) of a code object."""
    import struct
    secs = bench._elf_sections(co)
    symtab = [x for x in secs if x[0] == ".symtab"][0]
    strtab = secs[symtab[5]]
    out = {}
    for i in range(symtab[4] // 24):
        name, _info, _other, shndx, value, _size = struct.unpack_from("<IBBHQQ", co, symtab[3] + i * 24)
        end = co.index(b"\0", strtab[3] + name)
        nm = co[strtab[3] + name:end].decode()
        if nm.endswith(".kd") and 0 < shndx < len(secs):
            sec = secs[shndx]
            off = sec[3] + (value - sec[2])
            out[nm[:-3]] = co[off:off + 64]
    return out


def test_step_kernels_preload_their_leading_arguments():
    import struct
    if not os.path.exists(LIB):
        pytest.skip("libgdn.so is not built")
    kds = {}
    for co in bench.device_code_objects(LIB):
        kds.update(_kernel_descriptors(co))
    pre = {k: struct.unpack_from("<H", d, 58)[0] for k, d in kds.items()}
    tile = {k: v for k, v in pre.items() if "gdn_step_tile_kernel" in k}
    walk = {k: v for k, v in pre.items() if "15gdn_step_kernel" in k}
    probes = {k: v for k, v in pre.items() if "probe_" in k}
    assert len(tile) >= 18 and len(walk) >= 26 and len(probes) >= 40, "expected every step and probe kernel"
    # tile kernel: 4 pointers and 4 ints = 12 dwords from offset 0
    assert {v & 0x7F for v in tile.values()} == {12} and {v >> 7 for v in tile.values()} == {0}, tile
    # walk kernel: the read slots' pointer, H_k, N = 4 dwords
    assert {v & 0x7F for v in walk.values()} == {4} and {v >> 7 for v in walk.values()} == {0}, walk
    # copy probes: the pool, both slot arrays and five ints (+ the chunk size) = 11 or 12 dwords
    assert {v & 0x7F for v in probes.values()} <= {11, 12}, probes
    # kernels whose sources carry no preload flag preload nothing
    other = {k: v for k, v in pre.items() if k not in tile and k not in walk and k not in probes}
    assert other and not any(other.values()), {k: v for k, v in other.items() if v}
