"""Checks on the gfx950 machine code of the built libraries, no GPU needed: the
code object is read out of each library's .hip_fatbin section (the library
file is only read) and disassembled with the ROCm LLVM tools.

The data of a vector-memory store wider than 8 bytes is read from its VGPRs
after the store issues, so a vector instruction in the very next slot must not
write those registers (the store would write the new value).  The compiler
keeps that slot clear for its own stores; a store written in inline assembly
(the decode epilogue's streaming store, the probe's) carries its own wait
states.  These tests hold both to it, on the code the tests and the benchmark
actually load, and check that the decode library proper carries none of the
timeline build's instrumentation."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import mla_latent_kv_amd as mk
from mla_latent_kv_amd import _build

LLVM_BIN = "/opt/rocm/llvm/bin"


def _tool(name):
    path = os.path.join(LLVM_BIN, name)
    if os.path.exists(path):
        return path
    found = shutil.which(name)
    if found is None:
        pytest.skip(f"{name} not available")
    return found


BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _elf_section(path, name):
    """Bytes of section `name` of an ELF64 little-endian file, read directly (a
    tool such as objcopy would write the library back over itself)."""
    import struct
    data = open(path, "rb").read()
    assert data[:4] == b"\x7fELF" and data[4] == 2 and data[5] == 1, f"{path}: not an ELF64 LE file"
    shoff, = struct.unpack_from("<Q", data, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", data, 0x3A)

    def header(i):
        off = shoff + i * shentsize
        sh_name, = struct.unpack_from("<I", data, off)
        sh_offset, sh_size = struct.unpack_from("<QQ", data, off + 0x18)
        return sh_name, sh_offset, sh_size

    _, str_off, str_size = header(shstrndx)
    names = data[str_off:str_off + str_size]
    for i in range(shnum):
        sh_name, off, size = header(i)
        if names[sh_name:names.index(b"\0", sh_name)].decode() == name:
            return data[off:off + size]
    raise AssertionError(f"{path}: no section {name}")


def _disassemble(lib_path):
    """Disassembly of every gfx950 code object in the library: its .hip_fatbin
    section holds one offload bundle per source file, back to back."""
    bundler, objdump = _tool("clang-offload-bundler"), _tool("llvm-objdump")
    data = _elf_section(lib_path, ".hip_fatbin")
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
    assert starts and starts[0] == 0, "no offload bundle in the .hip_fatbin section"
    out = []
    with tempfile.TemporaryDirectory() as d:
        for k, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part, code = os.path.join(d, f"b{k}"), os.path.join(d, f"b{k}.co")
            with open(part, "wb") as f:
                f.write(data[a:b])
            subprocess.run([bundler, "--unbundle", "--type=o", f"--input={part}",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={code}"], check=True,
                           capture_output=True)
            out.append(subprocess.run([objdump, "-d", "--mcpu=gfx950", code], check=True, capture_output=True,
                                      text=True).stdout)
    return "\n".join(out)


def _functions(dis):
    """{symbol: [instruction text, ...]} in program order."""
    funcs, cur = {}, None
    for line in dis.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
            continue
        if cur is not None and line.startswith("\t"):
            ins = line.split("//")[0].strip()
            if ins:
                cur.append(ins)
    return funcs


def _vregs(text):
    """VGPR numbers named in an operand string (v7, v[4:7])."""
    regs = set()
    for m in re.finditer(r"\bv\[(\d+):(\d+)\]|\bv(\d+)\b", text):
        if m.group(3) is not None:
            regs.add(int(m.group(3)))
        else:
            regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    return regs


WIDE_STORE = re.compile(r"^(global|buffer|flat|scratch)_store_dwordx[34]\b")


def _wide_store_hazards(funcs):
    bad = []
    for name, code in funcs.items():
        for i, ins in enumerate(code[:-1]):
            if not WIDE_STORE.match(ins):
                continue
            ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
            data = _vregs(ops[1])   # vaddr, vdata, ... for global/flat/scratch; vdata first for buffer
            if ins.startswith("buffer_"):
                data = _vregs(ops[0])
            nxt = code[i + 1]
            if nxt.startswith("v_") and " " in nxt:
                dst = _vregs(nxt.split(None, 1)[1].split(",")[0])
                if dst & data:
                    bad.append(f"{name}: {ins} / {nxt}")
    return bad


@pytest.fixture(scope="module")
def decode_code():
    if not os.path.exists(mk.LIB_PATH):
        _build.build()
    return _functions(_disassemble(mk.LIB_PATH))


@pytest.fixture(scope="module")
def probe_code():
    if not os.path.exists(_build.PROBE_LIB):
        _build.build()
    return _functions(_disassemble(_build.PROBE_LIB))


def test_disassembly_holds_the_kernels(decode_code, probe_code):
    decode = [n for n in decode_code if "decode_kernel" in n]
    assert len(decode) == 16, sorted(decode_code)   # NB x SPLIT x OUT_F32 x SPARSE x FP8 instantiations
    assert any("merge_unabsorb_kernel" in n for n in decode_code)
    assert any("pipe_kernel" in n for n in probe_code)


def test_streaming_stores_carry_their_wait_states(decode_code, probe_code):
    """Every store with the streaming hint is the inline-assembly one, followed
    by s_nop 1 or more."""
    for funcs, where in ((decode_code, "decode library"), (probe_code, "probe library")):
        n = 0
        for name, code in funcs.items():
            for i, ins in enumerate(code[:-1]):
                if WIDE_STORE.match(ins) and re.search(r"\bnt\b", ins):
                    n += 1
                    m = re.match(r"^s_nop (\d+)$", code[i + 1])
                    assert m and int(m.group(1)) >= 1, f"{where}: {name}: {ins} / {code[i + 1]}"
        assert n > 0, f"no streaming store found in the {where}"


def test_no_vector_write_of_store_data_in_the_next_slot(decode_code, probe_code):
    bad = _wide_store_hazards(decode_code) + _wide_store_hazards(probe_code)
    assert not bad, "\n".join(bad[:10])


def test_hazard_check_detects_a_planted_case():
    """The checker itself: the sequence the compiler produced around a bare
    assembly store (a VALU write of the store's data register next) is flagged,
    the same store followed by s_nop is not."""
    planted = {"k": ["global_store_dwordx4 v[0:1], v[4:7], off nt", "v_mov_b32_e32 v4, v34", "s_endpgm"]}
    assert _wide_store_hazards(planted)
    fixed = {"k": ["global_store_dwordx4 v[0:1], v[4:7], off nt", "s_nop 1", "v_mov_b32_e32 v4, v34"]}
    assert not _wide_store_hazards(fixed)
    addr_only = {"k": ["global_store_dwordx4 v[0:1], v[4:7], off", "v_lshl_add_u64 v[0:1], s[0:1], 0, v[8:9]"]}
    assert not _wide_store_hazards(addr_only)


@pytest.fixture(scope="module")
def timeline_code():
    if not os.path.exists(_build.TIMELINE_LIB):
        _build.build()
    return _functions(_disassemble(_build.TIMELINE_LIB))


def test_timeline_points_only_in_the_timeline_build(decode_code, timeline_code):
    """The decode library proper carries no timeline point (the instrumented
    build of the same source is a library of its own); the timeline build's
    headline kernel reads the real-time counter at its eight points."""
    for name, code in decode_code.items():
        assert not any(i.startswith("s_memrealtime") for i in code), name
    head = [n for n in timeline_code if n.startswith("_ZN3mla13decode_kernelILi4ELb1ELb0ELb0ELb0E")]
    assert len(head) == 1
    assert sum(i.startswith("s_memrealtime") for i in timeline_code[head[0]]) == 8


def test_timeline_entry_point_only_in_the_timeline_build():
    import ctypes
    if not os.path.exists(_build.TIMELINE_LIB):
        _build.build()
    mk.load_library()   # (the HIP runtime first, as for the product library)
    assert not hasattr(ctypes.CDLL(mk.LIB_PATH), "mla_timeline_read")
    assert hasattr(ctypes.CDLL(_build.TIMELINE_LIB), "mla_timeline_read")
