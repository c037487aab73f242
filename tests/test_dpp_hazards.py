"""The DPP read hazard, checked on the built library's gfx950 code.

On gfx9-family GPUs a VALU instruction that writes a VGPR must be followed by
two wait states before a DPP instruction reads that VGPR as its DPP source;
the hardware does not interlock.  The compiler inserts those waits around the
DPP it generates itself, but not around DPP written in inline assembly (the
row kernel's broadcast fma, v_fmac_f32_dpp with row_newbcast), whose source
must come from a load.  This test disassembles every gfx950 code object of
libssmscan.so (code built here from this repository's sources) and checks
every DPP instruction: no VALU write of its source register within the two
wait states before it.  A planted listing checks that the checker finds such a
write.

The same holds for an MFMA's A and B operands: a VALU write needs two wait
states before an MFMA reads the VGPR (the compiler inserts s_nop 1 for its
own code; an operand last written inside inline assembly would get none).
Every MFMA of the library (the SSD and dt_proj kernels) is checked for that
hazard too."""
import os
import re
import shutil
import struct
import subprocess

import pytest

from selective_scan_ssm_amd import _lib

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
INST = re.compile(r"^(v_\w+|s_\w+|ds_\w+|buffer_\w+|global_\w+|flat_\w+|scratch_\w+)\s*(.*?)(\s*//.*)?$")
DPP_MARK = ("row_newbcast", "row_ror", "row_shl", "row_shr", "row_mirror", "row_half_mirror", "row_bcast",
            "quad_perm", "wave_shl", "wave_shr", "wave_rol", "wave_ror")


def parse(listing):
    """(opcode, operands) of each instruction; ('LABEL', name) at functions."""
    out = []
    for line in listing.splitlines():
        t = line.strip()
        m = re.match(r"^[0-9a-f]+ <(.*)>:$", t)
        if m:
            out.append(("LABEL", m.group(1)))
            continue
        m = INST.match(t)
        if m:
            out.append((m.group(1), m.group(2)))
    return out


def written_vgprs(operands):
    dst = operands.split(",")[0].strip()
    m = re.match(r"v\[(\d+):(\d+)\]", dst)
    if m:
        return {f"v{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
    return {dst} if re.match(r"^v\d+$", dst) else set()


def dpp_hazards(insts):
    """DPP instructions whose source register a VALU wrote less than two
    wait states before (an s_nop k counts k + 1, any other instruction 1)."""
    found, n_dpp = [], 0
    for i, (op, args) in enumerate(insts):
        if not op.startswith("v_") or not any(k in args for k in DPP_MARK):
            continue
        n_dpp += 1
        ops = [a.strip() for a in args.split(",")]
        if len(ops) < 2:
            continue
        src0 = ops[1].split()[0]
        waits, j = 0, i - 1
        while j >= 0 and waits < 2:
            pop, pargs = insts[j]
            if pop == "LABEL":
                break
            if pop == "s_nop":
                waits += int(pargs.split()[0], 0) + 1
            else:
                if pop.startswith("v_") and src0 in written_vgprs(pargs):
                    found.append((insts[j], insts[i]))
                waits += 1
            j -= 1
    return n_dpp, found


def mfma_src_hazards(insts):
    """MFMA instructions whose A or B operand register a VALU wrote less
    than two wait states before (counted as in dpp_hazards)."""
    found, n_mfma = [], 0
    for i, (op, args) in enumerate(insts):
        if not op.startswith("v_mfma"):
            continue
        n_mfma += 1
        ops = [a.strip() for a in args.split(",")]
        if len(ops) < 3:
            continue
        srcs = set()
        for a in ops[1:3]:
            m = re.match(r"v\[(\d+):(\d+)\]", a)
            if m:
                srcs |= {f"v{k}" for k in range(int(m.group(1)), int(m.group(2)) + 1)}
            elif re.match(r"^v\d+$", a):
                srcs.add(a)
        waits, j = 0, i - 1
        while j >= 0 and waits < 2:
            pop, pargs = insts[j]
            if pop == "LABEL":
                break
            if pop == "s_nop":
                waits += int(pargs.split()[0], 0) + 1
            else:
                if pop.startswith("v_") and not pop.startswith("v_mfma") and srcs & written_vgprs(pargs):
                    found.append((insts[j], insts[i]))
                waits += 1
            j -= 1
    return n_mfma, found


def code_objects(lib_path, tmp):
    """The gfx950 code objects of the library's .hip_fatbin (one bundle per
    translation unit)."""
    fat = os.path.join(tmp, "fatbin.bin")
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib_path, fat], check=True)
    data = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    paths = []
    for k, p in enumerate(starts):
        blob = data[p:starts[k + 1] if k + 1 < len(starts) else len(data)]
        n = struct.unpack_from("<Q", blob, len(MAGIC))[0]
        off = len(MAGIC) + 8
        for _ in range(n):
            o, size, idlen = struct.unpack_from("<QQQ", blob, off)
            off += 24
            ident = blob[off:off + idlen].decode()
            off += idlen
            if "gfx950" in ident:
                path = os.path.join(tmp, f"co{k}.o")
                open(path, "wb").write(blob[o:o + size])
                paths.append(path)
    return paths


def test_checker_finds_a_planted_hazard():
    listing = """0000000000001000 <k>:
    v_mul_f32_e32 v5, v1, v2
    v_fmac_f32_dpp v7, v5, v3 row_newbcast:1 row_mask:0xf bank_mask:0xf bound_ctrl:1
    v_mul_f32_e32 v6, v1, v2
    s_nop 1
    v_fmac_f32_dpp v8, v6, v3 row_newbcast:2 row_mask:0xf bank_mask:0xf bound_ctrl:1
    ds_read_b32 v9, v0
    v_fmac_f32_dpp v8, v9, v3 row_newbcast:3 row_mask:0xf bank_mask:0xf bound_ctrl:1
    v_mov_b32_e32 v[10:11], 0
    v_add_f32_dpp v4, v11, v4 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf
"""
    n, found = dpp_hazards(parse(listing))
    assert n == 4
    assert [f[1][1].split(",")[1].strip() for f in found] == ["v5", "v11"]


def test_checker_finds_a_planted_mfma_source_hazard():
    listing = """0000000000002000 <k>:
    v_fmac_f32_dpp v20, v23, v17 row_newbcast:7 row_mask:0xf bank_mask:0xf bound_ctrl:1
    v_mul_f32_e64 v5, |v4|, s96
    v_mfma_f32_16x16x4_f32 a[0:3], v57, v20, a[0:3]
    v_fmac_f32_dpp v21, v23, v17 row_newbcast:7 row_mask:0xf bank_mask:0xf bound_ctrl:1
    s_nop 1
    v_mfma_f32_16x16x4_f32 a[0:3], v57, v21, a[0:3]
    v_mov_b32_e32 v[30:31], 0
    v_mfma_f32_16x16x32_bf16 v[0:3], v[28:31], v[40:43], v[0:3]
    ds_read_b128 v[44:47], v1
    v_mfma_f32_16x16x32_bf16 v[0:3], v[44:47], v[40:43], v[0:3]
"""
    n, found = mfma_src_hazards(parse(listing))
    assert n == 4
    assert [f[0][1].split(",")[0].strip() for f in found] == ["v20", "v[30:31]"]


@pytest.mark.skipif(not (os.path.exists(OBJDUMP) and shutil.which("objcopy")), reason="no llvm-objdump / objcopy")
def test_no_mfma_source_hazard_in_the_built_library(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        from selective_scan_ssm_amd import build
        build.build()
    paths = code_objects(_lib.LIB_PATH, str(tmp_path))
    assert paths, "no gfx950 code object in the library"
    total, hazards = 0, []
    for path in paths:
        dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], capture_output=True, text=True,
                             check=True).stdout
        n, found = mfma_src_hazards(parse(dis))
        total += n
        hazards += found
    assert total > 100, total               # the SSD and dt_proj kernels' MFMAs are there
    assert not hazards, hazards[:5]


@pytest.mark.skipif(not (os.path.exists(OBJDUMP) and shutil.which("objcopy")), reason="no llvm-objdump / objcopy")
def test_no_dpp_read_hazard_in_the_built_library(tmp_path):
    if not os.path.exists(_lib.LIB_PATH):
        from selective_scan_ssm_amd import build
        build.build()
    paths = code_objects(_lib.LIB_PATH, str(tmp_path))
    assert paths, "no gfx950 code object in the library"
    total, hazards = 0, []
    for path in paths:
        dis = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", path], capture_output=True, text=True,
                             check=True).stdout
        n, found = dpp_hazards(parse(dis))
        total += n
        hazards += found
    assert total > 1000, total              # the row kernels' broadcasts are there
    assert not hazards, hazards[:5]
