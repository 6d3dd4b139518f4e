"""Register and scratch use of every gfx950 kernel in the built library (no GPU).

Reads the kernel metadata that the compiler stores in the library's own gfx950 code objects
(the offload bundles in its .hip_fatbin section).  A kernel whose accumulators or register
rings fall out of registers (vector spills, or an array the compiler had to place in private
memory) still passes every parity test but runs several times slower, so this is checked
here: no kernel may use private (scratch) memory or spill vector registers, and the
matrix-core kernels must fit two waves per SIMD (at most 256 registers) as their launch
bounds ask.  Scalar-register spills go to lanes of vector registers (no memory traffic) and
are allowed.
"""
import os
import re
import struct
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "moe_expert_offload_amd", "libmoe.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(fatbin):
    """gfx950 code objects of every offload bundle in the section (one per source file)."""
    out = []
    b = fatbin.find(MAGIC)
    while b >= 0:
        n = struct.unpack_from("<Q", fatbin, b + 24)[0]
        p = b + 32
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", fatbin, p)
            p += 24
            triple = fatbin[p:p + tl].decode()
            p += tl
            if triple.endswith("gfx950"):
                out.append(fatbin[b + off:b + off + size])
        b = fatbin.find(MAGIC, b + 1)
    return out


def _kernels(tmp_path):
    if not os.path.exists(LIB):
        pytest.fail("libmoe.so is not built (run __graft_entry__.build())")
    sec = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={sec}", LIB,
                    str(tmp_path / "lib.copy")], check=True, capture_output=True)
    kernels = {}
    for i, co in enumerate(_code_objects(sec.read_bytes())):
        f = tmp_path / f"co{i}.elf"
        f.write_bytes(co)
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(f)], check=True,
                               capture_output=True, text=True).stdout
        for block in notes.split("  - .agpr_count:")[1:]:
            field = lambda k: re.search(r"\." + k + r":\s+(\S+)", block).group(1)
            kernels[field("name")] = {
                "agpr": int(block.split("\n")[0]),
                "vgpr": int(field("vgpr_count")),
                "vgpr_spill": int(field("vgpr_spill_count")),
                "sgpr_spill": int(field("sgpr_spill_count")),
                "private": int(field("private_segment_fixed_size")),
            }
    return kernels


def test_no_kernel_spills_or_uses_scratch(tmp_path):
    ks = _kernels(tmp_path)
    names = " ".join(ks)
    for k in ("k1_logits", "k2_resolve", "k3_gate_up", "k4_down", "k2g_group", "k5_gate_up", "k5_down", "k5_combine"):
        assert k in names, k
    bad = {n: r for n, r in ks.items() if r["private"] or r["vgpr_spill"]}
    assert not bad, bad


def test_matrix_core_kernels_fit_two_waves_per_simd(tmp_path):
    ks = _kernels(tmp_path)
    mm = {n: r for n, r in ks.items() if "k5_gate_up" in n or "k5_down" in n}
    assert mm
    for n, r in mm.items():
        # on this target the metadata's vgpr_count is the whole unified register block of a wave
        # (architected VGPRs and AGPRs together; agpr_count is its AGPR part)
        assert r["agpr"] <= r["vgpr"] <= 256, (n, r)
