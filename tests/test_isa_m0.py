"""The built gfx950 code uses M0 only for the kernels' own direct-to-LDS loads.

Those loads are issued from inline assembly that writes M0 (the LDS address)
right before each load.  M0 is a register the compiler reserves and does not
track through inline assembly, so the loads are only correct while no other
instruction of the kernels reads or writes M0.  This test disassembles the
device code of every object of the library build (AMD assembly of code built
here) and checks that: every M0 write is one of ours, each followed by the
5-state wait and a direct-to-LDS load, every such load has its M0 write just
before it, and no instruction that reads M0 implicitly appears anywhere else.
A compiler update that starts using M0 fails here instead of corrupting
loads.  No GPU is used.
"""
import glob
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "memory_efficient_attention_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
# instructions that read M0 without naming it (gfx9 family)
IMPLICIT_M0 = re.compile(r"^(s_sendmsg|s_movrel|v_movrel|ds_gws|ds_ordered_count|ds_append|ds_consume|"
                         r"s_ttracedata)|\bgds\b")
LDS_DMA = re.compile(r"^(buffer_load_\w+ .*\blds$|global_load_lds_\w+)")


def _objects():
    objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    if not objs:
        if not os.path.exists(os.path.join(LLVM, "clang-offload-bundler")):
            pytest.skip("ROCm LLVM tools not installed")
        from memory_efficient_attention_amd import build
        build.build()
        objs = sorted(glob.glob(os.path.join(BUILD, "*.o")))
    return objs


def _disassemble(obj, tmp):
    fb = os.path.join(tmp, "fatbin")
    co = os.path.join(tmp, "co.o")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", f".hip_fatbin={fb}", obj],
                   check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o", f"--targets={TARGET}",
                    f"--input={fb}", f"--output={co}", "--unbundle"], check=True, capture_output=True)
    out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co], check=True,
                         capture_output=True, text=True).stdout
    # instruction text only (drop the encoding comment), in order
    ins = []
    for line in out.splitlines():
        if line.startswith("\t"):
            ins.append(line.strip().split("//")[0].strip())
    return ins


def test_m0_is_used_only_by_the_direct_to_lds_loads():
    if not os.path.exists(os.path.join(LLVM, "llvm-objdump")):
        pytest.skip("ROCm LLVM tools not installed")
    objs = _objects()
    assert objs, "no objects in the build directory"
    tmp = tempfile.mkdtemp()
    try:
        n_loads = 0
        for obj in objs:
            ins = _disassemble(obj, tmp)
            name = os.path.basename(obj)
            for i, x in enumerate(ins):
                assert not IMPLICIT_M0.search(x), f"{name}: {x!r} reads M0"
                if re.search(r"\bm0\b", x):
                    assert re.fullmatch(r"s_mov_b32 m0, s\d+", x), f"{name}: {x!r} uses M0"
                    assert ins[i + 1] == "s_nop 4", f"{name}: M0 write not followed by the wait: {ins[i + 1]!r}"
                    assert LDS_DMA.match(ins[i + 2]), f"{name}: M0 write not followed by an LDS load"
                if LDS_DMA.match(x):
                    n_loads += 1
                    assert i >= 2 and ins[i - 1] == "s_nop 4" and ins[i - 2].startswith("s_mov_b32 m0,"), \
                        f"{name}: LDS load without its own M0 write: {ins[i - 2:i + 1]}"
        assert n_loads > 0
    finally:
        shutil.rmtree(tmp)
