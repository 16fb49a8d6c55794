"""The built gfx950 code (disassembled on the CPU from libconvmi.so, which this
repository builds from source) touches M0 only inside the LDS-DMA copy blocks of
lds_dma.hpp: every instruction naming M0 is a write immediately followed by the
global/buffer load-to-LDS that consumes it, and no instruction that reads M0 implicitly
for another purpose (messages, GWS, indirect register moves, LDS append/consume)
appears.  So no M0 value the compiler relies on can be live across those blocks."""
import glob
import os
import re
import shutil
import subprocess

import pytest

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "convolution_layer_amd", "libconvmi.so")


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    if not os.path.exists(OBJDUMP) or not os.path.exists(LIB):
        pytest.skip("llvm-objdump or the built library is missing")
    d = tmp_path_factory.mktemp("isa")
    lib = os.path.join(d, "libconvmi.so")
    shutil.copy(LIB, lib)
    subprocess.run([OBJDUMP, "--offloading", lib], cwd=d, check=True, capture_output=True)
    objs = sorted(glob.glob(os.path.join(d, "*amdgcn-amd-amdhsa--gfx950")))
    assert objs, "no gfx950 code object in the library"
    text = []
    for o in objs:
        r = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", o], check=True, capture_output=True, text=True)
        text.extend(r.stdout.splitlines())
    return [ln.strip() for ln in text if ln.startswith("\t") or ln.startswith(" ")]


def test_m0_only_feeds_lds_copies(disassembly):
    ins = [ln for ln in disassembly if ln and not ln.startswith(";")]
    uses = [i for i, ln in enumerate(ins) if re.search(r"\bm0\b", ln)]
    assert uses, "expected the LDS-DMA copies to set M0"
    for i in uses:
        assert re.match(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)\b", ins[i]), ins[i]
        nxt = ins[i + 1]
        assert nxt.startswith("global_load_lds_dwordx4") or (nxt.startswith("buffer_load_dwordx4") and " lds" in nxt), \
            (ins[i], nxt)
    implicit = [ln for ln in ins if re.match(r"(s_sendmsg|s_movrel|v_movrel|ds_gws|ds_append|ds_consume)", ln)]
    assert not implicit, implicit[:5]
