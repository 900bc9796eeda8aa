"""Guards on the gfx950 code the library's kernels compile to.

A VMEM store wider than 64 bits reads its data registers after issue; a VALU
instruction that overwrites one of them right after the store needs a wait
state.  The compiler inserts it, except for buffer stores whose soffset field
holds a register, and on the GPU that case produced corrupted state entries.
The kernels therefore never give a wide buffer store a register soffset; this
test compiles every kernel source to assembly and checks both that rule and
the absence of the unprotected store/overwrite pair.  No GPU is needed.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_recurrence_decode_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["decode.hip", "prefill.hip", "copy.hip", "project.hip"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")),
                                reason="hipcc not available")

WIDE_STORE = re.compile(r"^\s*(buffer|global|flat)_store_dword(x3|x4)\s+(v\[(\d+):(\d+)\])(.*)$")
VALU_WRITE = re.compile(r"^\s*(v_\S+)\s+v(\d+)\b")


def assemble(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           "-x", "hip", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text().split("\n")


@pytest.mark.parametrize("src", SOURCES)
def test_no_unprotected_wide_store(src, tmp_path):
    lines = assemble(src, tmp_path)
    problems = []
    for i, line in enumerate(lines):
        m = WIDE_STORE.match(line)
        if not m:
            continue
        lo, hi, rest = int(m.group(4)), int(m.group(5)), m.group(6)
        if m.group(1) == "buffer":
            # operands after vdata: vaddr, srsrc, soffset, modifiers
            ops = [o.strip() for o in rest.lstrip(" ,").split(",")]
            soff = ops[2].split()[0] if len(ops) > 2 else "0"
            if re.match(r"^s\d+$|^s\[", soff):
                problems.append(f"register soffset: {line.strip()}")
        j = i + 1
        while j < len(lines) and (not lines[j].strip() or lines[j].strip().startswith(";")):
            j += 1
        w = VALU_WRITE.match(lines[j]) if j < len(lines) else None
        if w and lo <= int(w.group(2)) <= hi:
            problems.append(f"store data overwritten next: {line.strip()} | {lines[j].strip()}")
    assert not problems, "\n".join(problems[:10])
