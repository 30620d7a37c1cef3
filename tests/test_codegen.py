"""Checks on the compiled device code (gfx950 assembly from hipcc -S).

The kernels wait for their direct global-to-LDS loads with explicit vmcnt
counts, which hold only if the compiler emits the vector-memory operations
the source implies; and the pipelined kernel's launch parameters must stay in
scalar registers (an out-of-line call or scratch use puts them in memory and
turns every base pointer into a per-lane value).  These tests compile the
sources and check exactly that.  CPU only: hipcc cross-compiles.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_36_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def device_asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    subprocess.run([HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", f"-I{ROOT}/include", f"-I{CSRC}", "--cuda-device-only",
                    "-S", os.path.join(CSRC, src), "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


def functions(asm):
    """name -> body text of every function in the assembly."""
    bodies = {}
    for m in re.finditer(r"^(\S+):\s*;\s*@\1\n(.*?)^\.Lfunc_end", asm, re.M | re.S):
        bodies[m.group(1)] = m.group(2)
    return bodies


def kernel_metadata(asm):
    """kernel symbol -> dict of .vgpr_spill_count, .private_segment_fixed_size."""
    meta = {}
    for block in asm.split("  - .agpr_count:")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        meta[name] = {k: int(re.search(rf"\.{k}:\s+(\d+)", block).group(1))
                      for k in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size")}
    return meta


def opcodes(body):
    return [line.split()[0] for line in body.splitlines()
            if line.startswith("\t") and not line.lstrip().startswith((";", "."))]


def test_combine_memory_operations_match_its_waits(tmp_path):
    """scan_combine_kernel waits vmcnt(8) for a segment's direct loads,
    assuming that only the 8 single-dword stores of one segment step were
    issued after them: every store must be a global_store_dword, their
    number a multiple of 8, and no other vector-memory operation may appear
    besides the direct loads and the two loads of the starting state."""
    asm = device_asm("kda_scan.hip", tmp_path)
    fns = {k: v for k, v in functions(asm).items() if "scan_combine_kernel" in k}
    assert len(fns) == 1
    ops = opcodes(next(iter(fns.values())))
    vmem = [o for o in ops if o.startswith(("global_", "buffer_", "scratch_", "flat_"))]
    stores = [o for o in vmem if "store" in o]
    assert stores and all(o == "global_store_dword" for o in stores), sorted(set(stores))
    assert len(stores) % 8 == 0
    others = [o for o in vmem if "store" not in o and o != "global_load_lds_dwordx4"]
    assert others == ["global_load_dwordx4", "global_load_dwordx4"], others
    # the explicit waits (0, 8) and the compiler's own between the two
    # starting-state loads (1)
    waits = set(re.findall(r"s_waitcnt vmcnt\((\d+)\)", "\n".join(fns.values())))
    assert waits <= {"0", "1", "8"}, waits
    assert "s_swappc" not in ops


@pytest.mark.parametrize("src", ["kda_chunk_mfma.hip", "kda_scan.hip", "kda_decode.hip"])
def test_no_calls_scratch_or_spills(src, tmp_path):
    """Every kernel is one inlined function with no scratch memory: the
    launch parameters stay in scalar registers, which the direct loads' scalar
    base operand requires."""
    asm = device_asm(src, tmp_path)
    meta = kernel_metadata(asm)
    assert meta
    for name, m in meta.items():
        assert m["private_segment_fixed_size"] == 0, (name, m)
        assert m["vgpr_spill_count"] == 0 and m["sgpr_spill_count"] == 0, (name, m)
    assert "s_swappc" not in asm
    assert not [n for n in functions(asm) if n not in meta], "out-of-line device functions"
