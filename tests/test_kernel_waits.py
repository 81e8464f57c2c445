"""The streaming loops of the GEMM kernels keep their prefetched loads in flight.

The prefill K loop keeps PF steps of operand codes in flight and the decode
loop two register batches; both only pay off if each step waits for the loads
it consumes and not for the ones issued for later steps.  How the loop is
written decides what the compiler emits: an exit between the unrolled steps,
a load that may not be issued, or a 16-bit value widened where the loop's
register copies meet each made it wait for every load in flight
(`s_waitcnt vmcnt(0)`) inside the loop.  This test compiles gemm.hip for
gfx950 to assembly on the CPU, finds the main loop of each kernel below (the
loop with the most matrix instructions that also issues global loads) and
checks that no wait inside it drains the vector-memory counter.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S"]

# kernel symbol -> what it is
KERNELS = {
    "_ZN6splice18prefill_lds_kernelILb1EEEvNS_8GemmArgsE": "256 x 256 prefill tile",
    "_ZN6splice18prefill_seg_kernelILi256ELi4ELb1ELi2ELi1EEEvNS_8SegTableEiPjPf": "256 x 256 tile, segments",
    "_ZN6splice21prefill_lds128_kernelILb1ELi3ELi2EEEvNS_8GemmArgsEiPjPf": "128 x 128 tile",
    "_ZN6splice21prefill_lds128_kernelILb1ELi3ELi1EEEvNS_8GemmArgsEiPjPf": "128 x 128 tile, short K split",
    "_ZN6splice21prefill_lds128_kernelILb1ELi6ELi1EEEvNS_8GemmArgsEiPjPf": "128 x 128 tile, long K split",
    "_ZN6splice22grouped_prefill_kernelILi128ELi128ELb1EEEvNS_11GroupedArgsE": "grouped launch",
    "_ZN6splice14decode2_kernelILi1ELi3ELi8ELi1ELb1EEEvNS_8GemmArgsE": "decode, 48 columns",
    "_ZN6splice14decode2_kernelILi4ELi3ELi8ELi1ELb1EEEvNS_8GemmArgsE": "decode, 64 rows x 48 columns",
    "_ZN6splice15decode2s_kernelILi4ELi2ELi8ELi1ELb1EEEvNS_8GemmArgsEiPjPf": "decode, K split",
}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not available")
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    r = subprocess.run([HIPCC, *FLAGS, os.path.join(ROOT, "fp4_gemm_sparse_amd", "csrc", "gemm.hip"),
                        "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return open(out).read().split("\n")


def function_body(lines, sym):
    start = next((i for i, l in enumerate(lines) if l.startswith(sym + ":")), None)
    assert start is not None, f"{sym} not found in the assembly"
    end = next(i for i in range(start, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[start:end]


def loops(body):
    """Instructions of each innermost loop, keyed by its header block, from
    the compiler's block annotations (a block opens with its label, or with a
    `; %bb.N:` comment when it is only fallen into, and says which loop
    header it belongs to)."""
    out = {}
    cur = None
    for l in body:
        m = re.match(r"^(?:\.LBB(\w+):|; %bb\.\d+:)(.*)$", l)
        if m:
            name, note = m.group(1), m.group(2)
            h = re.search(r"in Loop: Header=BB(\w+)", note)
            if "Loop Header" in note and name:
                cur = name
            elif h:
                cur = h.group(1)
            else:
                cur = None
            continue
        if cur is not None:
            x = l.strip()
            if x and not x.startswith((";", ".")):
                out.setdefault(cur, []).append(x)
    return out


# Known: in the short K-split instance (three stages, one workgroup per CU,
# accumulators in AGPRs) the compiler still waits for every load once per
# group of three steps, at the top of the loop, for a reason not found in its
# source; the two- and four-stage forms do the same, and the
# six-stage instance, which does not, measured slower on ranges of 8 steps.
KNOWN_DRAIN = {"_ZN6splice21prefill_lds128_kernelILb1ELi3ELi1EEEvNS_8GemmArgsEiPjPf"}


@pytest.mark.parametrize("sym", [pytest.param(k, marks=pytest.mark.xfail(strict=True, reason="known drain"))
                                 if k in KNOWN_DRAIN else k for k in KERNELS])
def test_main_loop_keeps_loads_in_flight(asm, sym):
    body = function_body(asm, sym)
    best = None
    for ins in loops(body).values():
        nm = sum(1 for x in ins if x.startswith("v_mfma"))
        if any(x.startswith(("global_load", "buffer_load")) for x in ins) and (best is None or nm > best[0]):
            best = (nm, ins)
    assert best is not None and best[0] > 0, f"{KERNELS[sym]}: no streaming loop found"
    drains = [x for x in best[1] if x.startswith("s_waitcnt") and re.search(r"vmcnt\(0\)", x)]
    waits = [x for x in best[1] if x.startswith("s_waitcnt") and "vmcnt" in x]
    assert not drains, f"{KERNELS[sym]}: the main loop waits for every load in flight: {drains[:3]}"
    assert waits, f"{KERNELS[sym]}: the main loop never waits for its loads"
