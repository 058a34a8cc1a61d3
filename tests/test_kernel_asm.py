"""Static checks on the gfx950 assembly of the attention kernels (CPU only).

The LDS-filling buffer loads are inline assembly, so the compiler cannot pad
the hazards of their operands.  The ISA requires 5 wait states between a
VALU write of an SGPR (v_readfirstlane) and a vector-memory instruction that
reads it, and 1 wait state between a scalar write of M0 and a buffer load
that writes LDS.  This test compiles the kernels to assembly and checks every
such load: the instruction right before it must be the asm's own s_nop of at
least 4 (5 wait states), whatever the compiler put before the asm block, and
the distances are measured as well.  (A microbenchmark that issued these
loads without the padding made the GPU fault: the compiler had placed the
v_readfirstlane that writes the descriptor's base word directly before the
load, which then read a stale base address.)  It also checks that the
key-step loops run without scratch spills (the 384-row kernel may spill a few
per-item values outside them) and that no packed fp32 VALU instruction was
generated.
"""
import os
import re
import subprocess

import pytest

from conftest import load_builder

pabuild = load_builder()

pytestmark = pytest.mark.skipif(not os.path.exists(pabuild.HIPCC), reason="hipcc not installed")


@pytest.fixture(scope="module")
def attention_asm(tmp_path_factory):
    """The assembly of every source with LDS-filling loads."""
    text = []
    for src in ("pa_attention.hip", "pa_peak.hip"):
        out = tmp_path_factory.mktemp("asm") / src.replace(".hip", ".s")
        flags = [f for f in pabuild.FLAGS if f not in ("-fPIC",)]
        cmd = [pabuild.HIPCC, *flags, "--cuda-device-only", "-S",
               os.path.join(pabuild.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        text.append(out.read_text())
    return "\n".join(text)


def _functions(asm):
    """{kernel symbol: [instruction lines]} for every kernel body."""
    funcs = {}
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        body = asm[m.end():end].split("\n")
        funcs[name] = [l.strip() for l in body if l.strip() and not l.strip().startswith(";")]
    return funcs


def _sgprs(op):
    m = re.match(r"s\[(\d+):(\d+)\]$", op)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", op)
    return {int(m.group(1))} if m else set()


def _wait_states(line):
    op = line.split()[0]
    return int(line.split()[1], 0) + 1 if op == "s_nop" else 1


def test_lds_dma_hazards_padded(attention_asm):
    funcs = _functions(attention_asm)
    checked = 0
    for name, lines in funcs.items():
        for k, line in enumerate(lines):
            if not (line.startswith("buffer_load") and " lds" in line):
                continue
            checked += 1
            prev = lines[k - 1].split()
            assert prev[0] == "s_nop" and int(prev[1], 0) >= 4, f"{name}: unpadded LDS load: {line}"
            rsrc = _sgprs(line.split(None, 1)[1].split(",")[1].strip())
            assert rsrc, line
            dist, m0_done, sgpr_done = 0, False, False
            for prev in reversed(lines[max(0, k - 64):k]):
                if prev.endswith(":"):
                    break  # block boundary: only straight-line predecessors are checked
                parts = prev.split(None, 1)
                dst = parts[1].split(",")[0].strip() if len(parts) > 1 else ""
                if not m0_done and dst == "m0":
                    assert dist >= 1, f"{name}: M0 write too close to LDS load: {prev} -> {line}"
                    m0_done = True
                if not sgpr_done and parts[0].startswith("v_") and _sgprs(dst) & rsrc:
                    assert dist >= 5, f"{name}: VALU SGPR write too close to LDS load: {prev} -> {line}"
                    sgpr_done = True
                if m0_done and sgpr_done:
                    break
                dist += _wait_states(prev)
    assert checked > 0, "no LDS-filling buffer loads found"


def _loop_depths(asm, name):
    """[(depth, instruction)] of a kernel, depth from the compiler's loop comments."""
    i = asm.index(name + ":")
    body = asm[i:asm.find(".Lfunc_end", i)].split("\n")
    out, depth = [], 0
    for raw in body:
        t = raw.strip()
        if t.startswith(".LBB") or t.startswith("; %bb"):
            m = re.search(r"Depth=(\d+)", t)
            depth = int(m.group(1)) if m else 0
            continue
        if t and not t.startswith(";"):
            out.append((depth, t))
    return out


def test_no_scratch_in_loops_and_no_packed_fp32(attention_asm):
    """Spills are tolerated only outside loops and in per-item code: the
    384-row kernel's loop over a work-group's items (depth 1), and the
    one-launch step kernel's task loop and the items within a task (depths 1
    and 2); the key-step loops, where the time goes, must run from registers
    (the step kernel's inner loops are the same item code, checked in the
    standalone kernels).  One exception, bounded: the one-launch step with
    quantised KV holds its claim state beside a prefill that alone fills the
    register file, and may reload one value per key step."""
    for name in _functions(attention_asm):
        item_depth = 1 if "prefill_w48_kernel" in name else 2 if "step_kernel" in name else 0
        allowed = 1 if re.search(r"step_kernelILi\d+ELi[12]E", name) else 0
        in_loops = 0
        for depth, line in _loop_depths(attention_asm, name):
            op = line.split()[0]
            if op.startswith("scratch_") and depth > item_depth:
                in_loops += 1
                assert op.startswith("scratch_load_dword") and in_loops <= allowed, f"{name} spills in a loop: {line}"
            assert op not in ("v_pk_add_f32", "v_pk_mul_f32", "v_pk_fma_f32"), f"{name}: {line}"
