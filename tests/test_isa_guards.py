"""Guards on the compiled staged kernels (no GPU).

The chunk kernels issue their global->LDS copies from inline assembly (so
that the compiler adds no waits of its own for them).  Two things the
compiler would otherwise guarantee are checked here on the gfx950 assembly the
build flags produce:

* M0 belongs to the inline assembly: the compiler must not use it anywhere
  else in these kernels (the asm statements clobber it).
* A VALU write of an SGPR must be at least 5 wait states before a vector
  memory instruction that reads it (a GFX9 hazard the compiler does not check
  inside inline assembly).
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_03_amd", "csrc")
sys.path.insert(0, ROOT)

SOURCES = ["scan.hip", "prep.hip", "kda_chunk.hip"]


def _assembly(src, tmp_path):
    from gated_delta_rule_03_amd import build as gbuild
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    flags = [f for f in gbuild.HIPCC_FLAGS if f not in ("-fPIC",)]
    out = tmp_path / (src + ".s")
    subprocess.run([hipcc, *flags, "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", str(out)],
                   check=True, capture_output=True, cwd=CSRC)
    return out.read_text()


def _sregs(tok):
    m = re.match(r"s\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"s(\d+)$", tok)
    return {int(m.group(1))} if m else set()


@pytest.mark.parametrize("src", SOURCES)
def test_m0_only_in_inline_asm(src, tmp_path):
    text = _assembly(src, tmp_path)
    in_asm = False
    bad = []
    for line in text.split("\n"):
        t = line.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if in_asm or not t or t.startswith((";", ".")):
            continue
        if re.search(r"\bm0\b", t):
            bad.append(t)
    assert not bad, f"compiler-generated M0 uses in {src}: {bad[:5]}"


@pytest.mark.parametrize("src", SOURCES)
def test_no_valu_sgpr_write_before_asm_vmem(src, tmp_path):
    text = _assembly(src, tmp_path)
    kernels = re.findall(r"^(_Z\S+):", text, re.M)
    checked = 0
    bad = []
    for name in kernels:
        i = text.index(name + ":")
        j = text.index(".Lfunc_end", i)
        ins = [l.strip() for l in text[i:j].split("\n")]
        ins = [l for l in ins if l and not l.startswith((".", ";")) and not l.endswith(":")]
        for n, l in enumerate(ins):
            op = l.split()[0]
            if not (op.startswith("global_load_lds") or (op.startswith("buffer_load") and l.endswith("lds"))):
                continue
            checked += 1
            used = set()
            for tok in l.split(None, 1)[1].split(",")[1:]:
                used |= _sregs(tok.strip().split()[0])
            waits, k = 0, n - 1
            while k >= 0 and waits < 5:
                p = ins[k]
                pop = p.split()[0]
                if pop.startswith("v_") and _sregs(p.split(None, 1)[1].split(",")[0].strip()) & used:
                    bad.append((name, p, l))
                    break
                waits += int(p.split()[1], 0) + 1 if pop == "s_nop" else 1
                k -= 1
    assert checked > 0, f"no LDS-bound copies found in {src}"
    assert not bad, f"VALU-written SGPR read by a copy within 5 wait states: {bad[:3]}"
