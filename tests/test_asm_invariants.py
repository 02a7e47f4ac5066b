"""Invariants of the generated gfx950 code that the compiler cannot check
for the kernels that issue MFMAs and global->LDS copies as inline asm.

The compiler does not know such a statement is an MFMA, so it inserts no
wait states for the matrix-core latency: an accumulator register moved or
read by a compiler-generated instruction between two of these MFMAs, or
before the kernel's own `s_nop 7` guard after the last one, could read a
value the MFMA has not yet written.  These tests compile gemm.hip to
assembly (no GPU needed) and require that, in every kernel using inline-asm
MFMAs, no accumulator move/read/write appears from the first MFMA to the
guard, and that no such kernel spills to scratch memory (a spill reload
written just before an inline-asm MFMA reads it would miss the wait states
the compiler does not know to insert; a K/V-append kernel that spilled after
a change to the quantisation routine produced wrong outputs on the GPU)."""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_kv_amd", "csrc")


def _build_module():
    spec = importlib.util.spec_from_file_location("fq_build", os.path.join(ROOT, "bit_weight_kv_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    b = _build_module()
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not shutil.which(cc) and not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [cc] + [f for f in b.FLAGS if f not in ("-shared",)] + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
        os.path.join(CSRC, "gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return out.read_text()


def _kernels(text):
    """name -> body of every kernel function in an assembly listing."""
    bodies = {}
    for m in re.finditer(r"^(_Z\S+):\s*;\s*@\1\s*$", text, re.M):
        name = m.group(1)
        end = text.find("s_endpgm", m.end())
        bodies[name] = text[m.end():end]
    return bodies


def test_inline_asm_mfma_kernels_keep_accumulators_in_place(gemm_asm):
    kernels = _kernels(gemm_asm)
    checked = []
    for name, body in kernels.items():
        lines = body.split("\n")
        # a kernel with inline-asm MFMAs: an MFMA between ASMSTART and ASMEND
        inside, asm_mfma = False, False
        for l in lines:
            if ";;#ASMSTART" in l:
                inside = True
            elif ";;#ASMEND" in l:
                inside = False
            elif inside and "v_mfma" in l:
                asm_mfma = True
                break
        if not asm_mfma:
            continue
        checked.append(name)
        first = min(i for i, l in enumerate(lines) if "v_mfma" in l)
        guards = [i for i, l in enumerate(lines) if re.match(r"\s*s_nop 7\s*$", l) and i > first]
        assert guards, f"{name}: no s_nop 7 guard after the MFMAs"
        region = lines[first:guards[0]]
        # zero initialisation of the accumulators (a constant write the
        # compiler may lay out after the loop in text order) is not traffic
        bad = [l.strip() for l in region if re.search(r"v_accvgpr_(read|write|mov)", l)
               and not re.search(r"v_accvgpr_write_b32 a\d+, 0\s*$", l)]
        assert not bad, f"{name}: accumulator traffic between inline-asm MFMAs: {bad[:4]}"
        assert "scratch_" not in body, f"{name}: spills to scratch"
    # the 4-bit prefill kernel (plain and with the fused K/V append) and every
    # decode instantiation are covered
    assert sum("gemm_w4_kernel" in n for n in checked) >= 2, checked
    assert sum("gemm_decode_w4_kernel" in n for n in checked) >= 4, checked
    assert sum("gemm_decode8_kernel" in n for n in checked) >= 4, checked
