"""Build-level checks of the two-block prefill kernel (no GPU needed).

The kernel keeps its tile state (O^T and Q^T in AGPRs 64..255, scores and
operand ring in VGPRs 64..255) in registers the compiler may not allocate,
touched only by the generated inline-assembly blocks. That contract cannot be
seen by the compiler, so it is checked on the emitted gfx950 assembly: outside
the blocks no instruction names a register at or above 64, nothing spills to
scratch, and the kernel descriptor allocates the whole register file. The
generated header must also be what the generator writes today.
"""

import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_segmented_paged_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def test_generated_blocks_are_current():
    res = subprocess.run([sys.executable, os.path.join(CSRC, "gen_tile_asm.py"), "--check"],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "segkv_attn.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
           os.path.join(CSRC, "segkv_attn.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def _kernels(isa_text, name):
    """(symbol, body text up to its descriptor end) of every instantiation."""
    syms = sorted(set(re.findall(rf"^(_Z\S*{name}\S*):", isa_text, re.M)))
    out = []
    for sym in syms:
        start = isa_text.index(f"\n{sym}:")
        end = isa_text.index(".end_amdhsa_kernel", start)
        out.append((sym, isa_text[start:end]))
    return out


def test_two_block_kernel_register_discipline(isa):
    kernels = _kernels(isa, "attn_prefill_w2_kernel")
    assert len(kernels) == 8   # heads per unit {1, 2, 4, 8} x {fp32, bf16} output
    for sym, body in kernels:
        assert "scratch_" not in body, f"{sym} spills to scratch"
        assert re.search(r"\.amdhsa_next_free_vgpr 512\b", body), sym
        assert re.search(r"\.amdhsa_accum_offset 256\b", body), sym
        outside = re.sub(r";;#ASMSTART.*?;;#ASMEND", "", body, flags=re.S)
        code = [ln for ln in outside.splitlines() if ln.startswith("\t") and not ln.lstrip().startswith((";", "."))]
        bad = []
        for ln in code:
            for kind, a, b in re.findall(r"\b([va])(?:\[(\d+):\d+\]|(\d+))\b", ln):
                idx = int(a or b)
                if idx >= 64:
                    bad.append(ln.strip())
                    break
        assert not bad, f"{sym}: compiler code touches the blocks' registers: {bad[:5]}"
