"""Sanitizer build of the library's host code (no GPU): the table builder and
the C-ABI argument checks (segkv_tables.cpp, segkv_api.cpp, device launchers
replaced by host stubs) and the C oracle, compiled with the address and
undefined-behaviour sanitizers into one program that drives them with
randomised layers (tests/sanitize/fuzz_host.cpp). Any sanitizer report, or a
call returning other than the code expected of it, fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "head_segmented_paged_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stderr[-3000:]


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("needs gcc / g++")
    out = tmp_path_factory.mktemp("san")
    objs = []
    for src in (os.path.join(CSRC, "segkv_tables.cpp"), os.path.join(CSRC, "segkv_api.cpp"),
                os.path.join(HERE, "device_stubs.cpp"), os.path.join(HERE, "fuzz_host.cpp")):
        obj = str(out / (os.path.basename(src) + ".o"))
        _run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj])
        objs.append(obj)
    obj = str(out / "attn_fp64.o")
    _run(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "attn_fp64.c"), "-o", obj])
    objs.append(obj)
    exe = str(out / "fuzz_host")
    _run(["g++", *SAN, *objs, "-o", exe, "-lm"])
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_host_code_under_sanitizers(fuzz_bin, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([fuzz_bin, str(seed), "150"], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert "0 failures" in res.stdout, res.stdout
