"""Host-side argument validation under AddressSanitizer (CPU only, no GPU).

api.hip is compiled for the host alone (hipcc --offload-host-only) with
AddressSanitizer, linked with tests/asan/stubs.hip (HIP pointer queries that
report device memory, launchers that only count calls) and driven by
tests/asan/driver.cpp through every entry point that checks overlaps:

* the library as built: every valid call passes validation and reaches its
  launcher, every overlapping output is MP_ERR_ALIAS, and ASan stays silent;
* built with overlap lists too short for the calls (8 ranges): every call
  returns MP_ERR_INTERNAL, no list is written past its end, no abort;
* a mutant of that build whose list no longer refuses a range beyond its
  capacity: ASan reports the stack-buffer-overflow, which shows that this test
  would catch the overflow class behind a past GPU memory fault (the ranges of
  a host-side check written past a fixed stack array).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "gnn_sparse_message_amd", "csrc", "api.hip")
STUBS = os.path.join(ROOT, "tests", "asan", "stubs.hip")
DRIVER = os.path.join(ROOT, "tests", "asan", "driver.cpp")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
INC = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gnn_sparse_message_amd", "csrc")]
# host code only: the sanitizer flag applies to the host pass (there is no device pass)
HOST = ["--offload-host-only", "-x", "hip", "-std=c++17", "-O1", "-g", "-Xarch_host",
        "-fsanitize=address"]
GUARD = """        if (k < kCap) r[k++] = x;
        else refused = true;"""

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)),
                                reason="needs hipcc and ROCm's clang++")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


@pytest.fixture(scope="module")
def objs(tmp_path_factory):
    d = tmp_path_factory.mktemp("asan")
    stubs, driver = str(d / "stubs.o"), str(d / "driver.o")
    _run([HIPCC, *HOST, *INC, "-c", STUBS, "-o", stubs])
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address", "-I",
          os.path.join(ROOT, "include"), "-c", DRIVER, "-o", driver])
    return d, stubs, driver


def _program(objs, api_src, cap, name):
    d, stubs, driver = objs
    api = str(d / f"{name}.o")
    defines = [] if cap is None else [f"-DMP_RANGE_LIST_CAP={cap}"]
    _run([HIPCC, *HOST, *defines, *INC, "-c", api_src, "-o", api])
    exe = str(d / name)
    _run([CLANG, "-fsanitize=address", api, stubs, driver, "-o", exe])
    return exe


def test_validation_clean_under_asan(objs):
    exe = _program(objs, API, None, "full")
    res = subprocess.run([exe], capture_output=True, text=True)
    assert "AddressSanitizer" not in res.stderr, res.stderr
    assert res.returncode == 0, res.stdout + res.stderr
    assert "full lists: 0 failures" in res.stdout


def test_short_range_lists_return_internal_error(objs):
    exe = _program(objs, API, 8, "small")
    res = subprocess.run([exe, "small"], capture_output=True, text=True)
    assert "AddressSanitizer" not in res.stderr, res.stderr
    assert res.returncode == 0, res.stdout + res.stderr
    assert "small lists: 0 failures, 0 launches" in res.stdout


def test_asan_catches_an_unguarded_range_list(objs, tmp_path):
    src = open(API).read()
    assert GUARD in src, "the capacity guard of RangeList::add changed; update this test"
    mutant = tmp_path / "api_mutant.hip"
    mutant.write_text(src.replace(GUARD, "        r[k++] = x;"))
    exe = _program(objs, str(mutant), 8, "mutant")
    res = subprocess.run([exe, "small"], capture_output=True, text=True)
    assert res.returncode != 0
    assert "stack-buffer-overflow" in res.stderr, res.stderr[-2000:]
