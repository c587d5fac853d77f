"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two small drivers are built in a temporary directory and run as child processes:
  - tests/sanitize/oracle_driver.cpp: every C entry point of the CPU oracle (g++);
  - tests/sanitize/tuning_driver.cpp: the library's tuning-file parser, igc_tuning.cpp, compiled
    for the host only by hipcc with the sanitizers on the host side (clang's runtimes).
Any sanitizer finding aborts the driver (-fno-sanitize-recover=all), so the test passes only when
both exit 0 and print their "ok" line.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\nexit {r.returncode}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    return r


def _env(tmp):
    env = dict(os.environ)
    env["SAN_TMP"] = str(tmp)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("LD_PRELOAD", None)
    return env


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["g++", "-std=c++17", "-fopenmp", *SAN_FLAGS, os.path.join(SAN, "oracle_driver.cpp"), "-o", exe])
    r = _run([exe], env={**_env(tmp_path), "OMP_NUM_THREADS": "4"})
    assert "oracle driver: ok" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="hipcc / clang++ not available")
def test_tuning_parser_under_asan_ubsan(tmp_path):
    inc = ["-I", os.path.join(ROOT, "sparse_convolution_amd", "csrc"), "-I", os.path.join(ROOT, "include")]
    objs = []
    for src in (os.path.join(ROOT, "sparse_convolution_amd", "csrc", "igc_tuning.cpp"),
                os.path.join(SAN, "tuning_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        host_san = [x for f in SAN_FLAGS for x in (["-Xarch_host", f] if f.startswith("-fsanitize") or
                                                     f.startswith("-fno-sanitize") else [f])]
        _run([HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", *host_san, *inc, "-c", src, "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "tuning_driver")
    _run([CLANG, *SAN_FLAGS, *objs, "-o", exe, "-lpthread"])
    r = _run([exe], env=_env(tmp_path))
    assert "tuning driver: ok" in r.stdout
