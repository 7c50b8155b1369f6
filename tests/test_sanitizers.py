"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU.

* The fp64 C oracle built with gcc -fsanitize=address,undefined runs its pins (closed forms,
  hand-worked golden values, mutants, segment maps) in a child process with gcc's sanitizer
  runtimes preloaded.
* The host code of libkda.so (argument checks, workspace sizing, window planning, the C ABI)
  built with clang's sanitizers on the host side only (device code is compiled as usual and
  never runs here) runs the ABI contract tests in a child process with clang's runtime preloaded.

Any sanitizer report ends the child with a non-zero status (-fno-sanitize-recover=all), which
fails the test; the report is shown in the failure message.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_93_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run_child(code, preload, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", LD_PRELOAD=preload, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    assert r.returncode == 0, f"status {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r.stdout


def test_oracle_pins_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    lib = str(tmp_path / "libkda_oracle_san.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                           *SAN, os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", lib, "-lm"])
    rt = [subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
          for n in ("libasan.so", "libubsan.so")]
    code = f"""
import sys, oracle, pytest
oracle._LIB = {lib!r}; oracle._lib = None
rc = pytest.main(['-q', '-s', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py',
                  'tests/test_oracle_mutants.py', 'tests/test_oracle_kcp.py'])
assert oracle._load()._name == {lib!r}, 'the sanitized oracle was not the one loaded'
sys.exit(rc)
"""
    out = _run_child(code, ":".join(rt))
    assert " passed" in out and "failed" not in out


def test_library_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang's ASan runtime not found")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]  # host side only; device code as usual
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    procs, objs = [], []
    for s in srcs:
        o = str(tmp_path / s.replace(".hip", ".o"))
        objs.append(o)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *host_san,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             f"-I{os.path.join(ROOT, 'include')}", "-c", os.path.join(CSRC, s), "-o", o],
            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for s, p in zip(srcs, procs):
        _, err = p.communicate(timeout=600)
        assert p.returncode == 0, f"{s}: {err[-3000:]}"
    lib = str(tmp_path / "libkda_san.so")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", *objs, "-o", lib])
    code = f"""
import sys, pytest
import gated_delta_rule_93_amd as kda
kda.LIB_PATH = {lib!r}
rc = pytest.main(['-q', '-s', '-p', 'no:cacheprovider', 'tests/test_abi.py'])
assert kda.lib()._name == {lib!r}, 'the sanitized library was not the one loaded'
sys.exit(rc)
"""
    out = _run_child(code, rts[0])
    assert " passed" in out and "failed" not in out
