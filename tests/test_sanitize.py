"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

* The CPU oracle (oracle/kda_oracle.c) with a driver that runs every one of
  its entry points on small seeded inputs, edge sizes included
  (tests/sanitize/oracle_driver.c), built by gcc with
  -fsanitize=address,undefined and leak detection on.
* libkda's C-ABI layer (kda_api.hip) with its host side built the same way
  (-Xarch_host before each -fsanitize, so the GPU code is built as usual),
  linked with the library's other objects and a driver that calls every
  entry point with arguments the host validation must reject
  (tests/sanitize/abi_driver.cpp): all of it runs before any HIP call.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, env=None, **kw):
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, **kw)
    assert p.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), p.stdout[-4000:], p.stderr[-4000:])
    return p


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-g", "-O1", "-fopenmp"] + SAN + ["-I", os.path.join(ROOT, "oracle"),
         os.path.join(ROOT, "oracle", "kda_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", OMP_NUM_THREADS="2")
    p = _run([exe], env=env)
    assert "0 failure(s)" in p.stdout


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("g++") is None,
                    reason="needs hipcc and g++")
def test_abi_validation_under_sanitizers(tmp_path):
    from gated_delta_rule_kda_amd import build as kbuild
    objs = [o for o in glob.glob(os.path.join(kbuild.PKG, "_build", "*.o")) if "kda_api" not in o]
    if len(objs) < len(kbuild.sources()) - 1:
        kbuild.build()
        objs = [o for o in glob.glob(os.path.join(kbuild.PKG, "_build", "*.o")) if "kda_api" not in o]
    api = str(tmp_path / "kda_api_san.o")
    _run([kbuild.hipcc(), "-O1", "-g", "-std=c++17", "--offload-arch=" + kbuild.ARCH, "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-I", kbuild.INCLUDE, "-I", kbuild.CSRC, "-c", os.path.join(kbuild.CSRC, "kda_api.hip"), "-o", api])
    drv = str(tmp_path / "abi_driver.o")
    _run(["g++", "-g", "-std=c++17"] + SAN + ["-I", kbuild.INCLUDE, "-c", os.path.join(HERE, "abi_driver.cpp"),
                                              "-o", drv])
    exe = str(tmp_path / "abi_driver")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    _run(["g++"] + SAN + [drv, api] + objs + ["-L", os.path.join(rocm, "lib"), "-lamdhip64",
                                             "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1")
    p = _run([exe], env=env)
    assert "0 failure(s)" in p.stdout
