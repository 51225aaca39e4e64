"""Host sanitizer runs (CPU only, no kernel is launched).

* The C oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer:
  tests/sanitize/oracle_main.c runs it on batched and packed cases (empty and
  one-token sequences, several threads, absent S0) with exact-size heap buffers.
* The C ABI under AddressSanitizer on its host code: the library sources are
  compiled with hipcc, the host half instrumented (-Xarch_host) and the gfx950
  code as usual, and tests/sanitize/abi_main.cpp calls every entry point with
  rejected arguments of every kind and sweeps the workspace queries; on a host
  without a GPU it also passes valid arguments, which must stop at the device
  check.

A sanitizer report ends the driver with a non-zero status, which fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
CSRC = ROOT / "kda_gated_delta_chunk_amd" / "csrc"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/lib/llvm/bin/clang++"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s" % (" ".join(map(str, cmd)), r.stdout[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_asan"
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-std=c11", "-pthread", str(ROOT / "tests" / "sanitize" / "oracle_main.c"), str(ROOT / "oracle" / "kda_oracle.c"),
          "-o", str(exe), "-lm"])
    out = _run([str(exe)])
    assert "all checks passed" in out


@pytest.mark.timeout(900)
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="needs hipcc and ROCm clang++")
def test_abi_validation_under_address_sanitizer(tmp_path):
    sources = ["kda_api.hip", "kda_prefill.hip", "kda_decode.hip", "kda_backward.hip"]
    flags = ["-O2", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Wno-unused-command-line-argument",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = [tmp_path / (s.rsplit(".", 1)[0] + ".o") for s in sources]
    cmds = [[HIPCC, *flags, "-c", str(CSRC / s), "-o", str(o)] for s, o in zip(sources, objs)]
    main_o = tmp_path / "abi_main.o"
    cmds.append([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer",
                 "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", str(ROOT / "tests" / "sanitize" / "abi_main.cpp"),
                 "-o", str(main_o)])
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(_run, cmds))
    exe = tmp_path / "abi_asan"
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", str(main_o), *map(str, objs), "-o",
          str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")  # the HIP runtime keeps its allocations
    out = _run([str(exe)], env=env)
    assert "all checks passed" in out
