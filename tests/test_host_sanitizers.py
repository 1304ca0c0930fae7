"""Host code under the sanitizers (CPU only).

Four programs under ``tests/host/`` are built with g++/gcc and run:

* ``lookback_model.cpp`` (ThreadSanitizer): a thread-per-workgroup model of
  the segment look-back protocol (tickets, release/acquire flags, the
  fixed-shape walk over aggregates and inclusive states).  Checks that start
  states are bit-identical to a single-threaded walk and match the plain
  sequential chain; TSan reports any slot access the flags do not order.
* ``dual_segments_model.cpp`` (ThreadSanitizer): a thread-per-workgroup
  model of the segmented dual form's protocol (grouped tickets, started and
  published flag bits, segment 0's end state, the claim of the last segment
  by segment 0 or, failing that, segment n-2).  Checks every start state and
  the final state against a sequential chain bit for bit, that exactly one
  workgroup runs each last segment, and forces each claim path in turn.
* ``abi_driver.cpp`` (AddressSanitizer + UndefinedBehaviorSanitizer): the
  C-ABI's validation (``csrc/api.cpp``) with stubbed launchers, called with
  valid and invalid arguments, extreme sizes and strides.
* ``oracle_driver.c`` (AddressSanitizer + UndefinedBehaviorSanitizer): every
  routine of the C oracle on small edge-case inputs, with exact identities.

Every sanitizer report aborts the program (``-fno-sanitize-recover``), so a
non-zero exit fails the test.  None of this touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
ROCM = "/opt/rocm"


def build_and_run(tmp_path, cmd, exe):
    r = subprocess.run(cmd + ["-o", str(exe)], capture_output=True, text=True, cwd=tmp_path)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1", ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_lookback_protocol_under_tsan(tmp_path):
    out = build_and_run(tmp_path, ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
                                   os.path.join(HOST, "lookback_model.cpp")], tmp_path / "lookback_model")
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_dual_segment_protocol_under_tsan(tmp_path):
    out = build_and_run(tmp_path, ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread",
                                   os.path.join(HOST, "dual_segments_model.cpp")], tmp_path / "dual_segments_model")
    assert "0 failures" in out
    late = int(out.split("segment n-2 in ")[1].split(" late")[0])
    early = int(out.split(" late, ")[1].split(" early")[0])
    assert late > 0 and early == 0, "late runs take the second claim path, early runs the first"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_abi_validation_under_asan_ubsan(tmp_path):
    out = build_and_run(tmp_path, ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                                   "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
                                   os.path.join(HOST, "abi_driver.cpp"),
                                   os.path.join(ROOT, "linear_attention_chunked_amd", "csrc", "api.cpp"),
                                   f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"],
                        tmp_path / "abi_driver")
    assert "0 bad statuses" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    out = build_and_run(tmp_path, ["gcc", "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
                                   "-fno-sanitize-recover=all", "-ffp-contract=off",
                                   os.path.join(HOST, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ttt_oracle.c"),
                                   "-lm"], tmp_path / "oracle_driver")
    assert "0 failures" in out
