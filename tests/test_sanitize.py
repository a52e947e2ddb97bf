"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code
(no GPU needed): the library's argument checks and launch planning
(fa_api.cpp, fa_launch.cpp, driven by tests/sanitize/boundary_main.cpp with
the device launches stubbed out), and the CPU oracle (oracle.c) under a run
of its forward and backward pins."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_forward_05_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _clean_run(cmd, env=None):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "boundary_asan"
    cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "sanitize", "boundary_main.cpp"),
           os.path.join(CSRC, "fa_api.cpp"), os.path.join(CSRC, "fa_launch.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    out = _clean_run([str(exe)], env)
    assert "OK (0 failures)" in out


PINS = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
oracle.use_library({lib!r})
import test_oracle as f, test_oracle_bwd as b
f.test_single_key_gives_v0(True); f.test_causal_row0_and_last_row(); f.test_bottom_right_offset()
f.test_no_visible_key_rows(); f.test_merge_of_partials_equals_one_shot(True)
f.test_merge_identity_commutes_and_associates(); f.test_gqa_contiguous_grouping()
f.test_rows_equal_full(); f.test_against_softmax_definition(True)
b.test_finite_differences(True, 5, 11, 4, 2); b.test_golden_worked_example(); b.test_single_key(True)
b.test_no_visible_key_rows(); b.test_rows_equal_full()
print("PINS OK")
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    so = tmp_path / "liboracle_asan.so"
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", *SAN,
                    "-o", str(so), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], check=True)
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0",
               OMP_NUM_THREADS="4")
    script = PINS.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(so))
    out = _clean_run([sys.executable, "-c", script], env)
    assert "PINS OK" in out
