"""AddressSanitizer, LeakSanitizer and UndefinedBehaviorSanitizer runs of
the host code (CPU only): the C oracle through every entry point; the
library's planner and argument validation (fwt_api.cpp, with its kernel
entry points stubbed) through 20 000 random plans, every query and every
early-return error path; and fwt_execute's launch schedule against a fake
HIP runtime, checked tile by tile.  A sanitizer report makes the driver
exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(cmd, cwd, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.fixture
def workdir(tmp_path):
    return str(tmp_path)


def test_oracle_under_sanitizers(workdir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = os.path.join(workdir, "oracle_driver")
    rc, out = _run(["gcc"] + SAN + ["-ffp-contract=off", "-std=c99", "-D_POSIX_C_SOURCE=200809L",
                                    os.path.join(HERE, "oracle_driver.c"),
                                    os.path.join(ROOT, "oracle", "oracle.c"),
                                    "-o", exe, "-lm", "-lpthread"], workdir)
    assert rc == 0, out
    rc, out = _run([exe], workdir)
    assert rc == 0 and "oracle driver: ok" in out, out


def test_planner_under_sanitizers(workdir):
    if shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib",
                                                                       "libamdhip64.so")):
        pytest.skip("g++ or the HIP runtime library not found")
    exe = os.path.join(workdir, "planner_driver")
    rc, out = _run(["g++"] + SAN + ["-std=c++17", "-D__HIP_PLATFORM_AMD__",
                                    "-I", os.path.join(ROOT, "include"),
                                    "-I", os.path.join(ROCM, "include"),
                                    os.path.join(HERE, "planner_driver.cpp"),
                                    os.path.join(HERE, "kernel_stubs.cpp"),
                                    os.path.join(ROOT, "quantum_state_encoding_amd", "csrc",
                                                 "fwt_api.cpp"),
                                    "-o", exe, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                                    "-Wl,-rpath," + os.path.join(ROCM, "lib")], workdir)
    assert rc == 0, out
    rc, out = _run([exe], workdir)
    assert rc == 0 and "planner driver:" in out and " ok" in out, out


def test_launch_schedule_covers_every_tile_once(workdir):
    """fwt_execute with the kernels stubbed and a fake one-device HIP runtime
    (no GPU, no HIP library): for default plans and 3- and 4-factor splits
    of every n, at small, ragged and larger-than-cache batches, with and
    without im, each pass's launches cover every tile of the state exactly
    once, chunked passes stay inside their chunks, launches come in the
    order fwt_plan_call_schedule states, the scale and nontemporal flags
    sit on the right passes, and the XCD-affine workgroup placement of
    states below the Infinity Cache's size permutes each launch's
    workgroups so that every vector component stays on one XCD
    (tests/sanitize/schedule_driver.cpp)."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = os.path.join(workdir, "schedule_driver")
    rc, out = _run(["g++"] + SAN + ["-std=c++17", "-D__HIP_PLATFORM_AMD__",
                                    "-I", os.path.join(ROOT, "include"),
                                    "-I", os.path.join(ROCM, "include"),
                                    os.path.join(HERE, "schedule_driver.cpp"),
                                    os.path.join(HERE, "kernel_stubs.cpp"),
                                    os.path.join(ROOT, "quantum_state_encoding_amd", "csrc",
                                                 "fwt_api.cpp"),
                                    "-o", exe], workdir)
    assert rc == 0, out
    rc, out = _run([exe], workdir, timeout=900)
    assert rc == 0 and "schedule driver:" in out and " ok" in out, out
