"""AddressSanitizer / UndefinedBehaviorSanitizer builds of the host-side code,
run on the CPU:

* the fp64 C oracle (oracle/kda_oracle.c) and the seeded input generator
  (synth/synth.c), built with gcc and driven by tests/sanitize/san_c.c over
  every generator kind and output type and every oracle option;
* the library's host layer (gated_delta_rule_84_amd/csrc/kda_api.cpp), built
  with hipcc with the sanitizers on its host compilation only and driven by
  tests/sanitize/san_plan.cpp, which includes it to call the planning steps
  (descriptor validation, pipelined_segments, layout_for, make_plan,
  plan_launches) over a sweep of shapes and the C ABI's queries and argument
  checks, none of which needs a GPU.

A sanitizer finding makes the driver exit non-zero; its report is shown."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-8000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_and_generator_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "san_c")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(SAN, "san_c.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"),
          os.path.join(ROOT, "synth", "synth.c"), "-o", exe, "-lm"])
    assert "san_c: ok" in _run([exe], env=ENV).stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_host_planning_under_asan_ubsan(tmp_path):
    from gated_delta_rule_84_amd import _build

    objs = [os.path.join(_build.BUILD, s.rsplit(".", 1)[0] + ".o") for s in _build.SOURCES if s != "kda_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        _build.build()
    obj = str(tmp_path / "san_plan.o")
    exe = str(tmp_path / "san_plan")
    # sanitizers on the host compilation only (each flag right after -Xarch_host)
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    _run([HIPCC, "-x", "hip", "-std=c++17", "-O1", "-g", f"--offload-arch={_build.ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-I", os.path.join(ROOT, "include"), "-I", _build.CSRC, "-c", os.path.join(SAN, "san_plan.cpp"), "-o", obj])
    _run([HIPCC, f"--offload-arch={_build.ARCH}", *host_san, obj, *objs, "-o", exe])
    # the HIP runtime's own allocations at exit are not this code's: no leak check here
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")
    assert "san_plan: ok" in _run([exe], env=env).stdout
