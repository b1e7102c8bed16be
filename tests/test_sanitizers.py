"""AddressSanitizer / UndefinedBehaviorSanitizer runs of the host code (CPU).

The host C++ of the library (API validation, block pool and planner,
scheduler, prefix index, kernel-timing bookkeeping) and the C oracle are
rebuilt with g++/gcc -fsanitize=address,undefined -- host code only: the HIP
kernels are replaced by stub launchers that enqueue nothing, which the host
tests never reach -- and the host test files run against those builds in a
child process with the sanitizer runtimes preloaded.  Any report fails the
run (halt_on_error).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_paged_kv_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g",
       "-O1", "-fPIC"]

# Launchers that enqueue nothing: the host tests stop at argument
# validation, before any launch, so these only satisfy the linker.
STUBS = r"""
#include "zp_internal.h"
namespace zp {
hipError_t launch_score(const ScoreParams&, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_compact(const CompactParams&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode(const DecodeParams&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_append(const AppendParams&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_redundancy_all(const RedundancyParams&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_upload(const void*, void*, size_t, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_first_evict(const int32_t*, int32_t*, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t score_resident_per_cu(int, int, int, int, int, bool, int*) { return hipErrorInvalidValue; }
hipError_t decode_static_scratch(void**) { return hipErrorInvalidValue; }
}  // namespace zp
"""


def _runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


@pytest.fixture(scope="module")
def instrumented(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    stub = d / "stubs.cpp"
    stub.write_text(STUBS)
    host_lib = str(d / "libzp_host_san.so")
    srcs = [os.path.join(CSRC, f) for f in ("api.cpp", "block_pool.cpp", "sched.cpp",
                                             "prefix_index.cpp", "profile.cpp", "debug.cpp")] + [str(stub)]
    subprocess.run(["g++", "-std=c++17", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", f"-I{ROOT}/include", f"-I{CSRC}", "-o", host_lib, *srcs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-ldl", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    oracle_lib = str(d / "libzp_oracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-shared", *SAN, "-o", oracle_lib,
                    os.path.join(ROOT, "oracle", "zp_oracle.c"), "-lm"], check=True)
    return host_lib, oracle_lib


def test_host_code_and_oracle_are_clean_under_sanitizers(instrumented):
    host_lib, oracle_lib = instrumented
    env = dict(os.environ)
    env.update({
        "ZP_LIBRARY": host_lib,
        "ZP_ORACLE_LIBRARY": oracle_lib,
        # the sanitizer runtimes first, anything already preloaded kept after them
        "LD_PRELOAD": ":".join(x for x in (_runtime('libasan.so'), _runtime('libubsan.so'),
                                           os.environ.get("LD_PRELOAD", "")) if x),
        # the interpreter itself is not instrumented: no leak report for it
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_host_abi.py", "test_scheduler.py",
                                                      "test_prefix_index.py", "test_oracle_pins.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "not sanitizers", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out
