"""AddressSanitizer runs of the host code, on the CPU.

* The oracle (oracle/oracle.c), built by gcc with AddressSanitizer and
  UndefinedBehaviorSanitizer (no recovery: the first report aborts), runs
  every oracle pin (tests/test_oracle_pins.py) in a child process with the
  ASan runtime preloaded.
* The library's host code (sa_api.hip: argument checks, the plan and
  workspace layout, the far-list checker) built with AddressSanitizer on
  its host pass only and linked with the other objects of the regular
  build, runs the ABI, binding and far-list checker tests in a child
  process the same way.  No GPU is involved: every call there returns
  before a launch.

A report makes the child exit non-zero and print "AddressSanitizer" or
"runtime error"; both fail the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

RT_DIRS = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux"))


def gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def run_child(args, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["PYTHONDONTWRITEBYTECODE"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    return r.returncode, out


def test_oracle_under_asan_and_ubsan(tmp_path):
    asan = gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = str(tmp_path / "liboracle_asan.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]   # gcc, host code
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", *san, "-fPIC", "-shared",
                           "-Wno-unknown-pragmas", "-fno-fast-math", "-o", lib,
                           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    rc, out = run_child(["tests/test_oracle_pins.py"],
                        {"LD_PRELOAD": asan, "SA_ORACLE_LIB": lib}, timeout=600)
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert rc == 0, out[-4000:]
    assert " passed" in out


def test_library_host_code_under_asan(tmp_path):
    from sliding_window_long_amd import build as B
    rt = [d for d in RT_DIRS if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so"))]
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
            if s != "sa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build_library()
    api_obj = str(tmp_path / "sa_api_asan.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    r = subprocess.run([B.HIPCC, *B.FLAGS, *host_asan, "-c", os.path.join(B.CSRC, "sa_api.hip"),
                        "-o", api_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libsparse_attn_asan.so")
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_obj, *objs,
                        "-L" + rt[0], "-lclang_rt.asan-x86_64", "-Wl,-rpath," + rt[0]],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    rc, out = run_child(["tests/test_abi.py", "tests/test_binding_checks.py",
                         "tests/test_far_list_checker.py"],
                        {"LD_PRELOAD": os.path.join(rt[0], "libclang_rt.asan-x86_64.so"),
                         "SPARSE_ATTN_LIB": lib}, timeout=600)
    assert "AddressSanitizer" not in out, out[-4000:]
    assert rc == 0, out[-4000:]
    assert " passed" in out


# The runs above must be able to fail: the same harness on copies with one
# planted out-of-bounds read each must report it.
def test_oracle_harness_catches_planted_overflow(tmp_path):
    asan = gcc_runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "for (int64_t j = c * B; j < (c + 1) * B; ++j)"
    assert src.count(good) >= 1   # the first one is the mean pooling's key loop
    bad_src = tmp_path / "oracle_bad.c"
    bad_src.write_text(src.replace(good, "for (int64_t j = c * B; j <= (c + 1) * B; ++j)", 1))
    lib = str(tmp_path / "liboracle_bad.so")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]   # gcc, host code
    subprocess.check_call(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", *san, "-fPIC", "-shared",
                           "-Wno-unknown-pragmas", "-fno-fast-math", "-o", lib, str(bad_src), "-lm"])
    rc, out = run_child(["tests/test_oracle_pins.py", "-k", "pool"],
                        {"LD_PRELOAD": asan, "SA_ORACLE_LIB": lib}, timeout=600)
    assert rc != 0 and "AddressSanitizer" in out, out[-3000:]


def test_library_harness_catches_planted_overflow(tmp_path):
    from sliding_window_long_amd import build as B
    rt = [d for d in RT_DIRS if os.path.exists(os.path.join(d, "libclang_rt.asan-x86_64.so"))]
    if not rt:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    objs = [os.path.join(B.BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in B.SOURCES
            if s != "sa_api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build_library()
    src = open(os.path.join(B.CSRC, "sa_api.hip")).read()
    good = "    const long long total = off[lists];\n"
    assert src.count(good) >= 1   # the first one is the checker's
    bad_src = tmp_path / "sa_api_bad.hip"
    bad_src.write_text(src.replace(good, "    const long long total = off[lists] + (off[lists + 1] == 12345);\n", 1))
    api_obj = str(tmp_path / "sa_api_bad.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    r = subprocess.run([B.HIPCC, *B.FLAGS, *host_asan, "-c", str(bad_src), "-o", api_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libsparse_attn_bad.so")
    r = subprocess.run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib, api_obj, *objs,
                        "-L" + rt[0], "-lclang_rt.asan-x86_64", "-Wl,-rpath," + rt[0]],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    rc, out = run_child(["tests/test_far_list_checker.py"],
                        {"LD_PRELOAD": os.path.join(rt[0], "libclang_rt.asan-x86_64.so"),
                         "SPARSE_ATTN_LIB": lib}, timeout=600)
    assert rc != 0 and "AddressSanitizer" in out, out[-3000:]
