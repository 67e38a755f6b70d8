"""Host-side sanitizer runs (CPU only, no GPU needed).

* The oracle's C (bg_oracle.c) built with gcc's AddressSanitizer and
  UndefinedBehaviorSanitizer, driven by the oracle's own pin tests.
* The C-ABI's host code (argument validation, dispatch rules, workspace
  sizing, error strings) built with hipcc's host-side AddressSanitizer -- the
  device code is compiled as usual -- driven by the C-ABI CPU tests.

Each run is a child pytest process that preloads the sanitizer runtime and
loads the instrumented library in place of the normal one; any sanitizer
report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _child(env_extra, args, preload):
    env = dict(os.environ)
    env.update(env_extra)
    env["LD_PRELOAD"] = preload
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert not any(s in out for s in REPORTS), out[-4000:]
    assert " passed" in out
    return out


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc_asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(gcc_asan):
        pytest.skip("gcc has no libasan")
    lib = str(tmp_path / "liboracle_asan.so")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                           "-shared", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "bg_oracle.c"), "-o", lib,
                           "-lm"])
    tests = sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py")))
    tests.append(os.path.join(ROOT, "tests", "test_golden_pages.py"))
    # the exhaustive E4M3 sweep adds half a minute and no new code paths
    out = _child({"BG_ORACLE_LIB": lib}, [*tests, os.path.abspath(__file__) + "::test_child_loaded", "-k",
                                         "not exhaustive"], gcc_asan)
    assert "skipped" not in out


def test_capi_host_code_under_asan(tmp_path):
    sys.path.insert(0, ROOT)
    from bit_gemm_w4_amd import build as B
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt or not os.path.exists(B.HIPCC):
        pytest.skip("no hipcc / clang ASan runtime")
    os.makedirs(B.OBJDIR, exist_ok=True)
    headers = glob.glob(os.path.join(B.CSRC, "*.h"))
    newest_header = max(os.path.getmtime(h) for h in headers)
    objs = []
    for src in B.sources():
        if os.path.basename(src) == "capi.hip":
            continue
        obj = os.path.join(B.OBJDIR, os.path.basename(src) + ".o")
        if not os.path.exists(obj) or os.path.getmtime(obj) < max(os.path.getmtime(src), newest_header):
            obj = B._compile(src)
        objs.append(obj)
    capi_obj = str(tmp_path / "capi_asan.o")
    # host-side instrumentation only: each sanitizer flag is scoped to the host pass
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.check_call([B.HIPCC, *B.FLAGS, "-g", *host_asan, "-c", os.path.join(B.CSRC, "capi.hip"), "-o", capi_obj],
                          stderr=subprocess.DEVNULL)
    lib = str(tmp_path / "libbitgemm_asan.so")
    subprocess.check_call([B.HIPCC, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-fsanitize=address",
                           "-shared-libasan", capi_obj, *objs, "-o", lib])
    out = _child({"BG_LIB_PATH": lib}, [os.path.join(ROOT, "tests", "test_capi_cpu.py"),
                                        os.path.join(ROOT, "tests", "test_sanitizers_cpu.py") + "::test_child_loaded"],
                 rt[-1])
    assert "skipped" not in out


def test_child_loaded():
    """Inside an instrumented child: the library under test and the sanitizer
    runtime are the ones mapped."""
    if os.environ.get("BG_LIB_PATH"):
        from bit_gemm_w4_amd import ops
        ops.lib()
        lib = os.environ["BG_LIB_PATH"]
    elif os.environ.get("BG_ORACLE_LIB"):
        import oracle
        oracle._load()
        lib = os.environ["BG_ORACLE_LIB"]
    else:
        pytest.skip("runs inside the sanitizer children only")
    maps = open("/proc/self/maps").read()
    assert lib in maps and "asan" in maps
