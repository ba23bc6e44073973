"""Host-code sanitizer builds (no GPU needed):

* the CPU oracle, built with gcc under AddressSanitizer (with leak checks)
  and UndefinedBehaviorSanitizer, runs tests/sanitize/oracle_driver.c:
  MTTKRP of every mode for orders 2-5, row subsets against full outputs,
  CP-ALS sweeps and a failing Cholesky;
* the library's host code (C ABI, planner, allocation-free entry point),
  compiled with the sanitizers on the host side only (each -fsanitize
  behind -Xarch_host; the kernels are built as usual), is linked with the
  other objects of the library build into tests/sanitize/abi_driver.cpp,
  which plans thousands of shapes and runs every validation path that
  returns before a HIP call.

Either run fails on the first sanitizer report (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "mttkrp_matrix_free_amd")
CSRC = os.path.join(PKG, "csrc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
# the host code built with the sanitizers; every other object comes from the library build
SANITIZED = ("capi.cpp", "plan.cpp", "noalloc.hip")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(map(str, cmd)), r.stdout[-3000:], r.stderr[-3000:])
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_san"
    run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", str(exe),
         os.path.join(ROOT, "oracle", "mttkrp_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
         "-lm"])
    r = run([str(exe)], env=ENV, timeout=300)
    assert "0 failed checks" in r.stdout, r.stdout


def _library_objects():
    """Objects of the library build, rebuilt when a source is newer."""
    from mttkrp_matrix_free_amd import build as hipbuild
    objs = {}
    stale = False
    for src in hipbuild.sources():
        obj = os.path.join(hipbuild.OBJ, os.path.basename(src) + ".o")
        objs[os.path.basename(src)] = obj
        if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(src):
            stale = True
    hdrs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".h"))]
    hdrs.append(os.path.join(ROOT, "include", "mttkrp.h"))
    newest_hdr = max(os.path.getmtime(h) for h in hdrs)
    if any(os.path.exists(o) and os.path.getmtime(o) < newest_hdr for o in objs.values()):
        stale = True
    if stale:
        hipbuild.build()
    return objs


def test_library_host_code_under_asan_ubsan(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clangxx = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clangxx)):
        pytest.skip("ROCm toolchain not found")
    objs = _library_objects()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    link = []
    for name, obj in objs.items():
        if name in SANITIZED:
            out = tmp_path / (name + ".san.o")
            run([hipcc, "--offload-arch=gfx950", "-c", "-O1", "-g", "-std=c++17", "-fPIC",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + SAN_HOST + inc +
                ["-o", str(out), os.path.join(CSRC, name)])
            link.append(str(out))
        else:
            link.append(obj)
    drv = tmp_path / "abi_driver.o"
    run([clangxx, "-c", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined"] + inc + ["-o", str(drv), os.path.join(HERE, "abi_driver.cpp")])
    exe = tmp_path / "abi_san"
    run([clangxx, "-fsanitize=address,undefined", "-o", str(exe), str(drv)] + link +
        ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(ENV)
    env.pop("MTTKRP_FORCE_TILE", None)
    r = run([str(exe)], env=env, timeout=300)
    assert "0 failed checks" in r.stdout, r.stdout
