"""Host code of libgq under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU).

Every library source is compiled host-only (device code compiled out) with
both sanitizers, linked with tests/host_sanitize/host_checks.cpp and run.
The driver exercises the argument checks, size queries and grouped-decode
plan encoding on valid, edge and invalid inputs; none of its calls gets past
its checks, so nothing is launched.  A sanitizer finding aborts the driver.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
# host-side sanitizers only: each flag applies to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
LINK_SAN = "-fsanitize=address,undefined"


def test_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm toolchain not available")
    from quantized_gemm_groupwise_amd import _build as B
    inc = [f"-I{B.INCLUDE}", f"-I{B.CSRC}"]

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(os.path.basename(src))[0] + ".o"))
        lang = ["-x", "hip", "--offload-host-only"] if src.endswith(".hip") else []
        cmd = [HIPCC, "-std=c++17", "-O1", "-g", "-fPIC", f"--offload-arch={B.ARCH}", *inc, *HOST_SAN,
               *lang, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    srcs.append(os.path.join(ROOT, "tests", "host_sanitize", "host_checks.cpp"))
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    # the device images a host-only object refers to do not exist: define
    # each referenced image symbol as an empty array, and the registration
    # hooks that would hand them to the HIP runtime as no-ops
    nm = shutil.which("nm") or os.path.join(os.path.dirname(CLANGXX), "llvm-nm")
    images = set()
    for o in objs:
        r = subprocess.run([nm, "-u", o], capture_output=True, text=True)
        images.update(w for w in r.stdout.split() if w.startswith("__hip_fatbin_"))
    img_c = tmp_path / "images.c"
    img_c.write_text("".join(f"const char {n}[64] = {{0}};\n" for n in sorted(images)))
    stub_objs = []
    for src in (str(img_c), os.path.join(ROOT, "tests", "host_sanitize", "registration_stubs.c")):
        o = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([CLANGXX, "-x", "c", "-O1", "-fPIC", "-c", src, "-o", o], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        stub_objs.append(o)
    exe = str(tmp_path / "host_checks")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "lib")
    link = [CLANGXX, LINK_SAN, *objs, *stub_objs, "-o", exe, f"-L{rocm_lib}", "-lamdhip64",
            f"-Wl,-rpath,{rocm_lib}"]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all checks passed" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]


def test_header_is_plain_c(tmp_path):
    """include/gq.h compiles as C11 (the ABI is C; the C++-only enum type
    clause is behind __cplusplus)."""
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    src = tmp_path / "use_gq.c"
    src.write_text('#include "gq.h"\nint main(void) { gq_dtype d = GQ_BF16; gq_status s = GQ_OK; '
                   'return (int)d + (int)s; }\n')
    r = subprocess.run([gcc, "-x", "c", "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        f"-I{os.path.join(ROOT, 'include')}", "-fsyntax-only", str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
