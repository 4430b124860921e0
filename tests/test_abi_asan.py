"""Host-side AddressSanitizer run of the C ABI layer (CPU only, no GPU needed).

The library's host code (argument validation, workspace layout, status strings) is compiled with
AddressSanitizer into a separate shared library, linked with the normally built kernel objects,
and driven by tests/abi_check/abi_check.c, which calls every entry point with invalid arguments
and the size queries with extreme ones. Device code is compiled as usual; nothing is launched.
"""

import os
import shutil
import subprocess

import pytest

from exact_attention_94_amd import build as fabuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "abi_check", "abi_check.c")


def _clang():
    for cand in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if cand and os.path.exists(cand):
            return cand
    return None


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res


def build_asan(out_dir):
    """libfa_asan.so (ABI layer with host ASan + the kernel objects) and the driver program."""
    hipcc = fabuild.hipcc()
    os.makedirs(out_dir, exist_ok=True)
    api_src = os.path.join(fabuild.CSRC, "fa_api.hip")
    api_obj = os.path.join(out_dir, "fa_api_asan.o")
    _run([hipcc, "-c", api_src, "-o", api_obj] + fabuild.compile_flags() +
         ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"])
    objs = [api_obj]
    for src in fabuild.sources():
        if os.path.basename(src) == "fa_api.hip":
            continue
        obj = os.path.join(fabuild.BUILD_DIR, os.path.basename(src) + ".o")
        if not os.path.exists(obj):
            fabuild._compile(src, ())
        objs.append(obj)
    lib = os.path.join(out_dir, "libfa_asan.so")
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={fabuild.ARCH}", "-o", lib] + objs)
    exe = os.path.join(out_dir, "abi_check")
    cc = _clang()
    _run([cc, "-g", "-fsanitize=address", "-fno-omit-frame-pointer", "-I",
          os.path.join(ROOT, "include"), DRIVER, "-L", out_dir, "-lfa_asan",
          f"-Wl,-rpath,{out_dir}", "-o", exe])
    return exe


def test_abi_validation_under_asan(tmp_path):
    try:
        fabuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if _clang() is None:
        pytest.skip("clang not available")
    exe = build_asan(str(tmp_path / "asan"))
    # The ABI layer really is instrumented: the library calls into the ASan runtime.
    syms = subprocess.run(["nm", "-D", str(tmp_path / "asan" / "libfa_asan.so")],
                          capture_output=True, text=True).stdout
    assert "__asan_report" in syms or "__asan_init" in syms
    env = dict(os.environ)
    # The HIP runtime keeps process-lifetime allocations; leaks are not what this run checks.
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout)
    print(res.stderr[-4000:])
    assert res.returncode == 0, res.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "all" in res.stdout and "checks passed" in res.stdout
