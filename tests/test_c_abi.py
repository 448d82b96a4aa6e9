"""The C ABI from C (CPU only): include/kvc.h and include/kvc_probe.h compile as
strict C99, and a C program linked against libkvc.so drives a host-only cache
through the calls of "LingBot-Map Paged KV Cache", sections 2-3 (appends,
visible tables, rollback), checking the pages' invariants (tests/c/abi_host.c)."""
import os
import shutil
import subprocess

import pytest

from paged_sliding_window_kv_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_headers_compile_as_c99(tmp_path):
    src = tmp_path / "h.c"
    src.write_text('#include "kvc.h"\n#include "kvc_probe.h"\nint main(void) { return 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{INCLUDE}", "-c",
                        str(src), "-o", str(tmp_path / "h.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_c_program_drives_a_host_only_cache(tmp_path):
    lib = L.lib()  # builds nothing; raises if libkvc.so is missing
    libdir = os.path.dirname(os.path.abspath(L.LIB_PATH))
    exe = str(tmp_path / "abi_host")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", f"-I{INCLUDE}",
                        os.path.join(ROOT, "tests", "c", "abi_host.c"), "-o", exe, f"-L{libdir}", "-lkvc",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert lib is not None
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("OK")


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include/hip"),
                    reason="needs gcc and the HIP headers")
def test_device_program_compiles_as_c99(tmp_path):
    """tests/c/abi_device.c (run on the GPU by tests/test_gpu_c_abi.py) builds as strict C99 against
    libkvc.so and HIP's C API."""
    L.lib()
    libdir = os.path.dirname(os.path.abspath(L.LIB_PATH))
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
                        "-I/opt/rocm/include", os.path.join(ROOT, "tests", "c", "abi_device.c"),
                        "-o", str(tmp_path / "abi_device"), f"-L{libdir}", "-lkvc", f"-Wl,-rpath,{libdir}",
                        "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
