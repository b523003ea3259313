"""The C ABI's argument checks under the address and undefined-behaviour
sanitizers: api.cpp is built by the host compiler with both sanitizers and
stand-ins for the kernels and HIP calls (python -m attention_tiled_attn_amd.build
--sanitize), and every case of test_abi_cpu.py runs against that library in a
child process with the sanitizer runtime preloaded. A heap or stack overrun,
use after free, signed overflow, misaligned access or out-of-range shift in
the validation code ends the child with the sanitizer's report."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name: str) -> str | None:
    gcc = shutil.which("gcc")
    if not gcc:
        return None
    path = subprocess.run([gcc, f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_under_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("the fake-pointer validation cases run only without a GPU")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan and shutil.which("g++")):
        pytest.skip("no host compiler with sanitizer runtimes")
    from attention_tiled_attn_amd.build import build_sanitized
    lib = build_sanitized()
    env = dict(os.environ, FLEXATTN_LIB=lib, LD_PRELOAD=f"{asan} {ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import os, attention_tiled_attn_amd._lib as L, ctypes; ctypes.CDLL(L.LIB_PATH); "
             "maps = open('/proc/self/maps').read(); "
             "print(L.LIB_PATH, 'libasan' in maps, 'libflexattn_san' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.split() == [lib, "True", "True"], r.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-4000:], r.stderr[-4000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
