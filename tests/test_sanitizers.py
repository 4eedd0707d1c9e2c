"""CPU sanitizer tier: AddressSanitizer + UndefinedBehaviorSanitizer builds.

- The oracle (oracle/conv_oracle.c) with gcc, driven by
  tests/c/oracle_sanitized.c over ragged, strided, dilated and padded
  problems with exactly sized buffers.
- The library's host code (descriptor creation, planning, the selection
  model, argument checks) built by hipcc with the sanitizers on the host side
  only (the gfx950 device code is unsanitized), driven with no GPU by
  tests/c/host_sanitized.c and by the plain-C ABI program's host checks.

Any sanitizer report makes the program exit non-zero (no recovery); leak
detection is on for the oracle and for the library's own allocations.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CDIR = os.path.join(ROOT, "tests", "c")
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _run(exe, env=None):
    e = dict(os.environ)
    e.update(env or {})
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=e)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "all ok" in r.stdout
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-O1", "-ffp-contract=off", "-fopenmp", *SAN,
                    os.path.join(CDIR, "oracle_sanitized.c"),
                    os.path.join(ROOT, "oracle", "conv_oracle.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang not found")
    from convolution_forward_gemm_amd import build
    d = tmp_path_factory.mktemp("hostsan")
    return build.build_host_sanitized(str(d / "libconvfprop.so"))


def _clang_exe(lib, sources, exe):
    libdir = os.path.dirname(lib)
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                        capture_output=True, text=True, check=True).stdout.strip()
    subprocess.run([CLANG, "-std=c11", "-O1", "-ffp-contract=off", *SAN, "-shared-libsan",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROCM, "include"), *sources, "-o", exe,
                    "-L", libdir, "-lconvfprop", "-Wl,-rpath," + libdir,
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + os.path.join(ROCM, "lib"),
                    "-Wl,-rpath," + os.path.dirname(rt), "-lm"],
                   check=True, capture_output=True, text=True)
    return exe


def test_library_host_code_under_asan_ubsan(sanitized_lib, tmp_path):
    exe = _clang_exe(sanitized_lib, [os.path.join(CDIR, "host_sanitized.c")],
                     str(tmp_path / "host_san"))
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})


def test_c_abi_program_host_checks_under_asan_ubsan(sanitized_lib, tmp_path):
    exe = _clang_exe(sanitized_lib, [os.path.join(CDIR, "abi_from_c.c"),
                                     os.path.join(ROOT, "oracle", "conv_oracle.c")],
                     str(tmp_path / "abi_san"))
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})
