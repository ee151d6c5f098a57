"""The CPU oracle and the host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU is used).

* tests/sanitize/oracle_drive.c runs every oracle function on seeded inputs
  and edge cases (empty and ragged lengths, zero blocks, special floats,
  splits, causal masks), built with gcc -fsanitize=address,undefined.
* tests/sanitize/abi_drive.cpp runs the size queries and entry points of
  include/sage.h with valid and invalid descriptors, sequence tables and
  pointers, built with the library's sage_api.cpp and host-only stand-ins for
  the device launchers (tests/sanitize/launch_stubs.cpp), the sanitizers on
  the host side only.  Its calls stop at a host check or at the device check,
  so no fake pointer is ever dereferenced.
Any sanitizer report aborts the driver (no recovery), and the test fails.
Leak detection is off: the HIP runtime keeps allocations until exit.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    return res.returncode, res.stdout, err


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_drive")
    rc, out, err = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined",
                         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                         "-ffp-contract=off", os.path.join(ROOT, "oracle", "sage_oracle.c"),
                         os.path.join(SAN, "oracle_drive.c"), "-lm", "-o", exe])
    assert rc == 0, err
    rc, out, err = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"}, timeout=300)
    assert rc == 0 and "oracle drive: ok" in out, out + err


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_drive")
    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                 "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    csrc = os.path.join(ROOT, "quantized_attention_03_amd", "csrc")
    rc, out, err = _run([HIPCC, "-O1", "-g", "-std=c++17", *host_san,
                         "-I", os.path.join(ROOT, "include"), "-I", csrc,
                         os.path.join(csrc, "sage_api.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
                         os.path.join(SAN, "abi_drive.cpp"), "-o", exe])
    assert rc == 0, err
    rc, out, err = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=0"}, timeout=300)
    assert rc == 0 and "abi drive: ok" in out, out + err
