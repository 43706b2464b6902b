"""The host-side argument checks of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

The library's sources are compiled with both sanitizers on their host code
(the device code is compiled as usual and never runs here) and linked with
tests/sanitize/abi_driver.c into one executable. Every check of
tests/test_abi.py (bad pointers, shapes, sizes one past the limits,
alignment, overlap, workspace sizes, error strings) is then replayed through
that executable, one call per line. A sanitizer report ends the executable
with a non-zero status (nothing is recovered), so the check in flight fails,
and the last test asserts that the driver exited cleanly, leak check
included, with no report on its stderr.
"""

from __future__ import annotations

import ctypes
import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import tempfile

import pytest

import exact_attention_115_amd as fa
from exact_attention_115_amd import build as B
from tests import test_abi as T
# The checks themselves, collected again in this module, where the fixture
# below points them at the sanitized executable.
from tests.test_abi import (  # noqa: F401
    test_bwd_dropout_rejects_bad_arguments,
    test_bwd_noalloc_rejects_bad_arguments_before_any_hip_call,
    test_bwd_rejects_bad_arguments,
    test_dropout_mask_rejects_bad_arguments,
    test_extreme_sizes_are_refused_without_overflow,
    test_fwd_decode_needs_workspace,
    test_fwd_dropout_rejects_bad_arguments,
    test_fwd_empty_problems_are_noops,
    test_fwd_fp8_rejects_bad_arguments,
    test_fwd_rejects_bad_arguments,
    test_paged_rejects_bad_arguments,
    test_paged_workspace_matches_contiguous_decode,
    test_size_limits_are_enforced,
    test_version_and_strerror,
    test_workspace_sizes,
)

LLVM = "/opt/rocm/llvm/bin"
DRIVER_SRC = os.path.join(B.ROOT, "tests", "sanitize", "abi_driver.c")
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(
    not (os.path.exists(B.HIPCC) and os.path.exists(f"{LLVM}/clang")
         and os.path.exists(fa.LIB_PATH)),
    reason="needs hipcc, clang and a built libfa.so")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}")


def _build_driver() -> str:
    """Compile the sanitized executable (cached under _build/ by source hash)."""
    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    headers = [os.path.join(B.CSRC, f) for f in sorted(os.listdir(B.CSRC)) if f.endswith(".h")]
    h = hashlib.sha256()
    for f in srcs + headers + [os.path.join(B.INCLUDE, "fa.h"), DRIVER_SRC]:
        h.update(open(f, "rb").read())
    h.update(" ".join(SAN).encode())
    out_dir = os.path.join(B.BUILD, "sanitize", h.hexdigest()[:16])
    exe = os.path.join(out_dir, "abi_driver")
    if os.path.exists(exe):
        return exe
    os.makedirs(os.path.dirname(out_dir), exist_ok=True)
    tmp = tempfile.mkdtemp(dir=os.path.dirname(out_dir))
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]

    def lib_obj(src):
        name = os.path.basename(src)
        obj = os.path.join(tmp, os.path.splitext(name)[0] + ".o")
        lang = ["-x", "hip"] if name.endswith(".cpp") else []
        _run([B.HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
              "-I", B.INCLUDE, "-I", B.CSRC, *lang, "-c", src, "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lib_obj, srcs))
    drv = os.path.join(tmp, "abi_driver_main.o")
    _run([f"{LLVM}/clang", "-x", "c", "-std=c11", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I/opt/rocm/include", "-I", B.INCLUDE, "-c", DRIVER_SRC, "-o", drv])
    _run([f"{LLVM}/clang++", *SAN, *objs, drv, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", os.path.join(tmp, "abi_driver")])
    if os.path.isdir(out_dir):
        shutil.rmtree(out_dir)
    os.replace(tmp, out_dir)
    return exe


def _arg(value, ctype):
    if ctype is ctypes.c_float or ctype is ctypes.c_double:
        return float(value).hex()
    if isinstance(value, ctypes.c_void_p):
        value = value.value
    return str(int(value or 0))


class SanitizedLib:
    """Same entry points as the ctypes library; each call is one line to the
    sanitized driver, typed by the ctypes signatures the binding declares."""

    def __init__(self, exe: str):
        self.native = fa.load()
        self.stderr = tempfile.TemporaryFile(mode="w+")
        env = dict(os.environ)
        env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0"
        env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
        self.proc = subprocess.Popen([exe], stdin=subprocess.PIPE, stdout=subprocess.PIPE,
                                     stderr=self.stderr, text=True, env=env)
        self.calls = 0

    def report(self) -> str:
        self.stderr.seek(0)
        return self.stderr.read()

    def __getattr__(self, name):
        fn = getattr(self.native, name)

        def call(*args):
            line = " ".join([name] + [_arg(a, t) for a, t in zip(args, fn.argtypes)])
            self.proc.stdin.write(line + "\n")
            self.proc.stdin.flush()
            out = self.proc.stdout.readline()
            if not out or out.startswith("error:"):
                self.proc.wait(timeout=30)
                raise RuntimeError(f"sanitized driver failed on '{line}' "
                                   f"(status {self.proc.returncode}): {out}\n{self.report()}")
            self.calls += 1
            out = out.rstrip("\n")
            return out.encode() if fn.restype is ctypes.c_char_p else int(out)

        return call

    def close(self) -> int:
        self.proc.stdin.close()
        return self.proc.wait(timeout=60)


@pytest.fixture(scope="module", autouse=True)
def sanitized():
    drv = SanitizedLib(_build_driver())
    T.BACKEND["lib"] = drv
    try:
        yield drv
    finally:
        T.BACKEND["lib"] = None
        if drv.proc.poll() is None:
            drv.close()


def test_zz_driver_exits_clean(sanitized):
    """Runs last in this module: every replayed call went through, and the
    driver ends with status 0 and no sanitizer report (the leak check runs
    at exit)."""
    assert sanitized.calls > 100
    status = sanitized.close()
    report = sanitized.report()
    assert status == 0, report
    for marker in ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:"):
        assert marker not in report, report
