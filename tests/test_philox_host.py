"""The library's dropout generator, built for the host (CPU only).

fa_philox.h is the header the dropout kernels include; compiled here for the
CPU, its Philox4x64-10 must reproduce numpy's Philox (an independent
implementation of the same published generator) word for word, and its
128-bit multiply must equal the compiler's 128-bit product. The GPU tests
then compare the kernels' keep masks with the oracle's bit for bit.
"""

import os
import subprocess

import numpy as np
import pytest

from exact_attention_115_amd import build as B

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "philox_host", "philox_host.cpp")

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="needs hipcc")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("philox") / "philox_host")
    r = subprocess.run([B.HIPCC, "-O2", "-std=c++17", "-I", B.CSRC, SRC, "-o", out],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def test_128_bit_multiply(exe):
    r = subprocess.run([exe, "mul"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout


def test_matches_numpy_philox(exe):
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0, 0, 0, 0), (2**64 - 1,) * 6, (1, 2, 3, 4, 5, 6)]
    cases += [tuple(int(x) for x in rng.integers(0, 2**64, size=6, dtype=np.uint64))
              for _ in range(200)]
    text = "\n".join(" ".join(str(x) for x in c) for c in cases) + "\n"
    r = subprocess.run([exe], input=text, capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    got = r.stdout.split("\n")
    for c, line in zip(cases, got):
        # numpy adds one to the counter before each block: start one below.
        ctr = np.array([(c[0] - 1) % 2**64, c[1], c[2], c[3]], dtype=np.uint64)
        if c[0] == 0:  # the decrement borrowed: undo it in the higher words
            ctr[1:] = np.array([(c[1] - 1) % 2**64, c[2], c[3]], dtype=np.uint64)
            if c[1] == 0:
                ctr[2:] = np.array([(c[2] - 1) % 2**64, c[3]], dtype=np.uint64)
                if c[2] == 0:
                    ctr[3] = np.uint64((c[3] - 1) % 2**64)
        bg = np.random.Philox(key=np.array(c[4:], dtype=np.uint64), counter=ctr)
        want = " ".join("%016x" % x for x in bg.random_raw(4))
        assert line == want, (c, line, want)
