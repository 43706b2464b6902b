"""Every kernel of the library compiles for gfx950 without register spills
and without scratch memory (CPU only: hipcc cross-compiles the sources to
assembly and the test reads the code-object metadata). A spill would put
per-lane state in memory inside the hot loops."""

import concurrent.futures as cf
import os
import shutil

import pytest

from exact_attention_115_amd import build as B
from tests import isa_hazards as H

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and not shutil.which("hipcc"),
                                reason="needs hipcc")

KERNEL_SOURCES = [s for s in B.SOURCES if s.endswith(".hip")]


def test_no_kernel_spills_or_uses_scratch():
    with cf.ThreadPoolExecutor(max_workers=min(8, len(KERNEL_SOURCES))) as ex:
        asms = dict(zip(KERNEL_SOURCES, ex.map(H.library_asm, KERNEL_SOURCES)))
    bad, count = [], 0
    for src, asm in asms.items():
        for name, r in H.kernel_resources(asm).items():
            count += 1
            if r["vgpr_spill_count"] or r["private_segment_fixed_size"]:
                bad.append(f"{src}: {name}: {r}")
    print(f"{count} kernels checked")
    assert count >= 80
    assert not bad, "\n".join(bad)


def _count(asm, needle):
    return sum(1 for line in asm.splitlines() if line.strip().startswith(needle))


@pytest.mark.parametrize("src,needle", [("fa_fwd.hip", "s_barrier"), ("fa_bwd.hip", "s_barrier"),
                                        ("fa_bwd_dq.hip", "s_barrier"),
                                        ("fa_fwd_fp8.hip", "s_barrier"),
                                        ("fa_decode.hip", "s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)")])
def test_stage_barrier_build_adds_its_waits(src, needle):
    """The debug build (-DFA_STAGE_BARRIERS, compared bit for bit with the
    normal build by the GPU tests) really adds barriers, or full waits in
    the decode kernel, and still spills nothing."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    normal = H.library_asm(src)
    debug = H.compile_to_asm(os.path.join(B.CSRC, src), [os.path.join(root, "include"), B.CSRC],
                             ["-DFA_STAGE_BARRIERS"])
    n0, n1 = _count(normal, needle), _count(debug, needle)
    print(f"{src}: {needle}: {n0} -> {n1}")
    assert n1 > n0
    for name, r in H.kernel_resources(debug).items():
        assert not r["vgpr_spill_count"] and not r["private_segment_fixed_size"], (name, r)
