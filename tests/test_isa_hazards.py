"""The matrix-core hazards around the dK/dV kernel's inline-assembly
products, checked on the compiled gfx950 assembly (CPU only: hipcc
cross-compiles, nothing runs).

The compiler places no wait states around inline assembly, so these tests
check the code it generates: every product's operands must have been
written by the vector ALU, and every product's result read by anything else,
at least as many wait states earlier as the rules in tests/isa_hazards.py
require. The rule values are tied to the compiler's own hazard recognizer:
for the same producer / consumer pairs written with the builtins
(tests/isa/hazard_rules.hip) the compiler inserts no more wait states than
the rules ask for.
"""

import os
import shutil

import pytest

from tests import isa_hazards as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_115_amd", "csrc")
INC = [os.path.join(ROOT, "include"), CSRC]
PROBES = os.path.join(ROOT, "tests", "isa", "hazard_rules.hip")

pytestmark = pytest.mark.skipif(
    not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")) and not shutil.which("hipcc"),
    reason="needs hipcc")

# Probe kernel -> the hazard class its consumer exercises.
PROBE_KIND = {
    "probe_valu_to_srca": "valu_to_srcab",
    "probe_valu_to_srcb": "valu_to_srcab",
    "probe_valu_to_srcc": "valu_to_srcc",
    "probe_xdl_to_read": "xdl_to_read",
    "probe_xdl_to_srca": "xdl_to_read",
}


@pytest.fixture(scope="module")
def probe_functions():
    fns = H.functions(H.compile_to_asm(PROBES, INC))
    return {name: lines for name, lines in fns.items() if "probe_" in name}


def _short(name):
    return next(k for k in list(PROBE_KIND) + ["probe_chain"] if k in name)


def test_rules_are_at_least_the_compilers_wait_states(probe_functions):
    seen = {}
    for name, lines in probe_functions.items():
        key = _short(name)
        if key == "probe_chain":
            continue
        kind = PROBE_KIND[key]
        d = [ks[kind] for _, _, ks in H.distances(lines) if kind in ks]
        assert d, f"{key}: no {kind} pair found in the compiled probe"
        need = min(d)  # the compiler puts exactly what the pair needs
        seen[key] = need
        assert H.RULES[kind] >= need, (key, kind, need, H.RULES[kind])
    print("wait states the compiler inserts:", seen)
    assert len(seen) == len(PROBE_KIND)


def test_accumulation_chains_need_no_wait_state(probe_functions):
    lines = next(l for n, l in probe_functions.items() if "probe_chain" in n)
    text = "\n".join(lines)
    # The two products follow each other directly.
    body = [l.strip() for l in lines if l.strip() and not l.strip().startswith((";", "."))]
    i = next(k for k, l in enumerate(body) if l.startswith("v_mfma"))
    assert body[i + 1].startswith("v_mfma"), text
    assert H.check(lines) == []


def test_checker_flags_the_probes_without_their_wait_states(probe_functions):
    for name, lines in probe_functions.items():
        if "probe_chain" in name:
            continue
        stripped = [l for l in lines if "s_nop" not in l]
        assert H.check(stripped), f"{_short(name)}: removing the wait states went unnoticed"


def test_dkdv_kernels_have_no_matrix_core_hazards():
    fns = H.functions(H.library_asm("fa_bwd.hip"))
    kernels = {n: l for n, l in fns.items() if "bwd_dkdv_kernel" in n}
    assert len(kernels) == 16  # {bf16, f16} x {64, 128} x causal x dropout
    bad = {n: H.check(l) for n, l in kernels.items()}
    bad = {n: v for n, v in bad.items() if v}
    assert not bad, "\n".join(f"{n}: {v[:3]}" for n, v in bad.items())
