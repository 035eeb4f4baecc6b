"""Host-only checks of bench.py's profile helpers (no GPU)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def kinds_of(name):
    return [k for k, test in bench.KINDS.items() if test(name)]


def test_each_expert_kernel_has_exactly_one_kind():
    # the dot decode kernel's last template argument (ring depth 16) must not
    # be read as gate+up or down
    assert kinds_of("void strata::moe_decode_dot_kernel<1, true, 1, 1, false>(strata::GemmArgs)") == ["decode_gate_up"]
    assert kinds_of("void strata::moe_decode_dot_kernel<1, true, 1, 2, true>(strata::GemmArgs)") == ["decode_gate_up"]
    assert kinds_of("void strata::moe_decode_dot_kernel<2, false, 4, 1, true>(strata::GemmArgs)") == ["decode_down"]
    assert kinds_of("void strata::moe_decode_dot_kernel<4, false, 1, 1, false>(strata::GemmArgs)") == ["decode_down"]
    assert kinds_of("void strata::moe_decode_kernel<1, true, 2>(strata::GemmArgs, int)") == ["decode_gate_up"]
    assert kinds_of("void strata::moe_decode_kernel<4, false, 1>(strata::GemmArgs, int)") == ["decode_down"]
    assert kinds_of("void strata::moe_prefill_kernel<1, true>(strata::GemmArgs)") == ["prefill_gate_up"]
    assert kinds_of("void strata::moe_prefill_kernel<2, false>(strata::GemmArgs)") == ["prefill_down"]


def test_other_kernels_have_no_kind():
    for n in ("void strata::combine_kernel(float const*, int const*)", "__amd_rocclr_copyBuffer",
              "void strata::route_decode_kernel<2>(unsigned short const*)", "void strata::page_in_kernel(strata::PageBatch)"):
        assert kinds_of(n) == []


def test_code_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* doc */ int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_hash(a) == bench.code_hash(b)
    assert bench.code_hash(a) != bench.code_hash(c)
