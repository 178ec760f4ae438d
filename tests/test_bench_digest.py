"""CPU checks of bench.py's kernel-source digest, which ties the committed counter summaries to the
code they were taken on: comments and the probe build's code do not change it; code does."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

PRODUCT = """int f(int x)
{
#if X > 1
    x += 1;
#endif
    return x;  // done
}
"""

WITH_PROBE = """int f(int x)
{
#ifdef MOE_PHASE_PROBE
    stamp(0);
#else
    other();
#endif
    MOE_PROBE(a += g(h(1), 2);)
#if X > 1
    x += 1;   /* kept */
#endif
    MOE_PROBE(b = 1;)
    return x;
}
#ifdef MOE_PHASE_PROBE
#define MOE_PROBE(...) __VA_ARGS__
#else
#define MOE_PROBE(...)
#endif
"""


def test_probe_code_and_comments_leave_the_digest_alone():
    expect = bench._code_only(PRODUCT.replace("{\n", "{\n    other();\n", 1))
    assert bench._code_only(WITH_PROBE) == expect


def test_code_changes_the_digest():
    assert bench._code_only(PRODUCT) != bench._code_only(PRODUCT.replace("x += 1", "x += 2"))

