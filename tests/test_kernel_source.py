"""Static checks on the pipelined kernel sources (CPU only).

The consumer and producer waves of one workgroup run different code paths
that must execute the same number of workgroup barriers, or the workgroup
never finishes.  This counts __syncthreads() in each path, inside and outside
its chunk loop, straight from the source text, as a function a N + b of the
number of chunks N.
"""

import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "gated_delta_rule_17_amd", "csrc")
SOURCES = ["pipe_kernel.hpp", "chan_kernel.hpp"]
LOOP_RE = re.compile(r"for \(int n = 0; n (<|<=) nchunks; \+\+n\)")


def _block(text, start):
    """(brace block opened after `start`, text with that block removed)."""
    i = text.index(start)
    j = text.index("{", i)
    depth = 0
    for k in range(j, len(text)):
        if text[k] == "{":
            depth += 1
        elif text[k] == "}":
            depth -= 1
            if depth == 0:
                return text[j:k + 1], text[:i] + text[k + 1:]
    raise AssertionError("unbalanced braces")


def barrier_counts(src):
    """{role: (barriers in the chunk loop, barriers outside it)}."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    start = src.index("if (wave < NCW) {")
    cons, _ = _block(src, "if (wave < NCW) {")
    prod, _ = _block(src[start + len("if (wave < NCW) ") + len(cons):], "else {")
    out = {}
    for name, path in (("consumer", cons), ("producer", prod)):
        m = LOOP_RE.search(path)
        assert m, name
        loop, rest = _block(path, m.group(0))
        a = loop.count("__syncthreads()")
        extra = 1 if m.group(1) == "<=" else 0  # iterations: N or N + 1
        out[name] = (a, a * extra + rest.count("__syncthreads()"))
    return out


@pytest.mark.parametrize("name", SOURCES)
def test_consumer_and_producer_paths_have_equal_barrier_counts(name):
    counts = barrier_counts(open(os.path.join(CSRC, name)).read())
    assert counts["consumer"] == counts["producer"], counts
    assert counts["consumer"][0] >= 1


@pytest.mark.parametrize("name", SOURCES)
def test_count_detects_an_extra_producer_barrier(name):
    src = open(os.path.join(CSRC, name)).read()
    i = src.index("=================== producers")
    m = LOOP_RE.search(src, i)
    k = src.index("{", m.start()) + 1
    planted = src[:k] + "\n__syncthreads();\n" + src[k:]
    counts = barrier_counts(planted)
    assert counts["consumer"] != counts["producer"], counts
