"""Static checks on the pipelined kernel source (CPU only).

The consumer and producer waves of one workgroup run different code paths
that must execute the same number of workgroup barriers, or the workgroup
never finishes.  This counts __syncthreads() in each path, inside and outside
its chunk loop, straight from the source text.
"""

import os
import re

SRC = os.path.join(os.path.dirname(__file__), "..", "gated_delta_rule_17_amd", "csrc", "pipe_kernel.hpp")
LOOP = "for (int n = 0; n < nchunks; ++n)"


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
        loop, rest = _block(path, LOOP)
        out[name] = (loop.count("__syncthreads()"), rest.count("__syncthreads()"))
    return out


def test_consumer_and_producer_paths_have_equal_barrier_counts():
    counts = barrier_counts(open(SRC).read())
    assert counts["consumer"] == counts["producer"], counts
    assert counts["consumer"][0] >= 1


def test_count_detects_an_extra_producer_barrier():
    src = open(SRC).read()
    i = src.index("=================== producers")
    j = src.index(LOOP, i)
    k = src.index("{", j) + 1
    planted = src[:k] + "\n__syncthreads();\n" + src[k:]
    counts = barrier_counts(planted)
    assert counts["consumer"] != counts["producer"], counts
