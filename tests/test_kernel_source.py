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
SOURCES = ["pipe_kernel.hpp", "chan_kernel.hpp", "chan_split_kernel.hpp"]
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


def role_blocks(src):
    """The brace blocks of the role chain `if (wave < NCW) {..} else if (..) {..} else {..}`."""
    i = src.index("if (wave < NCW) {")
    blocks = []
    while True:
        j = src.index("{", i)
        block, _ = _block(src[j:], "{")
        blocks.append(block)
        rest = src[j + len(block):]
        m = re.match(r"\s*else\s*(if\s*\([^{]*\))?\s*\{", rest)
        if not m:
            return blocks
        i = j + len(block) + m.start()


def barrier_counts(src):
    """[(barriers in the chunk loop, barriers per sequence outside it)] per role.

    A loop `n < nchunks` runs N times and `n <= nchunks` N + 1 times; the
    second figure folds the extra iteration into the constant part."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    out = []
    for path in role_blocks(src):
        m = LOOP_RE.search(path)
        assert m, path[:200]
        loop, rest = _block(path, m.group(0))
        a = loop.count("__syncthreads()")
        extra = 1 if m.group(1) == "<=" else 0
        out.append((a, a * extra + rest.count("__syncthreads()")))
    return out


@pytest.mark.parametrize("name", SOURCES)
def test_every_role_executes_the_same_barriers(name):
    counts = barrier_counts(open(os.path.join(CSRC, name)).read())
    assert len(counts) >= 2, counts
    assert len(set(counts)) == 1, counts
    assert counts[0][0] >= 1


@pytest.mark.parametrize("name", SOURCES)
def test_count_detects_an_extra_producer_barrier(name):
    src = open(os.path.join(CSRC, name)).read()
    i = src.index("if (wave < NCW) {")
    i = src.index("} else", i + 1)  # the first producer role
    m = LOOP_RE.search(src, i)
    k = src.index("{", m.start()) + 1
    planted = src[:k] + "\n__syncthreads();\n" + src[k:]
    counts = barrier_counts(planted)
    assert len(set(counts)) > 1, counts
