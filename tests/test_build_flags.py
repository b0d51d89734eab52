"""The attention kernels are compiled without NaN semantics (the compiler may
assume no value is NaN), so no code in them may test for NaN by value: such a
test could be folded away.  NaN checks there use bit patterns."""
from __future__ import annotations

import os
import re

from paged_kv_cache_464_amd import build

CSRC = build.CSRC
NO_NAN_SOURCES = ["decode_kernels.hip", "decode_inst.hip", "decode_engine.hpp", "token_store.hpp", "layout.hpp",
                  "kernels.hpp"]


def test_attention_kernels_are_built_without_nan_semantics_and_nothing_else_is():
    assert build.FILE_FLAGS == {"decode_kernels.hip": ["-fno-honor-nans"], "decode_inst.hip": ["-fno-honor-nans"]}
    for src in build.HIP_SOURCES + build.HOST_SOURCES + [build.INST_SOURCE]:
        assert os.path.exists(os.path.join(CSRC, src)), src


def _code(path):
    text = open(path).read()
    text = re.sub(r"//[^\n]*", "", text)          # line comments
    return re.sub(r"/\*.*?\*/", "", text, flags=re.S)  # block comments


def test_no_value_nan_tests_in_sources_built_without_nan_semantics():
    self_cmp = re.compile(r"(?<![\w.])([A-Za-z_][\w.\[\]]*)\s*(==|!=)\s*\1(?![\w.\[])")
    for name in NO_NAN_SOURCES:
        code = _code(os.path.join(CSRC, name))
        assert not re.search(r"\b(isnan|isfinite|__builtin_isnan|__builtin_isfinite)\s*\(", code), name
        hits = [m.group(0) for m in self_cmp.finditer(code)]
        assert not hits, (name, hits)


def test_the_guard_finds_a_value_nan_test():
    """The pattern above does catch the forms it guards against."""
    self_cmp = re.compile(r"(?<![\w.])([A-Za-z_][\w.\[\]]*)\s*(==|!=)\s*\1(?![\w.\[])")
    assert self_cmp.search("r = (r == r) ? r : 0.0f;")
    assert self_cmp.search("if (x[i] != x[i]) return;")
    assert not self_cmp.search("if (a == b) return;")
