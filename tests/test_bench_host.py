"""Host-side pieces of bench.py (no GPU): the kernel-source hash that ties the stored
rocprofv3 traffic figures to the code they were measured on, and the stored figures'
validity for the current sources."""
from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_blank_lines_only():
    src = "int a = 1; // one\n\n/* a\n   block */ int b = 2;\n  return a + b;  \n"
    assert bench._code_only(src) == "int a = 1;\n int b = 2;\n  return a + b;"
    # a change of code changes the text, a change of comment does not
    assert bench._code_only(src.replace("// one", "// uno")) == bench._code_only(src)
    assert bench._code_only(src.replace("a + b", "a - b")) != bench._code_only(src)


def test_stored_traffic_matches_current_kernel_code():
    """Every committed FETCH/WRITE summary was taken on the current kernel code."""
    variants = {"c3": 6, "c5a": 6, "c5b": 3, "fa3": "attn", "fa4": "attn", "mx3": 9, "mx6": 9, "sp3": "sp",
                "w4a": "w4"}
    for w, v in variants.items():
        path = os.path.join(ROOT, "profiles", f"pmc_{w}.json")
        rec = json.load(open(path))
        assert rec["kernel_hash"] == bench.kernel_hash(v), f"{w}: profile taken on other kernel code"
        assert bench.stored_traffic(w, v) == rec["traffic_bytes_per_launch"]


def test_stored_kernel_traces_match_current_kernel_code():
    """Every committed rocprofv3 kernel-trace summary names the kernel-source hash it was
    taken on; that hash must be the current code's (a kernel change needs a new trace)."""
    import glob
    import re
    variants = {"gemm_lds_256x256": 6, "gemm_lds_32x128": 13, "gemm_lds_64x128": 10, "gemm_mx_256x256": 9,
                "gemm_skinny": 3, "gemm_sp_256x256": "sp", "gemm_w4": "w4", "attn_fwd": "attn"}
    seen = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        m = re.search(r"Kernel source hash \(bench\.kernel_hash\): (\w+)", open(path).read())
        if not m:
            continue
        name = os.path.basename(path)
        keys = [k for k in variants if name.startswith(k)]
        assert len(keys) == 1, f"{name}: no kernel family for this summary"
        assert m.group(1) == bench.kernel_hash(variants[keys[0]]), f"{name}: trace taken on other kernel code"
        seen += 1
    assert seen >= 10
