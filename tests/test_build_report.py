"""The compiler's per-kernel resource report of the last build: no kernel spills to
scratch, and the one-launch step is built only in its spill-free forms (4-head groups;
fp32 only at D = 64). build() itself refuses to link a spilling build; this test reads
the report it leaves in _build/."""
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORT = os.path.join(ROOT, "_build", "kernel_resources.txt")


def _rows():
    if not os.path.exists(REPORT):
        pytest.skip("no build report: run page_selected_sparse_amd.build first")
    with open(REPORT) as fh:
        next(fh)
        return [line.rstrip("\n").split(" ", 6) for line in fh if line.strip()]


def test_no_kernel_uses_scratch():
    rows = _rows()
    assert len(rows) > 50
    spills = [r[6] for r in rows if int(r[0]) != 0]
    assert not spills, spills


def test_fused_step_builds_are_spill_free_forms():
    fused = [r[6] for r in _rows() if "select_attn_kernel<" in r[6]]
    assert fused
    for name in fused:
        args = name.split("<", 1)[1].split(">", 1)[0].split(", ")
        bf16, d, hb = args[0] == "true", int(args[1]), int(args[2])
        assert hb == 4, name
        assert bf16 or d == 64, name
