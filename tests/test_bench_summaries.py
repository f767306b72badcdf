"""Host-side pieces of bench.py's profile summaries (no GPU): the workgroup
count of a rocprofv3 kernel-trace row and the phase table of a --phases
record."""
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("row,want", [
    # combine_kernel: grid (G, Hkv, rows * D/32) workgroups of one wave
    ({"Grid_Size_X": "384", "Grid_Size_Y": "1", "Grid_Size_Z": "32", "Workgroup_Size_X": "64",
      "Workgroup_Size_Y": "1", "Workgroup_Size_Z": "1"}, 6 * 32),
    # split_kernel: (splits, KV heads) workgroups of five waves
    ({"Grid_Size_X": "40960", "Grid_Size_Y": "1", "Grid_Size_Z": "1", "Workgroup_Size_X": "320",
      "Workgroup_Size_Y": "1", "Workgroup_Size_Z": "1"}, 128),
    ({"Grid_Size_X": "4096", "Workgroup_Size_X": "512"}, 8),  # a file without Y and Z columns
])
def test_trace_workgroups_counts_every_grid_dimension(row, want):
    assert bench.trace_workgroups(row) == want


def test_phase_table_lists_each_roles_waits(tmp_path, monkeypatch):
    case = dict(case="sweep 16K", splits=128, chunks_per_split=4.0, wait_c0=0.012, wait_c1=0.096,
                wait_c2=0.357, dma_prod=0.052, wait_prod=0.329)
    qcase = dict(case="quantised tree 64K", splits=64, wait_c0=0.1, wait_c1=0.2, dma_prod=0.06, wait_prod=0.43,
                 wait_dec=0.18, conv_dec=0.5)
    (tmp_path / "phases.log").write_text(json.dumps({"phases": [case, qcase], "kernel_hash": bench.kernel_hash()}) + "\n")
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    bench.phase_table(str(tmp_path), "python bench.py")
    text = (out / "split_kernel_phases.md").read_text()
    assert "| sweep 16K | 128 |" in text
    assert "0.012, 0.096, 0.357 / 0.329 (0.052) |" in text
    assert "0.100, 0.200 / 0.430 (0.060) / 0.180 (0.500) |" in text
