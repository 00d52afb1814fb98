"""Host-side arithmetic of the benchmark: the sweep's split counts, the
algorithmic bytes and flops behind the roofline, and the LDS bytes of the
partial kernel's dataflow. Worked by hand from the definitions in bench.py's
docstrings (no GPU)."""

import math

import pytest

import bench


@pytest.mark.parametrize("context,nodes,expect", [
    (4096, 9, 64), (4096, 16, 64), (4096, 32, 32),
    (16384, 9, 128), (16384, 16, 128), (16384, 32, 64),
    (65536, 9, 256), (65536, 32, 128), (184728, 9, 256), (184728, 32, 128),
    (1024, 9, 32), (256, 4, 16),
])
def test_sweep_nsplit_rule(context, nodes, expect):
    # about sqrt(keys) rounded down to a power of two, divided by the row
    # blocks (8 heads: 72 and 128 rows are one block, 256 rows two), at most
    # 256 workgroups
    assert bench.default_nsplit(1, nodes, 8, context + nodes) == expect


def test_sweep_nsplit_caps_at_one_workgroup_per_cu_for_batches():
    # 8 requests of 12 nodes x 8 heads (one row block): 256 / 8 = 32 per request
    assert bench.default_nsplit(8, 12, 8, 131072) == 32


def test_algorithmic_bytes_and_flops_c4a():
    keys = 184728 + 32
    rows = 32 * 8
    # KV rows, page-table entries (page size 1), queries, parents, one length
    expect = keys * 1152 + keys * 4 + rows * 1152 + 32 * 4 + 4
    assert bench.partial_algorithmic_bytes([keys], 32, 8, 1) == expect
    assert bench.algorithmic_flops([keys], 32, 8) == keys * rows * 2 * (576 + 512)


def test_lds_bytes_c4a_two_row_blocks_one_part():
    # 256 rows: two row blocks of four computing waves; 128 splits x 2 blocks
    # = 256 workgroups, so one column part. Per tile and block: four waves
    # read K (36,864 B) and V^T (32,768 B), and the tile arrives by DMA.
    tiles = math.ceil((184728 + 32) / 32)
    per = 4 * (36864 + 32768) + 36864
    assert bench.partial_lds_bytes([184728 + 32], 32, 8, 128) == tiles * 2 * per == 3642146816


def test_lds_bytes_c2_four_column_parts():
    # 128 rows, one block; 64 splits fill a quarter of the CUs, so four column
    # parts, each reading all of K and a quarter of V^T, each loading the tile
    tiles = math.ceil((4096 + 16) / 32)
    per_part = 4 * (36864 + 32768 // 4) + 36864
    assert bench.partial_lds_bytes([4096 + 16], 16, 8, 64) == tiles * 4 * per_part


def test_lds_bytes_t9_three_waves():
    # 72 rows: three computing waves; 256 splits, one column part
    tiles = math.ceil((184728 + 9) / 32)
    assert bench.partial_lds_bytes([184728 + 9], 9, 8, 256) == tiles * (3 * (36864 + 32768) + 36864)


def test_roof_bound_ridge():
    # intensity 1.89 flop/B per row against the 312.5 flop/B ridge
    assert bench.roof_bound(9, 8) == "hbm"
    assert bench.roof_bound(16, 8) == "hbm"
    assert bench.roof_bound(32, 8) == "mfma"
