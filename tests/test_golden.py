"""The verify-kernel page's printed arithmetic, recomputed with the bench's own
accounting (tests/golden/pages_arithmetic.json; page "The Custom sm_120 Verify
Kernel: From 0.7 tok/s to 3-6x Decode Speedup on Blackwell Consumer GPUs",
Parts I, V and VII). These tie the bench's bytes-per-key and its effective-
bandwidth definition to the numbers on the page."""

import json
import math
import os

import pytest

import bench
from workloads.gen import HEAD_DIM_QK, POOL_SLOTS_PAGES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_arithmetic.json")


def _entries():
    with open(GOLDEN) as f:
        return {e["name"]: e for e in json.load(f)["entries"]}


E = _entries()


def _close(value, entry):
    tol = entry["rel_tol"]
    assert math.isclose(value, entry["printed"], rel_tol=tol, abs_tol=0.0 if tol else 1e-9), (entry["name"], value)


def test_bytes_per_token_matches_part_i():
    e = E["latent_kv_bytes_per_token_all_layers"]
    assert bench.KV_ROW_BYTES == e["inputs"]["head_dim_qk"] * e["inputs"]["bytes_per_element"] == HEAD_DIM_QK * 2
    per_token = bench.kv_bytes([1]) * e["inputs"]["layers"]
    _close(per_token, e)


def test_pool_size_matches_part_i():
    _close(POOL_SLOTS_PAGES, E["kv_pool_tokens"])


def test_bytes_per_step_at_64k_matches_part_v():
    e = E["latent_bytes_per_decode_step_at_64k"]
    step_bytes = bench.kv_bytes([e["inputs"]["context"]]) * e["inputs"]["layers"]
    _close(step_bytes, e)


def test_effective_bandwidth_definition_matches_part_v():
    e = E["effective_kv_bandwidth_triton_at_64k"]
    # bench.effective_kv_gbs over 61 layers' worth of keys reproduces the page's ~14 GB/s
    layers = E["latent_bytes_per_decode_step_at_64k"]["inputs"]["layers"]
    gbs = bench.effective_kv_gbs([65536] * layers, e["inputs"]["step_seconds"])
    _close(gbs * 1e9, e)
    r = E["peak_over_effective"]
    _close(r["inputs"]["peak_bytes_per_s"] / r["inputs"]["effective_bytes_per_s"], r)


@pytest.mark.parametrize("name", ["grid_single_gpu_64_heads", "grid_tp8_8_heads_nsplit16", "grid_tp8_8_heads_nsplit64"])
def test_grid_arithmetic_matches_part_vii(name):
    e = E[name]
    i = e["inputs"]
    _close(i["batch"] * i["queries"] * i["heads"] * i["nsplit"], e)


@pytest.mark.parametrize("name", ["waves_nsplit16_on_188_sms", "waves_nsplit64_on_188_sms"])
def test_waves_match_part_vii(name):
    e = E[name]
    _close(e["inputs"]["blocks"] / e["inputs"]["sms"], e)


@pytest.mark.parametrize("name", ["speedup_4k", "speedup_16k", "speedup_65k"])
def test_speedups_match_part_vii(name):
    e = E[name]
    _close(e["inputs"]["after"] / e["inputs"]["before"], e)
