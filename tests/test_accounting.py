"""The benchmark's byte/FLOP accounting against the numbers the pages print (tests/golden/pages_numbers.json)."""
import json
import os

import numpy as np

from mla_decode_attention_amd import workloads as W

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_absorbed_intensity_matches_pages():
    # 128 heads, s_q = 1: FLOPs per key / bytes per key
    ai = 128 * W.FLOPS_PER_ROW_KEY / W.ROW_BYTES
    want = GOLDEN["absorbed_mqa_intensity_sq1"]["value"]
    assert abs(ai - want) / want < 0.005, ai


def test_cache_row_fraction_matches_pages():
    gqa_row = 8 * 128 * 2          # LLaMA-3-8B: 8 KV heads x 128 dims, K and V
    assert W.ROW_BYTES // 2 / gqa_row == GOLDEN["latent_cache_fraction_of_gqa"]["value"]


def test_speedups_are_the_throughput_ratios():
    g = GOLDEN["etap_throughput_64k_b16"]
    for k, s in g["speedups"].items():
        assert abs(g["tflops"]["etap"] / g["tflops"][k] - s) < 0.006, k


def test_headline_workload_sizes():
    lens = np.full(16, 65536)
    assert W.algorithmic_bytes(lens, 16, 1, 16) - 16 * 16 * (576 + 512) * 2 - 16 * 16 * 4 == 1207959552
    assert W.algorithmic_flops(lens, 1, 16, False) == 36507222016


def test_causal_visibility_rule():
    n = W.visible_keys(np.array([10, 1, 0]), 2, True)
    assert n.tolist() == [[9, 10], [0, 1], [0, 0]]
    assert W.visible_keys(np.array([10]), 2, False).tolist() == [[10, 10]]
