"""The bench's reporting arithmetic against the numbers the article prints."""
import json
import os

from speculative_verify_gemv_amd import metrics

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "byte_counts.json")


def g():
    with open(GOLDEN) as f:
        return json.load(f)


def test_lm_head_bytes():
    h = g()["lm_head"]
    b = metrics.weight_bytes(h["rows"], h["cols"])
    assert b == 655_564_800
    assert round(b / 1e9, 3) == h["gb_printed"]


def test_verify_pass_total():
    v = g()["verify_pass"]
    assert round(sum(v["parts_gb"]), 3) == v["total_gb_printed"]


def test_cycle_bandwidth_and_fraction():
    c = g()["cycle"]
    bw = metrics.gbps(c["gb"] * 1e9, c["ms"])
    assert round(bw) == c["gbps_printed"]
    assert round(metrics.fraction_of_peak(bw, c["peak_gbps"]), 2) == c["fraction_printed"]
    assert round(1000.0 / c["ms"], 1) == c["tok_s_printed"]


def test_decode_ceiling():
    c = g()["ceiling"]
    tok = metrics.decode_ceiling_tok_s(c["eta"], c["peak_gbps"], c["gb_per_cycle"])
    assert round(tok, 1) == c["tok_s_per_token_printed"]
    # the article's 276.7 tok/s then needs tau >= 276.7 / 53.74 ~ 5.15 tokens per cycle
    assert 5.1 < 276.7 / tok < 5.2


def test_body_pass_bytes():
    shapes = {"qkv": (7168, 5120), "o": (5120, 5120), "gate_up": (34816, 5120), "down": (5120, 17408)}
    per_layer = sum(metrics.weight_bytes(n, k) for n, k in shapes.values())
    assert 64 * per_layer == 10_899_947_520
    assert 64 * per_layer + metrics.weight_bytes(248320, 5120) == 11_555_512_320
