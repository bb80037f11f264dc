"""The byte model used for the roofline, pinned to the figures the article prints."""
import json
import os

from transformer_megakernel_amd import roofline
from transformer_megakernel_amd.synth import ModelShape

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_llama1b_weight_bytes_match_the_articles_2_48_GB():
    s = ModelShape.named("llama1b")
    w = roofline.weight_bytes(s)
    # 1,235,814,400 parameters at 2 bytes each
    assert w == 2 * 1_235_814_400
    got = (w + 2 * s.hidden) / 1e9
    assert abs(got / GOLD["llama1b_bytes_per_forward_GB"] - 1) < 0.004


def test_bubble_model_reproduces_the_articles_rates():
    bw = GOLD["h100_bandwidth_TBps"] * 1e12
    b = GOLD["llama1b_bytes_per_forward_GB"] * 1e9
    ideal = roofline.forwards_per_second(b, bw)
    assert abs(ideal - GOLD["theoretical_forwards_per_s"]) < 1.0
    stalled = roofline.forwards_per_second(
        b, bw, GOLD["kernels_per_layer"] * GOLD["layers"], GOLD["stall_per_kernel_us"] * 1e-6)
    assert stalled < GOLD["forwards_per_s_with_stalls_below"]
    assert stalled > 0.99 * GOLD["forwards_per_s_with_stalls_below"]
    # 78 % of H100 bandwidth on 2.48 GB is under 1 ms, as the results paragraph states
    assert b / (GOLD["h100_bandwidth_utilisation"] * bw) < GOLD["h100_latency_ms_below"] * 1e-3


def test_step_bytes_itemisation():
    s = ModelShape.named("llama1b")
    parts = roofline.step_bytes(s, 128)
    assert parts["kv_read"] == 16 * 129 * 2048
    assert parts["kv_write"] == 16 * 2048
    assert parts["logits"] == 4 * 128256
    assert parts["total"] == 2_476_405_760
    assert roofline.step_bytes(s, 8192)["total"] == 2_740_646_912
    s8 = ModelShape.named("llama8b")
    assert roofline.step_bytes(s8, 2048)["total"] == 15_279_068_160
