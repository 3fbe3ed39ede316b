"""The roofline calculator against every number the page prints (CPU).

Fixture: tests/golden/page_numbers.json, values from "GQLA: Group-Query Latent
Attention for Hardware-Adaptive LLM Decoding", technical summary sections 1, 2
and 4.  The device peaks are public spec values, not on the page; the ridges
they give must equal the page's.
"""
import json
import os

import pytest

from latent_kv_cache_amd import roofline as rf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def near(name, x):
    e = GOLD[name]
    assert abs(x - e["value"]) <= e["tol"], (name, x, e)


def test_ridges():
    near("ridge_h100_flops_per_byte", rf.H100.ridge)
    near("ridge_h20_flops_per_byte", rf.H20.ridge)


def test_absorb_intensity():
    near("absorb_intensity_sq1", rf.intensity("absorb", h_q=128, g=8, s_q=1))


@pytest.mark.parametrize("g,s_q", [(8, 2), (4, 1)])
def test_gqa_intensity_at_h20_ridge(g, s_q):
    near("gqa_intensity_h20", rf.intensity("gqa", h_q=128, g=g, s_q=s_q))


def test_cache_ratio():
    near("cache_ratio_absorb_vs_gqa", rf.cache_ratio(512, 64, 8, 128))


def test_throughput_projections():
    ctx = 8192
    a100 = rf.tokens_per_s(rf.H100, "absorb", 128, 8, 1, ctx)
    g20 = rf.tokens_per_s(rf.H20, "gqa", 128, 8, 2, ctx)
    m20 = rf.tokens_per_s(rf.H20, "absorb", 128, 8, 1, ctx)
    near("h100_absorb_tokens_per_s", a100)
    near("h20_gqa_g8_sq2_tokens_per_s", g20)
    near("h20_mla_tokens_per_s", m20)
    near("h20_gqa_over_mla", g20 / m20)
    # MTP gains nothing for the absorbed form on H20 (section 1, zero multi-token gain)
    assert rf.tokens_per_s(rf.H20, "absorb", 128, 8, 2, ctx) == pytest.approx(m20, rel=1e-9)


def test_step_work_counts():
    w = rf.step_work("gqa", 128, 8, 1, total_ctx=10, batch=1)
    assert w.bytes == 2 * (2 * 8 * 128 + 64) * 10 + 128 * (128 + 64 + 128) * 2
    assert w.flops == 2 * 128 * (2 * 128 + 64) * 10
    a = rf.step_work("absorb", 128, 8, 1, total_ctx=10, batch=1)
    assert a.flops == 2 * 128 * (2 * 512 + 64) * 10 + 4 * 128 * 128 * 512
