"""Roofline path selection (section 2, Path selection) on the CPU: the oracle's model
against the page's numbers and stated choices, and the library's gqla_select_path
against the oracle over a grid of devices and shapes.

Fixtures: tests/golden/page_numbers.json (ridges, intensities and throughput
projections printed on "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
Decoding", technical summary sections 1, 2 and 4) and tests/golden/path_selection.json
(the path the page assigns to each of its two devices).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import roofline as orf
from latent_kv_cache_amd import gqla

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PAGE = json.load(open(os.path.join(GOLD, "page_numbers.json")))
SEL = json.load(open(os.path.join(GOLD, "path_selection.json")))
DEV = SEL["devices"]
FLAG = dict(h_q=128, r_kv=512, d_r=64, d_h=128, e=2)


def near(name, x):
    e = PAGE[name]
    assert abs(x - e["value"]) <= e["tol"], (name, x, e)


def oracle_tps(dev, path, g, s_q, ctx=8192, batch=1):
    d = DEV[dev]
    return orf.step_tokens_per_s(path, FLAG["h_q"], g, s_q, FLAG["r_kv"], FLAG["d_r"], FLAG["d_h"], FLAG["e"],
                                 batch, ctx, d["peak_flops"], d["peak_bytes_per_s"])[0]


def test_oracle_reproduces_page_projections():
    near("ridge_h100_flops_per_byte", DEV["H100"]["peak_flops"] / DEV["H100"]["peak_bytes_per_s"])
    near("ridge_h20_flops_per_byte", DEV["H20"]["peak_flops"] / DEV["H20"]["peak_bytes_per_s"])
    h100 = oracle_tps("H100", orf.ABSORB, 8, 1)
    h20_gqa = oracle_tps("H20", orf.GQA, 8, 2)
    h20_mla = oracle_tps("H20", orf.ABSORB, 8, 1)
    near("h100_absorb_tokens_per_s", h100)
    near("h20_gqa_g8_sq2_tokens_per_s", h20_gqa)
    near("h20_mla_tokens_per_s", h20_mla)
    near("h20_gqa_over_mla", h20_gqa / h20_mla)
    # the absorbed form gains nothing from MTP on H20 (section 1, zero multi-token gain)
    assert oracle_tps("H20", orf.ABSORB, 8, 2) == pytest.approx(h20_mla, rel=1e-12)
    # and the per-token counts give the page's intensities
    near("absorb_intensity_sq1", orf.flops_per_token(orf.ABSORB, 128, 1, 512, 64, 128)
         / orf.cache_bytes_per_token(orf.ABSORB, 8, 512, 64, 128, 2))


@pytest.mark.parametrize("case", SEL["cases"], ids=lambda c: f"{c['device']}-g{c['g']}-sq{c['max_s_q']}")
def test_page_choices(case):
    d = DEV[case["device"]]
    want = orf.ABSORB if case["path"] == "absorb" else orf.GQA
    path, s_q, _, _ = orf.select_path(FLAG["h_q"], case["g"], case["max_s_q"], FLAG["r_kv"], FLAG["d_r"],
                                      FLAG["d_h"], FLAG["e"], 1, 8192, d["peak_flops"], d["peak_bytes_per_s"])
    assert (path, s_q) == (want, case["s_q"])
    sh = gqla.make_shape(128, case["g"], 512, 64, 128, case["max_s_q"])
    ch = gqla.select_path(sh, 1, 8192, d["peak_flops"], d["peak_bytes_per_s"])
    assert (ch.path, ch.s_q) == (want, case["s_q"])


def test_library_matches_oracle_on_a_grid():
    rng = np.random.default_rng(5)
    devices = [(d["peak_flops"], d["peak_bytes_per_s"]) for d in DEV.values()] + [(2.5e15, 8.0e12)]
    devices += [(10 ** rng.uniform(13, 16), 10 ** rng.uniform(11.5, 13.5)) for _ in range(12)]
    shapes = [(128, 8, 512, 64, 128), (32, 8, 512, 64, 128), (16, 2, 64, 16, 32), (64, 4, 256, 32, 64),
              (128, 1, 512, 64, 128), (128, 16, 512, 64, 128)]
    n = 0
    for flops, bw in devices:
        for h_q, g, r_kv, d_r, d_h in shapes:
            for max_sq in (1, 2, 3, 4):
                for dtype, e in ((gqla.BF16, 2), (gqla.F32, 4)):
                    batch, ctx = int(rng.integers(1, 300)), int(rng.integers(1, 10 ** 7))
                    want = orf.select_path(h_q, g, max_sq, r_kv, d_r, d_h, e, batch, ctx, flops, bw)
                    sh = gqla.make_shape(h_q, g, r_kv, d_r, d_h, max_sq, dtype=dtype)
                    got = gqla.select_path(sh, batch, ctx, flops, bw)
                    assert (got.path, got.s_q, bool(got.compute_bound)) == want[:2] + (want[3],), (flops, bw, h_q, g)
                    assert got.tokens_per_s == pytest.approx(want[2], rel=1e-12)
                    n += 1
    assert n > 500


def test_gqa_wins_where_absorb_is_compute_bound():
    """On a device whose ridge lies below the absorb intensity (H20), the GQA path at the
    same s_q always wins; on one above it at s_q = 1 (H100, MI355X), absorb does."""
    for max_sq in (1, 2):
        d = DEV["H20"]
        ch = gqla.select_path(gqla.make_shape(128, 8, 512, 64, 128, max_sq), 64, 8192 * 64, d["peak_flops"],
                              d["peak_bytes_per_s"])
        assert ch.path == gqla.GQA
    for flops, bw in ((DEV["H100"]["peak_flops"], DEV["H100"]["peak_bytes_per_s"]), (2.5e15, 8.0e12)):
        ch = gqla.select_path(gqla.make_shape(128, 8, 512, 64, 128, 1), 64, 8192 * 64, flops, bw)
        assert ch.path == gqla.ABSORB and ch.s_q == 1 and not ch.compute_bound


def test_selector_validation():
    sh = gqla.make_shape(128, 8, 512, 64, 128, 1)
    L = gqla.load()
    ch = gqla.PathChoice()
    import ctypes
    assert L.gqla_select_path(ctypes.byref(sh), 0, 10, 1e15, 1e12, ctypes.byref(ch)) == 1
    assert L.gqla_select_path(ctypes.byref(sh), 1, 0, 1e15, 1e12, ctypes.byref(ch)) == 1
    assert L.gqla_select_path(ctypes.byref(sh), 1, 10, -1.0, 1e12, ctypes.byref(ch)) == 1
    assert L.gqla_select_path(ctypes.byref(sh), 1, 10, 1e15, math.inf, ctypes.byref(ch)) == 1
    assert L.gqla_select_path(ctypes.byref(sh), 1, 10, 1e15, 1e12, None) == 1
    assert L.gqla_select_path(ctypes.byref(gqla.make_shape(128, 7, 512, 64, 128, 1)), 1, 10, 1e15, 1e12,
                              ctypes.byref(ch)) == 1
    assert L.gqla_measure_peaks(None, 1 << 30, ctypes.byref(ctypes.c_double()), ctypes.byref(ctypes.c_double()),
                                None) == 1
    assert L.gqla_measure_peaks(0x10000, 1 << 20, ctypes.byref(ctypes.c_double()), ctypes.byref(ctypes.c_double()),
                                None) == 1
