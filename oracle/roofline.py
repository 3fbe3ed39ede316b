"""Roofline path selection of GQLA decode (test infrastructure only).

Source: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM Decoding"
(gist.science explainer page), technical summary section 1 (Problem: the ridge
points of the two devices, about 295 and 37 FLOPs per byte), section 2
(Architecture: the intensity of the absorb path at s_q = 1; the GQA path's
intensity tuned through g and s_q; Path selection: the runtime picks the path per
device) and section 4 (Results: the throughput projections).

The page states the rule by its outcome (absorb on the device whose ridge sits just
above the absorb intensity, GQA on the device whose ridge is about 37) and the
projections by their values; the model that reproduces them is the plain roofline
of one attention layer in which every query token reads the whole cache once:

* absorb: bytes e (r_kv + d_R), flops 2 s_q h_q (2 r_kv + d_R) per cached token;
* GQA:    bytes e (2 g d_h + d_R), flops 2 s_q h_q (2 d_h + d_R) per cached token;
* a step over contexts summing to T takes max(bytes T / BW, flops T / F) and yields
  B s_q query tokens;
* the selected configuration is the (path, s_q) with the most query tokens per
  second, s_q ranging over 1 .. the most tokens the model proposes per step.

Reading where the page is silent: on equal throughput the smaller s_q wins (fewer
speculative tokens), then the absorb path (the smaller cache).
"""
from __future__ import annotations

from typing import Tuple

ABSORB, GQA = 0, 1


def cache_bytes_per_token(path: int, g: int, r_kv: int, d_r: int, d_h: int, e: int) -> int:
    return e * (r_kv + d_r) if path == ABSORB else e * (2 * g * d_h + d_r)


def flops_per_token(path: int, h_q: int, s_q: int, r_kv: int, d_r: int, d_h: int) -> int:
    return 2 * s_q * h_q * (2 * r_kv + d_r) if path == ABSORB else 2 * s_q * h_q * (2 * d_h + d_r)


def step_tokens_per_s(path: int, h_q: int, g: int, s_q: int, r_kv: int, d_r: int, d_h: int, e: int,
                      batch: int, total_ctx: int, peak_flops: float, peak_bw: float) -> Tuple[float, bool]:
    """(query tokens/s, compute-bound?) of one decode step under the roofline."""
    t_mem = cache_bytes_per_token(path, g, r_kv, d_r, d_h, e) * total_ctx / peak_bw
    t_cmp = flops_per_token(path, h_q, s_q, r_kv, d_r, d_h) * total_ctx / peak_flops
    t = max(t_mem, t_cmp)
    return (batch * s_q / t if t > 0 else float("inf")), t_cmp > t_mem


def select_path(h_q: int, g: int, max_s_q: int, r_kv: int, d_r: int, d_h: int, e: int,
                batch: int, total_ctx: int, peak_flops: float, peak_bw: float):
    """(path, s_q, tokens/s, compute-bound?) with the most query tokens per second."""
    best = None
    for s_q in range(1, max_s_q + 1):
        for path in (ABSORB, GQA):
            tps, comp = step_tokens_per_s(path, h_q, g, s_q, r_kv, d_r, d_h, e, batch, total_ctx,
                                          peak_flops, peak_bw)
            if best is None or tps > best[2]:
                best = (path, s_q, tps, comp)
    return best
