"""Roofline model of GQLA decode (host logic, no device code).

Source: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
Decoding", technical summary section 1 (ridge points of the two devices),
section 2 (arithmetic intensity of the absorb path at s_q = 1 and of the GQA
path tuned through g and s_q) and section 4 (throughput projections).  The page
prints the numbers but not the formulas; the per-token counts below are the
plain ones for one attention layer in which every query token reads the whole
cache once:

* absorb path:  bytes = e (r_kv + d_R) per cached token;
                flops = 2 s_q h_q (2 r_kv + d_R) per cached token
                (score over r_kv + d_R, latent accumulation over r_kv);
* GQA path:     bytes = e (2 g d_h + d_R) per cached token;
                flops = 2 s_q h_q (2 d_h + d_R) per cached token.

A step over context L takes max(bytes L / BW, flops L / F); throughput is
s_q / time query tokens per second per sequence.  Whole-step algorithmic bytes
for a batch add the queries, outputs and (absorb) the up-projection weights.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Device:
    name: str
    flops: float      # dense peak, FLOP/s, in the contraction dtype
    bw: float         # HBM bytes/s

    @property
    def ridge(self) -> float:
        return self.flops / self.bw


# Public spec values (not printed on the page).  H100 SXM dense bf16 and
# 3.35 TB/s; H20 dense bf16 and 4.0 TB/s; MI355X dense bf16 MFMA and HBM3E.
H100 = Device("H100", 989.4e12, 3.35e12)
H20 = Device("H20", 148e12, 4.0e12)
MI355X = Device("MI355X", 2.5e15, 8.0e12)
MI355X_FP32_MFMA = 157.3e12


def absorb_bytes_per_token(r_kv: int, d_r: int, e: int = 2) -> int:
    return e * (r_kv + d_r)


def absorb_flops_per_token(h_q: int, s_q: int, r_kv: int, d_r: int) -> int:
    return 2 * s_q * h_q * (2 * r_kv + d_r)


def gqa_bytes_per_token(g: int, d_h: int, d_r: int, e: int = 2) -> int:
    return e * (2 * g * d_h + d_r)


def gqa_flops_per_token(h_q: int, s_q: int, d_h: int, d_r: int) -> int:
    return 2 * s_q * h_q * (2 * d_h + d_r)


def intensity(path: str, h_q: int, g: int, s_q: int, r_kv: int = 512, d_r: int = 64,
              d_h: int = 128, e: int = 2) -> float:
    if path == "absorb":
        return absorb_flops_per_token(h_q, s_q, r_kv, d_r) / absorb_bytes_per_token(r_kv, d_r, e)
    if path == "gqa":
        return gqa_flops_per_token(h_q, s_q, d_h, d_r) / gqa_bytes_per_token(g, d_h, d_r, e)
    raise ValueError(path)


def tokens_per_s(dev: Device, path: str, h_q: int, g: int, s_q: int, ctx: int,
                 r_kv: int = 512, d_r: int = 64, d_h: int = 128, e: int = 2) -> float:
    """Query tokens/s of one sequence whose step reads ``ctx`` cached tokens (cache traffic only)."""
    if path == "absorb":
        by = absorb_bytes_per_token(r_kv, d_r, e) * ctx
        fl = absorb_flops_per_token(h_q, s_q, r_kv, d_r) * ctx
    else:
        by = gqa_bytes_per_token(g, d_h, d_r, e) * ctx
        fl = gqa_flops_per_token(h_q, s_q, d_h, d_r) * ctx
    return s_q / max(by / dev.bw, fl / dev.flops)


def cache_ratio(r_kv: int, d_r: int, n_kv: int, d_h: int) -> float:
    """Absorb-row cache size over the original GQA cache (2 n_kv d_h per token)."""
    return (r_kv + d_r) / (2 * n_kv * d_h)


@dataclasses.dataclass(frozen=True)
class StepWork:
    bytes: float   # algorithmic HBM bytes of one decode step (whole batch)
    flops: float   # algorithmic FLOPs of one decode step (whole batch)


def step_work(path: str, h_q: int, g: int, s_q: int, total_ctx: int, batch: int,
              r_kv: int = 512, d_r: int = 64, d_h: int = 128, e: int = 2) -> StepWork:
    """Algorithmic bytes and flops of one decode step over a batch whose contexts sum to total_ctx.

    Cache rows are read once; q is read and o written once per (sequence,
    query token, head); the absorb path also reads W_UK and W_UV once and
    spends 2 * 2 s_q h_q d_h r_kv flops per sequence on the query absorption
    and the output up-projection.
    """
    q_out = batch * s_q * h_q * (d_h + d_r + d_h) * e
    if path == "absorb":
        cache = absorb_bytes_per_token(r_kv, d_r, e) * total_ctx
        w = 2 * g * d_h * r_kv * e
        fl = absorb_flops_per_token(h_q, s_q, r_kv, d_r) * total_ctx + batch * 4 * s_q * h_q * d_h * r_kv
        return StepWork(cache + q_out + w, fl)
    cache = gqa_bytes_per_token(g, d_h, d_r, e) * total_ctx
    fl = gqa_flops_per_token(h_q, s_q, d_h, d_r) * total_ctx
    return StepWork(cache + q_out, fl)


def roofline_tokens_per_s(dev: Device, work: StepWork, query_tokens: int) -> float:
    return query_tokens / max(work.bytes / dev.bw, work.flops / dev.flops)
