"""Seeded synthetic workloads for GQLA decode attention.

The workload table mirrors the five decode configurations used for parity and
measurement (tiny fp32; the LLaMA-3-8B-derived TransGQLA shape; the h_q=128,
g=8 flagship; the multi-token step with ragged contexts; the long-context
split-K case).  The shapes follow "GQLA: Group-Query Latent Attention for
Hardware-Adaptive LLM Decoding", technical summary section 2 (Architecture):
group-indexed up-projections W_UK / W_UV over g groups, a latent cache of width
r_kv plus one shared RoPE key of width d^R_h per token, and a per-group key /
value width d_h.

Every array is produced per sequence from ``SeedSequence([cfg_id, tag, b])`` so
that any single sequence can be regenerated on its own (the oracle checks
sampled sequences of the large workloads this way).  Tags:

    0 context lengths   1 latent cKV    2 RoPE key k_R   3 query input x
    4 W_UK              5 W_UV          6 W_q

Weights use ``b := g`` so that a configuration run at two group counts draws
two different weight sets.

Value distributions (input recipe, not method arithmetic):

* cKV ~ N(0, 1); for the bf16 workloads each token's latent row is divided by
  its root-mean-square over r_kv (eps 1e-6, no learned gain).
* k_R ~ N(0, 1).  The decode operator consumes keys and queries after the
  rotary embedding has been applied.  A rotation of a pair of i.i.d. standard
  normals is again a pair of i.i.d. standard normals, so the draw stands in for
  the rotated key directly.
* W_UK, W_UV ~ N(0, 1/r_kv) (fan-in r_kv), shape [g][d_h][r_kv].
* queries: q = W_q x with x ~ N(0, 1)^{d_model}, d_model := r_kv and
  W_q ~ N(0, 1/d_model) of shape [h_q (d_h + d_R)] x d_model.  The first d_h
  entries of each head's slice are q^N, the last d_R are q^R (again standing
  in for the rotated value).
* draws are made in float64 and rounded once to the storage dtype (bf16 with
  round-to-nearest-even, or fp32).  Arrays are returned as float32 holding
  exactly representable values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

TAG_LENS, TAG_LATENT, TAG_KROPE, TAG_X, TAG_WUK, TAG_WUV, TAG_WQ = range(7)


@dataclasses.dataclass(frozen=True)
class GQLAConfig:
    """One decode workload.  ``ctx`` is a fixed length or an inclusive range."""

    cfg_id: int
    name: str
    dtype: str            # "f32" or "bf16"
    batch: int
    h_q: int
    g: int
    r_kv: int
    d_r: int
    d_h: int
    s_q: int
    ctx: Tuple[int, int]  # inclusive [lo, hi]; lo == hi for uniform contexts
    rms_norm: bool

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h + self.d_r)

    @property
    def max_ctx(self) -> int:
        return self.ctx[1]

    @property
    def heads_per_group(self) -> int:
        return self.h_q // self.g

    def with_(self, **kw) -> "GQLAConfig":
        return dataclasses.replace(self, **kw)


# The five decode workloads.  Config 4 runs three variants (GQA g=8 s_q=2,
# GQA g=4 s_q=1, absorb s_q=2); its g and s_q are set per variant with with_().
CONFIGS = {
    1: GQLAConfig(1, "tiny-fp32", "f32", 1, 16, 2, 64, 16, 32, 1, (256, 256), False),
    2: GQLAConfig(2, "llama3-8b-transgqla", "bf16", 64, 32, 8, 512, 64, 128, 1, (4096, 4096), True),
    3: GQLAConfig(3, "flagship-hq128-g8-ctx8k", "bf16", 128, 128, 8, 512, 64, 128, 1, (8192, 8192), True),
    4: GQLAConfig(4, "multi-token-ragged", "bf16", 256, 128, 8, 512, 64, 128, 2, (1024, 32768), True),
    5: GQLAConfig(5, "long-context-splitk", "bf16", 16, 128, 8, 512, 64, 128, 1, (65536, 131072), True),
}


def config(cfg_id: int, **overrides) -> GQLAConfig:
    c = CONFIGS[cfg_id]
    return c.with_(**overrides) if overrides else c


def _rng(cfg_id: int, tag: int, idx: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(tag), int(idx)]))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bfloat16 (round to nearest, ties to even).

    Values are first rounded to float32 (RNE), then the low 16 bits of the
    float32 pattern are rounded away (RNE).  Returns float32 holding the bf16
    values exactly.  NaN and inf are not expected in the draws.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def _store(cfg: GQLAConfig, x: np.ndarray) -> np.ndarray:
    if cfg.dtype == "bf16":
        return bf16_round(x)
    if cfg.dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(cfg.dtype)


def ctx_len(cfg: GQLAConfig, b: int) -> int:
    """Context length of sequence b: ctx[0] when uniform, else a seeded uniform integer on ctx (inclusive)."""
    lo, hi = cfg.ctx
    return lo if lo == hi else int(_rng(cfg.cfg_id, TAG_LENS, b).integers(lo, hi + 1))


def ctx_lens(cfg: GQLAConfig) -> np.ndarray:
    """Per-sequence context lengths, int32 [B]."""
    return np.array([ctx_len(cfg, b) for b in range(cfg.batch)], dtype=np.int32)


def latent_rows(cfg: GQLAConfig, b: int, length: Optional[int] = None) -> np.ndarray:
    """Latent cache rows of sequence b: float32 [L_b][r_kv + d_R] = [cKV | k_R]."""
    if length is None:
        length = ctx_len(cfg, b)
    c = _rng(cfg.cfg_id, TAG_LATENT, b).standard_normal((length, cfg.r_kv))
    if cfg.rms_norm:
        c = c / np.sqrt(np.mean(c * c, axis=1, keepdims=True) + 1e-6)
    k = _rng(cfg.cfg_id, TAG_KROPE, b).standard_normal((length, cfg.d_r))
    rows = np.empty((length, cfg.r_kv + cfg.d_r), dtype=np.float32)
    rows[:, : cfg.r_kv] = _store(cfg, c)
    rows[:, cfg.r_kv:] = _store(cfg, k)
    return rows


def query_weights(cfg: GQLAConfig) -> np.ndarray:
    """W_q ~ N(0, 1/d_model), float64 [h_q (d_h + d_R)][d_model], d_model := r_kv."""
    d_model = cfg.r_kv
    w = _rng(cfg.cfg_id, TAG_WQ, cfg.g).standard_normal((cfg.h_q * (cfg.d_h + cfg.d_r), d_model))
    return w / math.sqrt(d_model)


def queries(cfg: GQLAConfig, seqs: Optional[Sequence[int]] = None,
            w_q: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(q_nope [n][s_q][h_q][d_h], q_rope [n][s_q][h_q][d_R]) for the listed sequences."""
    if seqs is None:
        seqs = range(cfg.batch)
    seqs = list(seqs)
    if w_q is None:
        w_q = query_weights(cfg)
    x = np.stack([_rng(cfg.cfg_id, TAG_X, b).standard_normal((cfg.s_q, cfg.r_kv)) for b in seqs])
    q = (x.reshape(-1, cfg.r_kv) @ w_q.T).reshape(len(seqs), cfg.s_q, cfg.h_q, cfg.d_h + cfg.d_r)
    q_nope = _store(cfg, q[..., : cfg.d_h]).reshape(len(seqs), cfg.s_q, cfg.h_q, cfg.d_h)
    q_rope = _store(cfg, q[..., cfg.d_h:]).reshape(len(seqs), cfg.s_q, cfg.h_q, cfg.d_r)
    return q_nope, q_rope


def up_weights(cfg: GQLAConfig) -> Tuple[np.ndarray, np.ndarray]:
    """(W_UK, W_UV), each float32 [g][d_h][r_kv], N(0, 1/r_kv) rounded to the storage dtype."""
    s = 1.0 / math.sqrt(cfg.r_kv)
    w_uk = _rng(cfg.cfg_id, TAG_WUK, cfg.g).standard_normal((cfg.g, cfg.d_h, cfg.r_kv)) * s
    w_uv = _rng(cfg.cfg_id, TAG_WUV, cfg.g).standard_normal((cfg.g, cfg.d_h, cfg.r_kv)) * s
    return _store(cfg, w_uk), _store(cfg, w_uv)


def sample_sequences(cfg: GQLAConfig, n: int, seed: int = 0) -> List[int]:
    """A deterministic sample of sequence indices: first, last, and n-2 seeded others."""
    if cfg.batch <= n:
        return list(range(cfg.batch))
    rest = np.random.default_rng(np.random.SeedSequence([cfg.cfg_id, 99, seed])).choice(
        np.arange(1, cfg.batch - 1), size=n - 2, replace=False)
    return sorted({0, cfg.batch - 1, *map(int, rest)})
