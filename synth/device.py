"""Upload seeded synthetic workloads into device tensors (no method arithmetic).

The arrays come from ``synth.inputs`` (float32 holding values exactly
representable in the storage dtype), so converting them to torch.bfloat16 is
exact and the device path sees bit-identical inputs to the oracle.  Sequences
are generated independently (per-sequence seeds) on a thread pool and copied
one at a time, so a large workload never needs its whole cache in host memory.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

from .inputs import GQLAConfig, ctx_lens, latent_rows, queries, up_weights


@dataclasses.dataclass
class DeviceWorkload:
    cfg: GQLAConfig
    lens: np.ndarray          # int32 [B], host copy
    max_ctx: int
    ctx_lens: object          # torch int32 [B] on device
    latent: object            # torch [B][max_ctx][r_kv + d_R], rows >= L_b are zero
    q_nope: object            # torch [B][s_q][h_q][d_h]
    q_rope: object            # torch [B][s_q][h_q][d_R]
    w_uk: object              # torch [g][d_h][r_kv]
    w_uv: object

    @property
    def dtype(self):
        return self.latent.dtype


def torch_dtype(cfg: GQLAConfig):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[cfg.dtype]


def host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def make_workload(cfg: GQLAConfig, device="cuda", lens: Optional[Sequence[int]] = None,
                  max_ctx: Optional[int] = None, threads: Optional[int] = None) -> DeviceWorkload:
    """Seeded workload on ``device``.  ``lens`` overrides the drawn context lengths;
    ``max_ctx`` (>= max length) sets the row capacity per sequence."""
    import torch

    dt = torch_dtype(cfg)
    lens = np.asarray(ctx_lens(cfg) if lens is None else lens, dtype=np.int32)
    assert lens.shape == (cfg.batch,)
    cap = int(max_ctx if max_ctx is not None else max(int(lens.max(initial=0)), 1))
    assert cap >= int(lens.max(initial=0))
    width = cfg.r_kv + cfg.d_r
    latent = torch.zeros((cfg.batch, cap, width), dtype=dt, device=device)

    def gen(b):
        return b, latent_rows(cfg, b, int(lens[b]))

    with cf.ThreadPoolExecutor(max_workers=threads or host_threads()) as ex:
        for b, rows in ex.map(gen, range(cfg.batch)):
            if rows.shape[0]:
                latent[b, : rows.shape[0]].copy_(torch.from_numpy(rows).to(dt))
    qn, qr = queries(cfg)
    w_uk, w_uv = up_weights(cfg)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(device)  # noqa: E731
    return DeviceWorkload(cfg=cfg, lens=lens, max_ctx=cap,
                          ctx_lens=torch.from_numpy(lens.copy()).to(device),
                          latent=latent, q_nope=to(qn), q_rope=to(qr), w_uk=to(w_uk), w_uv=to(w_uv))
