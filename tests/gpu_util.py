"""Helpers of the GPU parity tests: run the HIP path through the C-ABI binding and
compare with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import numpy as np

import oracle
import synth
from synth.device import make_workload

# Tolerances (|gpu - oracle| <= atol + rtol |oracle|): bf16 storage, fp32 accumulation.
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}


def torch_mod():
    import torch
    return torch


def shape_of(cfg, gqla):
    return gqla.make_shape(cfg.h_q, cfg.g, cfg.r_kv, cfg.d_r, cfg.d_h, cfg.s_q, cfg.scale,
                           gqla.BF16 if cfg.dtype == "bf16" else gqla.F32)


def run_absorb(w, gqla, num_splits=0, workspace=None, poison=True):
    torch = torch_mod()
    cfg = w.cfg
    sh = shape_of(cfg, gqla)
    out = torch.empty((cfg.batch, cfg.s_q, cfg.h_q, cfg.d_h), dtype=w.dtype, device=w.latent.device)
    lse = torch.empty((cfg.batch, cfg.s_q, cfg.h_q), dtype=torch.float32, device=w.latent.device)
    if poison:
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    if workspace is None:
        workspace = gqla.alloc_workspace(sh, gqla.ABSORB, cfg.batch, w.max_ctx, num_splits, w.latent.device)
        if poison and workspace.numel() % 4 == 0:
            workspace.view(torch.float32).fill_(float("nan"))
    gqla.decode_absorb(sh, w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.latent, w.ctx_lens, out, lse, workspace, num_splits)
    return out, lse


def expand(w, gqla, group_cache=None, row_begin=0):
    torch = torch_mod()
    cfg = w.cfg
    sh = shape_of(cfg, gqla)
    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    if group_cache is None:
        group_cache = torch.zeros((cfg.batch, w.max_ctx, width), dtype=w.dtype, device=w.latent.device)
    gqla.expand_groups(sh, w.latent, w.w_uk, w.w_uv, w.ctx_lens, group_cache, row_begin)
    return group_cache


def run_gqa(w, gqla, group_cache, num_splits=0, poison=True):
    torch = torch_mod()
    cfg = w.cfg
    sh = shape_of(cfg, gqla)
    out = torch.empty((cfg.batch, cfg.s_q, cfg.h_q, cfg.d_h), dtype=w.dtype, device=w.latent.device)
    lse = torch.empty((cfg.batch, cfg.s_q, cfg.h_q), dtype=torch.float32, device=w.latent.device)
    ws = gqla.alloc_workspace(sh, gqla.GQA, cfg.batch, w.max_ctx, num_splits, w.latent.device)
    if poison:
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        if ws.numel() % 4 == 0:
            ws.view(torch.float32).fill_(float("nan"))
    gqla.decode_gqa(sh, w.q_nope, w.q_rope, group_cache, w.ctx_lens, out, lse, ws, num_splits)
    return out, lse


def host(t):
    return t.float().cpu().numpy()


def oracle_seq(cfg, b, length, q_nope, q_rope, w_uk, w_uv):
    """fp64 oracle output (o [s_q][h_q][d_h], lse [s_q][h_q]) for sequence b."""
    rows = synth.latent_rows(cfg, b, length)
    return oracle.textbook_decode(rows, q_nope[b], q_rope[b], w_uk, w_uv, length, cfg.scale)


def stored_group_rows(cfg, b, length):
    """The oracle's fp64 expansion of sequence b rounded once to the storage dtype:
    the rows a group cache holds, [L][2 g d_h + d_R] float32."""
    w_uk, w_uv = synth.up_weights(cfg)
    gr = oracle.expand_groups(synth.latent_rows(cfg, b, length), w_uk, w_uv)
    return synth.bf16_round(gr) if cfg.dtype == "bf16" else gr.astype(np.float32)


def upload_stored_group_cache(w):
    """Device group cache [B][max_ctx][width] holding stored_group_rows of every sequence."""
    torch = torch_mod()
    cfg = w.cfg
    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    gc = torch.zeros((cfg.batch, w.max_ctx, width), dtype=w.dtype, device=w.latent.device)
    rows = {}
    for b in range(cfg.batch):
        L = int(w.lens[b])
        rows[b] = stored_group_rows(cfg, b, L)
        if L:
            gc[b, :L].copy_(torch.from_numpy(rows[b]).to(w.dtype))
    return gc, rows


def gqa_reference(cfg, rows):
    """Reference of the GQA decode entry point: the oracle's GQA form over the stored rows."""
    qn, qr = synth.queries(cfg)

    def ref(b, length):
        return oracle.gqa_decode(rows[b], qn[b], qr[b], cfg.g, length, cfg.scale)
    return ref


def compare(cfg, out, lse, seqs, lens, what="", ref=None):
    """Element-wise comparison of device outputs against the oracle on the listed sequences.
    ref(b, L) -> (o, lse) overrides the default reference (the textbook definition)."""
    rtol, atol = TOL[cfg.dtype]
    qn, qr = synth.queries(cfg)
    w_uk, w_uv = synth.up_weights(cfg)
    o_dev, l_dev = host(out), host(lse)
    worst = 0.0
    for b in seqs:
        if ref is None:
            o_ref, l_ref = oracle_seq(cfg, b, int(lens[b]), qn, qr, w_uk, w_uv)
        else:
            o_ref, l_ref = ref(b, int(lens[b]))
        got = o_dev[b].astype(np.float64)
        assert np.all(np.isfinite(got)), f"{what} b={b}: non-finite output"
        err = np.abs(got - o_ref)
        lim = atol + rtol * np.abs(o_ref)
        ratio = float(np.max(err / lim)) if err.size else 0.0
        worst = max(worst, ratio)
        assert ratio <= 1.0, (f"{what} b={b} L={lens[b]}: max |err|/tol = {ratio:.3f}, "
                              f"max err {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}")
        # lse: same tolerance form on the natural-log value; -inf where nothing is visible
        lr = l_dev[b].astype(np.float64)
        fin = np.isfinite(l_ref)
        assert np.array_equal(np.isfinite(lr), fin), f"{what} b={b}: lse finiteness differs"
        assert np.all(lr[~fin] == -np.inf)
        if fin.any():
            lerr = np.abs(lr[fin] - l_ref[fin])
            assert np.all(lerr <= atol + rtol * np.abs(l_ref[fin])), f"{what} b={b}: lse max err {lerr.max():.3e}"
    return worst


def workload(cfg, lens=None, max_ctx=None):
    return make_workload(cfg, device="cuda", lens=lens, max_ctx=max_ctx)
