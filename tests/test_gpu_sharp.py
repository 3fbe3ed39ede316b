"""Parity with sharp softmaxes and at the edges of the operand range, through the C-ABI
(MI355X only).

Every decode path must meet |gpu - oracle| <= 2e-3 + 2e-2 |oracle| on the same inputs,
however peaked the attention is: the page's two decode paths are algebraically equal
("GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM Decoding", technical
summary section 2, Architecture), so their results differ from the definition only by
rounding, and the bound is written for bf16 storage, not for a particular logit range.

Sequence b of a batch gets input kind b % 4 (seeded rows of the workload, then):
  0  latent rows scaled by a ramp 0.1 -> 6 over the last 70 % of the context (peak logits
     around 30-35 in log2 units), so the online softmax's reference rises many times;
  1  a jump: rows scaled 0.15 up to 40 % of the context, 6 after it;
  2  unscaled rows, queries x 4;
  3  unscaled rows, queries x 8 (peak logits near 40 in log2 units).
The absorb path is compared with the textbook definition; the GQA and sparse paths with
the oracle's GQA form over the stored (bf16-rounded) expanded rows they read.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def gqla():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from latent_kv_cache_amd import gqla as mod
    mod.load()
    return mod


def row_scale(kind, L):
    t = np.arange(L, dtype=np.float64)
    if kind == 0:
        a = int(0.3 * L)
        return np.where(t < a, 0.1, 0.1 + 5.9 * (t - a) / max(L - a, 1))
    if kind == 1:
        return np.where(t < int(0.4 * L), 0.15, 6.0)
    return np.ones(L)


def sharp_workload(cfg, lens, kinds=None, latent_scale=None):
    """Device workload with the rows and queries of the kinds above (or every row scaled by
    latent_scale); returns (workload, host rows per sequence, q_nope, q_rope)."""
    torch = gu.torch_mod()
    w = gu.workload(cfg, lens=lens)
    qn, qr = synth.queries(cfg)
    qn, qr = qn.astype(np.float64), qr.astype(np.float64)
    rows = {}
    for b, L in enumerate(lens):
        kind = (b % 4) if kinds is None else kinds[b]
        base = synth.latent_rows(cfg, b, L).astype(np.float64)
        f = row_scale(kind, L) if latent_scale is None else np.full(L, latent_scale)
        rows[b] = synth.bf16_round(base * f[:, None])
        if L:
            w.latent[b, :L].copy_(torch.from_numpy(rows[b]).to(w.dtype))
        if latent_scale is None and kind >= 2:
            m = 4.0 if kind == 2 else 8.0
            qn[b] = synth.bf16_round(qn[b] * m)
            qr[b] = synth.bf16_round(qr[b] * m)
    qn, qr = qn.astype(np.float32), qr.astype(np.float32)
    w.q_nope.copy_(torch.from_numpy(qn).to(w.dtype))
    w.q_rope.copy_(torch.from_numpy(qr).to(w.dtype))
    return w, rows, qn, qr


def stored_cache(cfg, w, rows):
    torch = gu.torch_mod()
    w_uk, w_uv = synth.up_weights(cfg)
    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    gc = torch.zeros((cfg.batch, w.max_ctx, width), dtype=w.dtype, device="cuda")
    stored = {}
    for b, L in enumerate(w.lens):
        stored[b] = synth.bf16_round(oracle.expand_groups(rows[b], w_uk, w_uv))
        if L:
            gc[b, :L].copy_(torch.from_numpy(stored[b]).to(w.dtype))
    return gc, stored


def check_absorb(cfg, gqla, w, rows, qn, qr, num_splits, what):
    w_uk, w_uv = synth.up_weights(cfg)
    note(f"{what} absorb h_q={cfg.h_q} g={cfg.g} s_q={cfg.s_q} lens={list(w.lens)} splits={num_splits}")
    out, lse = gu.run_absorb(w, gqla, num_splits)
    return gu.compare(cfg, out, lse, list(range(cfg.batch)), w.lens, f"{what} absorb",
                      ref=lambda b, L: oracle.textbook_decode(rows[b], qn[b], qr[b], w_uk, w_uv, L, cfg.scale))


def check_gqa(cfg, gqla, w, rows, qn, qr, num_splits, what):
    gc, stored = stored_cache(cfg, w, rows)
    note(f"{what} gqa g={cfg.g} s_q={cfg.s_q} lens={list(w.lens)} splits={num_splits}")
    out, lse = gu.run_gqa(w, gqla, gc, num_splits)
    return gu.compare(cfg, out, lse, list(range(cfg.batch)), w.lens, f"{what} gqa",
                      ref=lambda b, L: oracle.gqa_decode(stored[b], qn[b], qr[b], cfg.g, L, cfg.scale))


# Absorb workgroups hold 16, 32, 48 or 64 query rows (s_q * h_q rows per sequence, in
# blocks of at most 64): every block size, one and several blocks per sequence.
@pytest.mark.parametrize("h_q,g,s_q,splits", [
    (128, 8, 1, 0),     # flagship shape: two 64-row blocks, one chunk per sequence
    (128, 8, 2, 3),     # four 64-row blocks, three chunks (split-K combine)
    (32, 8, 1, 0),      # one 32-row block (four heads per group)
    (16, 2, 3, 2),      # one 48-row block, three query tokens
    (16, 1, 1, 0),      # one 16-row block (g = 1: every head in one group)
    (48, 4, 2, 0),      # 96 rows: a 64-row block and a 32-row remainder
])
def test_sharp_absorb(gqla, h_q, g, s_q, splits):
    cfg = synth.config(3, g=g, s_q=s_q).with_(batch=4, h_q=h_q)
    w, rows, qn, qr = sharp_workload(cfg, [1000, 1000, 1000, 1000])
    check_absorb(cfg, gqla, w, rows, qn, qr, splits, "sharp")


@pytest.mark.parametrize("g,s_q,splits", [(8, 1, 0), (8, 2, 3), (4, 1, 0), (4, 2, 2), (2, 1, 1)])
def test_sharp_gqa(gqla, g, s_q, splits):
    cfg = synth.config(3, g=g, s_q=s_q).with_(batch=4)
    w, rows, qn, qr = sharp_workload(cfg, [1000, 1000, 1000, 1000])
    check_gqa(cfg, gqla, w, rows, qn, qr, splits, "sharp")


@pytest.mark.parametrize("s_q", [1, 2])
def test_sharp_sparse(gqla, s_q):
    """Sparse decode over 320 listed rows per (sequence, token, group): the last 64 rows of
    the context (where the ramp and the jump put the largest scores) plus 256 others."""
    torch = gu.torch_mod()
    cfg = synth.config(3, s_q=s_q).with_(batch=4)
    lens = [1000, 1000, 1000, 1000]
    w, rows, qn, qr = sharp_workload(cfg, lens)
    gc, stored = stored_cache(cfg, w, rows)
    rng = np.random.default_rng(11 + s_q)
    topk = 320
    idx = np.empty((cfg.batch, cfg.s_q, cfg.g, topk), dtype=np.int32)
    for b, L in enumerate(lens):
        for s in range(cfg.s_q):
            for j in range(cfg.g):
                idx[b, s, j, :64] = np.arange(L - 64, L)
                idx[b, s, j, 64:] = rng.choice(L - 64, size=topk - 64, replace=False)
    sh = gu.shape_of(cfg, gqla)
    out = torch.full((cfg.batch, cfg.s_q, cfg.h_q, cfg.d_h), float("nan"), dtype=w.dtype, device="cuda")
    lse = torch.full((cfg.batch, cfg.s_q, cfg.h_q), float("nan"), dtype=torch.float32, device="cuda")
    note(f"sharp sparse s_q={s_q} topk={topk}")
    gqla.decode_gqa_sparse(sh, w.q_nope, w.q_rope, gc, w.ctx_lens, torch.from_numpy(idx).cuda(), out, lse)
    gu.compare(cfg, out, lse, list(range(cfg.batch)), w.lens, "sharp sparse",
               ref=lambda b, L: oracle.sparse_gqa_decode(stored[b], qn[b], qr[b], cfg.g, idx[b], L, cfg.scale))


# Operand range.  Some products run on fp16 copies of the bf16 inputs (the GQA path's
# queries and expanded rows, the absorb path's latent rows in u): exact for magnitudes in
# fp16's normal range [2^-14, 65504]; smaller values keep fp16's subnormal spacing 2^-24.
#   Small values: latent rows of RMS 1e-4 and 1e-5 (mostly below 2^-14) meet the bound
#   as it is written (their outputs are small; the absolute term covers the subnormal
#   rounding).
#   Large values: latent rows scaled by S = 2^11 (values up to about 1e4, expanded rows
#   alike) and queries by 1/S leave every logit unchanged, and the method is then linear
#   in S: o(S c, q / S) = S o(c, q).  The outputs are compared as o / S (exact: S is a
#   power of two) with the bound as written, the reading of the bound that does not
#   depend on the unit of the values.  (Compared unscaled, the absolute term 2e-3 would
#   ask for 2^-20 of the data's own scale wherever o cancels to near zero, finer than
#   the fp32 accumulation of any decode kernel.)
@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("scale", [1e-4, 1e-5])
def test_operand_range_small(gqla, scale, s_q):
    cfg = synth.config(3, s_q=s_q).with_(batch=2)
    w, rows, qn, qr = sharp_workload(cfg, [700, 333], latent_scale=scale)
    check_absorb(cfg, gqla, w, rows, qn, qr, 0, f"range {scale:g}")
    check_gqa(cfg, gqla, w, rows, qn, qr, 0, f"range {scale:g}")


@pytest.mark.parametrize("s_q", [1, 2])
def test_operand_range_large(gqla, s_q):
    torch = gu.torch_mod()
    S = 2.0 ** 11
    cfg = synth.config(3, s_q=s_q).with_(batch=2)
    w, rows, qn, qr = sharp_workload(cfg, [700, 333], latent_scale=S)
    qn = (qn.astype(np.float64) / S).astype(np.float32)
    qr = (qr.astype(np.float64) / S).astype(np.float32)
    w.q_nope.copy_(torch.from_numpy(qn).to(w.dtype))
    w.q_rope.copy_(torch.from_numpy(qr).to(w.dtype))
    assert max(float(np.abs(r).max()) for r in rows.values()) > 5e3
    w_uk, w_uv = synth.up_weights(cfg)
    note(f"range x{S:g} absorb s_q={s_q}")
    out, lse = gu.run_absorb(w, gqla, 0)

    def ref_a(b, L):
        o, l = oracle.textbook_decode(rows[b], qn[b], qr[b], w_uk, w_uv, L, cfg.scale)
        return o / S, l
    gu.compare(cfg, out / S, lse, [0, 1], w.lens, f"range x{S:g} absorb", ref=ref_a)
    gc, stored = stored_cache(cfg, w, rows)
    note(f"range x{S:g} gqa s_q={s_q}")
    out2, lse2 = gu.run_gqa(w, gqla, gc, 0)

    def ref_g(b, L):
        o, l = oracle.gqa_decode(stored[b], qn[b], qr[b], cfg.g, L, cfg.scale)
        return o / S, l
    gu.compare(cfg, out2 / S, lse2, [0, 1], w.lens, f"range x{S:g} gqa", ref=ref_g)
