"""Sparse GQLA decode (gqla_decode_gqa_sparse) vs the fp64 oracle, through the C-ABI (MI355X only).

Query token s of every head of group j attends to the rows listed in
indices[b][s][j]: the oracle's ``sparse_gqa_decode`` over the stored (bf16-rounded)
expanded rows is the reference, as for the dense GQA decode.  Index lists are seeded
synthetic selections (distinct rows drawn from the visible range, the shape of a
top-k selection), with padding (-1), repeated rows, rows past the sequence and rows
past the causal window mixed in where a case says so.  Tolerances as for the dense
paths: |gpu - oracle| <= 2e-3 + 2e-2 |oracle| (bf16), 1e-4 + 1e-4 |oracle| (fp32).
"""
import numpy as np
import pytest

import oracle
import synth
from synth.inputs import sample_sequences
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


def make_indices(cfg, lens, topk, seed, extras=False):
    """[B][s_q][g][topk] int32: distinct rows of [0, L_b) per (b, s, j) (shorter lists padded
    with -1); with extras, some slots get a repeated row, a row past L_b, a row past the
    token's causal window, and -1."""
    rng = np.random.default_rng(seed)
    idx = np.full((cfg.batch, cfg.s_q, cfg.g, topk), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        for s in range(cfg.s_q):
            for j in range(cfg.g):
                k = min(topk, L)
                if k:
                    idx[b, s, j, :k] = rng.choice(L, size=k, replace=False)
                if extras and topk >= 8 and L >= 2:
                    idx[b, s, j, 0] = idx[b, s, j, 1]          # repeated row
                    idx[b, s, j, 2] = L + 5                    # past the sequence
                    idx[b, s, j, 3] = L - 1                    # past the window of token s < s_q - 1
                    idx[b, s, j, 4] = -1
    return idx


def run_sparse(gqla, w, gc, idx, num_splits=0):
    import torch
    cfg = w.cfg
    sh = gu.shape_of(cfg, gqla)
    out = torch.full((cfg.batch, cfg.s_q, cfg.h_q, cfg.d_h), float("nan"), dtype=w.dtype, device="cuda")
    lse = torch.full((cfg.batch, cfg.s_q, cfg.h_q), float("nan"), dtype=torch.float32, device="cuda")
    ws = gqla.alloc_workspace(sh, gqla.SPARSE, cfg.batch, int(idx.shape[3]), num_splits, "cuda")
    if ws.numel() % 4 == 0:
        ws.view(torch.float32).fill_(float("nan"))
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).cuda()
    gqla.decode_gqa_sparse(sh, w.q_nope, w.q_rope, gc, w.ctx_lens, idx_d, out, lse, ws, num_splits)
    return out, lse


def check(gqla, cfg, lens, topk, seed, num_splits=0, extras=False, max_ctx=None):
    w = gu.workload(cfg, lens=lens, max_ctx=max_ctx)
    gc, rows = gu.upload_stored_group_cache(w)
    idx = make_indices(cfg, lens, topk, seed, extras)
    note(f"sparse cfg={cfg.name} g={cfg.g} s_q={cfg.s_q} lens={lens} topk={topk} splits={num_splits} extras={extras}")
    out, lse = run_sparse(gqla, w, gc, idx, num_splits)
    qn, qr = synth.queries(cfg)

    def ref(b, L):
        return oracle.sparse_gqa_decode(rows[b], qn[b], qr[b], cfg.g, idx[b], L, cfg.scale)
    gu.compare(cfg, out, lse, list(range(cfg.batch)), w.lens, "sparse", ref=ref)
    return w, gc, idx, out, lse


@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_sparse_flagship_shape(gqla, num_splits):
    cfg = synth.config(3).with_(batch=3)
    check(gqla, cfg, [1000, 300, 40], 256, 81, num_splits)


def test_sparse_ragged_list_and_extras(gqla):
    cfg = synth.config(4, s_q=2).with_(batch=3)
    check(gqla, cfg, [700, 77, 3], 77, 82, 0, extras=True)


@pytest.mark.parametrize("g,h_q", [(4, 128), (2, 32), (8, 64)])
def test_sparse_group_layouts(gqla, g, h_q):
    """h_q/g = 32 (two 16-head tiles per group), 16, and 8 (a partial tile)."""
    cfg = synth.config(4, g=g, s_q=1).with_(batch=2, h_q=h_q)
    check(gqla, cfg, [500, 64], 96, 83, 0, extras=True)


def test_sparse_every_row_is_dense(gqla):
    """Listing every row once (in a shuffled order) gives the dense GQA decode."""
    import torch
    cfg = synth.config(3).with_(batch=2)
    lens = [333, 64]
    w, gc, idx, out, lse = check(gqla, cfg, lens, 333, 84)
    for b, L in enumerate(lens):
        for j in range(cfg.g):
            assert sorted(idx[b, 0, j][idx[b, 0, j] >= 0].tolist()) == list(range(L))
    dense, dlse = gu.run_gqa(w, gqla, gc, 0)
    d = np.abs(gu.host(out) - gu.host(dense))
    assert np.all(d <= 4e-3 + 4e-2 * np.abs(gu.host(dense)))
    assert torch.isfinite(lse).all()


def test_sparse_empty_lists(gqla):
    import torch
    cfg = synth.config(3).with_(batch=2)
    w = gu.workload(cfg, lens=[100, 0], max_ctx=128)
    gc, _ = gu.upload_stored_group_cache(w)
    note("sparse: all entries -1, and topk = 0")
    for topk in (40, 0):
        idx = np.full((2, 1, cfg.g, topk), -1, dtype=np.int32)
        out, lse = run_sparse(gqla, w, gc, idx)
        assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_sparse_fp32(gqla):
    cfg = synth.config(1, s_q=2).with_(batch=2)
    check(gqla, cfg, [256, 30], 50, 85, 0, extras=True)
    check(gqla, cfg, [256, 30], 200, 86, 3)


def test_sparse_full_size_sampled(gqla):
    """The flagship batch (128 sequences at 8192 rows) with 2048 listed rows per (sequence,
    group), checked on sampled sequences."""
    cfg = synth.config(3)
    w = gu.workload(cfg)
    note("sparse full size: expand, then 2048 rows per (b, j)")
    gc = gu.expand(w, gqla)
    idx = make_indices(cfg, w.lens, 2048, 87)
    out, lse = run_sparse(gqla, w, gc, idx)
    seqs = sample_sequences(cfg, 3)
    qn, qr = synth.queries(cfg)
    gch = {b: gu.host(gc[b, : int(w.lens[b])]) for b in seqs}

    def ref(b, L):
        return oracle.sparse_gqa_decode(gch[b], qn[b], qr[b], cfg.g, idx[b], L, cfg.scale)
    gu.compare(cfg, out, lse, seqs, w.lens, "sparse full", ref=ref)
