"""Seeded randomized parity sweep of the decode entry points against the fp64 oracle
(MI355X only).

Each case draws a shape the C-ABI accepts and the oracle finishes in about a second:
- bf16 at r_kv = 512, d_R = 64, d_h = 128, with h_q in {16, 32, 64, 128} and g in
  {1, 2, 4, 8};
- fp32 at the tiny widths, with any g dividing h_q.

It also draws s_q in 1..4 (the causal window of every query token), a batch of ragged
lengths with the edge values 0, 1, s_q, 31, 32 and 33 mixed in, and the number of
split-K chunks (0 lets the library choose). Every case runs the absorb decode (against
the textbook definition), the GQA decode over the stored expanded rows (against the
oracle's GQA form over those rows) and the sparse decode over seeded index lists with
padding, repeats and out-of-window entries (against the oracle's sparse form).

Tolerances as elsewhere: 2e-3 + 2e-2 |oracle| for bf16 storage, 1e-4 + 1e-4 |oracle|
for fp32.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_CASES = 16
EDGE_LENS = (0, 1, 31, 32, 33)


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def gqla():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from latent_kv_cache_amd import gqla as mod
    mod.load()
    return mod


def draw_case(i):
    """(cfg, lens, num_splits, topk) of sweep case i."""
    rng = np.random.default_rng(7000 + i)
    s_q = int(rng.integers(1, 5))
    batch = int(rng.integers(1, 4))
    if i % 4 == 3:                       # every fourth case in fp32 at the tiny widths
        h_q = int(rng.choice([4, 8, 16, 32]))
        g = int(rng.choice([d for d in (1, 2, 4, 8, 16) if h_q % d == 0]))
        cfg = synth.config(1, g=g, s_q=s_q).with_(batch=batch, h_q=h_q)
        cap = 300
    else:
        h_q = int(rng.choice([16, 32, 64, 128]))
        g = int(rng.choice([d for d in (1, 2, 4, 8) if h_q % d == 0]))
        cfg = synth.config(2, g=g, s_q=s_q).with_(batch=batch, h_q=h_q)
        cap = 700
    lens = []
    for _ in range(batch):
        if rng.random() < 0.35:
            lens.append(int(rng.choice(EDGE_LENS + (s_q,))))
        else:
            lens.append(int(rng.integers(s_q, cap + 1)))
    num_splits = int(rng.choice([0, 0, 1, 2, 3, 5]))
    topk = int(rng.choice([1, 17, 64, 200]))
    return cfg, lens, num_splits, topk


def sparse_indices(cfg, lens, topk, seed):
    """[B][s_q][g][topk]: distinct rows of [0, L_b) (padded with -1), then a repeated row,
    a row past the sequence, a row past the window of the first token and a -1."""
    rng = np.random.default_rng(seed)
    idx = np.full((cfg.batch, cfg.s_q, cfg.g, topk), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        for s in range(cfg.s_q):
            for j in range(cfg.g):
                k = min(topk, L)
                if k:
                    idx[b, s, j, :k] = rng.choice(L, size=k, replace=False)
                if topk >= 8 and L >= 2:
                    idx[b, s, j, 0] = idx[b, s, j, 1]
                    idx[b, s, j, 2] = L + 3
                    idx[b, s, j, 3] = L - 1
                    idx[b, s, j, 4] = -1
    return idx


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep(gqla, case):
    import torch
    cfg, lens, num_splits, topk = draw_case(case)
    max_ctx = max(max(lens), 1)
    note(f"sweep case {case}: dtype={cfg.dtype} B={cfg.batch} h_q={cfg.h_q} g={cfg.g} s_q={cfg.s_q} "
         f"lens={lens} splits={num_splits} topk={topk}")
    w = gu.workload(cfg, lens=lens, max_ctx=max_ctx)
    seqs = list(range(cfg.batch))

    out, lse = gu.run_absorb(w, gqla, num_splits)
    gu.compare(cfg, out, lse, seqs, w.lens, f"sweep {case} absorb")

    gc, rows = gu.upload_stored_group_cache(w)
    out2, lse2 = gu.run_gqa(w, gqla, gc, num_splits)
    gu.compare(cfg, out2, lse2, seqs, w.lens, f"sweep {case} gqa", ref=gu.gqa_reference(cfg, rows))

    idx = sparse_indices(cfg, lens, topk, 9000 + case)
    sh = gu.shape_of(cfg, gqla)
    out3 = torch.full((cfg.batch, cfg.s_q, cfg.h_q, cfg.d_h), float("nan"), dtype=w.dtype, device="cuda")
    lse3 = torch.full((cfg.batch, cfg.s_q, cfg.h_q), float("nan"), dtype=torch.float32, device="cuda")
    ws = gqla.alloc_workspace(sh, gqla.SPARSE, cfg.batch, topk, num_splits, "cuda")
    gqla.decode_gqa_sparse(sh, w.q_nope, w.q_rope, gc, w.ctx_lens, torch.from_numpy(idx).cuda(), out3, lse3, ws,
                           num_splits)
    qn, qr = synth.queries(cfg)

    def ref(b, L):
        return oracle.sparse_gqa_decode(rows[b], qn[b], qr[b], cfg.g, idx[b], L, cfg.scale)
    gu.compare(cfg, out3, lse3, seqs, w.lens, f"sweep {case} sparse", ref=ref)
