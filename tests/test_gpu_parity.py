"""HIP path vs the fp64 oracle, element by element, through the C-ABI (MI355X only).

Sizes span several 32-token tiles, ragged tails and several split-K chunks at
shapes the oracle finishes in seconds; the full-size launches (the ones the
benchmark times) are checked on sampled sequences.  Tolerance: |gpu - oracle|
<= 2e-3 + 2e-2 |oracle| for bf16 storage, 1e-4 + 1e-4 |oracle| for fp32.

References.  The absorb decode reads the latent rows themselves, so it is
compared with the textbook definition at every length.  The GQA decode reads
an expanded cache that is itself stored in bf16; its reference is the oracle's
GQA form over those stored rows (the oracle's fp64 expansion rounded once to
the storage dtype), uploaded as its input.  The expansion kernel is checked
against the same stored rows, and the whole expand-then-decode chain against
the textbook definition at the workloads' context lengths (>= 1024 tokens,
where the rounding of the stored K/V averages out far below the tolerance).
"""
import sys

import numpy as np
import pytest

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


def both_paths(cfg, lens, gqla, num_splits=0, seqs=None, max_ctx=None, what="", end_to_end=False):
    """Absorb decode vs the textbook oracle; GQA decode vs the oracle's GQA form over
    stored rows (end_to_end: device expansion, then GQA decode vs the textbook)."""
    w = gu.workload(cfg, lens=lens, max_ctx=max_ctx)
    seqs = list(range(cfg.batch)) if seqs is None else seqs
    note(f"{what} absorb cfg={cfg.name} B={cfg.batch} g={cfg.g} s_q={cfg.s_q} lens={list(w.lens[:6])} splits={num_splits}")
    out, lse = gu.run_absorb(w, gqla, num_splits)
    gu.compare(cfg, out, lse, seqs, w.lens, f"{what} absorb")
    if end_to_end:
        note(f"{what} device expand + gqa vs textbook")
        gc = gu.expand(w, gqla)
        ref = None
    else:
        note(f"{what} gqa over stored rows")
        gc, rows = gu.upload_stored_group_cache(w)
        ref = gu.gqa_reference(cfg, rows)
    out2, lse2 = gu.run_gqa(w, gqla, gc, num_splits)
    gu.compare(cfg, out2, lse2, seqs, w.lens, f"{what} gqa", ref=ref)
    return w, (out, lse), (out2, lse2)


# ---------------------------------------------------------------- tiny fp32 (config 1, full size)
@pytest.mark.parametrize("num_splits", [0, 1, 3, 256])
def test_tiny_fp32(gqla, num_splits):
    cfg = synth.config(1)
    both_paths(cfg, None, gqla, num_splits, what="tiny")


def test_tiny_fp32_ragged_multi(gqla):
    cfg = synth.config(1).with_(batch=4, s_q=2)
    both_paths(cfg, [256, 1, 0, 97], gqla, 2, max_ctx=256, what="tiny-ragged")


@pytest.mark.parametrize("d_h", [48, 256])
def test_fp32_head_widths(gqla, d_h):
    """d_h = 48 and 256: the combine's one- and four-outputs-per-lane layouts (upper lanes
    idle at 48), with three chunks per sequence so every row is merged.  d_h = 48 is not a
    whole MFMA tile (vector-ALU kernels on both paths); at 256 the absorb path runs the
    MFMA kernel and the GQA path, whose staged queries would pass the MFMA kernel's
    64 KB of LDS, the vector-ALU one."""
    cfg = synth.config(1).with_(batch=2, d_h=d_h)
    both_paths(cfg, [256, 77], gqla, 3, max_ctx=256, what=f"tiny d_h={d_h}")


# ---------------------------------------------------------------- bf16 shapes at reduced batch/context
@pytest.mark.parametrize("num_splits", [0, 1, 3])
def test_llama3_shape(gqla, num_splits):
    cfg = synth.config(2).with_(batch=3)
    both_paths(cfg, [4096, 1000, 33], gqla, num_splits, what="cfg2")


@pytest.mark.parametrize("num_splits", [0, 1, 5])
def test_flagship_shape_ragged(gqla, num_splits):
    cfg = synth.config(3).with_(batch=3)
    both_paths(cfg, [1000, 8192, 31], gqla, num_splits, max_ctx=8192, what="cfg3")


@pytest.mark.parametrize("g", [1, 2])
def test_flagship_heads_few_groups(gqla, g):
    """h_q = 128 with g = 1 (every head shares one K/V: the MQA special case, 320-wide
    expanded rows) and g = 2, through the device expansion and both decode paths."""
    cfg = synth.config(3, g=g).with_(batch=2)
    both_paths(cfg, [1500, 77], gqla, 0, max_ctx=1536, what=f"g={g}")
    # the chain against the textbook at the long sequence, where the stored rows' rounding averages out
    both_paths(cfg, [1500, 77], gqla, 0, seqs=[0], max_ctx=1536, what=f"g={g} e2e", end_to_end=True)


@pytest.mark.parametrize("h_q,s_q", [(16, 4), (32, 3)])
def test_fp32_row_tiles(gqla, h_q, s_q):
    """fp32 at g = 1, h_q s_q query rows per group: the MFMA kernels' four 16-row waves at
    64 rows, and past their 64 rows (96) the vector-ALU kernels."""
    cfg = synth.config(1, g=1, s_q=s_q).with_(batch=2, h_q=h_q)
    both_paths(cfg, [256, 45], gqla, 3, max_ctx=256, what=f"fp32 rows h_q={h_q} s_q={s_q}")


@pytest.mark.parametrize("g", [1, 16])
def test_tiny_fp32_group_extremes(gqla, g):
    """fp32 at g = 1 (MQA) and g = h_q = 16 (one head per group: MLA's per-head
    up-projections)."""
    cfg = synth.config(1, g=g).with_(batch=2)
    both_paths(cfg, [256, 40], gqla, 2, max_ctx=256, what=f"tiny g={g}")


@pytest.mark.parametrize("g,s_q", [(8, 2), (4, 1), (8, 1)])
def test_multi_token_shapes(gqla, g, s_q):
    cfg = synth.config(4, g=g, s_q=s_q).with_(batch=4)
    lens = [int(x) for x in synth.ctx_lens(synth.config(4))[:4]]
    lens = [min(x, 3000) for x in lens[:3]] + [2]
    both_paths(cfg, lens, gqla, 0, what=f"cfg4 g{g} s_q{s_q}")


@pytest.mark.parametrize("h_q,g,s_q", [(128, 1, 2), (128, 2, 2), (128, 4, 2), (128, 8, 2), (32, 8, 1), (128, 8, 1),
                                       (128, 8, 4), (64, 4, 3), (128, 2, 1)])
def test_gqa_direct_load_tiles(gqla, h_q, g, s_q):
    """The GQA kernels that load tiles straight into LDS (two 32-row buffers at g = 2 and
    4, two 16-row ones at g = 8; g = 1 stays on register-staged tiles): one and two row
    tiles per wave, several workgroups per item (g = 8, s_q = 4), lengths that end one
    row into a tile, on a tile boundary and mid-tile, over three chunks of at most 1024
    tokens."""
    cfg = synth.config(3, g=g, s_q=s_q).with_(batch=5, h_q=h_q)
    w = gu.workload(cfg, lens=[1000, 77, 33, 17, s_q], max_ctx=1000)
    note(f"direct-load gqa h_q={h_q} g={g} s_q={s_q} lens={list(w.lens)}")
    gc, rows = gu.upload_stored_group_cache(w)
    out, lse = gu.run_gqa(w, gqla, gc, 3)
    gu.compare(cfg, out, lse, list(range(cfg.batch)), w.lens, f"direct-load gqa g={g} s_q={s_q}",
               ref=gu.gqa_reference(cfg, rows))


def test_absorb_sq2_long(gqla):
    cfg = synth.config(4, s_q=2).with_(batch=2)
    w = gu.workload(cfg, lens=[4097, 1])
    note("absorb s_q=2 lens [4097, 1]")
    out, lse = gu.run_absorb(w, gqla, 0)
    gu.compare(cfg, out, lse, [0, 1], w.lens, "absorb sq2")


def test_long_context_shape(gqla):
    cfg = synth.config(5).with_(batch=2)
    lens = [int(x) for x in synth.ctx_lens(synth.config(5))[:2]]
    both_paths(cfg, lens, gqla, 0, what="cfg5", end_to_end=True)


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("s_q", [1, 2])
def test_edge_lengths(gqla, s_q):
    """Empty, single-row, shorter-than-s_q and exactly-one-chunk contexts in one batch."""
    cfg = synth.config(3, s_q=s_q).with_(batch=7)
    lens = [0, 1, 2, 32, 33, 64, 95]
    both_paths(cfg, lens, gqla, 3, max_ctx=96, what=f"edges s_q{s_q}")


@pytest.mark.parametrize("batch,seed", [(12, 0), (300, 2), (1040, 1)])
def test_item_order(gqla, batch, seed):
    """Both split-K item layouts.  12 sequences in 3 splits make at most 36 items, which
    run at once: every sequence is cut into chunks of equal size (rounded up to 32
    rows), so chunk boundaries fall off the uniform grid.  300 and 1040 sequences make
    more items than the device runs at once: full chunks first, then the shorter last
    chunks, longest first (300 sequences) or in sequence order (1040).  Lengths mix
    full chunks, tails of equal length, single rows and empty sequences."""
    cfg = synth.config(2).with_(batch=batch)
    rng = np.random.default_rng(7 + seed)
    if batch <= 16:
        lens = [700, 256, 300, 556, 44, 300, 0, 512, 44, 699, 1, 257][:batch]
        max_ctx, splits = 700, 3      # chunks of 256 tokens
    else:
        lens = [int(x) for x in rng.integers(0, 97, size=batch)]
        lens[::7] = [64] * len(lens[::7])
        max_ctx, splits = 96, 3       # chunks of 32 tokens
    both_paths(cfg, lens, gqla, splits, max_ctx=max_ctx, what=f"order B{batch}")


@pytest.mark.parametrize("lens,max_ctx", [([97, 65], 129), ([33, 20], 64)])
def test_chunk_boundary_causal(gqla, lens, max_ctx):
    """s_q = 2 with a chunk boundary near row L - 1, which only query 1 sees.  In 2
    splits max_ctx 129 gives chunks of at most 96 rows, cut evenly into 64 + 33 at
    L = 97; max_ctx 64 gives chunks of 32, and L = 33 puts row L - 1 alone in chunk 1
    (query 0 sees nothing there)."""
    cfg = synth.config(4, s_q=2).with_(batch=2)
    both_paths(cfg, lens, gqla, 2, max_ctx=max_ctx, what=f"causal-boundary {lens}")


@pytest.mark.parametrize("s_q", [1, 2])
def test_rising_scores(gqla, s_q):
    """Latent rows whose scale grows along the sequence, so the softmax maximum rises by
    more than the online softmax's slack (10 log2 units) after rows have accumulated:
    the kernels must raise their reference and rescale what they hold (a ramp on
    sequence 0, a sudden jump on sequence 1; a replay of the lazy-reference rule on the
    CPU counts 24 and 57 such raises over the heads).  Sharper softmaxes (peak logits of
    30-40 in log2 units) are covered by test_gpu_sharp.py.  At s_q = 2 the GQA path runs
    its 16-token kernel (two row tiles per wave) and the absorb path four row blocks."""
    import oracle
    torch = gu.torch_mod()
    cfg = synth.config(3, s_q=s_q).with_(batch=2)
    lens = [1000, 700]
    w = gu.workload(cfg, lens=lens)
    qn, qr = synth.queries(cfg)
    w_uk, w_uv = synth.up_weights(cfg)
    rows = {}
    for b, L in enumerate(lens):
        t = np.arange(L, dtype=np.float64)
        if b == 0:
            f = np.where(t < 300, 0.1, 0.1 + 2.5 * (t - 300) / (L - 300))
        else:
            f = np.where(t < 400, 0.15, 2.4)
        rows[b] = synth.bf16_round(synth.latent_rows(cfg, b, L).astype(np.float64) * f[:, None])
        w.latent[b, :L].copy_(torch.from_numpy(rows[b]).to(w.dtype))
    note("rising scores absorb")
    out, lse = gu.run_absorb(w, gqla, 1)
    gu.compare(cfg, out, lse, [0, 1], w.lens, "rising absorb",
               ref=lambda b, L: oracle.textbook_decode(rows[b], qn[b], qr[b], w_uk, w_uv, L, cfg.scale))
    note("rising scores gqa over stored rows")
    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    gc = torch.zeros((2, w.max_ctx, width), dtype=w.dtype, device="cuda")
    stored = {}
    for b, L in enumerate(lens):
        stored[b] = synth.bf16_round(oracle.expand_groups(rows[b], w_uk, w_uv))
        gc[b, :L].copy_(torch.from_numpy(stored[b]).to(w.dtype))
    out2, lse2 = gu.run_gqa(w, gqla, gc, 1)
    gu.compare(cfg, out2, lse2, [0, 1], w.lens, "rising gqa",
               ref=lambda b, L: oracle.gqa_decode(stored[b], qn[b], qr[b], cfg.g, L, cfg.scale))


# ---------------------------------------------------------------- properties
def test_split_invariance_and_determinism(gqla):
    cfg = synth.config(3).with_(batch=2)
    w = gu.workload(cfg, lens=[3000, 2049])
    note("split invariance absorb/gqa")
    a1, _ = gu.run_absorb(w, gqla, 1)
    a2, _ = gu.run_absorb(w, gqla, 0)
    a3, _ = gu.run_absorb(w, gqla, 0)
    assert gu.torch_mod().equal(a2, a3), "absorb is not bitwise deterministic"
    d = np.abs(gu.host(a1) - gu.host(a2))
    assert d.max() <= 2e-3 + 2e-2 * np.abs(gu.host(a1)).max()
    gc = gu.expand(w, gqla)
    g1, _ = gu.run_gqa(w, gqla, gc, 1)
    g2, _ = gu.run_gqa(w, gqla, gc, 0)
    g3, _ = gu.run_gqa(w, gqla, gc, 0)
    assert gu.torch_mod().equal(g2, g3), "gqa is not bitwise deterministic"
    # the two paths agree with each other (algebraic equivalence, section 2); the GQA
    # side reads bf16-stored K/V, hence twice the tolerance
    dd = np.abs(gu.host(a2) - gu.host(g2))
    assert np.all(dd <= 4e-3 + 4e-2 * np.abs(gu.host(g2)))


def test_expand_matches_oracle(gqla):
    """Expanded rows equal the fp64 expansion rounded once to bf16 (within one bf16 ulp)."""
    cfg = synth.config(3).with_(batch=2)
    w = gu.workload(cfg, lens=[300, 77], max_ctx=320)
    note("expand rows")
    torch = gu.torch_mod()
    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    gc = torch.full((2, 320, width), 7.0, dtype=torch.bfloat16, device="cuda")
    gu.expand(w, gqla, gc, row_begin=0)
    gch = gu.host(gc)
    for b, L in enumerate(w.lens):
        stored = gu.stored_group_rows(cfg, b, int(L)).astype(np.float64)
        got = gch[b, :L].astype(np.float64)
        # equal to the once-rounded oracle value, or one bf16 ulp away where fp32
        # accumulation lands on the other side of a rounding boundary; the absolute
        # term covers fp32 accumulation of 512 products (|sum of terms| ~ 20) where
        # cancellation leaves a value far smaller than its terms
        assert np.all(np.abs(got - stored) <= 2.0 ** -7 * np.abs(stored) + 1e-4), f"b={b}"
        assert np.mean(got == stored) > 0.99, f"b={b}: {np.mean(got == stored):.4f} exact"
        assert np.all(gch[b, L:] == 7.0), "rows past L_b were written"


def test_expand_row_begin(gqla):
    """row_begin expands only rows [row_begin, L_b): the decode-step append of s_q new rows."""
    cfg = synth.config(4, g=4).with_(batch=2)
    w = gu.workload(cfg, lens=[130, 64], max_ctx=130)
    torch = gu.torch_mod()
    full = gu.expand(w, gqla)
    width = 2 * cfg.g * cfg.d_h + cfg.d_r
    part = torch.full((2, 130, width), 3.0, dtype=torch.bfloat16, device="cuda")
    note("expand row_begin=62")
    gu.expand(w, gqla, part, row_begin=62)
    fh, ph = gu.host(full), gu.host(part)
    assert np.all(ph[:, :62] == 3.0)
    assert np.array_equal(ph[0, 62:130], fh[0, 62:130])
    assert np.array_equal(ph[1, 62:64], fh[1, 62:64])
    assert np.all(ph[1, 64:] == 3.0)


# ---------------------------------------------------------------- full-size launches, sampled sequences
@pytest.mark.parametrize("cfg_id", [2, 3])
def test_full_size_sampled(gqla, cfg_id):
    cfg = synth.config(cfg_id)
    seqs = sample_sequences(cfg, 4)
    both_paths(cfg, None, gqla, 0, seqs=seqs, what=f"full cfg{cfg_id}", end_to_end=True)


def test_full_size_multi_token_sampled(gqla):
    torch = gu.torch_mod()
    for g, s_q, paths in ((8, 2, ("gqa", "absorb")), (4, 1, ("gqa",))):
        cfg = synth.config(4, g=g, s_q=s_q)
        seqs = sample_sequences(cfg, 3)
        w = gu.workload(cfg)
        if "absorb" in paths:
            note(f"full cfg4 absorb s_q={s_q}")
            out, lse = gu.run_absorb(w, gqla, 0)
            gu.compare(cfg, out, lse, seqs, w.lens, "full cfg4 absorb")
            del out, lse
        note(f"full cfg4 gqa g={g} s_q={s_q}")
        gc = gu.expand(w, gqla)
        out, lse = gu.run_gqa(w, gqla, gc, 0)
        gu.compare(cfg, out, lse, seqs, w.lens, f"full cfg4 gqa g{g}")
        del gc, out, lse, w
        torch.cuda.empty_cache()


def test_full_size_long_context_sampled(gqla):
    cfg = synth.config(5)
    both_paths(cfg, None, gqla, 0, seqs=[0, 15], what="full cfg5", end_to_end=True)


@pytest.mark.parametrize("h_q,g,s_q", [(16, 8, 2), (64, 8, 1), (32, 4, 2), (32, 1, 1)])
def test_absorb_column_split_rows(gqla, h_q, g, s_q):
    """32 and 64 query rows per sequence (s_q * h_q), the workgroups whose eight waves
    split u's latent columns in two or four parts and reduce the W_UV epilogue in LDS:
    groups narrower than a 16-row block (h_q / g = 2 or 8: several W_UV groups per
    block), one group wider than a block (g = 1), two query tokens per step, ragged
    lengths across tiles and chunks."""
    cfg = synth.config(2, g=g, s_q=s_q).with_(batch=3, h_q=h_q)
    both_paths(cfg, [1500, 70, s_q], gqla, 3, max_ctx=1500, what=f"colsplit h_q={h_q} g={g} s_q={s_q}")


def test_binding_rejects_mismatched_tensors(gqla):
    """A host ctx_lens, int64 lengths, an output of the wrong dtype or size, or weights of
    the wrong shape raise ValueError in the binding; nothing is launched."""
    torch = gu.torch_mod()
    cfg = synth.config(3).with_(batch=2)
    w = gu.workload(cfg, lens=[40, 3], max_ctx=64)
    sh = gu.shape_of(cfg, gqla)
    out = torch.zeros((2, 1, cfg.h_q, cfg.d_h), dtype=torch.bfloat16, device="cuda")
    args = (sh, w.q_nope, w.q_rope, w.w_uk, w.w_uv, w.latent)
    for lens, o, msg in ((w.ctx_lens.cpu(), out, "ctx_lens"), (w.ctx_lens.long(), out, "ctx_lens must be"),
                         (w.ctx_lens, out.float(), "out must be"), (w.ctx_lens, out[:1], "out must have shape")):
        with pytest.raises(ValueError, match=msg):
            gqla.decode_absorb(*args, lens, o)
    with pytest.raises(ValueError, match="w_uk must have shape"):
        gqla.decode_absorb(sh, w.q_nope, w.q_rope, w.w_uk[:4], w.w_uv, w.latent, w.ctx_lens, out)
    torch.cuda.synchronize()
    assert bool(torch.all(out == 0))


if __name__ == "__main__":  # pragma: no cover
    sys.exit(pytest.main([__file__, "-v"]))
