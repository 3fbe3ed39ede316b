"""gqla_decode_gqa_noalloc (the GQA decode whose split-K partials live in the library's
static device scratch) against gqla_decode_gqa with a caller workspace, through the C-ABI.

Two calls in a row, the second with a smaller input, so the second runs on scratch that
still holds the first call's partials.  Each result must equal the workspace call's
bit for bit (same kernels, same split plan) and the oracle's GQA form over the stored
rows within the bf16 tolerance."""
import numpy as np
import pytest

import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gqla():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from latent_kv_cache_amd import gqla as mod
    mod.load()
    return mod


def _one(gqla, cfg, lens, max_ctx, num_splits):
    torch = gu.torch_mod()
    print(f"[gpu-case] noalloc g={cfg.g} s_q={cfg.s_q} B={cfg.batch} lens={lens} splits={num_splits}", flush=True)
    w = gu.workload(cfg, lens=lens, max_ctx=max_ctx)
    gc, rows = gu.upload_stored_group_cache(w)
    sh = gu.shape_of(cfg, gqla)
    need = gqla.workspace_size(sh, gqla.GQA, cfg.batch, w.max_ctx, num_splits)
    assert need <= gqla.NOALLOC_SCRATCH_BYTES
    ref_out, ref_lse = gu.run_gqa(w, gqla, gc, num_splits)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    gqla.decode_gqa_noalloc(sh, w.q_nope, w.q_rope, gc, w.ctx_lens, out, lse, num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "no-allocation output differs from the workspace call's"
    assert torch.equal(lse, ref_lse), "no-allocation lse differs from the workspace call's"
    gu.compare(cfg, out, lse, list(range(cfg.batch)), w.lens, "gqa noalloc", ref=gu.gqa_reference(cfg, rows))
    return need


def test_noalloc_matches_workspace_call_twice(gqla):
    big = synth.config(3).with_(batch=4)
    need1 = _one(gqla, big, [3000, 8192, 1, 0], 8192, 0)
    small = synth.config(4, g=4, s_q=2).with_(batch=2)
    need2 = _one(gqla, small, [700, 33], 704, 3)
    assert need2 < need1
