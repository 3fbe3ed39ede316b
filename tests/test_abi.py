"""The C-ABI library loads and exports every declared symbol; host-side
validation and split planning (CPU only: no call here launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

from latent_kv_cache_amd import gqla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqla.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gqla.LIB_PATH):
        from latent_kv_cache_amd import build
        build.build()
    return gqla.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gqla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("gqla_expand_groups", "gqla_decode_absorb", "gqla_decode_gqa", "gqla_workspace_size",
              "gqla_status_string"):
        assert n in names
    assert set(names) == set(gqla.EXPORTS)


def test_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(5):
        assert lib.gqla_status_string(code)
    assert lib.gqla_status_string(99) == b"unknown status"


FLAG = gqla.make_shape(128, 8, 512, 64, 128, 1)
FAKE = 0x10000   # aligned non-null stand-in: validation never dereferences device pointers


def ws_size(shape, path=gqla.ABSORB, batch=128, ctx=8192, splits=0):
    n = ctypes.c_size_t(0)
    st = gqla.load().gqla_workspace_size(ctypes.byref(shape), path, batch, ctx, splits, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(h_q=128, g=7), 1),                           # h_q % g
    (dict(s_q=0), 1), (dict(s_q=5), 1),
    (dict(d_h=0), 1),
    (dict(r_kv=256), 2), (dict(d_h=64), 2),            # bf16 kernels are built for 512/64/128
    (dict(g=16), 2),                                   # GQA template groups
])
def test_shape_validation(lib, kw, status):
    base = dict(h_q=128, g=8, r_kv=512, d_r=64, d_h=128, s_q=1)
    base.update(kw)
    sh = gqla.make_shape(**base)
    st, _ = ws_size(sh, path=gqla.GQA)
    assert st == status, lib.gqla_last_error()
    assert lib.gqla_last_error()


def test_dtype_and_path_validation(lib):
    bad = gqla.make_shape(128, 8, 512, 64, 128, 1, dtype=7)
    assert ws_size(bad)[0] == 1
    assert ws_size(FLAG, path=3)[0] == 1
    nan_scale = gqla.make_shape(128, 8, 512, 64, 128, 1, scale=float("nan"))
    assert ws_size(nan_scale)[0] == 1
    f32_big = gqla.make_shape(16, 2, 2048, 16, 32, 1, dtype=gqla.F32)
    assert ws_size(f32_big)[0] == 2
    f32_ok = gqla.make_shape(16, 2, 64, 16, 32, 1, dtype=gqla.F32)
    assert ws_size(f32_ok, batch=1, ctx=256)[0] == 0


def test_workspace_size_formula(lib):
    st, n = ws_size(FLAG, gqla.GQA, 128, 8192, 2)
    assert st == 0
    n_split, chunk = gqla.plan_splits(FLAG, gqla.GQA, 128, 8192, 2)
    rows = 128 * 1 * 128
    assert n_split == 2 and chunk == 4096
    assert n >= n_split * rows * (128 + 1) * 4
    st, na = ws_size(FLAG, gqla.ABSORB, 128, 8192, 2)
    assert na >= n + rows * 576 * 2     # plus the absorbed queries


@pytest.mark.parametrize("ctx,splits", [(8192, 0), (8192, 1), (8192, 3), (131072, 0), (1, 0), (33, 2), (0, 0),
                                        (32768, 0), (100, 1000)])
def test_plan_covers_context(lib, ctx, splits):
    n, c = gqla.plan_splits(FLAG, gqla.GQA, 16, ctx, splits)
    assert c % 32 == 0 and c > 0
    assert n * c >= max(ctx, 1) and (n - 1) * c < max(ctx, 1)
    if splits:
        assert n <= splits
    if splits == 0:
        assert c <= 4096


def test_plan_fp32_chunk_cap(lib):
    sh = gqla.make_shape(16, 2, 64, 16, 32, 1, dtype=gqla.F32)
    n, c = gqla.plan_splits(sh, gqla.ABSORB, 1, 5000, 1)
    assert c <= 1024 and n * c >= 5000


def test_decode_argument_validation(lib):
    """Bad pointers, strides and workspace are rejected before any launch."""
    L = gqla.load()
    sh = FLAG
    B, S = 2, 64
    ws_ok = ws_size(sh, gqla.ABSORB, B, S)[1]

    def call(**over):
        a = dict(q_nope=FAKE, q_rope=FAKE, w_uk=FAKE, w_uv=FAKE, latent=FAKE, lbs=S * 576, lens=FAKE,
                 out=FAKE, lse=None, ws=FAKE, wsb=ws_ok, splits=0)
        a.update(over)
        return L.gqla_decode_absorb(ctypes.byref(sh), B, S, a["q_nope"], a["q_rope"], a["w_uk"], a["w_uv"],
                                    a["latent"], a["lbs"], a["lens"], a["out"], a["lse"], a["ws"], a["wsb"],
                                    a["splits"], None)

    assert call(q_nope=None) == 1
    assert call(latent=FAKE + 2) == 1            # misaligned
    assert call(lbs=S * 576 - 8) == 1            # stride shorter than max_ctx rows
    assert call(lbs=S * 576 + 4) == 1            # stride not a multiple of 8
    assert call(lens=None) == 1
    assert call(ws=None) == 3
    assert call(wsb=ws_ok - 1) == 3
    assert b"workspace" in L.gqla_last_error()
    assert call(splits=-1) == 1
    # batch 0 is a no-op that succeeds without touching any pointer
    assert L.gqla_decode_absorb(ctypes.byref(sh), 0, S, None, None, None, None, None, 0, None, None, None, None,
                                0, 0, None) == 0


def test_noalloc_validation_and_limit(lib):
    """The no-allocation GQA decode validates like the workspace call and rejects a call
    whose partials exceed the static scratch (GQLA_ERR_WORKSPACE) before any launch."""
    L = gqla.load()
    sh = FLAG
    width = 2 * 8 * 128 + 64

    def call(B, S, splits, **over):
        a = dict(q_nope=FAKE, q_rope=FAKE, gc=FAKE, gbs=S * width, lens=FAKE, out=FAKE, lse=None)
        a.update(over)
        return L.gqla_decode_gqa_noalloc(ctypes.byref(sh), B, S, a["q_nope"], a["q_rope"], a["gc"], a["gbs"],
                                         a["lens"], a["out"], a["lse"], splits, None)

    assert call(2, 64, 0, q_nope=None) == 1
    assert call(2, 64, 0, gbs=64 * width - 8) == 1
    assert call(2, 64, 0, lens=None) == 1
    assert call(2, 64, -1) == 1
    B, S, splits = 64, 32768, 64
    assert ws_size(sh, gqla.GQA, B, S, splits)[1] > gqla.NOALLOC_SCRATCH_BYTES
    assert call(B, S, splits) == 3
    assert b"static maximum" in L.gqla_last_error()
    assert L.gqla_decode_gqa_noalloc(ctypes.byref(sh), 0, S, None, None, None, 0, None, None, None, 0, None) == 0


def test_expand_argument_validation(lib):
    L = gqla.load()
    sh = FLAG
    S = 64
    assert L.gqla_expand_groups(ctypes.byref(sh), 2, S, FAKE, S * 576, FAKE, FAKE, FAKE, -1, FAKE, S * 2112,
                                None) == 1
    assert L.gqla_expand_groups(ctypes.byref(sh), 2, S, FAKE, S * 576, FAKE, FAKE, FAKE, 0, FAKE, S * 2112 - 8,
                                None) == 1
    assert L.gqla_expand_groups(ctypes.byref(sh), 2, S, FAKE, S * 576, None, FAKE, FAKE, 0, FAKE, S * 2112,
                                None) == 1
    # nothing to expand: row_begin past max_ctx
    assert L.gqla_expand_groups(ctypes.byref(sh), 2, S, FAKE, S * 576, FAKE, FAKE, FAKE, S, FAKE, S * 2112,
                                None) == 0


def test_append_argument_validation(lib):
    L = gqla.load()
    sh = FLAG
    S = 64
    F = FAKE

    def call(c=F, kr=F, qraw=F, qout=F + 4096, theta=10000.0, lens=F, lat=F, lbs=S * 576, wuk=F, wuv=F, gc=F,
             gbs=S * 2112, batch=2, shape=sh):
        return L.gqla_append_rows(ctypes.byref(shape), batch, S, c, kr, qraw, qout, theta, lens, lat, lbs, wuk, wuv,
                                  gc, gbs, None)
    assert call(theta=0.0) == 1
    assert call(theta=float("inf")) == 1
    assert call(qout=None) == 1                    # q_rope_raw without q_rope_out
    assert call(qraw=None) == 1
    assert call(qout=F) == 1                       # aliasing
    assert call(c=None) == 1
    assert call(kr=F + 8) == 1                     # misaligned
    assert call(lens=None) == 1
    assert call(lbs=S * 576 - 8) == 1
    assert call(wuk=None) == 1                     # expansion needs the weights
    assert call(gbs=S * 2112 - 8) == 1
    assert call(shape=gqla.make_shape(128, 8, 512, 64, 128, 1, dtype=9)) == 1
    odd = gqla.make_shape(16, 2, 64, 14, 32, 1, dtype=gqla.F32)
    assert call(shape=odd, lbs=S * 78, gbs=S * 142) == 1     # odd rotary width
    # the group layout is only checked when rows are expanded
    g16 = gqla.make_shape(128, 16, 512, 64, 128, 1)
    assert call(shape=g16, gbs=S * (2 * 16 * 128 + 64)) == 2
    # nothing to append
    assert call(batch=0) == 0


def test_sparse_argument_validation(lib):
    L = gqla.load()
    sh = FLAG
    S, K = 64, 48
    n = ctypes.c_size_t(0)
    assert L.gqla_workspace_size(ctypes.byref(sh), gqla.SPARSE, 2, K, 0, ctypes.byref(n)) == 0
    need = n.value
    assert need >= 2 * 128 * 128 * 4

    def call(qn=FAKE, gc=FAKE, gbs=S * 2112, lens=FAKE, idx=FAKE, topk=K, out=FAKE, lse=None, ws=FAKE, wsb=need,
             splits=0, shape=sh, batch=2):
        return L.gqla_decode_gqa_sparse(ctypes.byref(shape), batch, S, qn, FAKE, gc, gbs, lens, idx, topk, out, lse, ws,
                                        wsb, splits, None)
    assert call(topk=-1) == 1
    assert call(idx=None) == 1
    assert call(idx=FAKE + 2) == 1                 # misaligned int32 list
    assert call(gbs=S * 2112 - 8) == 1
    assert call(lens=None) == 1
    assert call(qn=None) == 1
    assert call(wsb=need - 1) == 3
    assert call(ws=None) == 3
    assert call(splits=-2) == 1
    assert call(batch=0) == 0                      # nothing to do
    # any g dividing h_q is accepted on this path (g = 16 has no dense GQA kernel)
    g16 = gqla.make_shape(128, 16, 512, 64, 128, 1)
    assert L.gqla_workspace_size(ctypes.byref(g16), gqla.SPARSE, 2, K, 0, ctypes.byref(n)) == 0
    assert L.gqla_workspace_size(ctypes.byref(g16), gqla.GQA, 2, K, 0, ctypes.byref(n)) == 2


def test_binding_raises_without_status_ok(lib):
    with pytest.raises(gqla.GQLAError):
        gqla.workspace_size(gqla.make_shape(128, 7, 512, 64, 128, 1), gqla.GQA, 1, 1)


def test_plan_lens_long_ragged_context(lib):
    # 16 sequences of 64K-128K tokens: the automatic rule (chunks <= 4096 tokens) makes
    # about 388 (chunk, sequence) units, a second round on 256 compute units; planned
    # from the lengths, every unit fits in one round and the count is a valid num_splits
    rng = np.random.default_rng(5)
    lens = rng.integers(65536, 131073, size=16).astype(np.int32)
    cap = int(lens.max())
    for path, blocks in ((gqla.ABSORB, 2), (gqla.GQA, 1)):
        # absorb workgroups hold 64 of the 128 query rows: two per (chunk, sequence)
        w, n, c = gqla.plan_splits_lens(FLAG, path, lens, cap)
        assert w > 0 and (n, c) == gqla.plan_splits(FLAG, path, 16, cap, w)
        units = blocks * sum((int(L) + c - 1) // c for L in lens)
        assert units <= 256 and n * c >= cap
        assert c > gqla.plan_splits(FLAG, path, 16, cap, 0)[1]


def test_plan_lens_uniform_flagship(lib):
    # 128 sequences of 8192 tokens on 256 compute units, one workgroup per CU: GQA cuts
    # two chunks per sequence; absorb keeps one chunk and runs the two 64-row blocks
    lens = np.full(128, 8192, dtype=np.int32)
    for path, want in ((gqla.ABSORB, (1, 8192)), (gqla.GQA, (2, 4096))):
        w, n, c = gqla.plan_splits_lens(FLAG, path, lens, 8192)
        assert (n, c) == want


def test_plan_lens_edges(lib):
    # empty batch, zero and clamped lengths, fp32 (automatic plan), null lengths
    assert gqla.plan_splits_lens(FLAG, gqla.ABSORB, [], 8192)[0] == 0
    w, n, c = gqla.plan_splits_lens(FLAG, gqla.GQA, [0, 0, 100000], 4096)
    assert n * c >= 4096 and c % 32 == 0
    sh = gqla.make_shape(16, 2, 64, 16, 32, 1, dtype=gqla.F32)
    assert gqla.plan_splits_lens(sh, gqla.ABSORB, [300], 300)[0] == 0
    w, n, c = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = lib.gqla_plan_splits_lens(ctypes.byref(FLAG), gqla.GQA, 2, 64, None, ctypes.byref(w), ctypes.byref(n),
                                   ctypes.byref(c))
    assert st == 1
