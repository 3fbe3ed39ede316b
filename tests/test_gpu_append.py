"""Decode-step append (gqla_append_rows) vs the fp64 oracle, through the C-ABI (MI355X only).

The append writes the s_q new latent rows of every sequence with their rotary keys
turned to the rows' positions, turns the new queries' rotary parts to the same
positions, and expands the new rows into the group cache.  References: the oracle's
``append_rows`` (fp64) rounded once to the storage dtype (fp64 -> fp32 -> bf16, round
to nearest even, the kernel's rounding), and ``expand_groups`` of the rounded rows.
Rotations are computed in fp64 on both sides, by different sine/cosine routines, so
a result may land one unit in the last place away where the fp64 values straddle a
rounding boundary: the test allows one bf16 (or fp32) ulp and requires nearly every
value to be bit-identical.  Rows that are not new must stay untouched.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SENTINEL = 5.0


def note(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.fixture(scope="module")
def gqla():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    from latent_kv_cache_amd import gqla as mod
    mod.load()
    return mod


def _store(dtype, x):
    return synth.bf16_round(x) if dtype == "bf16" else np.asarray(x, np.float32)


def _ulp(dtype, x):
    """Spacing of the storage dtype at |x| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if dtype == "bf16" else 24
    e = np.floor(np.log2(np.maximum(np.abs(x), 1e-30)))
    return 2.0 ** (e - (bits - 1))


def _close_to_ulp(dtype, got, ref, what, exact_frac=0.999):
    """got (storage dtype) within one ulp of the fp64 reference, and nearly always equal
    to the reference rounded to the storage dtype."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    assert np.all(diff <= _ulp(dtype, ref) * 1.0001 + 1e-30), f"{what}: max diff {diff.max():.3e}"
    frac = float(np.mean(got == _store(dtype, ref).astype(np.float64)))
    assert frac >= exact_frac, f"{what}: only {frac:.5f} equal to the rounded reference"


def _inputs(cfg, lens, seed):
    rng = np.random.default_rng(seed)
    B, s_q = cfg.batch, cfg.s_q
    c = rng.standard_normal((B, s_q, cfg.r_kv))
    c = c / np.sqrt(np.mean(c * c, axis=2, keepdims=True) + 1e-6)
    kr = rng.standard_normal((B, s_q, cfg.d_r))
    qr = rng.standard_normal((B, s_q, cfg.h_q, cfg.d_r))
    return _store(cfg.dtype, c), _store(cfg.dtype, kr), _store(cfg.dtype, qr)


def _dev(torch, x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda()


def _run_append(gqla, cfg, lens, max_ctx, seed, with_group=True, theta=10000.0):
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    c, kr, qr = _inputs(cfg, lens, seed)
    w_uk, w_uv = synth.up_weights(cfg)
    width = cfg.r_kv + cfg.d_r
    gwidth = 2 * cfg.g * cfg.d_h + cfg.d_r
    latent = torch.full((cfg.batch, max_ctx, width), SENTINEL, dtype=dt, device="cuda")
    group = torch.full((cfg.batch, max_ctx, gwidth), SENTINEL, dtype=dt, device="cuda") if with_group else None
    q_out = torch.full((cfg.batch, cfg.s_q, cfg.h_q, cfg.d_r), SENTINEL, dtype=dt, device="cuda")
    sh = gu.shape_of(cfg, gqla)
    gqla.append_rows(sh, _dev(torch, c, dt), _dev(torch, kr, dt), _dev(torch, np.asarray(lens, np.int32), torch.int32),
                     latent, q_rope_raw=_dev(torch, qr, dt), q_rope_out=q_out, rope_theta=theta,
                     w_uk=_dev(torch, w_uk, dt), w_uv=_dev(torch, w_uv, dt), group_cache=group)
    torch.cuda.synchronize()
    return (c, kr, qr, w_uk, w_uv), gu.host(latent), (gu.host(group) if with_group else None), gu.host(q_out)


def _check(cfg, lens, max_ctx, inputs, lat, grp, qo, theta=10000.0):
    c, kr, qr, w_uk, w_uv = inputs
    s_q = cfg.s_q
    for b, L in enumerate(lens):
        L = min(max(int(L), 0), max_ctx)
        keep = [s for s in range(s_q) if L - s_q + s >= 0]
        new_t = [L - s_q + s for s in keep]
        untouched = np.ones(max_ctx, bool)
        untouched[new_t] = False
        assert np.all(lat[b, untouched] == SENTINEL), f"b={b}: latent rows outside the new ones written"
        if grp is not None:
            assert np.all(grp[b, untouched] == SENTINEL), f"b={b}: group rows outside the new ones written"
        if not keep:
            assert np.all(qo[b] == SENTINEL), f"b={b}: queries written for tokens without a row"
            continue
        # the oracle appends the tokens that have a row (the first ones are skipped when L < s_q)
        _, rows, q_rot = oracle.append_rows(c[b, keep], kr[b, keep], qr[b, keep], L, theta)
        # positions of the kept tokens: L - s_q + s for s in keep, i.e. the last len(keep) rows
        rows_st = _store(cfg.dtype, rows)
        np.testing.assert_array_equal(lat[b, new_t, :cfg.r_kv], rows_st[:, :cfg.r_kv])
        _close_to_ulp(cfg.dtype, lat[b, new_t, cfg.r_kv:], rows[:, cfg.r_kv:], f"b={b} rotated k_R")
        _close_to_ulp(cfg.dtype, qo[b, keep], q_rot, f"b={b} rotated q_R")
        skipped = [s for s in range(s_q) if s not in keep]
        assert np.all(qo[b, skipped] == SENTINEL)
        if grp is not None:
            ref = oracle.expand_groups(lat[b, new_t].astype(np.float64), w_uk, w_uv)
            got = grp[b, new_t].astype(np.float64)
            gw = 2 * cfg.g * cfg.d_h
            np.testing.assert_array_equal(got[:, gw:], lat[b, new_t, cfg.r_kv:])
            stored = _store(cfg.dtype, ref[:, :gw]).astype(np.float64)
            rel = 2.0 ** -7 if cfg.dtype == "bf16" else 1e-5
            assert np.all(np.abs(got[:, :gw] - stored) <= rel * np.abs(stored) + 1e-4), f"b={b}: expanded rows"


@pytest.mark.parametrize("s_q", [1, 2])
def test_append_bf16(gqla, s_q):
    cfg = synth.config(3, s_q=s_q).with_(batch=5)
    lens = [100, 37, 2, 1, 64]
    note(f"append bf16 s_q={s_q} lens={lens}")
    inputs, lat, grp, qo = _run_append(gqla, cfg, lens, 128, seed=31 + s_q)
    _check(cfg, lens, 128, inputs, lat, grp, qo)


def test_append_bf16_g4_no_group_no_query(gqla):
    import torch
    cfg = synth.config(4, g=4, s_q=2).with_(batch=3)
    lens = [9, 2, 0]
    note("append bf16 g=4 without group cache")
    c, kr, _ = _inputs(cfg, lens, 41)
    latent = torch.full((3, 16, cfg.r_kv + cfg.d_r), SENTINEL, dtype=torch.bfloat16, device="cuda")
    gqla.append_rows(gu.shape_of(cfg, gqla), _dev(torch, c, torch.bfloat16), _dev(torch, kr, torch.bfloat16),
                     _dev(torch, np.asarray(lens, np.int32), torch.int32), latent)
    torch.cuda.synchronize()
    lat = gu.host(latent)
    for b, L in enumerate(lens):
        for s in range(cfg.s_q):
            t = L - cfg.s_q + s
            if t < 0:
                continue
            _, rows, _ = oracle.append_rows(c[b, s:s + 1], kr[b, s:s + 1], np.zeros((1, 1, cfg.d_r)), t + 1)
            np.testing.assert_array_equal(lat[b, t, :cfg.r_kv], c[b, s])
            _close_to_ulp("bf16", lat[b, t:t + 1, cfg.r_kv:], rows[:, cfg.r_kv:], f"b={b} s={s}")
    assert np.all(lat[2] == SENTINEL)


def test_append_fp32(gqla):
    cfg = synth.config(1, s_q=2).with_(batch=3)
    lens = [256, 1, 40]
    note(f"append fp32 lens={lens}")
    inputs, lat, grp, qo = _run_append(gqla, cfg, lens, 256, seed=51, theta=500.0)
    _check(cfg, lens, 256, inputs, lat, grp, qo, theta=500.0)


def test_append_long_positions(gqla):
    """Positions near 131072 (the long-context workload): fp64 angles keep the rotation exact."""
    cfg = synth.config(5).with_(batch=2)
    lens = [131072, 65537]
    note(f"append bf16 long positions {lens}")
    inputs, lat, grp, qo = _run_append(gqla, cfg, lens, 131072, seed=61, with_group=False)
    # only the new rows matter here; checking the untouched rows of a 131072-row cache is the slow part
    c, kr, qr, _, _ = inputs
    for b, L in enumerate(lens):
        _, rows, q_rot = oracle.append_rows(c[b], kr[b], qr[b], L)
        _close_to_ulp("bf16", lat[b, L - 1:L, cfg.r_kv:], rows[:, cfg.r_kv:], f"b={b} k_R at {L - 1}")
        _close_to_ulp("bf16", qo[b], q_rot, f"b={b} q_R at {L - 1}")
        assert np.all(lat[b, L - 2] == SENTINEL)


def test_decode_step_end_to_end(gqla):
    """A whole decode step: the cached prefix, the append of s_q = 2 new tokens (rows,
    rotary keys and queries), then both decode paths, against the oracle's append and
    textbook attention over the same rows."""
    import torch
    cfg = synth.config(4, s_q=2).with_(batch=2)
    lens = [300, 1000]
    max_ctx = 1024
    note("decode step: append then absorb and gqa")
    w = gu.workload(cfg, lens=lens, max_ctx=max_ctx)     # prefix rows (rows L-2, L-1 get overwritten)
    c, kr, qr = _inputs(cfg, lens, 71)
    sh = gu.shape_of(cfg, gqla)
    dt = torch.bfloat16
    gc = torch.zeros((2, max_ctx, 2 * cfg.g * cfg.d_h + cfg.d_r), dtype=dt, device="cuda")
    gqla.expand_groups(sh, w.latent, w.w_uk, w.w_uv, w.ctx_lens, gc)      # expand the prefix once
    q_rope = torch.empty((2, cfg.s_q, cfg.h_q, cfg.d_r), dtype=dt, device="cuda")
    gqla.append_rows(sh, _dev(torch, c, dt), _dev(torch, kr, dt), w.ctx_lens, w.latent,
                     q_rope_raw=_dev(torch, qr, dt), q_rope_out=q_rope, w_uk=w.w_uk, w_uv=w.w_uv, group_cache=gc)
    w.q_rope = q_rope
    out_a, lse_a = gu.run_absorb(w, gqla, 0)
    out_g, lse_g = gu.run_gqa(w, gqla, gc, 0)
    qn, _ = synth.queries(cfg)
    w_uk, w_uv = synth.up_weights(cfg)
    q_dev = gu.host(q_rope)
    rows_dev = gu.host(w.latent)
    gc_dev = gu.host(gc)
    rows_of = {}
    for b, L in enumerate(lens):
        # the device's rows are the prefix plus the oracle's appended rows (one ulp at most
        # in the rotary key); the references below run on exactly what the device holds
        prefix = synth.latent_rows(cfg, b, L)[: L - cfg.s_q]
        _, new_rows, q_rot = oracle.append_rows(c[b], kr[b], qr[b], L)
        np.testing.assert_array_equal(rows_dev[b, : L - cfg.s_q], prefix)
        _close_to_ulp("bf16", rows_dev[b, L - cfg.s_q:L], new_rows, f"b={b} appended rows", exact_frac=0.99)
        _close_to_ulp("bf16", q_dev[b], q_rot, f"b={b} rotated queries", exact_frac=0.99)
        rows_of[b] = rows_dev[b, :L].astype(np.float64)
        stored = synth.bf16_round(oracle.expand_groups(rows_of[b], w_uk, w_uv)).astype(np.float64)
        assert np.all(np.abs(gc_dev[b, :L] - stored) <= 2.0 ** -7 * np.abs(stored) + 1e-4), f"b={b} group rows"

    def ref_absorb(b, L):
        return oracle.textbook_decode(rows_of[b], qn[b], q_dev[b], w_uk, w_uv, L, cfg.scale)

    def ref_gqa(b, L):
        return oracle.gqa_decode(gc_dev[b, :L].astype(np.float64), qn[b], q_dev[b], cfg.g, L, cfg.scale)
    gu.compare(cfg, out_a, lse_a, [0, 1], w.lens, "step absorb", ref=ref_absorb)
    gu.compare(cfg, out_g, lse_g, [0, 1], w.lens, "step gqa", ref=ref_gqa)


def test_append_full_size(gqla):
    """The benchmark's batch: 128 sequences of 8192 rows, one new token each, with the
    group cache; only the new rows are read back."""
    import torch
    cfg = synth.config(3)
    B, S = cfg.batch, 8192
    lens = np.full(B, S, dtype=np.int32)
    note("append full size: 128 x 8192, group rows")
    c, kr, qr = _inputs(cfg, lens, 91)
    w_uk, w_uv = synth.up_weights(cfg)
    dt = torch.bfloat16
    latent = torch.zeros((B, S, cfg.r_kv + cfg.d_r), dtype=dt, device="cuda")
    group = torch.zeros((B, S, 2 * cfg.g * cfg.d_h + cfg.d_r), dtype=dt, device="cuda")
    q_out = torch.empty((B, 1, cfg.h_q, cfg.d_r), dtype=dt, device="cuda")
    gqla.append_rows(gu.shape_of(cfg, gqla), _dev(torch, c, dt), _dev(torch, kr, dt),
                     _dev(torch, lens, torch.int32), latent, q_rope_raw=_dev(torch, qr, dt), q_rope_out=q_out,
                     w_uk=_dev(torch, w_uk, dt), w_uv=_dev(torch, w_uv, dt), group_cache=group)
    torch.cuda.synchronize()
    lat = gu.host(latent[:, S - 1])
    grp = gu.host(group[:, S - 1])
    qo = gu.host(q_out)
    assert float(latent[:, S - 2].abs().max()) == 0.0 and float(group[:, S - 2].abs().max()) == 0.0
    gw = 2 * cfg.g * cfg.d_h
    for b in range(B):
        _, rows, q_rot = oracle.append_rows(c[b], kr[b], qr[b], S)
        np.testing.assert_array_equal(lat[b, :cfg.r_kv], c[b, 0])
        _close_to_ulp("bf16", lat[b:b + 1, cfg.r_kv:], rows[:, cfg.r_kv:], f"b={b} k_R", exact_frac=0.99)
        _close_to_ulp("bf16", qo[b], q_rot, f"b={b} q_R", exact_frac=0.99)
        stored = synth.bf16_round(oracle.expand_groups(lat[b:b + 1].astype(np.float64), w_uk, w_uv)).astype(np.float64)
        assert np.all(np.abs(grp[b:b + 1, :gw] - stored[:, :gw]) <= 2.0 ** -7 * np.abs(stored[:, :gw]) + 1e-4)
        np.testing.assert_array_equal(grp[b, gw:], lat[b, cfg.r_kv:])
