"""Pins of the fp64 oracle against facts it does not compute itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with a closed form, a library routine, brute force, or an
invariant the definition implies.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutations.py`` runs them on copies of the oracle
with one planted mistake each and checks that some pin fails.

Source of the definition: "GQLA: Group-Query Latent Attention for
Hardware-Adaptive LLM Decoding", technical summary section 2 (Architecture,
Path selection) and section 1 (Problem).
"""
from __future__ import annotations

import math

import numpy as np


def small_problem(seed=0, h_q=8, g=2, r_kv=16, d_r=8, d_h=8, length=13, s_q=1, rows_extra=3):
    rng = np.random.default_rng(seed)
    rows = rng.standard_normal((length + rows_extra, r_kv + d_r))
    q_nope = rng.standard_normal((s_q, h_q, d_h))
    q_rope = rng.standard_normal((s_q, h_q, d_r))
    w_uk = rng.standard_normal((g, d_h, r_kv)) / math.sqrt(r_kv)
    w_uv = rng.standard_normal((g, d_h, r_kv)) / math.sqrt(r_kv)
    scale = 1.0 / math.sqrt(d_h + d_r)
    return dict(rows=rows, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv, length=length, scale=scale)


def _tb(orc, p):
    return orc.textbook_decode(p["rows"], p["q_nope"], p["q_rope"], p["w_uk"], p["w_uv"], p["length"], p["scale"])


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


SHAPES = [
    dict(h_q=8, g=2, s_q=1, length=13),
    dict(h_q=8, g=8, s_q=1, length=9),    # g = h_q: one up-projection per head (MLA)
    dict(h_q=8, g=1, s_q=1, length=11),   # g = 1: one group (MQA)
    dict(h_q=8, g=4, s_q=2, length=10),   # multi-token step
    dict(h_q=6, g=3, s_q=2, length=2),
    dict(h_q=4, g=2, s_q=1, length=1),
]


def pin_three_forms_agree(orc):
    """The absorb and GQA paths are algebraically equal to the textbook form (section 2)."""
    for k, sh in enumerate(SHAPES):
        p = small_problem(seed=10 + k, **sh)
        o, lse = _tb(orc, p)
        oa, la = orc.absorb_decode(p["rows"], p["q_nope"], p["q_rope"], p["w_uk"], p["w_uv"], p["length"], p["scale"])
        gr = orc.expand_groups(p["rows"][: p["length"]], p["w_uk"], p["w_uv"])
        og, lg = orc.gqa_decode(gr, p["q_nope"], p["q_rope"], sh["g"], p["length"], p["scale"])
        assert _rel(oa, o) < 1e-12 and _rel(og, o) < 1e-12, sh
        assert _rel(la, lse) < 1e-12 and _rel(lg, lse) < 1e-12, sh


def pin_torch_sdpa(orc):
    """Softmax attention of each head over its materialised K/V equals torch's fp64 SDPA on the CPU."""
    import torch
    import torch.nn.functional as F

    for k, sh in enumerate(SHAPES):
        p = small_problem(seed=20 + k, **sh)
        o, _ = _tb(orc, p)
        h_q, g, s_q, length = sh["h_q"], sh["g"], sh["s_q"], sh["length"]
        r_kv = p["w_uk"].shape[2]
        rows = torch.tensor(p["rows"][:length], dtype=torch.float64)
        c, k_r = rows[:, :r_kv], rows[:, r_kv:]
        w_uk = torch.tensor(p["w_uk"], dtype=torch.float64)
        w_uv = torch.tensor(p["w_uv"], dtype=torch.float64)
        hpg = h_q // g
        keys = torch.stack([torch.cat([c @ w_uk[i // hpg].T, k_r], dim=1) for i in range(h_q)])  # [h][L][D]
        vals = torch.stack([c @ w_uv[i // hpg].T for i in range(h_q)])                            # [h][L][d_h]
        q = torch.cat([torch.tensor(p["q_nope"]), torch.tensor(p["q_rope"])], dim=2).permute(1, 0, 2)  # [h][s_q][D]
        pos = torch.arange(length)
        allowed = torch.stack([pos <= length - s_q + s for s in range(s_q)])  # [s_q][L]
        ref = F.scaled_dot_product_attention(q.contiguous(), keys.contiguous(), vals.contiguous(),
                                             attn_mask=allowed, scale=p["scale"])
        assert _rel(o, ref.permute(1, 0, 2).numpy()) < 1e-12, sh


def pin_bruteforce_scalar(orc):
    """Pure-Python scalar loops with exactly rounded sums on a tiny shape."""
    sh = dict(h_q=4, g=2, r_kv=8, d_r=4, d_h=4, length=7, s_q=2)
    p = small_problem(seed=3, **sh)
    o, lse = _tb(orc, p)
    rows, w_uk, w_uv = p["rows"].tolist(), p["w_uk"].tolist(), p["w_uv"].tolist()
    qn, qr = p["q_nope"].tolist(), p["q_rope"].tolist()
    L, s_q, r_kv, d_h = sh["length"], sh["s_q"], sh["r_kv"], sh["d_h"]
    for s in range(s_q):
        for i in range(sh["h_q"]):
            j = i // (sh["h_q"] // sh["g"])
            sc = []
            vs = []
            for t in range(L - s_q + s + 1):
                key = [math.fsum(w_uk[j][d][r] * rows[t][r] for r in range(r_kv)) for d in range(d_h)]
                dot = math.fsum([qn[s][i][d] * key[d] for d in range(d_h)] +
                                [qr[s][i][e] * rows[t][r_kv + e] for e in range(sh["d_r"])])
                sc.append(p["scale"] * dot)
                vs.append([math.fsum(w_uv[j][d][r] * rows[t][r] for r in range(r_kv)) for d in range(d_h)])
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            z = math.fsum(w)
            for d in range(d_h):
                ref = math.fsum(w[t] * vs[t][d] for t in range(len(w))) / z
                assert abs(o[s, i, d] - ref) <= 1e-13 * max(1.0, abs(ref)), (s, i, d)
            assert abs(lse[s, i] - (m + math.log(z))) <= 1e-13 * max(1.0, abs(m)), (s, i)


def pin_single_row(orc):
    """L = 1: the softmax weight is 1, so o = W_UV[j] c_0 and lse is the scaled score of that row."""
    p = small_problem(seed=4, length=1)
    o, lse = _tb(orc, p)
    r_kv = p["w_uk"].shape[2]
    c0, kr0 = p["rows"][0, :r_kv], p["rows"][0, r_kv:]
    hpg = 8 // 2
    for i in range(8):
        j = i // hpg
        np.testing.assert_allclose(o[0, i], p["w_uv"][j] @ c0, rtol=1e-13, atol=1e-15)
        score = p["scale"] * (p["q_nope"][0, i] @ (p["w_uk"][j] @ c0) + p["q_rope"][0, i] @ kr0)
        assert abs(lse[0, i] - score) < 1e-13


def pin_zero_query(orc):
    """q = 0: uniform weights, so o = W_UV[j] mean_t c_t and lse = ln(number of visible rows)."""
    for s_q in (1, 2):
        p = small_problem(seed=5, length=9, s_q=s_q)
        p["q_nope"][:] = 0.0
        p["q_rope"][:] = 0.0
        o, lse = _tb(orc, p)
        r_kv = p["w_uk"].shape[2]
        for s in range(s_q):
            n = 9 - s_q + s + 1
            mean_c = p["rows"][:n, :r_kv].mean(axis=0)
            for i in range(8):
                np.testing.assert_allclose(o[s, i], p["w_uv"][i // 4] @ mean_c, rtol=1e-12, atol=1e-14)
                assert abs(lse[s, i] - math.log(n)) < 1e-13


def pin_constant_rows(orc):
    """Every latent row equal to c: any weights average to W_UV[j] c, whatever the RoPE keys."""
    p = small_problem(seed=6, length=12)
    r_kv = p["w_uk"].shape[2]
    p["rows"][:, :r_kv] = p["rows"][0, :r_kv]
    o, _ = _tb(orc, p)
    for i in range(8):
        np.testing.assert_allclose(o[0, i], p["w_uv"][i // 4] @ p["rows"][0, :r_kv], rtol=1e-12, atol=1e-14)


def pin_two_rows_sigmoid(orc):
    """L = 2: o = sigmoid(d) v_0 + (1 - sigmoid(d)) v_1 with d = the difference of the scaled scores."""
    p = small_problem(seed=7, length=2)
    o, _ = _tb(orc, p)
    r_kv = p["w_uk"].shape[2]
    for i in range(8):
        j = i // 4
        ks = [np.concatenate([p["w_uk"][j] @ p["rows"][t, :r_kv], p["rows"][t, r_kv:]]) for t in (0, 1)]
        vs = [p["w_uv"][j] @ p["rows"][t, :r_kv] for t in (0, 1)]
        q = np.concatenate([p["q_nope"][0, i], p["q_rope"][0, i]])
        d = p["scale"] * (q @ ks[0] - q @ ks[1])
        sig = 1.0 / (1.0 + math.exp(-d))
        np.testing.assert_allclose(o[0, i], sig * vs[0] + (1 - sig) * vs[1], rtol=1e-12, atol=1e-14)


def pin_mtp_causal(orc):
    """s_q = 2: query 0 does not see the newest row; query 1 sees every row (section 2, Path selection)."""
    p = small_problem(seed=8, length=10, s_q=2)
    o, lse = _tb(orc, p)
    q = dict(p)
    q["rows"] = p["rows"].copy()
    q["rows"][9] += 3.0
    o2, lse2 = _tb(orc, q)
    assert np.array_equal(o[0], o2[0]) and np.array_equal(lse[0], lse2[0])
    assert np.max(np.abs(o[1] - o2[1])) > 1e-3
    # query 1 of an s_q = 2 step equals a single-token step over all rows,
    # query 0 equals a single-token step over the first L - 1 rows
    one = dict(p, q_nope=p["q_nope"][1:], q_rope=p["q_rope"][1:])
    o1, _ = _tb(orc, one)
    assert _rel(o[1], o1[0]) < 1e-13
    zero = dict(p, q_nope=p["q_nope"][:1], q_rope=p["q_rope"][:1], length=9)
    o0, _ = _tb(orc, zero)
    assert _rel(o[0], o0[0]) < 1e-13


def pin_group_map(orc):
    """Head i depends on its own group's W_UK / W_UV only (contiguous grouping, section 2)."""
    p = small_problem(seed=9, h_q=8, g=4, length=8)
    o, _ = _tb(orc, p)
    for jj in range(4):
        q = dict(p)
        q["w_uk"] = p["w_uk"].copy()
        q["w_uv"] = p["w_uv"].copy()
        q["w_uk"][jj] *= 1.7
        q["w_uv"][jj] += 0.5
        o2, _ = _tb(orc, q)
        changed = [i for i in range(8) if np.max(np.abs(o2[0, i] - o[0, i])) > 1e-9]
        assert changed == [2 * jj, 2 * jj + 1], (jj, changed)


def pin_key_permutation(orc):
    """s_q = 1: attention is a set function of the cached rows."""
    p = small_problem(seed=11, length=12)
    o, lse = _tb(orc, p)
    perm = np.random.default_rng(0).permutation(12)
    q = dict(p)
    q["rows"] = p["rows"].copy()
    q["rows"][:12] = p["rows"][perm]
    o2, lse2 = _tb(orc, q)
    assert _rel(o2, o) < 1e-13 and _rel(lse2, lse) < 1e-13


def pin_lse_merge(orc):
    """Merging per-chunk partials with their log-sum-exp reproduces the unsplit result, empty chunks included."""
    for s_q, bounds in ((1, [0, 3, 3, 8, 13]), (2, [0, 12, 13, 20]), (1, [0, 13])):
        p = small_problem(seed=12, length=13, s_q=s_q)
        o, lse = _tb(orc, p)
        parts, lses = orc.split_partials(p["rows"], p["q_nope"], p["q_rope"], p["w_uk"], p["w_uv"],
                                         p["length"], p["scale"], bounds)
        om, lm = orc.lse_merge(parts, lses)
        assert _rel(om, o) < 1e-12 and _rel(lm, lse) < 1e-12


def pin_empty(orc):
    """A query that sees no cached row yields o = 0 and lse = -inf."""
    p = small_problem(seed=13, length=0)
    o, lse = _tb(orc, p)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    p = small_problem(seed=13, length=1, s_q=2)
    o, lse = _tb(orc, p)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


def pin_expanded_row(orc):
    """The expanded row has 2 g d_h + d_R entries: [K_0..K_{g-1} | V_0..V_{g-1} | k_R] (section 2, GQA path)."""
    p = small_problem(seed=14, h_q=8, g=4, length=5)
    gr = orc.expand_groups(p["rows"][:5], p["w_uk"], p["w_uv"])
    g, d_h, r_kv = p["w_uk"].shape
    assert gr.shape == (5, 2 * g * d_h + p["rows"].shape[1] - r_kv)
    np.testing.assert_array_equal(gr[:, 2 * g * d_h:], p["rows"][:5, r_kv:])
    # the value block of group j reproduces W_UV[j] c for a unit latent
    unit = np.zeros((1, p["rows"].shape[1]))
    unit[0, 3] = 1.0
    gu = orc.expand_groups(unit, p["w_uk"], p["w_uv"])
    for j in range(g):
        np.testing.assert_array_equal(gu[0, j * d_h:(j + 1) * d_h], p["w_uk"][j][:, 3])
        np.testing.assert_array_equal(gu[0, (g + j) * d_h:(g + j + 1) * d_h], p["w_uv"][j][:, 3])


def pin_rope_closed_form(orc):
    """Hand-computed rotations fix the pairing (k with k + d_R/2), the frequency
    theta^(-2k/d_R) and the direction of the turn."""
    # d_R = 2: the single pair turns by the position itself
    np.testing.assert_allclose(orc.rope_rotate(np.array([1.0, 0.0]), 3), [math.cos(3), math.sin(3)], rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.rope_rotate(np.array([0.0, 1.0]), 3), [-math.sin(3), math.cos(3)], rtol=0, atol=1e-15)
    # d_R = 4, theta = 10000: pair (x_1, x_3) turns at 10000^(-1/2) = 0.01 rad per position
    x = np.array([0.0, 1.0, 0.0, 0.0])
    np.testing.assert_allclose(orc.rope_rotate(x, 100), [0.0, math.cos(1.0), 0.0, math.sin(1.0)], rtol=0, atol=1e-14)
    # pair (x_0, x_2) at frequency 1 and another base
    x = np.array([2.0, 0.0, -1.0, 0.0])
    a = 5.0
    np.testing.assert_allclose(orc.rope_rotate(x, 5, theta=500.0),
                               [2 * math.cos(a) + math.sin(a), 0.0, 2 * math.sin(a) - math.cos(a), 0.0], rtol=0, atol=1e-14)


def pin_rope_rotation_properties(orc):
    """Position 0 is the identity, every pair keeps its length, and scores depend only on
    the distance between query and key positions (the defining property of rotary
    embeddings): <R(p) q, R(t) k> = <R(p - t) q, k>."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((6, 16))
    np.testing.assert_array_equal(orc.rope_rotate(x, np.zeros(6, dtype=np.int64)), x)
    pos = rng.integers(0, 100000, 6)
    y = orc.rope_rotate(x, pos)
    np.testing.assert_allclose(x[:, :8] ** 2 + x[:, 8:] ** 2, y[:, :8] ** 2 + y[:, 8:] ** 2, rtol=1e-12)
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    for p, t in ((7, 3), (1000, 999), (5, 40), (70000, 12)):
        lhs = orc.rope_rotate(q, p) @ orc.rope_rotate(k, t)
        rhs = orc.rope_rotate(q, p - t) @ k
        assert abs(lhs - rhs) <= 1e-9 * (1 + abs(rhs)), (p, t, lhs, rhs)


def pin_append_positions(orc):
    """Appending s_q tokens at once equals appending them one at a time, and the cache
    ends up holding every key rotated at its own row index; the new queries sit at the
    positions of the new rows."""
    rng = np.random.default_rng(22)
    L, s_q, h_q, r_kv, d_r = 9, 3, 4, 6, 8
    c = rng.standard_normal((L, r_kv))
    kr = rng.standard_normal((L, d_r))
    qr = rng.standard_normal((s_q, h_q, d_r))
    pos, rows, q_rot = orc.append_rows(c[L - s_q:], kr[L - s_q:], qr, L)
    assert list(pos) == [L - 3, L - 2, L - 1]
    whole = np.concatenate([c, orc.rope_rotate(kr, np.arange(L))], axis=1)
    np.testing.assert_array_equal(rows, whole[L - s_q:])
    for s in range(s_q):
        _, row1, q1 = orc.append_rows(c[L - s_q + s:L - s_q + s + 1], kr[L - s_q + s:L - s_q + s + 1],
                                      qr[s:s + 1], L - s_q + s + 1)
        np.testing.assert_array_equal(row1[0], rows[s])
        np.testing.assert_array_equal(q1[0], q_rot[s])
    # the newest query against the newest key: zero distance, so the rotary score is
    # the unrotated dot product
    np.testing.assert_allclose(q_rot[-1] @ rows[-1, r_kv:], qr[-1] @ kr[-1], rtol=1e-12)


def _sparse_problem(seed, h_q=8, g=2, length=11, s_q=1, topk=6):
    p = small_problem(seed=seed, h_q=h_q, g=g, length=length, s_q=s_q)
    rng = np.random.default_rng(seed + 100)
    p["gr"] = rng.standard_normal((length + 3, 2 * g * p["w_uk"].shape[1] + p["q_rope"].shape[2]))
    p["idx"] = rng.integers(0, length, size=(s_q, g, topk))
    return p


def _sp(orc, p, idx=None):
    g = p["w_uk"].shape[0]
    return orc.sparse_gqa_decode(p["gr"], p["q_nope"], p["q_rope"], g, p["idx"] if idx is None else idx,
                                 p["length"], p["scale"])


def pin_sparse_all_rows_is_dense(orc):
    """Listing every visible row once gives the dense GQA form (and, over expanded rows,
    the textbook form), for s_q = 1 and 2 and in any order."""
    for s_q in (1, 2):
        p = _sparse_problem(30 + s_q, s_q=s_q)
        g = p["w_uk"].shape[0]
        L = p["length"]
        idx = np.stack([np.stack([np.random.default_rng(s * 7 + j).permutation(L) for j in range(g)])
                        for s in range(s_q)])
        o, lse = _sp(orc, p, idx)
        od, ld = orc.gqa_decode(p["gr"], p["q_nope"], p["q_rope"], g, L, p["scale"])
        np.testing.assert_allclose(o, od, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, ld, rtol=1e-12)


def pin_sparse_bruteforce(orc):
    """Scalar loops over the listed rows (math.fsum) with repeated, out-of-range and
    future indices in the lists."""
    p = _sparse_problem(41, h_q=4, g=2, length=7, s_q=2, topk=9)
    p["idx"][0, 0, :4] = [3, 3, -1, 6]          # a duplicate, an empty slot, a row past query 0's window
    p["idx"][1, 1, :3] = [8, 0, 0]              # a row past L, a duplicate
    o, lse = _sp(orc, p)
    g, d_h = p["w_uk"].shape[0], p["w_uk"].shape[1]
    L, s_q, h_q = p["length"], 2, 4
    gr = p["gr"]
    for s in range(s_q):
        n = L - s_q + s + 1
        for i in range(h_q):
            j = i // (h_q // g)
            q = list(p["q_nope"][s, i]) + list(p["q_rope"][s, i])
            rows = [int(t) for t in p["idx"][s, j] if 0 <= t < n]
            sc = []
            for t in rows:
                k = list(gr[t, j * d_h:(j + 1) * d_h]) + list(gr[t, 2 * g * d_h:])
                sc.append(p["scale"] * math.fsum(a * b for a, b in zip(q, k)))
            m = max(sc)
            w = [math.exp(x - m) for x in sc]
            z = math.fsum(w)
            for d in range(d_h):
                ref = math.fsum(wt * gr[t, (g + j) * d_h + d] for wt, t in zip(w, rows)) / z
                assert abs(o[s, i, d] - ref) <= 1e-12 * (1 + abs(ref))
            assert abs(lse[s, i] - (m + math.log(z))) <= 1e-12 * (1 + abs(m))


def pin_sparse_single_and_empty(orc):
    """One listed row: o is that row's value block and lse its score; no usable row:
    o = 0, lse = -inf."""
    p = _sparse_problem(42, topk=1)
    g, d_h = p["w_uk"].shape[0], p["w_uk"].shape[1]
    p["idx"][0, :, 0] = [5, 2]
    o, lse = _sp(orc, p)
    for i in range(8):
        j = i // 4
        t = p["idx"][0, j, 0]
        np.testing.assert_array_equal(o[0, i], p["gr"][t, (g + j) * d_h:(g + j + 1) * d_h])
        k = np.concatenate([p["gr"][t, j * d_h:(j + 1) * d_h], p["gr"][t, 2 * g * d_h:]])
        q = np.concatenate([p["q_nope"][0, i], p["q_rope"][0, i]])
        assert abs(lse[0, i] - p["scale"] * (q @ k)) <= 1e-12
    o, lse = _sp(orc, p, np.full((1, g, 3), -1))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def pin_sparse_duplicate_weight(orc):
    """A row listed twice weighs as if its score were raised by ln 2."""
    p = _sparse_problem(43, topk=3)
    g, d_h = p["w_uk"].shape[0], p["w_uk"].shape[1]
    idx = np.array([[[1, 4, 4], [2, 7, 7]]])
    o, lse = _sp(orc, p, idx)
    for i in range(8):
        j = i // 4
        q = np.concatenate([p["q_nope"][0, i], p["q_rope"][0, i]])
        rows = idx[0, j, :2]
        sc = np.array([p["scale"] * (q @ np.concatenate([p["gr"][t, j * d_h:(j + 1) * d_h], p["gr"][t, 2 * g * d_h:]]))
                       for t in rows])
        sc[1] += math.log(2.0)
        w = np.exp(sc - sc.max())
        ref = (w @ p["gr"][rows, (g + j) * d_h:(g + j + 1) * d_h]) / w.sum()
        np.testing.assert_allclose(o[0, i], ref, rtol=1e-12, atol=1e-13)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
