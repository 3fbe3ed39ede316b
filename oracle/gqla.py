"""fp64 oracle for GQLA decode attention (test infrastructure only).

Source: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
Decoding" (gist.science explainer page), technical summary, section 2
(Methodology, Architecture and Path selection) and section 1 (Problem).

What the method computes.  GQLA keeps one latent row cKV (width r_kv) and one
shared RoPE key k_R (width d^R_h) per cached token, and group-indexed
up-projections W_UK, W_UV (one d_h x r_kv matrix per group, g groups) instead
of one per query head (section 2, Architecture).  Query head i of h_q belongs
to group j(i).  Its key for token t is [W_UK[j] c_t || k_R,t] and its value is
W_UV[j] c_t.  Decode attention is ordinary softmax attention of each query head
over all cached tokens (section 1: every generated token reads the whole KV
history).  The two decode paths of section 2 (MQA-absorb and GQA) are stated to
be algebraically equivalent over the same weights, so the result has a plain
definition, and ``textbook_decode`` writes that definition out.  The two path
forms are written out too (``absorb_decode``, ``gqa_decode``); agreement of all
three is one of the oracle's pins.

Readings where the page is silent (each is also listed in the design notes):

* head -> group map is contiguous: j(i) = floor(i / (h_q / g));
* the decode operator receives q^R and k_R with the rotary embedding already
  applied (the page gives no RoPE convention; applying it is the cache-append
  step, not part of attention);
* only the latent part of a cached row is value; k_R is key-only;
* the expanded group row is laid out [K_0 .. K_{g-1} | V_0 .. V_{g-1} | k_R];
* with s_q query tokens per step (multi-token prediction, section 2 Path
  selection), the s_q new tokens are the last s_q cached rows, and query s
  sees rows t <= L - s_q + s (causal among the new tokens);
* a query that sees no row returns o = 0 and lse = -inf;
* lse is the natural-log log-sum-exp of the scaled scores;
* sparse GQLA (section 2, Sparse GQLA: fine-grained sparse attention keeps the
  GQA path because a group's h_q/g = 16 heads fill one 16-row matrix tile):
  every query token s and group j has its own list of selected cached rows,
  shared by the group's heads; a head attends to the listed rows only, each
  listing counting once (a row listed twice weighs twice); entries outside
  [0, L) or past the query's causal window are skipped;
* the decode-step append (``rope_rotate``, ``append_rows``), the step that
  feeds the path, rotates with the half-split pairing (x_k, x_{k + d_R/2}) at
  frequency theta^(-2k/d_R), theta = 10000 unless given; cache row t sits at
  position t, so the s_q new tokens of a sequence of length L take positions
  L - s_q .. L - 1, and their queries the same positions.

Everything is computed in float64 from the stored (bf16- or fp32-rounded)
inputs; nothing is blocked, fused or reordered beyond the definition.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

F64 = np.float64


def group_of_head(i: int, h_q: int, g: int) -> int:
    """Group index j(i) of query head i (contiguous grouping; section 2, Architecture)."""
    if h_q % g:
        raise ValueError("h_q must be a multiple of g")
    return i // (h_q // g)


def visible_rows(length: int, s_q: int, s: int) -> int:
    """Number of cached rows query token s of s_q sees: rows t <= L - s_q + s."""
    return max(0, min(length, length - s_q + s + 1))


def _softmax_attend(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Textbook softmax over the last axis of ``scores`` [m][n], then the weighted sum of value rows [n][d].

    Returns (o [m][d], lse [m]).  With n = 0 every row returns o = 0, lse = -inf.
    """
    m_rows = scores.shape[0]
    if scores.shape[1] == 0:
        return np.zeros((m_rows, values.shape[1]), dtype=F64), np.full(m_rows, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    w = np.exp(scores - m)
    z = w.sum(axis=1, keepdims=True)
    return (w @ values) / z, (m + np.log(z))[:, 0]


def _heads_of_group(j: int, h_q: int, g: int) -> List[int]:
    return [i for i in range(h_q) if group_of_head(i, h_q, g) == j]


def textbook_decode(rows, q_nope, q_rope, w_uk, w_uv, length: int, scale: float):
    """Plain definition for one sequence: materialise the keys and values, then softmax attention.

    rows    [>= L][r_kv + d_R]  cached [cKV | k_R]
    q_nope  [s_q][h_q][d_h]     query part contracted with the up-projected key
    q_rope  [s_q][h_q][d_R]     query part contracted with the shared RoPE key
    w_uk, w_uv [g][d_h][r_kv]
    returns o [s_q][h_q][d_h], lse [s_q][h_q]  (float64)

    Head i's key for token t is [W_UK[j(i)] c_t | k_R,t] and its value W_UV[j(i)] c_t.
    Heads of one group have identical keys and values, so they are materialised
    once per group and shared by that group's heads.
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    s_q, h_q, d_h = q_nope.shape
    g, _, r_kv = w_uk.shape
    rows = np.asarray(rows[:length], F64)
    c, k_r = rows[:, :r_kv], rows[:, r_kv:]
    o = np.zeros((s_q, h_q, d_h), F64)
    lse = np.full((s_q, h_q), -np.inf, F64)
    for j in range(g):
        heads = _heads_of_group(j, h_q, g)
        k_j = np.concatenate([c @ w_uk[j].T, k_r], axis=1)  # [L][d_h + d_R]
        v_j = c @ w_uv[j].T                                 # [L][d_h]
        for s in range(s_q):
            n = visible_rows(length, s_q, s)
            q = np.concatenate([q_nope[s, heads], q_rope[s, heads]], axis=1)  # [heads][d_h + d_R]
            o[s, heads], lse[s, heads] = _softmax_attend(scale * (q @ k_j[:n].T), v_j[:n])
    return o, lse


def absorb_decode(rows, q_nope, q_rope, w_uk, w_uv, length: int, scale: float):
    """MQA-absorb form (section 2, Architecture, memory-friendly path).

    W_UK is folded into the query: q~ = W_UK[j]^T q^N (width r_kv).  Every head
    scores the shared row [cKV | k_R] with [q~ | q^R], accumulates the latent
    u = sum_t p_t cKV_t, and only then applies its group's W_UV: o = W_UV[j] u.
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    s_q, h_q, d_h = q_nope.shape
    g, _, r_kv = w_uk.shape
    rows = np.asarray(rows[:length], F64)
    c = rows[:, :r_kv]
    o = np.zeros((s_q, h_q, d_h), F64)
    lse = np.full((s_q, h_q), -np.inf, F64)
    for j in range(g):
        heads = _heads_of_group(j, h_q, g)
        for s in range(s_q):
            n = visible_rows(length, s_q, s)
            q_hat = np.concatenate([q_nope[s, heads] @ w_uk[j], q_rope[s, heads]], axis=1)  # [heads][r_kv + d_R]
            u, lse[s, heads] = _softmax_attend(scale * (q_hat @ rows[:n].T), c[:n])     # u [heads][r_kv]
            o[s, heads] = u @ w_uv[j].T
    return o, lse


def expand_groups(rows, w_uk, w_uv) -> np.ndarray:
    """Expand latent rows once into g groups of K and V plus the shared k_R (section 2, GQA path).

    rows [L][r_kv + d_R] -> [L][2 g d_h + d_R] laid out [K_0..K_{g-1} | V_0..V_{g-1} | k_R],
    K_j,t = W_UK[j] c_t and V_j,t = W_UV[j] c_t, in float64.
    """
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    g, d_h, r_kv = w_uk.shape
    rows = np.asarray(rows, F64)
    c, k_r = rows[:, :r_kv], rows[:, r_kv:]
    out = np.empty((rows.shape[0], 2 * g * d_h + k_r.shape[1]), F64)
    for j in range(g):
        out[:, j * d_h:(j + 1) * d_h] = c @ w_uk[j].T
        out[:, (g + j) * d_h:(g + j + 1) * d_h] = c @ w_uv[j].T
    out[:, 2 * g * d_h:] = k_r
    return out


def gqa_decode(group_rows, q_nope, q_rope, g: int, length: int, scale: float):
    """GQA form over expanded rows (section 2, compute-friendly path).

    Head i of group j scores [K_j,t | k_R,t] with [q^N | q^R] and averages V_j,t.
    group_rows [>= L][2 g d_h + d_R] as produced by ``expand_groups``.
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    s_q, h_q, d_h = q_nope.shape
    gr = np.asarray(group_rows[:length], F64)
    k_r = gr[:, 2 * g * d_h:]
    o = np.zeros((s_q, h_q, d_h), F64)
    lse = np.full((s_q, h_q), -np.inf, F64)
    for j in range(g):
        heads = _heads_of_group(j, h_q, g)
        k_j = np.concatenate([gr[:, j * d_h:(j + 1) * d_h], k_r], axis=1)
        v_j = gr[:, (g + j) * d_h:(g + j + 1) * d_h]
        for s in range(s_q):
            n = visible_rows(length, s_q, s)
            q = np.concatenate([q_nope[s, heads], q_rope[s, heads]], axis=1)
            o[s, heads], lse[s, heads] = _softmax_attend(scale * (q @ k_j[:n].T), v_j[:n])
    return o, lse


def split_partials(rows, q_nope, q_rope, w_uk, w_uv, length: int, scale: float,
                   bounds: Sequence[int]) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """Per-chunk normalised partials of the textbook form over token chunks [bounds[k], bounds[k+1]).

    Each partial is the softmax attention of every (s, head) restricted to the
    visible rows of that chunk, with its own log-sum-exp (-inf where empty).
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    w_uk = np.asarray(w_uk, F64)
    w_uv = np.asarray(w_uv, F64)
    s_q, h_q, d_h = q_nope.shape
    g, _, r_kv = w_uk.shape
    rows = np.asarray(rows[:length], F64)
    c, k_r = rows[:, :r_kv], rows[:, r_kv:]
    parts, lses = [], []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        o = np.zeros((s_q, h_q, d_h), F64)
        lse = np.full((s_q, h_q), -np.inf, F64)
        for j in range(g):
            heads = _heads_of_group(j, h_q, g)
            k_j = np.concatenate([c @ w_uk[j].T, k_r], axis=1)
            v_j = c @ w_uv[j].T
            for s in range(s_q):
                n = visible_rows(length, s_q, s)
                a, b = min(lo, n), min(hi, n)
                q = np.concatenate([q_nope[s, heads], q_rope[s, heads]], axis=1)
                o[s, heads], lse[s, heads] = _softmax_attend(scale * (q @ k_j[a:b].T), v_j[a:b])
        parts.append(o)
        lses.append(lse)
    return parts, lses


def lse_merge(parts: Sequence[np.ndarray], lses: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Merge normalised partials: lse = log sum_p exp(lse_p), o = sum_p exp(lse_p - lse) o_p.

    Entries whose every partial is empty (lse_p = -inf) stay o = 0, lse = -inf.
    """
    lse_stack = np.stack([np.asarray(x, F64) for x in lses])       # [P][...]
    o_stack = np.stack([np.asarray(x, F64) for x in parts])         # [P][...][d]
    m = lse_stack.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(lse_stack), np.exp(lse_stack - m_safe), 0.0)
    z = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, z, 1.0)), -np.inf)
    o = np.where(finite[..., None],
                 np.einsum("p...,p...d->...d", w, o_stack) / np.where(finite, z, 1.0)[..., None], 0.0)
    return o, lse


def rope_rotate(x, positions, theta: float = 10000.0) -> np.ndarray:
    """Rotary embedding of vectors x [..., n][d_R] at integer positions [..., n] (float64).

    Half-split pairing: component k < d_R/2 pairs with k + d_R/2 and the pair turns by
    the angle position * theta^(-2k/d_R):
        x'_k        = x_k cos a - x_{k+d/2} sin a
        x'_{k+d/2}  = x_k sin a + x_{k+d/2} cos a
    Section 2 (Architecture) keeps one shared rotary key per token and a rotary part
    per query head; the rotation itself is the standard one, applied before attention.
    """
    x = np.asarray(x, F64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("rotary width must be even")
    half = d // 2
    freq = theta ** (-2.0 * np.arange(half, dtype=F64) / d)                 # [half]
    ang = np.asarray(positions, F64)[..., None] * freq                      # [..., half]
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def append_rows(c_new, kr_raw, q_rope_raw, length: int, theta: float = 10000.0):
    """The decode-step append of one sequence: its s_q new tokens enter the cache.

    c_new       [s_q][r_kv]         new latent rows
    kr_raw      [s_q][d_R]          new rotary keys before rotation
    q_rope_raw  [s_q][h_q][d_R]     rotary query parts before rotation
    length      L, the sequence length including the new tokens (L >= s_q)
    returns (positions [s_q], cache rows [s_q][r_kv + d_R] = [c | rotated k_R],
             rotated q_rope [s_q][h_q][d_R])
    New token s sits at position L - s_q + s; its key and its queries are rotated there.
    """
    c_new = np.asarray(c_new, F64)
    s_q = c_new.shape[0]
    pos = np.arange(length - s_q, length, dtype=np.int64)
    rows = np.concatenate([c_new, rope_rotate(kr_raw, pos, theta)], axis=1)
    q_rot = rope_rotate(q_rope_raw, np.broadcast_to(pos[:, None], np.asarray(q_rope_raw).shape[:2]), theta)
    return pos, rows, q_rot


def sparse_gqa_decode(group_rows, q_nope, q_rope, g: int, indices, length: int, scale: float):
    """Sparse GQLA over expanded rows (section 2, Sparse GQLA).

    group_rows [>= L][2 g d_h + d_R] as produced by ``expand_groups``
    indices    [s_q][g][topk] integer row indices; query token s of a head of group j
               attends to the rows listed in indices[s][j] that lie in [0, L) and in its
               causal window t <= L - s_q + s, each listing counting once
    returns o [s_q][h_q][d_h], lse [s_q][h_q]  (float64; o = 0, lse = -inf with no row)
    """
    q_nope = np.asarray(q_nope, F64)
    q_rope = np.asarray(q_rope, F64)
    s_q, h_q, d_h = q_nope.shape
    gr = np.asarray(group_rows[:length], F64)
    k_r = gr[:, 2 * g * d_h:]
    idx = np.asarray(indices)
    o = np.zeros((s_q, h_q, d_h), F64)
    lse = np.full((s_q, h_q), -np.inf, F64)
    for j in range(g):
        heads = _heads_of_group(j, h_q, g)
        k_j = np.concatenate([gr[:, j * d_h:(j + 1) * d_h], k_r], axis=1)
        v_j = gr[:, (g + j) * d_h:(g + j + 1) * d_h]
        for s in range(s_q):
            n = visible_rows(length, s_q, s)
            sel = np.array([int(t) for t in idx[s, j] if 0 <= t < n], dtype=np.int64)
            q = np.concatenate([q_nope[s, heads], q_rope[s, heads]], axis=1)
            o[s, heads], lse[s, heads] = _softmax_attend(scale * (q @ k_j[sel].T), v_j[sel])
    return o, lse
