"""Plant one mistake at a time in a copy of the oracle and check that some pin catches it (CPU only)."""
import importlib.util
import os
import types

import pytest

from tests.oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "gqla.py")).read()

# (description, original text, mutated text); each original must occur in the oracle source
MUTATIONS = [
    ("group map off by one", "return i // (h_q // g)", "return (i // (h_q // g) + 1) % g"),
    ("causal window too wide", "length - s_q + s + 1", "length - s_q + s + 2"),
    ("causal window too narrow", "length - s_q + s + 1", "length - s_q + s"),
    ("RoPE query term dropped", "q = np.concatenate([q_nope[s, heads], q_rope[s, heads]], axis=1)  # [heads][d_h + d_R]",
     "q = np.concatenate([q_nope[s, heads], 0 * q_rope[s, heads]], axis=1)"),
    ("key up-projection uses W_UV", "k_j = np.concatenate([c @ w_uk[j].T, k_r], axis=1)  # [L][d_h + d_R]",
     "k_j = np.concatenate([c @ w_uv[j].T, k_r], axis=1)"),
    ("softmax max not subtracted consistently", "w = np.exp(scores - m)", "w = np.exp(scores - 0.5 * m)"),
    ("lse uses log2", "(m + np.log(z))[:, 0]", "(m + np.log2(z))[:, 0]"),
    ("no normalisation", "return (w @ values) / z,", "return (w @ values),"),
    ("scale applied twice", "_softmax_attend(scale * (q @ k_j[:n].T), v_j[:n])",
     "_softmax_attend(scale * scale * (q @ k_j[:n].T), v_j[:n])"),
    ("value block order swapped in expansion", "out[:, (g + j) * d_h:(g + j + 1) * d_h] = c @ w_uv[j].T",
     "out[:, (g + j) * d_h:(g + j + 1) * d_h] = c @ w_uk[j].T"),
    ("merge weights not renormalised", "/ np.where(finite, z, 1.0)[..., None]", ""),
    ("RoPE pairs interleaved", "a, b = x[..., :half], x[..., half:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    ("RoPE frequency exponent halved", "freq = theta ** (-2.0 * np.arange(half, dtype=F64) / d)",
     "freq = theta ** (-1.0 * np.arange(half, dtype=F64) / d)"),
    ("RoPE turns the other way", "return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)",
     "return np.concatenate([a * cos + b * sin, -a * sin + b * cos], axis=-1)"),
    ("sparse rows past L kept", "sel = np.array([int(t) for t in idx[s, j] if 0 <= t < n], dtype=np.int64)",
     "sel = np.array([int(t) for t in idx[s, j] if 0 <= t < length + 1], dtype=np.int64)"),
    ("sparse duplicates collapsed", "sel = np.array([int(t) for t in idx[s, j] if 0 <= t < n], dtype=np.int64)",
     "sel = np.unique(np.array([int(t) for t in idx[s, j] if 0 <= t < n], dtype=np.int64))"),
    ("sparse lists of the wrong group", "sel = np.array([int(t) for t in idx[s, j] if 0 <= t < n], dtype=np.int64)",
     "sel = np.array([int(t) for t in idx[s, (j + 1) % g] if 0 <= t < n], dtype=np.int64)"),
    ("appended rows one position late", "pos = np.arange(length - s_q, length, dtype=np.int64)",
     "pos = np.arange(length - s_q + 1, length + 1, dtype=np.int64)"),
]


def _mutant(orig, new):
    assert SRC.count(orig) >= 1, orig
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(orig, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,orig,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_some_pin_catches(desc, orig, new):
    mod = _mutant(orig, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception:  # noqa: BLE001 - any failure of a pin counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin catches: {desc}"
