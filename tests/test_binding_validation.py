"""The Python binding checks every tensor (shape, dtype, contiguity, device) before it
calls the library, so a mistaken argument raises ValueError instead of reaching a
kernel.  CPU-only: the checks run on CPU tensors (which then fail the device check)."""
import pytest

torch = pytest.importorskip("torch")

from latent_kv_cache_amd import gqla  # noqa: E402

SH = gqla.make_shape(128, 8, 512, 64, 128, 2)
B = 3


def good():
    q = (B, 2, 128)
    return dict(q_nope=torch.zeros(q + (128,), dtype=torch.bfloat16), q_rope=torch.zeros(q + (64,), dtype=torch.bfloat16),
                ctx_lens=torch.zeros(B, dtype=torch.int32), out=torch.zeros(q + (128,), dtype=torch.bfloat16),
                lse=torch.zeros(q, dtype=torch.float32))


def specs(**over):
    a = good()
    a.update(over)
    return gqla._decode_specs(SH, B, a["q_nope"], a["q_rope"], a["ctx_lens"], a["out"], a["lse"])


def test_correct_tensors_fail_only_on_device():
    with pytest.raises(ValueError, match="CUDA device"):
        gqla._validate(torch.device("cuda", 0), **specs())


@pytest.mark.parametrize("over,msg", [
    (dict(q_nope=torch.zeros((B, 1, 128, 128), dtype=torch.bfloat16)), "q_nope must have shape"),
    (dict(q_rope=torch.zeros((B, 2, 128, 32), dtype=torch.bfloat16)), "q_rope must have shape"),
    (dict(ctx_lens=torch.zeros(B, dtype=torch.int64)), "ctx_lens must be torch.int32"),
    (dict(ctx_lens=torch.zeros(B + 1, dtype=torch.int32)), "ctx_lens must have shape"),
    (dict(out=torch.zeros((B, 2, 128, 128), dtype=torch.float32)), "out must be torch.bfloat16"),
    (dict(out=torch.zeros((B, 2, 64, 128), dtype=torch.bfloat16)), "out must have shape"),
    (dict(lse=torch.zeros((B, 2, 128), dtype=torch.bfloat16)), "lse must be torch.float32"),
    (dict(q_nope=torch.zeros((B, 2, 128, 256), dtype=torch.bfloat16)[..., ::2]), "q_nope must be contiguous"),
])
def test_mismatch_raises(over, msg):
    with pytest.raises(ValueError, match=msg):
        gqla._validate(torch.device("cuda", 0), **specs(**over))


def test_lse_optional():
    s = specs(lse=None)
    with pytest.raises(ValueError, match="CUDA device"):
        gqla._validate(torch.device("cuda", 0), **s)


def test_cache_dtype_and_device():
    lat = torch.zeros((B, 64, 576), dtype=torch.float32)
    with pytest.raises(ValueError, match="shape.dtype"):
        gqla._cache("latent", lat, SH, 576)
    with pytest.raises(ValueError, match="CUDA tensor"):
        gqla._cache("latent", lat.to(torch.bfloat16), SH, 576)
    with pytest.raises(ValueError, match="CUDA tensor"):
        gqla.decode_gqa(SH, *[good()[k] for k in ("q_nope", "q_rope")],
                        torch.zeros((B, 64, 2112), dtype=torch.bfloat16), good()["ctx_lens"], good()["out"])
