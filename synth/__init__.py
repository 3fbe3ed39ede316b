"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side callers.

This package draws random numbers and rounds them to the storage dtype.  It
holds none of the attention arithmetic: no scores, no softmax, no
up-projection, no rotation.  Both the oracle and the HIP path receive the
arrays it returns, so they see bit-identical inputs.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    GQLAConfig,
    bf16_round,
    config,
    ctx_len,
    ctx_lens,
    latent_rows,
    queries,
    up_weights,
)
