"""ctypes binding of libgqla (include/gqla.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels.  Torch is
used for device memory and the current stream: tensors are passed as raw
device pointers plus element strides.  There is no fallback: if the built
library is missing, or a call returns a non-zero status, this module raises.

Method: "GQLA: Group-Query Latent Attention for Hardware-Adaptive LLM
Decoding", technical summary section 2 (the MQA-absorb and GQA decode paths
over the same group-indexed up-projections).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgqla.so")

BF16, F32 = 0, 1
ABSORB, GQA, SPARSE = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20   # GQLA_NOALLOC_SCRATCH_BYTES
STATUS = {0: "GQLA_OK", 1: "GQLA_ERR_INVALID_ARG", 2: "GQLA_ERR_UNSUPPORTED", 3: "GQLA_ERR_WORKSPACE", 4: "GQLA_ERR_HIP"}

EXPORTS = ("gqla_workspace_size", "gqla_plan_splits", "gqla_plan_splits_lens", "gqla_expand_groups", "gqla_decode_absorb",
           "gqla_decode_gqa", "gqla_decode_gqa_noalloc", "gqla_decode_gqa_sparse", "gqla_append_rows", "gqla_select_path", "gqla_measure_peaks",
           "gqla_set_kernel_events", "gqla_status_string", "gqla_last_error")


class Shape(ctypes.Structure):
    """Mirror of struct gqla_shape."""

    _fields_ = [("h_q", ctypes.c_int32), ("g", ctypes.c_int32), ("r_kv", ctypes.c_int32),
                ("d_r", ctypes.c_int32), ("d_h", ctypes.c_int32), ("s_q", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class PathChoice(ctypes.Structure):
    """Mirror of struct gqla_path_choice."""

    _fields_ = [("path", ctypes.c_int32), ("s_q", ctypes.c_int32), ("compute_bound", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("tokens_per_s", ctypes.c_double)]


class GQLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgqla.so (once) and declare its signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m latent_kv_cache_amd.build` "
                           "(or __graft_entry__.build()) first")
    # torch first: its bundled HIP runtime then satisfies the library's libamdhip64.so.7
    # dependency, so device pointers, streams and events are shared with one runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    c_i32, c_i64, c_vp, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    sp = ctypes.POINTER(Shape)
    lib.gqla_workspace_size.argtypes = [sp, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_sz)]
    lib.gqla_plan_splits.argtypes = [sp, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]
    lib.gqla_plan_splits_lens.argtypes = [sp, c_i32, c_i32, c_i32, c_vp, ctypes.POINTER(c_i32), ctypes.POINTER(c_i32),
                                          ctypes.POINTER(c_i32)]
    lib.gqla_expand_groups.argtypes = [sp, c_i32, c_i32, c_vp, c_i64, c_vp, c_vp, c_vp, c_i32, c_vp, c_i64, c_vp]
    lib.gqla_decode_absorb.argtypes = [sp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp,
                                       c_vp, c_sz, c_i32, c_vp]
    lib.gqla_decode_gqa.argtypes = [sp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp, c_sz,
                                    c_i32, c_vp]
    lib.gqla_decode_gqa_noalloc.argtypes = [sp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_vp, c_i32, c_vp]
    lib.gqla_decode_gqa_sparse.argtypes = [sp, c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_vp, c_vp,
                                           c_vp, c_sz, c_i32, c_vp]
    lib.gqla_append_rows.argtypes = [sp, c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, ctypes.c_float, c_vp, c_vp, c_i64,
                                     c_vp, c_vp, c_vp, c_i64, c_vp]
    lib.gqla_select_path.argtypes = [sp, c_i32, c_i64, ctypes.c_double, ctypes.c_double, ctypes.POINTER(PathChoice)]
    lib.gqla_measure_peaks.argtypes = [c_vp, c_sz, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                       c_vp]
    lib.gqla_set_kernel_events.argtypes = [c_vp, c_vp]
    for name in ("gqla_workspace_size", "gqla_plan_splits", "gqla_plan_splits_lens", "gqla_expand_groups", "gqla_decode_absorb",
                 "gqla_decode_gqa", "gqla_decode_gqa_noalloc", "gqla_decode_gqa_sparse", "gqla_append_rows", "gqla_select_path", "gqla_measure_peaks",
                 "gqla_set_kernel_events"):
        getattr(lib, name).restype = ctypes.c_int
    lib.gqla_status_string.argtypes = [ctypes.c_int]
    lib.gqla_status_string.restype = ctypes.c_char_p
    lib.gqla_last_error.argtypes = []
    lib.gqla_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().gqla_last_error().decode()
        raise GQLAError(status, msg)


def make_shape(h_q: int, g: int, r_kv: int, d_r: int, d_h: int, s_q: int, scale: Optional[float] = None,
               dtype: int = BF16) -> Shape:
    if scale is None:
        scale = 1.0 / math.sqrt(d_h + d_r)
    return Shape(h_q, g, r_kv, d_r, d_h, s_q, scale, dtype)


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def workspace_size(shape: Shape, path: int, batch: int, max_ctx: int, num_splits: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check(load().gqla_workspace_size(ctypes.byref(shape), path, batch, max_ctx, num_splits, ctypes.byref(n)))
    return int(n.value)


def plan_splits(shape: Shape, path: int, batch: int, max_ctx: int, num_splits: int = 0) -> Tuple[int, int]:
    n, c = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().gqla_plan_splits(ctypes.byref(shape), path, batch, max_ctx, num_splits, ctypes.byref(n),
                                   ctypes.byref(c)))
    return int(n.value), int(c.value)


def plan_splits_lens(shape: Shape, path: int, ctx_lens, max_ctx: int) -> Tuple[int, int, int]:
    """gqla_plan_splits_lens over host context lengths (any int sequence or array):
    returns (num_splits to pass to the decode call, n_split, chunk)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(ctx_lens, dtype=np.int32))
    w, n, c = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    ptr = lens.ctypes.data if lens.size else None
    _check(load().gqla_plan_splits_lens(ctypes.byref(shape), path, int(lens.size), max_ctx, ptr, ctypes.byref(w),
                                        ctypes.byref(n), ctypes.byref(c)))
    return int(w.value), int(n.value), int(c.value)


def set_kernel_events(before=None, after=None) -> None:
    """Record two torch.cuda.Event objects around the main attention kernel of later decode
    calls on this thread (None, None turns it off).  The events must already exist on the
    device, i.e. have been recorded once."""
    b = None if before is None else int(before.cuda_event)
    a = None if after is None else int(after.cuda_event)
    _check(load().gqla_set_kernel_events(b, a))


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _rows(t, width: int) -> Tuple[int, int]:
    """(batch stride in elements, max_ctx) of a [B][S][width] cache tensor with packed rows."""
    if t.dim() != 3 or t.shape[2] != width or t.stride(2) != 1 or t.stride(1) != width:
        raise ValueError(f"cache tensor must be [B][S][{width}] with packed rows, got {tuple(t.shape)} "
                         f"strides {t.stride()}")
    return int(t.stride(0)), int(t.shape[1])


def _torch_dtype(shape: Shape):
    import torch
    if shape.dtype == BF16:
        return torch.bfloat16
    if shape.dtype == F32:
        return torch.float32
    raise ValueError(f"shape.dtype {shape.dtype} is neither BF16 ({BF16}) nor F32 ({F32})")


def _validate(device, **specs) -> None:
    """Check tensors before any library call: each spec is (tensor, expected shape, dtype);
    a tensor must have exactly that shape and dtype, be contiguous, and live on `device`
    (a CUDA device).  A None tensor is skipped.  Raises ValueError naming the argument."""
    for name, (t, want_shape, want_dtype) in specs.items():
        if t is None:
            continue
        if tuple(t.shape) != tuple(want_shape):
            raise ValueError(f"{name} must have shape {tuple(want_shape)}, got {tuple(t.shape)}")
        if t.dtype != want_dtype:
            raise ValueError(f"{name} must be {want_dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, (t, _, _) in specs.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} is on {t.device}; every tensor of the call must be on the cache's "
                             f"CUDA device ({device})")


def _cache(name: str, t, shape: Shape, width: int) -> Tuple[int, int, int]:
    """(batch, batch stride, max_ctx) of a cache tensor, checked for dtype and CUDA placement."""
    if t.dtype != _torch_dtype(shape):
        raise ValueError(f"{name} must be {_torch_dtype(shape)} (shape.dtype), got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor, got {t.device}")
    bs, max_ctx = _rows(t, width)
    return int(t.shape[0]), bs, max_ctx


def _decode_specs(shape: Shape, batch: int, q_nope, q_rope, ctx_lens, out, lse, workspace=None):
    import torch
    dt = _torch_dtype(shape)
    q = (batch, shape.s_q, shape.h_q)
    specs = dict(q_nope=(q_nope, q + (shape.d_h,), dt), q_rope=(q_rope, q + (shape.d_r,), dt),
                 ctx_lens=(ctx_lens, (batch,), torch.int32), out=(out, q + (shape.d_h,), dt),
                 lse=(lse, q, torch.float32))
    if workspace is not None:
        specs["workspace"] = (workspace, (workspace.numel(),), workspace.dtype)
    return specs


def alloc_workspace(shape: Shape, path: int, batch: int, max_ctx: int, num_splits: int = 0, device=None):
    import torch
    n = workspace_size(shape, path, batch, max_ctx, num_splits)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device or "cuda")


def expand_groups(shape: Shape, latent, w_uk, w_uv, ctx_lens, group_cache, row_begin: int = 0, stream=None):
    """Write group rows [row_begin, L_b) of group_cache [B][S][2 g d_h + d_r] from latent [B][S][r_kv + d_r]."""
    import torch
    batch, lbs, max_ctx = _cache("latent", latent, shape, shape.r_kv + shape.d_r)
    gb, gbs, gctx = _cache("group_cache", group_cache, shape, 2 * shape.g * shape.d_h + shape.d_r)
    if gb != batch or gctx < max_ctx:
        raise ValueError("group_cache must hold as many sequences and at least as many rows as latent")
    w = (shape.g, shape.d_h, shape.r_kv)
    _validate(latent.device, w_uk=(w_uk, w, latent.dtype), w_uv=(w_uv, w, latent.dtype),
              ctx_lens=(ctx_lens, (batch,), torch.int32), group_cache=(group_cache, group_cache.shape, latent.dtype))
    _check(load().gqla_expand_groups(ctypes.byref(shape), latent.shape[0], max_ctx, _ptr(latent), lbs, _ptr(w_uk),
                                     _ptr(w_uv), _ptr(ctx_lens), row_begin, _ptr(group_cache), gbs, _stream(stream)))


def decode_absorb(shape: Shape, q_nope, q_rope, w_uk, w_uv, latent, ctx_lens, out, lse=None, workspace=None,
                  num_splits: int = 0, stream=None):
    """MQA-absorb decode into out [B][s_q][h_q][d_h] (and lse [B][s_q][h_q] if given)."""
    batch, lbs, max_ctx = _cache("latent", latent, shape, shape.r_kv + shape.d_r)
    w = (shape.g, shape.d_h, shape.r_kv)
    _validate(latent.device, w_uk=(w_uk, w, latent.dtype), w_uv=(w_uv, w, latent.dtype),
              **_decode_specs(shape, batch, q_nope, q_rope, ctx_lens, out, lse, workspace))
    if workspace is None:
        workspace = alloc_workspace(shape, ABSORB, batch, max_ctx, num_splits, latent.device)
    _check(load().gqla_decode_absorb(ctypes.byref(shape), batch, max_ctx, _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                     _ptr(w_uv), _ptr(latent), lbs, _ptr(ctx_lens), _ptr(out), _ptr(lse),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), num_splits,
                                     _stream(stream)))
    return out


def decode_gqa(shape: Shape, q_nope, q_rope, group_cache, ctx_lens, out, lse=None, workspace=None,
               num_splits: int = 0, stream=None):
    """GQA decode over expanded rows into out [B][s_q][h_q][d_h] (and lse if given)."""
    batch, gbs, max_ctx = _cache("group_cache", group_cache, shape, 2 * shape.g * shape.d_h + shape.d_r)
    _validate(group_cache.device, **_decode_specs(shape, batch, q_nope, q_rope, ctx_lens, out, lse, workspace))
    if workspace is None:
        workspace = alloc_workspace(shape, GQA, batch, max_ctx, num_splits, group_cache.device)
    _check(load().gqla_decode_gqa(ctypes.byref(shape), batch, max_ctx, _ptr(q_nope), _ptr(q_rope),
                                  _ptr(group_cache), gbs, _ptr(ctx_lens), _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), num_splits, _stream(stream)))
    return out


def decode_gqa_noalloc(shape: Shape, q_nope, q_rope, group_cache, ctx_lens, out, lse=None, num_splits: int = 0,
                       stream=None):
    """decode_gqa with the split-K partials in the library's static device scratch (no
    workspace, no allocation by the library; overlapping calls on one device race)."""
    batch, gbs, max_ctx = _cache("group_cache", group_cache, shape, 2 * shape.g * shape.d_h + shape.d_r)
    _validate(group_cache.device, **_decode_specs(shape, batch, q_nope, q_rope, ctx_lens, out, lse))
    _check(load().gqla_decode_gqa_noalloc(ctypes.byref(shape), batch, max_ctx, _ptr(q_nope), _ptr(q_rope),
                                          _ptr(group_cache), gbs, _ptr(ctx_lens), _ptr(out), _ptr(lse), num_splits,
                                          _stream(stream)))
    return out


def decode_gqa_sparse(shape: Shape, q_nope, q_rope, group_cache, ctx_lens, indices, out, lse=None, workspace=None,
                      num_splits: int = 0, stream=None):
    """Sparse GQLA decode: query token s of group j attends to the rows listed in
    indices [B][s_q][g][topk] (int32; -1 pads) of group_cache [B][S][2 g d_h + d_r]."""
    import torch
    batch, gbs, max_ctx = _cache("group_cache", group_cache, shape, 2 * shape.g * shape.d_h + shape.d_r)
    if indices.dim() != 4 or tuple(indices.shape[:3]) != (batch, shape.s_q, shape.g) or not indices.is_contiguous():
        raise ValueError(f"indices must be a contiguous [B][s_q][g][topk] tensor, got {tuple(indices.shape)}")
    topk = int(indices.shape[3])
    _validate(group_cache.device, indices=(indices, indices.shape, torch.int32),
              **_decode_specs(shape, batch, q_nope, q_rope, ctx_lens, out, lse, workspace))
    if workspace is None:
        workspace = alloc_workspace(shape, SPARSE, batch, topk, num_splits, group_cache.device)
    _check(load().gqla_decode_gqa_sparse(ctypes.byref(shape), batch, max_ctx, _ptr(q_nope), _ptr(q_rope),
                                         _ptr(group_cache), gbs, _ptr(ctx_lens), _ptr(indices), topk, _ptr(out),
                                         _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         num_splits, _stream(stream)))
    return out


def append_rows(shape: Shape, c_new, kr_new, ctx_lens, latent, q_rope_raw=None, q_rope_out=None,
                rope_theta: float = 10000.0, w_uk=None, w_uv=None, group_cache=None, stream=None):
    """Decode-step append: write the s_q new rows of every sequence into latent [B][S][r_kv + d_r]
    (c_new [B][s_q][r_kv], kr_new [B][s_q][d_r] rotated at t = L_b - s_q + s), rotate q_rope_raw
    into q_rope_out, and expand the new rows into group_cache [B][S][2 g d_h + d_r] if given."""
    import torch
    batch, lbs, max_ctx = _cache("latent", latent, shape, shape.r_kv + shape.d_r)
    gbs = 0
    if group_cache is not None:
        gb, gbs, gctx = _cache("group_cache", group_cache, shape, 2 * shape.g * shape.d_h + shape.d_r)
        if gb != batch or gctx < max_ctx:
            raise ValueError("group_cache must hold as many sequences and at least as many rows as latent")
    dt = latent.dtype
    qr = (batch, shape.s_q, shape.h_q, shape.d_r)
    w = (shape.g, shape.d_h, shape.r_kv)
    _validate(latent.device, c_new=(c_new, (batch, shape.s_q, shape.r_kv), dt),
              kr_new=(kr_new, (batch, shape.s_q, shape.d_r), dt), ctx_lens=(ctx_lens, (batch,), torch.int32),
              q_rope_raw=(q_rope_raw, qr, dt), q_rope_out=(q_rope_out, qr, dt),
              w_uk=(w_uk, w, dt), w_uv=(w_uv, w, dt),
              group_cache=(group_cache, None if group_cache is None else group_cache.shape, dt))
    _check(load().gqla_append_rows(ctypes.byref(shape), latent.shape[0], max_ctx, _ptr(c_new), _ptr(kr_new),
                                   _ptr(q_rope_raw), _ptr(q_rope_out), float(rope_theta), _ptr(ctx_lens),
                                   _ptr(latent), lbs, _ptr(w_uk), _ptr(w_uv), _ptr(group_cache), gbs,
                                   _stream(stream)))


def select_path(shape: Shape, batch: int, total_ctx: int, peak_flops: float, peak_bytes_per_s: float) -> PathChoice:
    """Roofline choice of (path, s_q <= shape.s_q) for a step over contexts summing to total_ctx."""
    ch = PathChoice()
    _check(load().gqla_select_path(ctypes.byref(shape), batch, total_ctx, float(peak_flops), float(peak_bytes_per_s),
                                   ctypes.byref(ch)))
    return ch


def measure_peaks(scratch, stream=None) -> Tuple[float, float]:
    """(HBM read bytes/s, dense bf16 MFMA flop/s) of the current device; scratch is a device
    tensor of at least 64 MiB whose contents are overwritten.  Waits for the measurement."""
    bw, fl = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(load().gqla_measure_peaks(_ptr(scratch), scratch.numel() * scratch.element_size(), ctypes.byref(bw),
                                     ctypes.byref(fl), _stream(stream)))
    return bw.value, fl.value
