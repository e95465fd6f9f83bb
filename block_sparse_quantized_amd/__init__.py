"""SpargeAttn hot path for AMD Instinct MI355X (gfx950): Python binding.

Thin ctypes layer over ``libsparge.so`` (C ABI in ``include/sparge.h``).  It only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors, workspace) and the current
stream.  There is no fallback: if the library is not built, or a tensor is not on
a GPU, the calls raise.

Functions share the C names:
    sparge_topk_attn(q, k, v, topk=0.5, is_causal=False, ...)
    sparge_topk_attn_noalloc(q, k, v, topk=0.5, is_causal=False, ...)
    sparge_cdf_attn(q, k, v, cdf_threshold, is_causal=False, ...)
    block_sparse_attn(q, k, v, mask_id=None, ...)
    sparge_predict_mask(q, k, topk, is_causal, ...)
    sparge_quantize_qk(q, k)
    sparge_hilbert_perm3d(T, H, W)
    sparge_reorder(x, perm, offset, count, inverse=False)
    sparge_workspace_bytes(B, H, N, D, dtype)
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

from ._lib import (  # noqa: F401
    SPARGE_BF16,
    SPARGE_F16,
    SPARGE_F32,
    SpargeError,
    SpargeOpts,
    SpargeStats,
    SpargeTensor,
    lib,
    lib_path,
)

__all__ = [
    "sparge_topk_attn",
    "sparge_topk_attn_noalloc",
    "sparge_cdf_attn",
    "block_sparse_attn",
    "sparge_predict_mask",
    "sparge_quantize_qk",
    "sparge_hilbert_perm3d",
    "sparge_reorder",
    "sparge_workspace_bytes",
    "SpargeError",
]

_DTYPES = {torch.float32: SPARGE_F32, torch.float16: SPARGE_F16, torch.bfloat16: SPARGE_BF16}


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().sparge_status_str(status).decode()
        raise SpargeError(status, f"{what}: {msg} (status {status})")


def _desc(t: torch.Tensor, name: str) -> SpargeTensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dim() != 4:
        raise ValueError(f"{name} must have shape (B, H, N, D)")
    if t.dtype not in _DTYPES:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    B, H, N, D = t.shape
    sB, sH, sN, _ = t.stride()
    return SpargeTensor(t.data_ptr(), _DTYPES[t.dtype], 0, B, H, N, D, sB, sH, sN)


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def sparge_workspace_bytes(B: int, H: int, N: int, D: int, dtype: torch.dtype) -> int:
    n = lib().sparge_workspace_bytes(B, H, N, D, _DTYPES[dtype], None)
    if n == 0:
        raise ValueError("invalid shape or dtype for sparge_workspace_bytes")
    return int(n)


def _workspace(q: torch.Tensor, workspace: Optional[torch.Tensor]) -> Tuple[torch.Tensor, int]:
    need = sparge_workspace_bytes(*q.shape, q.dtype)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    return workspace, workspace.numel() * workspace.element_size()


def _head_array(vals, H: int, name: str):
    """A host double array of H per-head values (kept alive by the caller), or None."""
    if vals is None:
        return None
    vals = [float(x) for x in vals]
    if len(vals) != H:
        raise ValueError(f"{name} needs {H} values (one per head), got {len(vals)}")
    return (ctypes.c_double * H)(*vals)


def _opts(scale, sim_threshold, filter_lambda, filter_on, qk_int8, pv_fp16, mask_out, stats,
          prof=None, pv_fp8=False, heads=None):
    """sparge_opts plus the stats struct; ``heads`` = (H, select, sim_threshold,
    filter_lambda) per-head sequences (or None each); their ctypes arrays are kept on
    the returned struct so they outlive the call."""
    o = SpargeOpts()
    lib().sparge_default_opts(ctypes.byref(o))
    o.scale = 0.0 if scale is None else float(scale)
    o.sim_threshold = float(sim_threshold)
    o.filter_lambda = float(filter_lambda)
    o.filter_on = int(bool(filter_on))
    o.qk_int8 = int(bool(qk_int8))
    o.pv_fp16 = int(bool(pv_fp16))
    o.pv_fp8 = int(bool(pv_fp8))
    o.mask_out = None if mask_out is None else ctypes.c_void_p(mask_out.data_ptr())
    st = SpargeStats() if stats else None
    o.stats = ctypes.pointer(st) if st is not None else None
    if prof is not None:  # raw hipEvent_t handles (start, attention begin, attention end)
        o.prof_start, o.prof_attn_begin, o.prof_attn_end = prof
    if heads is not None:
        H, sel, th, lam = heads
        o._keep = [_head_array(sel, H, "head_select"), _head_array(th, H, "head_sim_threshold"),
                   _head_array(lam, H, "head_filter_lambda")]
        dbl = ctypes.POINTER(ctypes.c_double)
        o.head_select, o.head_sim_threshold, o.head_filter_lambda = (
            ctypes.cast(a, dbl) if a is not None else None for a in o._keep)
    return o, st


def _stats_dict(st: Optional[SpargeStats]) -> Optional[Dict[str, int]]:
    if st is None:
        return None
    return dict(valid_blocks=st.valid_blocks, kept_blocks=st.kept_blocks,
                group_updates=st.group_updates, skipped_updates=st.skipped_updates)


def _mask_shape(q: torch.Tensor):
    B, H, N, _ = q.shape
    return (B, H, (N + 127) // 128, (N + 63) // 64)


def _predicted_attn(fn, name, q, k, v, sel, is_causal, scale, sim_threshold, filter_lambda,
                    filter_on, qk_int8, pv_fp16, pv_fp8, return_mask, stats, out, workspace, prof,
                    head_select, head_sim_threshold, head_filter_lambda):
    if out is None:
        out = torch.empty_like(q)
    mask = torch.empty(_mask_shape(q), dtype=torch.uint8, device=q.device) if return_mask else None
    o, st = _opts(scale, sim_threshold, filter_lambda, filter_on, qk_int8, pv_fp16, mask, stats,
                  prof, pv_fp8, (q.shape[1], head_select, head_sim_threshold, head_filter_lambda))
    ws, nbytes = _workspace(q, workspace)
    dq, dk, dv, do = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    _check(fn(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(do),
              ctypes.c_double(sel), int(bool(is_causal)), ctypes.byref(o),
              ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes), _stream(q)), name)
    res = [out]
    if return_mask:
        res.append(mask)
    if stats:
        res.append(_stats_dict(st))
    return res[0] if len(res) == 1 else tuple(res)


def sparge_topk_attn(q, k, v, topk: float = 0.5, is_causal: bool = False, *, scale=None,
                     sim_threshold: float = 0.1, filter_lambda: float = -10.0,
                     filter_on: bool = True, qk_int8: bool = False, pv_fp16: bool = False,
                     pv_fp8: bool = False, return_mask: bool = False, stats: bool = False,
                     out=None, workspace=None, prof=None, head_select=None,
                     head_sim_threshold=None, head_filter_lambda=None):
    """Sparse attention with the on-the-fly block-mask predictor (two-stage filter).

    Returns ``out`` (same shape/dtype as q), plus the predicted uint8 block mask
    when ``return_mask`` and a counters dict when ``stats`` (which synchronises).
    ``head_*``: optional per-head sequences (H values) replacing topk,
    sim_threshold and filter_lambda head by head.
    """
    return _predicted_attn(lib().sparge_topk_attn, "sparge_topk_attn", q, k, v, topk, is_causal,
                           scale, sim_threshold, filter_lambda, filter_on, qk_int8, pv_fp16,
                           pv_fp8, return_mask, stats, out, workspace, prof, head_select,
                           head_sim_threshold, head_filter_lambda)


def sparge_topk_attn_noalloc(q, k, v, topk: float = 0.5, is_causal: bool = False, *, scale=None,
                             sim_threshold: float = 0.1, filter_lambda: float = -10.0,
                             filter_on: bool = True, qk_int8: bool = False, pv_fp16: bool = False,
                             pv_fp8: bool = False, return_mask: bool = False, stats: bool = False,
                             out=None):
    """``sparge_topk_attn`` on the library's own static device scratch (no workspace, no
    allocation in the call: for graph capture and loops that may not allocate).  Calls
    that overlap on one GPU race on that scratch; problems beyond it raise."""
    if out is None:
        out = torch.empty_like(q)
    mask = torch.empty(_mask_shape(q), dtype=torch.uint8, device=q.device) if return_mask else None
    o, st = _opts(scale, sim_threshold, filter_lambda, filter_on, qk_int8, pv_fp16, mask, stats,
                  None, pv_fp8)
    dq, dk, dv, do = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    _check(lib().sparge_topk_attn_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                                          ctypes.byref(do), ctypes.c_double(topk), int(bool(is_causal)),
                                          ctypes.byref(o), _stream(q)), "sparge_topk_attn_noalloc")
    res = [out]
    if return_mask:
        res.append(mask)
    if stats:
        res.append(_stats_dict(st))
    return res[0] if len(res) == 1 else tuple(res)


def sparge_cdf_attn(q, k, v, cdf_threshold: float, is_causal: bool = False, *, scale=None,
                    sim_threshold: float = 0.1, filter_lambda: float = -10.0,
                    filter_on: bool = True, qk_int8: bool = False, pv_fp16: bool = False,
                    pv_fp8: bool = False, return_mask: bool = False, stats: bool = False,
                    out=None, workspace=None, prof=None, head_select=None,
                    head_sim_threshold=None, head_filter_lambda=None):
    """Like ``sparge_topk_attn``, but each block row keeps the shortest ranked prefix of
    its candidate blocks whose compressed-softmax mass reaches ``cdf_threshold``."""
    return _predicted_attn(lib().sparge_cdf_attn, "sparge_cdf_attn", q, k, v, cdf_threshold,
                           is_causal, scale, sim_threshold, filter_lambda, filter_on, qk_int8,
                           pv_fp16, pv_fp8, return_mask, stats, out, workspace, prof, head_select,
                           head_sim_threshold, head_filter_lambda)


def block_sparse_attn(q, k, v, mask_id=None, *, scale=None, filter_lambda: float = -10.0,
                      filter_on: bool = False, qk_int8: bool = False, pv_fp16: bool = False,
                      pv_fp8: bool = False, stats: bool = False, out=None, workspace=None,
                      prof=None, head_filter_lambda=None):
    """Attention under a caller-given (B, H, ceil(N/128), ceil(N/64)) 0/1 block mask."""
    if out is None:
        out = torch.empty_like(q)
    mptr = None
    if mask_id is not None:
        if mask_id.device != q.device or tuple(mask_id.shape) != _mask_shape(q):
            raise ValueError(f"mask_id must be a {_mask_shape(q)} tensor on {q.device}")
        mask_id = mask_id.to(torch.uint8).contiguous()
        mptr = ctypes.c_void_p(mask_id.data_ptr())
    o, st = _opts(scale, 0.1, filter_lambda, filter_on, qk_int8, pv_fp16, None, stats, prof,
                  pv_fp8, (q.shape[1], None, None, head_filter_lambda))
    ws, nbytes = _workspace(q, workspace)
    dq, dk, dv, do = _desc(q, "q"), _desc(k, "k"), _desc(v, "v"), _desc(out, "out")
    _check(lib().block_sparse_attn(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), mptr,
                                   ctypes.byref(do), ctypes.byref(o), ctypes.c_void_p(ws.data_ptr()),
                                   ctypes.c_size_t(nbytes), _stream(q)), "block_sparse_attn")
    return (out, _stats_dict(st)) if stats else out


def sparge_predict_mask(q, k, topk: float = 0.5, is_causal: bool = False, *, scale=None,
                        sim_threshold: float = 0.1, stats: bool = False, workspace=None,
                        head_select=None, head_sim_threshold=None):
    """Stage 1 only: the predicted (B, H, ceil(N/128), ceil(N/64)) uint8 block mask."""
    mask = torch.empty(_mask_shape(q), dtype=torch.uint8, device=q.device)
    o, st = _opts(scale, sim_threshold, -10.0, True, False, False, None, stats,
                  heads=(q.shape[1], head_select, head_sim_threshold, None))
    ws, nbytes = _workspace(q, workspace)
    dq, dk = _desc(q, "q"), _desc(k, "k")
    _check(lib().sparge_predict_mask(ctypes.byref(dq), ctypes.byref(dk), ctypes.c_double(topk),
                                     int(bool(is_causal)), ctypes.byref(o),
                                     ctypes.c_void_p(mask.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                     ctypes.c_size_t(nbytes), _stream(q)), "sparge_predict_mask")
    return (mask, _stats_dict(st)) if stats else mask


def sparge_quantize_qk(q, k, workspace=None) -> Dict[str, torch.Tensor]:
    """int8 operands of the qk_int8 option: codes, steps and K block means."""
    B, H, N, D = q.shape
    dev = q.device
    res = dict(
        q_codes=torch.empty((B, H, N, D), dtype=torch.int8, device=dev),
        q_scales=torch.empty((B, H, (N + 31) // 32), dtype=torch.float32, device=dev),
        k_codes=torch.empty((B, H, N, D), dtype=torch.int8, device=dev),
        k_scales=torch.empty((B, H, (N + 63) // 64), dtype=torch.float32, device=dev),
        k_means=torch.empty((B, H, (N + 63) // 64, D), dtype=torch.float32, device=dev),
    )
    ws, nbytes = _workspace(q, workspace)
    dq, dk = _desc(q, "q"), _desc(k, "k")
    p = {n: ctypes.c_void_p(t.data_ptr()) for n, t in res.items()}
    _check(lib().sparge_quantize_qk(ctypes.byref(dq), ctypes.byref(dk), p["q_codes"], p["q_scales"],
                                    p["k_codes"], p["k_scales"], p["k_means"],
                                    ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(nbytes),
                                    _stream(q)), "sparge_quantize_qk")
    return res


def sparge_hilbert_perm3d(T: int, H: int, W: int) -> torch.Tensor:
    """Hilbert order of a T x H x W grid as an int32 CPU tensor (host computation)."""
    out = torch.empty(T * H * W, dtype=torch.int32)
    _check(lib().sparge_hilbert_perm3d(int(T), int(H), int(W),
                                       ctypes.c_void_p(out.data_ptr())), "sparge_hilbert_perm3d")
    return out


def sparge_reorder(x, perm, offset: int, count: int, inverse: bool = False, out=None):
    """Gather (or, with ``inverse``, scatter) token rows [offset, offset+count) by perm."""
    if out is None:
        out = torch.empty_like(x)
    if perm.device != x.device or perm.dtype != torch.int32:
        raise ValueError("perm must be an int32 tensor on the same device as x")
    perm = perm.contiguous()
    dx, dy = _desc(x, "x"), _desc(out, "out")
    _check(lib().sparge_reorder(ctypes.byref(dx), ctypes.byref(dy), ctypes.c_void_p(perm.data_ptr()),
                                ctypes.c_int64(offset), ctypes.c_int64(count), int(bool(inverse)),
                                _stream(x)), "sparge_reorder")
    return out
