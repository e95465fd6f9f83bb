"""The allocation-free entry point (sparge_topk_attn_noalloc), through the C ABI.

It runs the kernels of sparge_topk_attn on the library's static per-GPU scratch, so
its outputs, masks and counters must equal sparge_topk_attn's bit for bit, call
after call, whatever the previous call left in the scratch: two calls in a row
here, the second on a smaller problem (and a third, larger again, with other
options).  Problems beyond the scratch are rejected before any work is queued.
"""
import ctypes

import pytest
import torch

import block_sparse_quantized_amd as bsq
from block_sparse_quantized_amd import _lib as L
from block_sparse_quantized_amd import synth


def _inputs(dev, H, N, D, seed):
    wl = synth.workload("llm8k", H=H, N=N, D=D, seed=seed)
    return synth.make_qkv(wl, device=dev)


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point(dev):
    cases = [  # (H, N, D, options): larger, then smaller, then larger with other options
        (8, 4000, 128, dict(qk_int8=True, pv_fp16=True)),
        (3, 777, 64, dict()),
        (16, 8192, 128, dict(qk_int8=True, pv_fp8=True)),
    ]
    for n, (H, N, D, kw) in enumerate(cases):
        q, k, v = _inputs(dev, H, N, D, seed=40 + n)
        want, wmask, wst = bsq.sparge_topk_attn(q, k, v, 0.5, True, return_mask=True, stats=True, **kw)
        got, gmask, gst = bsq.sparge_topk_attn_noalloc(q, k, v, 0.5, True, return_mask=True, stats=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(gmask, wmask), f"call {n}: masks differ"
        assert torch.equal(got, want), f"call {n}: outputs differ"
        assert gst == wst, f"call {n}: counters differ"
        # and without stats (no counter clearing), the same output again
        again = bsq.sparge_topk_attn_noalloc(q, k, v, 0.5, True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(again, want), f"call {n}: repeated call differs"
        print(f"noalloc call {n}: H={H} N={N} D={D} {kw}: identical, density "
              f"{wmask.float().mean().item():.3f}", flush=True)


def test_noalloc_rejects_problems_beyond_the_scratch():
    lib = L.lib()
    FAKE = 0x7f0000000000
    N, D, H = 131072, 128, 32
    ts = [L.SpargeTensor(FAKE + i * (1 << 36), L.SPARGE_BF16, 0, 1, H, N, D, H * N * D, N * D, D)
          for i in range(4)]
    r = lib.sparge_topk_attn_noalloc(*(ctypes.byref(t) for t in ts), 0.5, 1, None, None)
    assert r == -6                                   # SPARGE_E_WORKSPACE, nothing queued
    r = lib.sparge_topk_attn_noalloc(*(ctypes.byref(t) for t in ts), 1.5, 1, None, None)
    assert r == -4                                   # argument errors first
