"""The single-launch pipeline (sparge_topk_attn_fused) against the separate launches.

The fused kernel runs the preparation pass, the pooled scores, the selection and the
attention as phases of one cooperative grid, with the same device code as the
separate kernels, so its output, block mask and counters must equal those of
sparge_topk_attn bit for bit: on ragged and boundary lengths, both head sizes, both
input types, every supported option (int8 Q.K^T, fp16 P.V, filter on and off, per-head
knobs), every width of the selector (N up to 131072) and the full 8K and 128K
workloads.  A second call checks that the kernel's own reset of its work counters
and statistics leaves nothing behind.  Small shapes are also checked against the
oracle directly, to the bars of the separate path.

The entry point is not in the library: its first run on the GPU (the first case
below) returned a HIP error and left the GPU faulted, and no cause was found in the
kernel by reading it.  These tests stay, skipped, as the acceptance bar for a
single-launch path.
"""
import sys

import numpy as np
import pytest
import torch

import block_sparse_quantized_amd as bsq
from block_sparse_quantized_amd import synth
from oracle import sparge_oracle as so
from test_gpu_parity import TOL16, f64, oracle_outputs, oracle_predict, unexcused_mismatches

pytestmark = [pytest.mark.gpu,
              pytest.mark.skip(reason="single-launch entry point taken out: its first GPU run left the GPU faulted, cause not found")]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def same_as_separate(q, k, v, topk, causal, tag, **kw):
    say(f"[fused] {tag}: B,H,N,D={tuple(q.shape)} {q.dtype} causal={causal} {kw}")
    want, wmask, wst = bsq.sparge_topk_attn(q, k, v, topk, causal, return_mask=True, stats=True, **kw)
    got, gmask, gst = bsq.sparge_topk_attn_fused(q, k, v, topk, causal, return_mask=True, stats=True,
                                                 **kw)
    torch.cuda.synchronize()
    assert torch.equal(gmask, wmask), f"{tag}: masks differ"
    assert gst == wst, f"{tag}: counters differ: {gst} vs {wst}"
    assert torch.equal(got, want), f"{tag}: outputs differ, max |d| = " \
        f"{(got.float() - want.float()).abs().max().item():.3e}"
    again = bsq.sparge_topk_attn_fused(q, k, v, topk, causal, **kw)
    torch.cuda.synchronize()
    assert torch.equal(again, want), f"{tag}: second call differs"
    say(f"[fused] {tag}: identical, density {wmask.float().mean().item():.3f}, stats {wst}")


CASES = [  # (H, N, D, dtype, causal, options)
    (2, 1, 64, torch.bfloat16, True, dict()),
    (2, 64, 128, torch.float16, False, dict()),
    (3, 129, 64, torch.bfloat16, False, dict(filter_on=False)),
    (4, 1000, 128, torch.bfloat16, True, dict()),
    (3, 2500, 64, torch.bfloat16, False, dict(qk_int8=True, pv_fp16=True)),
    (2, 777, 128, torch.float16, True, dict(qk_int8=True)),
    (2, 3001, 128, torch.float16, False, dict(pv_fp16=True)),
    (8, 8192, 128, torch.bfloat16, True, dict(qk_int8=True, pv_fp16=True)),
    (4, 3000, 64, torch.bfloat16, True, dict(head_select=[0.2, 0.5, 0.8, 1.0],
                                             head_sim_threshold=[0.1, 0.3, -1.0, 0.1],
                                             head_filter_lambda=[-10.0, -5.0, -20.0, -8.0])),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_matches_separate_launches(dev, case):
    H, N, D, dtype, causal, kw = CASES[case]
    wl = synth.workload("tiny", H=H, N=N, D=D, dtype=dtype)
    q, k, v = synth.make_qkv(wl, device=dev)
    same_as_separate(q, k, v, 0.5, causal, f"case {case}", **kw)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N", [20000, 40000, 100000])
def test_fused_selector_widths(dev, N):
    """Block rows of up to 2048 candidate blocks (every width of the selector past the
    small cases above), one head."""
    wl = synth.workload("llm128k", H=1, N=N)
    q, k, v = synth.make_qkv(wl, device=dev)
    same_as_separate(q, k, v, wl.topk, True, f"N={N}", qk_int8=True, pv_fp16=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llm8k", "llm128k"])
def test_fused_full_workload(dev, name):
    """The full workloads, on the options bench.py times for them."""
    wl = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(wl, device=dev)
    same_as_separate(q, k, v, wl.topk, wl.causal, name, filter_on=wl.filter_on,
                     qk_int8=wl.qk_int8, pv_fp16=wl.pv_fp16)


@pytest.mark.parametrize("N,D,causal", [(1, 64, True), (65, 128, False), (129, 64, True),
                                        (1000, 128, True), (1000, 64, False)])
def test_fused_small_shapes_match_oracle(dev, N, D, causal):
    """The fused call against the oracle: mask bit-exact, output within the 16-bit bar."""
    wl = synth.workload("tiny", H=2, N=N, D=D, dtype=torch.bfloat16)
    q, k, v = synth.make_qkv(wl, device=dev)
    say(f"[fused] oracle N={N} D={D} causal={causal}")
    out, gm = bsq.sparge_topk_attn_fused(q, k, v, 0.5, causal, return_mask=True)
    torch.cuda.synchronize()
    om, infos = oracle_predict(q, k, so.OracleParams(topk=0.5, causal=causal))
    bad, exc = unexcused_mismatches(gm.cpu().numpy(), om, infos)
    assert bad == 0 and exc == 0
    ref, _ = oracle_outputs(q, k, v, om, causal, lam=-10.0)
    err = np.abs(f64(out) - ref).max()
    say(f"[fused] oracle N={N} D={D} causal={causal}: density {om.mean():.3f}, err {err:.3e}")
    assert err < TOL16


def test_fused_rejects_what_it_does_not_cover(dev):
    wl = synth.workload("tiny", H=1, N=300, D=64, dtype=torch.float32)
    q, k, v = synth.make_qkv(wl, device=dev)
    with pytest.raises(bsq.SpargeError) as e:
        bsq.sparge_topk_attn_fused(q, k, v, 0.5, True)
    assert e.value.status == -5
