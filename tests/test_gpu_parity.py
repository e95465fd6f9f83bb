"""GPU parity of the HIP path against the fp64 CPU oracle (needs an MI355X).

Bars: the block mask is bit-exact except documented near-ties (a mismatch at
(i, j) is excused only when s_ij lies within 1e-6 * max(1, scale * sum_c |qbar_ic
kbar_jc|) of the row's k-th largest candidate score, or a block's similarity lies
within 1e-6 of theta); outputs are within max-abs 2e-2 of the fp64 oracle for the
16-bit paths and 5e-2 for the int8 Q K^T path, plus, where the output is stored in
a 16-bit type, half an ulp of that type at the oracle's value (the storage rounding
of a correct fp32 result); the fp8 P.V path is gated element by element against
exact attention on its own logits by the bound derived from E4M3's rounding steps
(tests/fp8_bounds.py), and, after the int8 Q K^T, also against plain fp64 within
5e-2 plus that bound; int8 codes and block lists are bit-exact.  Full-size
workloads are checked on the whole mask and, in the launch configuration bench.py
times, on whole output tensors (8K, image, video) or one 32-row group per head.
"""

import math
import sys

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import block_sparse_quantized_amd as bsq
import fp8_bounds as fb
from oracle_pool import head_reference
from block_sparse_quantized_amd import synth
from oracle import sparge_oracle as so
from oracle.hilbert_ref import hilbert_cell_order

pytestmark = pytest.mark.gpu

TOL16 = 2e-2
TOL8 = 5e-2
TOLF8 = 2e-2     # fp8 P.V (exact logits) against the oracle's fp8 P.V simulation

_STORE = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}


def bar(ref, dtype, tol):
    """Elementwise bar: the path's tolerance plus the storage rounding of its output
    type at the oracle's value (half an ulp; none for fp32)."""
    return tol + fb.half_ulp(ref, _STORE[dtype])


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def rand_qkv(B, H, N, D, dtype, dev, seed, scale=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    out = [(torch.randn((B, H, N, D), generator=g) * scale).to(dtype).to(dev) for _ in range(3)]
    return out


def oracle_predict(q, k, params):
    """Per-head oracle masks and infos for (B, H, N, D) tensors."""
    qn, kn = f64(q), f64(k)
    B, H = qn.shape[:2]
    masks, infos = [], []
    for b in range(B):
        for h in range(H):
            m, info = so.predict_mask(qn[b, h], kn[b, h], params)
            masks.append(m)
            infos.append(info)
    nQ, nK = masks[0].shape
    return np.stack(masks).reshape(B, H, nQ, nK), infos


def unexcused_mismatches(gpu_mask, ora_mask, infos, theta=0.1):
    """Count mask mismatches not covered by the near-tie rule."""
    B, H, nQ, nK = ora_mask.shape
    g = gpu_mask.reshape(B * H, nQ, nK).astype(bool)
    o = ora_mask.reshape(B * H, nQ, nK)
    bad, excused = 0, 0
    for bh in range(B * H):
        diff = np.argwhere(g[bh] != o[bh])
        if diff.size == 0:
            continue
        info = infos[bh]
        S, valid = info["scores"], info["valid"]
        cand_all = valid & info["simk"][None, :]
        for i, j in diff:
            ok = abs(info["qsim"][i] - theta) <= 1e-6 or abs(info["ksim"][j] - theta) <= 1e-6
            if not ok and cand_all[i, j] and info["kcount"][i] > 0:
                srow = np.sort(S[i][cand_all[i]])[::-1]
                thr = srow[info["kcount"][i] - 1]
                mag = info["scale"] * np.abs(info["qmean"][i] * info["kmean"][j]).sum()
                ok = abs(S[i, j] - thr) <= 1e-6 * max(1.0, mag)
            if ok:
                excused += 1
            else:
                bad += 1
    return bad, excused


def oracle_mask_and_rows(q, k, gm, topk, causal):
    """The oracle's own block mask (the GPU mask must match it up to excused near-ties)
    and a (B, H, N) flag of the query rows whose block row is identical on both sides:
    outputs are compared on those rows, with the oracle's mask as its input."""
    om, infos = oracle_predict(q, k, so.OracleParams(topk=topk, causal=causal))
    g = gm.cpu().numpy().astype(bool)
    bad, exc = unexcused_mismatches(g, om, infos)
    assert bad == 0
    same = (g == om).all(axis=3)                                   # (B, H, nQ)
    N = q.shape[2]
    rows = np.repeat(same, so.BQ, axis=2)[:, :, :N]
    assert rows.mean() > 0.9
    return om, rows


def oracle_outputs(q, k, v, mask, causal, lam=None, scale=None):
    qn, kn, vn = f64(q), f64(k), f64(v)
    B, H = qn.shape[:2]
    out = np.zeros_like(qn)
    skipped = 0
    for b in range(B):
        for h in range(H):
            o, sk = so.attend_head(qn[b, h], kn[b, h], vn[b, h], mask[b, h], causal, scale=scale,
                                   lam=lam, return_skips=True)
            out[b, h] = o
            skipped += sum(len(x) for x in sk.values())
    return out, skipped


def all_groups(B, H, N):
    nQ = (N + 127) // 128
    return [(b, h, i, g) for b in range(B) for h in range(H) for i in range(nQ) for g in range(4)
            if 128 * i + 32 * g < N]


def fp8_gate(out, q, k, v, mask, causal, lam, qk8, groups=None):
    """The fp8 P.V output against exact attention on the path's own logits (the exact
    ones, or the int8 option's), element by element within the E4M3 bound B of
    tests/fp8_bounds.py; after the int8 Q.K^T also against plain fp64 within 5e-2 + B.
    groups: (b, h, block row, 32-row group) picks, default all.  Returns the largest
    error / bound ratio."""
    qn, kn, vn = f64(q), f64(k), f64(v)
    got = f64(out)
    _, _, N, D = qn.shape
    scale = 1.0 / math.sqrt(D)
    dt = _STORE[out.dtype]
    groups = all_groups(*qn.shape[:3]) if groups is None else groups
    heads, worst = {}, 0.0
    for (b, h, i, g) in groups:
        if (b, h) not in heads:
            i8, slack = None, 1e-4
            if qk8:
                q32, k32 = qn[b, h].astype(np.float32), kn[b, h].astype(np.float32)
                i8 = so.int8_qk_inputs(q32, k32)
                slack += fb.int8_logit_slack(q32, i8[4], scale)
            heads[(b, h)] = (i8, slack, np.abs(vn[b, h]).max(axis=0))
        i8, slack, vmax = heads[(b, h)]
        t0 = 128 * i + 32 * g
        t1 = min(N, t0 + 32, 128 * i + 128)
        js = np.flatnonzero(mask[b, h, i])
        Z = fb.group_logits(qn[b, h], kn[b, h], js, t0, t1, causal, scale, lam, i8)
        O, Bd = fb.fp8_bound(Z, vn[b, h], vmax, dt, slack)
        err = np.abs(got[b, h, t0:t1] - O)
        ratio = float((err / np.where(Bd > 0, Bd, 1.0)).max())
        assert np.all(err <= Bd), f"fp8 bound exceeded at b={b} h={h} i={i} g={g}: ratio {ratio:.3f}"
        worst = max(worst, ratio)
        if qk8:
            O64 = fb.exact_attention(fb.group_logits(qn[b, h], kn[b, h], js, t0, t1, causal, scale, lam),
                                     vn[b, h])
            assert np.all(np.abs(got[b, h, t0:t1] - O64) <= TOL8 + Bd)
    return worst


# ------------------------------------------------------------ block_sparse_attn

@pytest.mark.parametrize("N,D,dtype", [
    (64, 64, torch.bfloat16), (65, 128, torch.bfloat16), (127, 64, torch.float16),
    (129, 128, torch.bfloat16), (300, 64, torch.float32), (1000, 128, torch.bfloat16),
    (1, 64, torch.bfloat16), (513, 128, torch.float16)])
def test_block_sparse_attn_matches_oracle(dev, N, D, dtype):
    say(f"block_sparse_attn N={N} D={D} {dtype}")
    B, H = 2, 3
    q, k, v = rand_qkv(B, H, N, D, dtype, dev, seed=N + D)
    nQ, nK = so.num_blocks(N)
    g = torch.Generator().manual_seed(7)
    mask = (torch.rand((B, H, nQ, nK), generator=g) < 0.45).to(torch.uint8)
    mask[0, 0, 0] = 0                       # an empty block row -> zero output
    if nK > 1:
        mask[1, 2, :, -1] = 1               # ragged last K block kept
    out = bsq.block_sparse_attn(q, k, v, mask.to(dev))
    torch.cuda.synchronize()
    ref, _ = oracle_outputs(q, k, v, mask.numpy().astype(bool), causal=False)
    err = np.abs(f64(out) - ref).max()
    say(f"  max abs err {err:.3e}")
    assert err < TOL16
    assert np.all(f64(out)[0, 0, :min(N, 128)] == 0)


@pytest.mark.parametrize("D", [64, 128])
def test_block_sparse_dense_equals_sdpa(dev, D):
    B, H, N = 1, 4, 777
    q, k, v = rand_qkv(B, H, N, D, torch.bfloat16, dev, seed=3)
    out = bsq.block_sparse_attn(q, k, v, None)
    ref = F.scaled_dot_product_attention(q.double().cpu(), k.double().cpu(), v.double().cpu())
    err = (out.double().cpu() - ref).abs().max().item()
    say(f"dense D={D} err {err:.3e}")
    assert err < TOL16


def test_block_sparse_stats_and_lists(dev):
    B, H, N, D = 1, 2, 1000, 64
    q, k, v = rand_qkv(B, H, N, D, torch.bfloat16, dev, seed=5)
    nQ, nK = so.num_blocks(N)
    mask = (torch.rand((B, H, nQ, nK), generator=torch.Generator().manual_seed(1)) < 0.3).to(torch.uint8)
    out, st = bsq.block_sparse_attn(q, k, v, mask.to(dev), stats=True)
    assert st["valid_blocks"] == B * H * nQ * nK
    assert st["kept_blocks"] == int(mask.sum())
    groups = sum(int(mask[0, h, i].sum()) * len(range(128 * i, min(N, 128 * i + 128), 32))
                 for h in range(H) for i in range(nQ))
    assert st["group_updates"] == groups and st["skipped_updates"] == 0


# ------------------------------------------------------------------ predictor

@pytest.mark.parametrize("N,D,causal", [(512, 64, False), (1000, 128, True), (1000, 64, False),
                                        (65, 64, True), (4000, 128, True)])
def test_predict_mask_bit_exact(dev, N, D, causal):
    wl = synth.workload("llm8k", H=4, N=N, D=D)
    q, k, _ = synth.make_qkv(wl, device=dev)
    for topk in (0.3, 0.5, 1.0):
        params = so.OracleParams(topk=topk, causal=causal)
        gm, st = bsq.sparge_predict_mask(q, k, topk, causal, stats=True)
        om, infos = oracle_predict(q, k, params)
        bad, exc = unexcused_mismatches(gm.cpu().numpy(), om, infos)
        say(f"mask N={N} D={D} causal={causal} topk={topk}: unexcused {bad}, excused {exc}")
        assert bad == 0
        assert st["kept_blocks"] == int(gm.sum())
        assert st["valid_blocks"] == int(sum(i["valid"].sum() for i in infos))


@pytest.mark.parametrize("dtype,N,D", [(torch.float32, 4000, 128), (torch.float16, 4000, 128),
                                       (torch.float32, 4000, 64)])
def test_predict_mask_other_dtypes(dev, dtype, N, D):
    """fp32 inputs take the separate block-statistics kernel and fp16 inputs the
    fp16 branch of the fused preparation pass; both must give the oracle's mask on
    the exact stored values (long enough that K blocks pass the similarity gate)."""
    wl = synth.workload("llm8k", H=2, N=N, D=D, dtype=dtype)
    q, k, _ = synth.make_qkv(wl, device=dev)
    gm = bsq.sparge_predict_mask(q, k, 0.5, True)
    om, infos = oracle_predict(q, k, so.OracleParams(topk=0.5, causal=True))
    bad, exc = unexcused_mismatches(gm.cpu().numpy(), om, infos)
    simk = np.mean([i["simk"].mean() for i in infos])
    say(f"mask {dtype} N={N} D={D}: unexcused {bad}, excused {exc}, similar K blocks {simk:.2f}")
    assert simk > 0.1
    assert bad == 0


def test_predict_mask_degenerate_blocks(dev):
    B, H, N, D = 1, 2, 640, 64
    q, k, _ = rand_qkv(B, H, N, D, torch.bfloat16, dev, seed=11)
    q[0, 0, :128] = 0                          # zero block: similarity 0 -> forced row
    k[0, 0, 64:128] = 0
    k[0, 1, 128:192] = k[0, 1, 128:129]        # identical rows: similarity 1
    q[0, 1, 256:384] = q[0, 1, 256:257]
    for causal in (False, True):
        gm = bsq.sparge_predict_mask(q, k, 0.4, causal)
        om, infos = oracle_predict(q, k, so.OracleParams(topk=0.4, causal=causal))
        bad, exc = unexcused_mismatches(gm.cpu().numpy(), om, infos)
        assert bad == 0


# ------------------------------------------------------------- sparge_topk_attn

def test_tiny_workload_end_to_end(dev):
    wl = synth.WORKLOADS["tiny"]
    q, k, v = synth.make_qkv(wl, device=dev)
    out, gm = bsq.sparge_topk_attn(q, k, v, wl.topk, wl.causal, filter_on=False, return_mask=True)
    om, infos = oracle_predict(q, k, so.OracleParams(topk=wl.topk, causal=wl.causal))
    bad, exc = unexcused_mismatches(gm.cpu().numpy(), om, infos)
    assert bad == 0 and exc == 0
    ref, _ = oracle_outputs(q, k, v, om, wl.causal)
    err = np.abs(f64(out) - ref).max()
    say(f"tiny workload err {err:.3e}, density {gm.float().mean().item():.3f}")
    assert err < TOL16


@pytest.mark.parametrize("N", [1, 63, 64, 65, 127, 128, 129, 1000])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_topk_attn_small_shapes(dev, N, D, causal):
    """The whole call on ragged and boundary lengths: mask bit-exact, output within the
    16-bit bar (block-correlated inputs, so that the similarity gate and the top-k
    selection are both live)."""
    wl = synth.workload("tiny", H=2, N=N, D=D, dtype=torch.bfloat16)
    q, k, v = synth.make_qkv(wl, device=dev)
    out, gm = bsq.sparge_topk_attn(q, k, v, 0.5, causal, return_mask=True)
    torch.cuda.synchronize()
    om, infos = oracle_predict(q, k, so.OracleParams(topk=0.5, causal=causal))
    bad, exc = unexcused_mismatches(gm.cpu().numpy(), om, infos)
    assert bad == 0 and exc == 0
    ref, _ = oracle_outputs(q, k, v, om, causal, lam=-10.0)
    err = np.abs(f64(out) - ref).max()
    say(f"small shape N={N} D={D} causal={causal}: density {om.mean():.3f}, err {err:.3e}")
    assert err < TOL16


@pytest.mark.parametrize("N,D,causal", [(700, 64, True), (1000, 128, False), (129, 128, True)])
def test_topk_attn_topk1_filter_off_is_dense(dev, N, D, causal):
    q, k, v = rand_qkv(1, 2, N, D, torch.bfloat16, dev, seed=N)
    out = bsq.sparge_topk_attn(q, k, v, 1.0, causal, filter_on=False)
    ref = F.scaled_dot_product_attention(q.double().cpu(), k.double().cpu(), v.double().cpu(),
                                         is_causal=causal)
    assert (out.double().cpu() - ref).abs().max().item() < TOL16


def _filter_inputs(dev, N=1024, D=64, H=2):
    g = torch.Generator().manual_seed(2)
    u = torch.randn(D, generator=g)
    u = u / u.norm() * 8.0
    q = torch.randn((1, H, N, D), generator=g) + u
    k = torch.randn((1, H, N, D), generator=g) * 0.5
    k[:, :, :64] += 3 * u      # block 0: logits ~24 above the rest for every row (margin >> |lambda|)
    v = torch.randn((1, H, N, D), generator=g)
    return [t.to(torch.bfloat16).to(dev) for t in (q, k, v)]


@pytest.mark.parametrize("causal", [True, False])
def test_filter_skips_match_oracle(dev, causal):
    q, k, v = _filter_inputs(dev)
    # topk attention with topk=1 keeps every valid block, so the filter alone decides;
    # the oracle runs on its own mask, which the GPU's must equal
    out, gm, st = bsq.sparge_topk_attn(q, k, v, 1.0, causal, filter_on=True, return_mask=True,
                                        stats=True)
    om, _ = oracle_predict(q, k, so.OracleParams(topk=1.0, causal=causal))
    assert np.array_equal(gm.cpu().numpy().astype(bool), om)
    ref, skipped = oracle_outputs(q, k, v, om, causal, lam=-10.0)
    err = np.abs(f64(out) - ref).max()
    say(f"filter causal={causal}: skipped gpu {st['skipped_updates']} oracle {skipped}, err {err:.3e}")
    assert skipped > 0
    assert st["skipped_updates"] == skipped
    assert err < TOL16


# -------------------------------------------------------------------- int8 path

@pytest.mark.parametrize("dtype,N,D", [(torch.bfloat16, 1000, 128), (torch.float32, 333, 64),
                                       (torch.float16, 64, 64), (torch.bfloat16, 700, 64),
                                       (torch.float16, 1000, 128)])
def test_int8_codes_bit_exact(dev, dtype, N, D):
    """The int8 operands as the attention path multiplies them (the Q codes written by
    the attention kernel itself), bit for bit against the oracle's quantizer; fp32
    inputs are rounded to bfloat16 for the attention products, so their codes are
    those of the rounded values."""
    wl = synth.workload("llm8k", H=3, N=N, D=D, dtype=dtype)
    q, k, _ = synth.make_qkv(wl, device=dev)
    q[0, 1, :32] = 0                                   # an all-zero Q group
    r = bsq.sparge_quantize_qk(q, k)
    if dtype == torch.float32:
        q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    qn = q.float().cpu().numpy()
    kn = k.float().cpu().numpy()
    for h in range(3):
        qc, qd, kc, kd, kbar = so.int8_qk_inputs(qn[0, h], kn[0, h], 32)
        assert np.array_equal(r["q_codes"][0, h].cpu().numpy(), qc)
        assert np.array_equal(r["q_scales"][0, h].cpu().numpy(), qd)
        assert np.array_equal(r["k_means"][0, h].cpu().numpy(), kbar)
        assert np.array_equal(r["k_scales"][0, h].cpu().numpy(), kd)
        assert np.array_equal(r["k_codes"][0, h].cpu().numpy(), kc)


@pytest.mark.parametrize("N,D,causal,pv16", [(2000, 128, True, True), (1500, 64, False, False),
                                             (300, 128, False, True)])
def test_int8_attention(dev, N, D, causal, pv16):
    wl = synth.workload("llm8k", H=2, N=N, D=D)
    q, k, v = synth.make_qkv(wl, device=dev)
    out, gm = bsq.sparge_topk_attn(q, k, v, 0.5, causal, qk_int8=True, pv_fp16=pv16,
                                   filter_on=False, return_mask=True)
    mask, rows = oracle_mask_and_rows(q, k, gm, 0.5, causal)
    ref, _ = oracle_outputs(q, k, v, mask, causal)
    err = np.abs(f64(out) - ref)[rows].max()
    qn, kn, vn = f64(q), f64(k), f64(v)
    sim_err = 0.0
    for h in range(2):
        o8 = so.attend_head_int8_sim(qn[0, h].astype(np.float32), kn[0, h].astype(np.float32),
                                     vn[0, h], mask[0, h], causal,
                                     pv_round="fp16" if pv16 else "bf16")
        sim_err = max(sim_err, np.abs(f64(out)[0, h] - o8)[rows[0, h]].max())
    say(f"int8 N={N} D={D}: err vs fp64 {err:.3e}, vs int8 simulation {sim_err:.3e}")
    assert err < TOL8
    assert sim_err < TOL16


@pytest.mark.parametrize("D", [64, 128])
def test_int8_attention_fp32_inputs(dev, D):
    """fp32 inputs on the int8 path (K codes and block means from quant_k_kernel, the
    q . kbar codes from those means), top-k mask and outputs against fp64."""
    q, k, v = rand_qkv(1, 2, 700, D, torch.float32, dev, seed=5 + D)
    out, gm = bsq.sparge_topk_attn(q, k, v, 0.5, True, qk_int8=True, pv_fp16=True,
                                   filter_on=False, return_mask=True)
    torch.cuda.synchronize()
    mask, rows = oracle_mask_and_rows(q, k, gm, 0.5, True)
    ref, _ = oracle_outputs(q, k, v, mask, True)
    err = np.abs(f64(out) - ref)[rows].max()
    say(f"int8 fp32 inputs D={D}: max abs err vs fp64 {err:.3e}")
    assert err < TOL8


@pytest.mark.parametrize("D", [64, 128])
def test_int8_zero_means_and_rows(dev, D):
    """int8 Q.K^T edge cases of the q . kbar term: a head whose K is all zero (every
    block mean zero, so the per-head code step is 0), and in another head an all-zero
    K block and all-zero Q rows (zero int8 steps); dense, filter off, against fp64."""
    B, H, N = 1, 2, 300
    q, k, v = rand_qkv(B, H, N, D, torch.bfloat16, dev, seed=77 + D)
    k[0, 0] = 0
    k[0, 1, 64:128] = 0
    q[0, 1, 32:64] = 0
    out = bsq.block_sparse_attn(q, k, v, None, qk_int8=True, pv_fp16=True, filter_on=False)
    torch.cuda.synchronize()
    nQ, nK = so.num_blocks(N)
    ref, _ = oracle_outputs(q, k, v, np.ones((B, H, nQ, nK), dtype=bool), False)
    err = np.abs(f64(out) - ref).max()
    say(f"int8 zero means/rows D={D}: max abs err vs fp64 {err:.3e}")
    assert np.all(np.isfinite(f64(out)))
    assert err < TOL8


@pytest.mark.parametrize("D,qk8,pv", [(128, True, "fp16"), (64, True, "fp16"), (128, False, "bf16"),
                                       (64, False, "bf16"), (64, False, "fp16"), (128, True, "fp8")])
def test_rescale_per_row(dev, D, qk8, pv):
    """Scores that grow along the keys at a different rate in every query row (and fall
    in others), so that the reference max of the exponentials moves often, and at
    different blocks for the rows of one wavefront: each row's O and row sum must be
    rescaled by that row's own factor.  All blocks kept, filter off: dense attention."""
    B, H, N = 1, 2, 2048
    g = torch.Generator().manual_seed(21 + D)
    q, k, v = (torch.randn(B, H, N, D, generator=g, dtype=torch.float64) for _ in range(3))
    u = torch.randn(D, generator=g, dtype=torch.float64)
    u /= u.norm()
    alpha = torch.rand(B, H, N, 1, generator=g, dtype=torch.float64) * 8.0 - 4.0
    # +2 (log2 units) per 64 keys for a row with |alpha| = 4
    kappa = 2.0 / (64 * 4 * math.log2(math.e) / math.sqrt(D))
    t = kappa * torch.arange(N, dtype=torch.float64).view(1, 1, N, 1)
    q, k = q + alpha * u, k + t * u
    q, k, v = (x.to(torch.bfloat16).to(dev) for x in (q, k, v))
    out = bsq.block_sparse_attn(q, k, v, None, qk_int8=qk8, pv_fp16=(pv == "fp16"),
                                pv_fp8=(pv == "fp8"), filter_on=False)
    torch.cuda.synchronize()
    nQ, nK = so.num_blocks(N)
    ones = np.ones((B, H, nQ, nK), dtype=bool)
    exact, _ = oracle_outputs(q, k, v, ones, False)
    err = np.abs(f64(out) - exact).max()
    say(f"rescale per row D={D} int8={qk8} P.V {pv}: max abs err vs fp64 {err:.3e}")
    if pv == "fp8":
        ratio = fp8_gate(out, q, k, v, ones, False, None, qk8)
        say(f"  fp8 error / E4M3 bound at most {ratio:.3f}")
        if not qk8:
            assert np.abs(f64(out) - pv8_oracle(q, k, v, ones, False, None, "exact")).max() < TOLF8
    else:
        assert err < (TOL8 if qk8 else TOL16)


# ------------------------------------------------------------------ fp8 P.V

def pv8_oracle(q, k, v, mask, causal, lam, qk):
    qn, kn, vn = f64(q), f64(k), f64(v)
    B, H = qn.shape[:2]
    out = np.zeros_like(qn)
    for b in range(B):
        for h in range(H):
            out[b, h] = so.attend_head_pv8_sim(qn[b, h], kn[b, h], vn[b, h], mask[b, h], causal,
                                               lam=lam, qk=qk)
    return out


@pytest.mark.parametrize("N,D,dtype,qk8,filt", [
    (1000, 128, torch.bfloat16, False, False), (700, 64, torch.float16, True, True),
    (129, 128, torch.bfloat16, True, False), (64, 64, torch.bfloat16, False, True),
    (513, 128, torch.float16, False, True), (1, 128, torch.bfloat16, True, False)])
def test_fp8_pv_block_sparse_matches_oracle(dev, N, D, dtype, qk8, filt):
    say(f"fp8 P.V block_sparse N={N} D={D} {dtype} qk_int8={qk8} filter={filt}")
    B, H = 2, 2
    q, k, v = rand_qkv(B, H, N, D, dtype, dev, seed=N + D + 7)
    nQ, nK = so.num_blocks(N)
    g = torch.Generator().manual_seed(8)
    mask = (torch.rand((B, H, nQ, nK), generator=g) < 0.45).to(torch.uint8)
    mask[0, 0, 0] = 0                       # an empty block row -> zero output
    mask[1, 1, :, -1] = 1                   # ragged last K block kept
    out = bsq.block_sparse_attn(q, k, v, mask.to(dev), pv_fp8=True, qk_int8=qk8, filter_on=filt)
    torch.cuda.synchronize()
    mnp = mask.numpy().astype(bool)
    lam = -10.0 if filt else None
    exact, _ = oracle_outputs(q, k, v, mnp, False, lam=lam)
    ratio = fp8_gate(out, q, k, v, mnp, False, lam, qk8)
    say(f"  max abs err vs fp64 {np.abs(f64(out) - exact).max():.3e}, error / E4M3 bound at most {ratio:.3f}")
    if not qk8:
        ref = pv8_oracle(q, k, v, mnp, False, lam, "exact")
        err = np.abs(f64(out) - ref).max()
        say(f"  max abs err vs fp8 simulation {err:.3e}")
        assert err < TOLF8
    assert np.all(f64(out)[0, 0, :min(N, 128)] == 0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_fp8_pv_exact_when_p_and_v_are_representable(dev, dtype):
    # logits n ln 2 (integers n in [-6, 2]) and V on the E4M3 grid times 1/8 with
    # every channel's max |v| = 56: every P and V code is exact, so the fp8 path
    # equals dense attention up to fp32 accumulation
    B, H, N, D = 1, 2, 1000, 128
    r = np.random.default_rng(21)
    q = np.zeros((B, H, N, D))
    q[..., 0] = 1.0
    k = np.zeros((B, H, N, D))
    k[..., 0] = r.integers(-6, 3, size=(B, H, N))
    e = np.array([(1 + m / 8) * 2.0 ** (x - 7) for x in range(1, 16) for m in range(8)
                  if not (x == 15 and m == 7)])
    v = r.choice(e, size=(B, H, N, D)) * r.choice([-1.0, 1.0], size=(B, H, N, D)) * 0.125
    v[:, :, 5, :] = 56.0
    qt, kt, vt = (torch.from_numpy(x).to(dtype).to(dev) for x in (q, k, v))
    out = bsq.block_sparse_attn(qt, kt, vt, None, scale=math.log(2.0), pv_fp8=True)
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x) for x in (q, k, v)),
                                         scale=math.log(2.0)).numpy()
    got = f64(out)
    err = np.abs(got - ref).max()
    say(f"fp8 P.V exact case {dtype}: err {err:.3e}")
    # only the output's rounding to the input type (half an ulp) and fp32 sums remain
    rel = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    assert np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-4)


@pytest.mark.parametrize("N,D,causal,qk8", [(2000, 128, True, True), (1500, 64, False, False),
                                            (300, 128, True, False)])
def test_fp8_pv_topk(dev, N, D, causal, qk8):
    wl = synth.workload("llm8k", H=2, N=N, D=D)
    q, k, v = synth.make_qkv(wl, device=dev)
    out, gm = bsq.sparge_topk_attn(q, k, v, 0.5, causal, qk_int8=qk8, pv_fp8=True,
                                   filter_on=True, return_mask=True)
    mask, rows = oracle_mask_and_rows(q, k, gm, 0.5, causal)
    same = rows[:, :, ::128]
    groups = [(b, h, i, g) for (b, h, i, g) in all_groups(*q.shape[:3]) if same[b, h, i]]
    ratio = fp8_gate(out, q, k, v, mask, causal, -10.0, qk8, groups)
    msg = f"fp8 P.V topk N={N} D={D} causal={causal} int8={qk8}: error / E4M3 bound at most {ratio:.3f}"
    if not qk8:
        err = np.abs(f64(out) - pv8_oracle(q, k, v, mask, causal, -10.0, "exact"))[rows].max()
        msg += f", err vs fp8 simulation {err:.3e}"
        assert err < TOLF8
    say(msg)


@pytest.mark.parametrize("path", ["fp8_int8", "fp8_bf16", "cdf", "cdf_fp8_int8"])
def test_strided_inputs_match_contiguous(dev, path):
    # (B, N, H, D) storage viewed as (B, H, N, D): every kernel that reads Q, K or V
    # (preparation, V scales and E4M3 tiles, attention) must give bit-identical
    # results to the contiguous copies
    B, H, N, D = 2, 3, 777, 128
    g = torch.Generator(device="cpu").manual_seed(31)
    base = [(torch.randn((B, N, H, D), generator=g)).to(torch.bfloat16).to(dev) for _ in range(3)]
    qs, ks, vs = (t.transpose(1, 2) for t in base)
    qc, kc, vc = (t.contiguous() for t in (qs, ks, vs))
    assert not qs.is_contiguous()
    kw = dict(qk_int8=path.endswith("int8"), pv_fp8="fp8" in path, return_mask=True)
    fn = (lambda *a, **k: bsq.sparge_cdf_attn(*a, 0.9, True, **k)) if path.startswith("cdf") else \
         (lambda *a, **k: bsq.sparge_topk_attn(*a, 0.5, True, **k))
    o1, m1 = fn(qs, ks, vs, **kw)
    o2, m2 = fn(qc, kc, vc, **kw)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2)
    assert torch.equal(o1, o2)
    say(f"strided == contiguous for {path}: density {m1.float().mean().item():.3f}")


@pytest.mark.parametrize("pv_fp8", [False, True])
def test_graph_replay_matches_eager(dev, pv_fp8):
    """The library's launches captured in a HIP graph (no allocation, no host sync, no
    memset in the call): every replay, with eager work and synchronisations between
    the replays, reproduces the eager result bit for bit."""
    wl = synth.workload("llm8k", H=4, N=3000, D=128)
    q, k, v = synth.make_qkv(wl, device=dev)
    ws = torch.empty(bsq.sparge_workspace_bytes(*q.shape, q.dtype), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    kw = dict(qk_int8=True, pv_fp16=not pv_fp8, pv_fp8=pv_fp8, out=out, workspace=ws)
    eager = bsq.sparge_topk_attn(q, k, v, 0.5, True, **kw).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        bsq.sparge_topk_attn(q, k, v, 0.5, True, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bsq.sparge_topk_attn(q, k, v, 0.5, True, **kw)
    for rep in range(3):
        out.fill_(float("nan"))            # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"
    say(f"graph replay == eager (pv_fp8={pv_fp8}) over 3 replays")


def test_fp8_pv_fp32_inputs_unsupported(dev):
    q, k, v = rand_qkv(1, 1, 256, 64, torch.float32, dev, seed=1)
    with pytest.raises(Exception):
        bsq.sparge_topk_attn(q, k, v, 0.5, False, pv_fp8=True)
    with pytest.raises(Exception):
        bsq.sparge_topk_attn(*rand_qkv(1, 1, 256, 64, torch.bfloat16, dev, seed=1), 0.5, False,
                             pv_fp8=True, pv_fp16=True)


# ------------------------------------------- threshold selection, per-head knobs

def cdf_mismatches(gpu_mask, om, infos, tau, theta=0.1):
    """Unexcused mask mismatches under the threshold selection: a row may differ only
    when the GPU kept the oracle's ranked prefix of a length that the oracle's
    cumulative masses allow within 1e-9 of tau, or by the top-k near-tie rule."""
    B, H, nQ, nK = om.shape
    g = gpu_mask.reshape(B * H, nQ, nK).astype(bool)
    o = om.reshape(B * H, nQ, nK)
    bad = 0
    for bh in range(B * H):
        info = infos[bh]
        S, valid, simk = info["scores"], info["valid"], info["simk"]
        t = tau[bh % H] if np.ndim(tau) else tau
        for i in np.flatnonzero((g[bh] != o[bh]).any(axis=1)):
            cand = valid[i] & simk
            js = np.flatnonzero(cand)
            order = np.lexsort((js, -S[i][js]))
            e = np.exp(S[i][js][order] - S[i][js].max())
            cum = np.cumsum(e / e.sum())
            lo = min(js.size, 1 + int((cum < t - 1e-9).sum()))
            hi = min(js.size, 1 + int((cum < t + 1e-9).sum()))
            kg = int((g[bh][i] & cand).sum())
            row = valid[i] & (~info["simq"][i] | ~simk)
            row[so.select_row(S[i], cand, kg)] = True
            if not (lo <= kg <= hi and np.array_equal(row, g[bh][i])):
                bad += 1
    return bad


@pytest.mark.parametrize("N,D,causal,tau,theta", [
    (1000, 128, True, 0.9, 0.1), (1500, 64, False, 0.5, 0.0), (129, 128, True, 0.99, 0.0),
    (4000, 128, True, 0.3, 0.1), (3000, 64, False, 0.8, 0.0), (5000, 128, True, 0.95, 0.0)])
def test_cdf_selection_matches_oracle(dev, N, D, causal, tau, theta):
    # theta = 0 makes every block similar, so every valid block competes
    wl = synth.workload("llm8k", H=3, N=N, D=D)
    q, k, v = synth.make_qkv(wl, device=dev)
    out, gm = bsq.sparge_cdf_attn(q, k, v, tau, causal, filter_on=True, return_mask=True,
                                  sim_threshold=theta)
    torch.cuda.synchronize()
    om, infos = oracle_predict(q, k, so.OracleParams(cdf=tau, causal=causal, theta=theta))
    g = gm.cpu().numpy().astype(bool)
    bad = cdf_mismatches(g, om, infos, tau, theta)
    same = (g == om).all(axis=3)
    say(f"cdf N={N} D={D} causal={causal} tau={tau} theta={theta}: unexcused {bad}, rows "
        f"differing {int((~same).sum())}, density {om.mean():.3f}")
    assert bad == 0
    rows = np.repeat(same, so.BQ, axis=2)[:, :, :N]
    ref, _ = oracle_outputs(q, k, v, om, causal, lam=-10.0)
    err = np.abs(f64(out) - ref)[rows].max()
    say(f"  output err {err:.3e}")
    assert err < TOL16


def test_per_head_knobs(dev):
    B, H, N, D = 1, 4, 1200, 128
    wl = synth.workload("llm8k", H=H, N=N, D=D)
    q, k, v = synth.make_qkv(wl, device=dev)
    sel = [0.2, 0.5, 0.8, 1.0]
    theta = [0.05, 0.1, 0.3, 0.1]
    lam = [-10.0, -3.0, -float("inf"), -20.0]
    out, gm, st = bsq.sparge_topk_attn(q, k, v, 0.5, True, head_select=sel, head_sim_threshold=theta,
                                       head_filter_lambda=lam, return_mask=True, stats=True)
    g = gm.cpu().numpy().astype(bool)
    qn, kn, vn = f64(q), f64(k), f64(v)
    skipped = 0
    for h in range(H):
        p = so.OracleParams(topk=sel[h], causal=True, theta=theta[h])
        m, info = so.predict_mask(qn[0, h], kn[0, h], p)
        bad, _ = unexcused_mismatches(g[:, h:h + 1], m[None, None], [info], theta=theta[h])
        assert bad == 0
        rows = np.repeat((g[0, h] == m).all(axis=1), so.BQ)[:N]
        o, sk = so.attend_head(qn[0, h], kn[0, h], vn[0, h], m, True, lam=lam[h], return_skips=True)
        skipped += sum(len(x) for x in sk.values())
        err = np.abs(f64(out)[0, h] - o)[rows].max()
        say(f"per-head knobs head {h}: topk {sel[h]} theta {theta[h]} lambda {lam[h]}: err {err:.3e}")
        assert err < TOL16
    say(f"  skipped updates gpu {st['skipped_updates']} oracle {skipped}")
    assert st["skipped_updates"] == skipped
    # equal per-head values reproduce the scalar call exactly
    a = bsq.sparge_topk_attn(q, k, v, 0.3, True, sim_threshold=0.2, filter_lambda=-5.0)
    b = bsq.sparge_topk_attn(q, k, v, 0.7, True, head_select=[0.3] * H, head_sim_threshold=[0.2] * H,
                             head_filter_lambda=[-5.0] * H)
    assert torch.equal(a, b)
    # per-head cdf thresholds
    taus = [0.5, 0.9, 0.99, 0.3]
    out2, gm2 = bsq.sparge_cdf_attn(q, k, v, 0.9, True, head_select=taus, return_mask=True)
    for h in range(H):
        m, info = so.predict_mask(qn[0, h], kn[0, h], so.OracleParams(cdf=taus[h], causal=True))
        assert cdf_mismatches(gm2.cpu().numpy()[:, h:h + 1], m[None, None], [info], taus[h]) == 0
    # block_sparse_attn takes the per-head lambda
    nQ, nK = so.num_blocks(N)
    mask = (torch.rand((B, H, nQ, nK), generator=torch.Generator().manual_seed(3)) < 0.6).to(torch.uint8)
    out3 = bsq.block_sparse_attn(q, k, v, mask.to(dev), filter_on=True, head_filter_lambda=lam)
    for h in range(H):
        o = so.attend_head(qn[0, h], kn[0, h], vn[0, h], mask[0, h].numpy().astype(bool), False,
                           lam=lam[h])
        assert np.abs(f64(out3)[0, h] - o).max() < TOL16


# -------------------------------------------------------------- Hilbert reorder

def test_reorder_gather_scatter(dev):
    T, Hg, W, text = 3, 8, 10, 17
    N = text + T * Hg * W
    x = torch.randn((2, 3, N, 64), device=dev).to(torch.bfloat16)
    perm = bsq.sparge_hilbert_perm3d(T, Hg, W)
    assert np.array_equal(perm.numpy().astype(np.int64), hilbert_cell_order(T, Hg, W))
    pd = perm.to(dev)
    y = bsq.sparge_reorder(x, pd, text, T * Hg * W)
    full = torch.cat([torch.arange(text), text + perm.long()]).to(dev)
    assert torch.equal(y, x[:, :, full])
    back = bsq.sparge_reorder(y, pd, text, T * Hg * W, inverse=True)
    assert torch.equal(back, x)


@pytest.mark.parametrize("qk8", [False, True])
def test_video_pipeline_small(dev, qk8):
    # the int8 variant runs with the filter off: its decisions on int8 logits may
    # differ from the oracle's exact ones near the threshold
    wl = synth.workload("video", B=1, H=2, N=10 + 3 * 16 * 16, text=10, grid=(3, 16, 16))
    q, k, v = synth.make_qkv(wl, device=dev)
    cells = 3 * 16 * 16
    perm = bsq.sparge_hilbert_perm3d(3, 16, 16).to(dev)
    qr, kr, vr = (bsq.sparge_reorder(t, perm, 10, cells) for t in (q, k, v))
    o_r, gm = bsq.sparge_topk_attn(qr, kr, vr, 0.3, False, return_mask=True, qk_int8=qk8,
                                   pv_fp16=qk8, filter_on=not qk8)
    out = bsq.sparge_reorder(o_r, perm, 10, cells, inverse=True)
    fullp = np.concatenate([np.arange(10), 10 + hilbert_cell_order(3, 16, 16)])
    qn, kn, vn = f64(q)[:, :, fullp], f64(k)[:, :, fullp], f64(v)[:, :, fullp]
    om = np.zeros(gm.shape, dtype=bool)
    for h in range(2):
        m, info = so.predict_mask(qn[0, h], kn[0, h], so.OracleParams(topk=0.3))
        om[0, h] = m
        o, _ = so.attend_head(qn[0, h], kn[0, h], vn[0, h], m, False, lam=None if qk8 else -10.0,
                              return_skips=True)
        back = np.empty_like(o)
        back[fullp] = o
        err = np.abs(f64(out)[0, h] - back).max()
        say(f"video small head {h} int8={qk8}: err {err:.3e}")
        assert err < (TOL8 if qk8 else TOL16)
    assert np.array_equal(gm.cpu().numpy().astype(bool), om)


# ------------------------------------------------------ full-size workloads

def run_workload(wl, q, k, v, mask=None, stats=False):
    """The exact call sequence bench.py times for a workload."""
    if wl.api == "block_sparse":
        return bsq.block_sparse_attn(q, k, v, mask, filter_on=wl.filter_on, qk_int8=wl.qk_int8,
                                     pv_fp16=wl.pv_fp16, pv_fp8=wl.pv_fp8, stats=stats)
    return bsq.sparge_topk_attn(q, k, v, wl.topk, wl.causal, filter_on=wl.filter_on,
                                qk_int8=wl.qk_int8, pv_fp16=wl.pv_fp16, pv_fp8=wl.pv_fp8,
                                return_mask=True, stats=stats)


def sample_groups(B, H, N, n, seed, causal, ok=None):
    """n (b, h, block row, 32-row group) picks, the ragged last group first; with
    ok (B, H, nQ) only block rows where ok holds."""
    r = np.random.default_rng(seed)
    nQ = (N + 127) // 128
    picks = []
    if ok is None or ok[0, 0, nQ - 1]:
        picks.append((0, 0, nQ - 1, (N - 1 - 128 * (nQ - 1)) // 32))   # the ragged last group
    while len(picks) < n:
        b, h = int(r.integers(B)), int(r.integers(H))
        i = int(r.integers(nQ)) if not causal or r.random() < 0.5 else nQ - 1 - int(r.integers(4))
        if ok is not None and not ok[b, h, i]:
            continue
        gmax = (min(N, 128 * i + 128) - 128 * i + 31) // 32
        picks.append((b, h, i, int(r.integers(gmax))))
    return picks


def per_head_groups(B, H, N, seed, causal, ok=None):
    """One (b, h, block row, 32-row group) pick per head, in block rows where ok
    (B, H, nQ) holds, plus the ragged last group of head (0, 0) when N is not a
    multiple of 32; causal picks favour the longest rows (the sequence's end)."""
    r = np.random.default_rng(seed)
    nQ = (N + 127) // 128
    picks = []
    if N % 32 and (ok is None or ok[0, 0, nQ - 1]):
        picks.append((0, 0, nQ - 1, (N - 1 - 128 * (nQ - 1)) // 32))
    for b in range(B):
        for h in range(H):
            for _ in range(1000):
                i = int(r.integers(nQ)) if not causal or r.random() < 0.5 else nQ - 1 - int(r.integers(4))
                if ok is None or ok[b, h, i]:
                    break
            else:
                continue
            gmax = (min(N, 128 * i + 128) - 128 * i + 31) // 32
            picks.append((b, h, i, int(r.integers(gmax))))
    return picks


def check_groups(out, q, k, v, mask, causal, lam, tol, groups, tag):
    """Sampled 32-row groups of out against the oracle, within bar(ref, out.dtype, tol)."""
    cur, worst = None, 0.0
    for (b, h, i, g) in groups:
        if cur is None or cur[0] != (b, h):
            cur = ((b, h), f64(q[b, h]), f64(k[b, h]), f64(v[b, h]))   # one head in memory at a time
        _, qn, kn, vn = cur
        ref = so.attend_rows(qn, kn, vn, mask[b, h], [(i, g)], causal, lam=lam)[(i, g)]
        t0 = 128 * i + 32 * g
        err = np.abs(f64(out[b, h, t0:t0 + ref.shape[0]]) - ref)
        worst = max(worst, float((err / bar(ref, out.dtype, tol)).max()))
    say(f"  {tag}: {len(groups)} groups, error / bar at most {worst:.3f}")
    assert worst < 1.0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cdf", [None, 0.9])
def test_max_sequence_length(dev, cdf):
    """N = 262144, the largest the ABI accepts: 4096 K blocks per row fill the
    selector's per-thread key slots and the uint16 block lists.  The random walk drifts
    far at this length (|O| reaches 10, where a bfloat16 ulp is 2^-4), so outputs are
    compared in fp32: the same bfloat16 values given as fp32 tensors take the same
    attention kernel (rounded to bfloat16 on load, exactly) and an fp32 store, and the
    bfloat16 call must store exactly the bfloat16 rounding of that fp32 result."""
    N = 262144
    wl = synth.workload("llm8k", H=1, N=N, D=64, seed=9)
    q, k, v = synth.make_qkv(wl, device=dev)
    if cdf is None:
        call = lambda a, b, c: bsq.sparge_topk_attn(a, b, c, 0.5, True, return_mask=True)
        params = so.OracleParams(topk=0.5, causal=True)
    else:
        call = lambda a, b, c: bsq.sparge_cdf_attn(a, b, c, cdf, True, return_mask=True)
        params = so.OracleParams(cdf=cdf, causal=True)
    out, gm = call(q, k, v)
    out32, gm32 = call(q.float(), k.float(), v.float())
    torch.cuda.synchronize()
    assert torch.equal(gm, gm32)
    assert torch.equal(out, out32.to(torch.bfloat16))
    g = gm.cpu().numpy().astype(bool)
    om, infos = oracle_predict(q, k, params)
    bad = unexcused_mismatches(g, om, infos)[0] if cdf is None else cdf_mismatches(g, om, infos, cdf)
    same = (g == om).all(axis=3)
    say(f"N=262144 cdf={cdf}: unexcused {bad}, rows differing {int((~same).sum())}, "
        f"density {om.mean():.3f}, longest row {int(om.sum(axis=3).max())} blocks, "
        f"max|v| {float(v.abs().max()):.2f}")
    assert bad == 0
    check_groups(out32, q, k, v, om, True, -10.0, TOL16,
                 sample_groups(1, 1, N, 6, seed=11, causal=True, ok=same), "fp32 output")


@pytest.mark.parametrize("N", [16384, 32768, 65536])
def test_selection_mid_sizes(dev, N):
    """The selector's register layouts between the small tests and the full
    workloads (rows of 4, 8 and 16 chunks of 64 K blocks): the top-k mask and the
    threshold-selection mask against the oracle."""
    wl = synth.workload("llm8k", H=1, N=N, D=64, seed=N % 97)
    q, k, v = synth.make_qkv(wl, device=dev)
    gm = bsq.sparge_predict_mask(q, k, 0.5, True)
    _, gc = bsq.sparge_cdf_attn(q, k, v, 0.9, True, return_mask=True)
    torch.cuda.synchronize()
    om, infos = oracle_predict(q, k, so.OracleParams(topk=0.5, causal=True))
    bad_topk = unexcused_mismatches(gm.cpu().numpy(), om, infos)[0]
    oc, infc = oracle_predict(q, k, so.OracleParams(cdf=0.9, causal=True))
    bad_cdf = cdf_mismatches(gc.cpu().numpy().astype(bool), oc, infc, 0.9)
    say(f"selection N={N}: top-k unexcused {bad_topk} (density {om.mean():.3f}), "
        f"cdf unexcused {bad_cdf} (density {oc.mean():.3f})")
    assert bad_topk == 0 and bad_cdf == 0


_SWEEP = {}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("N", [16384, 32768, 65536])
@pytest.mark.parametrize("path", ["i8-qk/f16-pv", "i8-qk/fp8-pv", "bf16"])
def test_sweep_point_outputs(dev, N, path):
    """The bench's N sweep (LLM generator, 32 heads, D = 128, causal, top-k 0.5, filter
    on) at 16K, 32K and 64K for each of its three paths: the whole mask, and one 32-row
    group of every head against the oracle."""
    wl = synth.workload("llm8k", N=N)
    if _SWEEP.get("N") != N:
        _SWEEP.clear()
        _SWEEP["N"] = N
        _SWEEP["qkv"] = synth.make_qkv(wl, device=dev)
        _SWEEP["oracle"] = oracle_predict(*_SWEEP["qkv"][:2], so.OracleParams(topk=0.5, causal=True))
    q, k, v = _SWEEP["qkv"]
    om, infos = _SWEEP["oracle"]
    qk8 = path.startswith("i8")
    out, gm = bsq.sparge_topk_attn(q, k, v, 0.5, True, filter_on=True, qk_int8=qk8,
                                   pv_fp16=path == "i8-qk/f16-pv", pv_fp8=path.endswith("fp8-pv"),
                                   return_mask=True)
    torch.cuda.synchronize()
    g = gm.cpu().numpy().astype(bool)
    bad, exc = unexcused_mismatches(g, om, infos)
    say(f"sweep N={N} {path}: mask unexcused {bad}, excused {exc}, density {om.mean():.3f}")
    assert bad == 0
    same = (g == om).all(axis=3)
    groups = per_head_groups(1, wl.H, N, seed=N + len(path), causal=True, ok=same)
    if path.endswith("fp8-pv"):
        say(f"  fp8 error / E4M3 bound at most {fp8_gate(out, q, k, v, om, True, -10.0, True, groups):.3f}")
    else:
        check_groups(out, q, k, v, om, True, -10.0, TOL8 if qk8 else TOL16, groups, path)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,variant", [("llm128k", "fp8"), ("llm128k", "bf16"), ("llm8k", "cdf"),
                                          ("llm128k", "cdf")])
def test_full_workload_variant(dev, name, variant):
    """The bench's extra paths at full size: int8 Q.K^T with fp8 P.V, the 16-bit path
    (the one the bf16 roofline is quoted on), and the threshold selection (mass 0.95)
    -- the whole mask, and one 32-row group of every head."""
    wl = synth.WORKLOADS[name]
    say(f"full workload {name} ({variant}): generating on {dev}")
    q, k, v = synth.make_qkv(wl, device=dev)
    lam = -10.0 if wl.filter_on else None
    if variant in ("fp8", "bf16"):
        out, gm, st = bsq.sparge_topk_attn(q, k, v, wl.topk, wl.causal, filter_on=wl.filter_on,
                                           qk_int8=variant == "fp8", pv_fp8=variant == "fp8",
                                           return_mask=True, stats=True)
        params = so.OracleParams(topk=wl.topk, causal=wl.causal)
        tol = TOL16
    else:
        out, gm, st = bsq.sparge_cdf_attn(q, k, v, 0.95, wl.causal, filter_on=wl.filter_on,
                                          qk_int8=wl.qk_int8, pv_fp16=wl.pv_fp16, return_mask=True,
                                          stats=True)
        params = so.OracleParams(cdf=0.95, causal=wl.causal)
        tol = TOL8 if wl.qk_int8 else TOL16
    torch.cuda.synchronize()
    g = gm.cpu().numpy().astype(bool)
    om, infos = oracle_predict(q, k, params)
    if variant == "cdf":
        bad, exc = cdf_mismatches(g, om, infos, 0.95), None
    else:
        bad, exc = unexcused_mismatches(g, om, infos)
    same = (g == om).all(axis=3)
    say(f"  mask: unexcused {bad}, excused {exc}, rows differing {int((~same).sum())}, "
        f"density {om.mean():.3f}, stats {st}")
    assert bad == 0
    assert st["kept_blocks"] == int(g.sum())
    B, H, N, D = q.shape
    groups = per_head_groups(B, H, N, seed=len(name) + 7, causal=wl.causal, ok=same)
    if variant == "fp8":
        say(f"  fp8 error / E4M3 bound at most {fp8_gate(out, q, k, v, om, wl.causal, lam, True, groups):.3f}")
    else:
        check_groups(out, q, k, v, om, wl.causal, lam, tol, groups, variant)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llm8k", "image", "video", "llm128k"])
def test_full_workload(dev, name, oracle_pool):
    """Each workload at full size through the call sequence bench.py times (for the
    video workload: the Hilbert gather of Q, K and V, attention in that order, and the
    scatter of O back, all at full size): the whole mask against the oracle's, and the
    whole output tensor against the oracle's (one 32-row group per head at 128K)."""
    wl = synth.WORKLOADS[name]
    say(f"full workload {name}: generating on {dev}")
    q, k, v = synth.make_qkv(wl, device=dev)
    mask_in = synth.make_block_mask(wl, device=dev) if wl.api == "block_sparse" else None
    B, H, N, D = q.shape
    tok = np.arange(N)                       # token of each attention row
    if wl.hilbert:
        cells = int(np.prod(wl.grid))
        perm = bsq.sparge_hilbert_perm3d(*wl.grid).to(dev)
        tok = np.concatenate([np.arange(wl.text), wl.text + hilbert_cell_order(*wl.grid)])
        fidx = torch.from_numpy(tok).to(dev)
        gathered = [bsq.sparge_reorder(t, perm, wl.text, cells) for t in (q, k, v)]
        assert all(torch.equal(a, t[:, :, fidx]) for a, t in zip(gathered, (q, k, v)))
        q, k, v = gathered
    res = run_workload(wl, q, k, v, mask_in, stats=True)
    torch.cuda.synchronize()
    if wl.api == "block_sparse":
        out, st = res
        mask = mask_in.cpu().numpy().astype(bool)
        assert st["kept_blocks"] == int(mask.sum())
        same = np.ones(mask.shape[:3], dtype=bool)
    else:
        out, gm, st = res
        om, infos = oracle_predict(q, k, so.OracleParams(topk=wl.topk, causal=wl.causal))
        g = gm.cpu().numpy().astype(bool)
        bad, exc = unexcused_mismatches(g, om, infos)
        say(f"  mask: unexcused {bad}, excused {exc}, density {om.mean():.3f}")
        assert bad == 0
        assert st["kept_blocks"] == int(g.sum())
        same = (g == om).all(axis=3)
        mask = om
    say(f"  stats {st}")
    lam = -10.0 if wl.filter_on else None
    tol = TOL8 if wl.qk_int8 else TOL16
    if wl.hilbert:
        # the full-size scatter of O back to token order equals indexing
        out_tok = bsq.sparge_reorder(out, perm, wl.text, cells, inverse=True)
        back = torch.empty_like(out)
        back[:, :, fidx] = out
        assert torch.equal(out_tok, back)
    if name == "llm128k":
        check_groups(out, q, k, v, mask, wl.causal, lam, tol,
                     per_head_groups(B, H, N, seed=len(name), causal=wl.causal, ok=same), "one group per head")
        return
    # whole tensors: the oracle per head (in a pool of CPU workers when one is available)
    qn, kn, vn = f64(q), f64(k), f64(v)
    tasks = [(qn[b, h], kn[b, h], vn[b, h], mask[b, h], wl.causal, lam) for b in range(B) for h in range(H)]
    refs = (oracle_pool.imap(head_reference, tasks) if oracle_pool is not None
            else map(head_reference, tasks))
    got = f64(out_tok if wl.hilbert else out)
    worst, rows_checked = 0.0, 0
    for n, ref in enumerate(refs):
        b, h = divmod(n, H)
        rows = np.repeat(same[b, h], so.BQ)[:N]          # attention rows whose mask row agrees
        ref_tok = np.empty_like(ref)
        ref_tok[tok] = ref                                # back to token order
        rows_tok = np.empty_like(rows)
        rows_tok[tok] = rows
        err = np.abs(got[b, h] - ref_tok)[rows_tok]
        worst = max(worst, float((err / bar(ref_tok[rows_tok], out.dtype, tol)).max()))
        rows_checked += int(rows_tok.sum())
    say(f"  whole tensor: {rows_checked} of {B * H * N} rows, error / bar at most {worst:.3f}")
    assert rows_checked >= 0.99 * B * H * N
    assert worst < 1.0
