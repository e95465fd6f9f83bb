"""The fp8 P.V error bound of tests/fp8_bounds.py, pinned on the CPU.

The GPU tests gate the fp8 P.V path against exact attention (fp64, on the path's
logits) with the elementwise bound B derived from E4M3's rounding steps.  Here the
derivation itself is checked: the distance e(y) is the real worst-case E4M3
rounding distance (against the format decoded from its bit fields), the oracle's
fp8 simulation stays within B on causal and non-causal, filtered, int8-logit and
long-row inputs, B is not vacuous (the simulation comes close to it), a coarser
rounding than E4M3's planted in the simulation breaks it, and the int8 path's
two-level q . kbar term shifts logits by far less than the slack B allows for it.
"""
import math

import numpy as np
import pytest
import torch

import fp8_bounds as fb
from oracle import sparge_oracle as so


def _e4m3_table():
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_half_step_is_the_worst_rounding_distance():
    t = _e4m3_table()
    r = np.random.default_rng(3)
    y = np.concatenate([np.exp2(r.uniform(-14, 8.8, 20000)), (t[:-1] + t[1:]) / 2, t])
    y = y[y <= 448]
    dist = np.abs(t[np.abs(y[:, None] - t[None, :]).argmin(axis=1)] - y)
    bound = fb.e4m3_half_step(y)
    assert np.all(dist <= bound * (1 + 1e-12))
    mids = (t[:-1] + t[1:]) / 2
    # the bound is reached (up to one part in 17) at the first midpoint of each
    # binade and in the subnormal range: it is the tightest of its form
    assert (np.abs(mids - t[:-1]) / fb.e4m3_half_step(mids)).max() > 0.94
    sub = mids < 2.0 ** -6
    assert np.allclose(np.abs(mids - t[:-1])[sub], fb.e4m3_half_step(mids)[sub])


def _case(N, D, causal, lam, qk, seed, dens=0.5, drift=False):
    r = np.random.default_rng(seed)
    if drift:
        nb = (N + 63) // 64
        mu = np.cumsum(r.standard_normal((nb, D)) * 0.05, axis=0)
        q, k, v = [np.repeat(mu, 64, axis=0)[:N] + r.standard_normal((N, D)) for _ in range(3)]
    else:
        q, k, v = [r.standard_normal((N, D)) for _ in range(3)]
    q, k, v = [torch.from_numpy(x).to(torch.bfloat16).double().numpy() for x in (q, k, v)]
    nQ, nK = so.num_blocks(N)
    mask = (r.random((nQ, nK)) < dens) & so.block_valid(N, causal)
    return q, k, v, mask


CASES = [(129, 128, False, None, "exact", 1), (700, 64, True, -10.0, "exact", 2),
         (1000, 128, False, None, "int8", 3), (2000, 128, True, -10.0, "int8", 4, 1.0, True),
         (4096, 64, True, None, "exact", 5, 1.0, True)]


def _ratios(case):
    N, D, causal, lam, qk = case[:5]
    q, k, v, mask = _case(*case)
    scale = 1.0 / math.sqrt(D)
    nQ = mask.shape[0]
    groups = [(i, g) for i in range(nQ) for g in range(4) if 128 * i + 32 * g < N]
    if N > 2000:       # long rows: the last block rows only
        groups = [(i, g) for (i, g) in groups if i >= nQ - 2]
    sim = so.attend_rows_pv8(q, k, v, mask, groups, causal, lam=lam, qk=qk)
    i8 = so.int8_qk_inputs(q.astype(np.float32), k.astype(np.float32)) if qk == "int8" else None
    if qk == "int8":
        ref_head = so.attend_head_int8_sim(q.astype(np.float32), k.astype(np.float32), v, mask, causal,
                                           lam=lam, pv_round=None)
    vmax = np.abs(v).max(axis=0)
    worst, bmax = 0.0, 0.0
    for (i, g), o8 in sim.items():
        t0 = 128 * i + 32 * g
        t1 = min(N, t0 + 32, 128 * i + 128)
        Z = fb.group_logits(q, k, np.flatnonzero(mask[i]), t0, t1, causal, scale, lam, i8)
        O, B = fb.fp8_bound(Z, v, vmax, "fp32")
        # the helper's exact attention is the oracle's
        ref = (so.attend_rows(q, k, v, mask, [(i, g)], causal, lam=lam)[(i, g)] if qk == "exact"
               else ref_head[t0:t1])
        assert np.abs(O - ref).max() < 1e-10
        err = np.abs(o8 - O)
        assert np.all(err <= B), (case, (i, g), float((err / np.where(B > 0, B, 1)).max()))
        worst = max(worst, float((err[B > 0] / B[B > 0]).max()) if (B > 0).any() else 0.0)
        bmax = max(bmax, float(B.max()))
    return worst, bmax


@pytest.mark.parametrize("case", CASES)
def test_oracle_fp8_simulation_within_bound(case):
    worst, bmax = _ratios(case)
    assert bmax < 0.5


def test_bound_is_not_vacuous():
    worst = max(_ratios(c)[0] for c in CASES[:2])
    assert worst > 0.3


def test_planted_coarser_rounding_breaks_bound(monkeypatch):
    orig = so.e4m3_round

    def two_bits(x):           # E4M3's exponent range, but 2 fraction bits
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        _, e2 = np.frexp(a)
        ulp = np.ldexp(1.0, np.maximum(e2 - 3, -9))
        return np.copysign(np.minimum(np.rint(a / ulp) * ulp, 448.0), x)
    monkeypatch.setattr(so, "e4m3_round", two_bits)
    with pytest.raises(AssertionError):
        for c in CASES[:2]:
            _ratios(c)
    monkeypatch.setattr(so, "e4m3_round", orig)


def test_two_level_qkbar_slack_is_small():
    """On drifting data (large block means) the two-level q . kbar term shifts a logit
    by under 1e-3 relative in P; the int8 comparisons add it to the per-numerator slack."""
    q, k, v, mask = _case(4096, 128, True, None, "int8", 6, 1.0, True)
    kbar = so.k_block_means(k.astype(np.float32))
    s = fb.int8_logit_slack(q.astype(np.float32), kbar, 1.0 / math.sqrt(128))
    assert 0 < s < 1e-3
