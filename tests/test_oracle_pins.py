"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a library routine
(torch SDPA and cosine similarity in fp64), a closed form, brute-force enumeration
on tiny inputs, or an invariant of the method.  A final group plants plausible
mistakes in the oracle and checks that a pin catches each one.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import sparge_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa64(q, k, v, causal=False, attn_mask=None, scale=None):
    """torch SDPA in fp64 on CPU for one head: (N, D) arrays."""
    Q = torch.from_numpy(np.asarray(q, np.float64))[None, None]
    K = torch.from_numpy(np.asarray(k, np.float64))[None, None]
    V = torch.from_numpy(np.asarray(v, np.float64))[None, None]
    am = None if attn_mask is None else torch.from_numpy(attn_mask)[None, None]
    o = F.scaled_dot_product_attention(Q, K, V, attn_mask=am, is_causal=causal, scale=scale)
    return o[0, 0].numpy()


def rnd(N, D, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return [r.standard_normal((N, D)) * scale for _ in range(3)]


def expand_mask(mask_bh, N):
    """Block mask -> (N, N) token mask."""
    rows = np.repeat(mask_bh, so.BQ, axis=0)[:N]
    return np.repeat(rows, so.BK, axis=1)[:, :N]


# ---------------------------------------------------------------- block geometry

def test_mask_shapes_golden():
    with open(os.path.join(GOLDEN, "mask_shapes.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert rows
    for N, nq, nk in rows:
        assert so.num_blocks(int(N)) == (int(nq), int(nk))


def test_causal_validity_enumeration():
    # valid(i, j) iff some query t in block i and key s in block j have s <= t
    for N in (1, 64, 100, 128, 129, 300, 512):
        V = so.block_valid(N, True)
        nQ, nK = so.num_blocks(N)
        for i in range(nQ):
            for j in range(nK):
                ts = range(128 * i, min(N, 128 * i + 128))
                ss = range(64 * j, min(N, 64 * j + 64))
                assert V[i, j] == any(s <= t for t in ts for s in ss)
        assert so.block_valid(N, False).all()


# ------------------------------------------------------- stage 2: masked attention

@pytest.mark.parametrize("N,D,causal", [(512, 64, False), (300, 64, True), (129, 128, False),
                                        (200, 32, True), (1, 64, False), (65, 64, True)])
def test_all_ones_mask_equals_sdpa(N, D, causal):
    q, k, v = rnd(N, D, N + D)
    nQ, nK = so.num_blocks(N)
    mask = so.block_valid(N, causal)
    o = so.attend_head(q, k, v, mask, causal)
    ref = sdpa64(q, k, v, causal=causal)
    assert np.abs(o - ref).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_block_mask_equals_sdpa_with_token_mask(causal):
    N, D = 333, 64
    q, k, v = rnd(N, D, 7)
    nQ, nK = so.num_blocks(N)
    r = np.random.default_rng(3)
    mask = r.random((nQ, nK)) < 0.4
    for i in range(nQ):
        mask[i, min(2 * i, nK - 1)] = True      # every row keeps a block that has allowed keys
    mask &= so.block_valid(N, causal)
    o = so.attend_head(q, k, v, mask, causal)
    tok = expand_mask(mask, N)
    if causal:
        tok = tok & np.tril(np.ones((N, N), dtype=bool))
    has = tok.any(axis=1)
    ref = sdpa64(q, k, v, attn_mask=tok)
    assert np.abs(o[has] - ref[has]).max() < 1e-12
    assert np.all(o[~has] == 0)


def test_empty_rows_are_zero():
    N, D = 256, 64
    q, k, v = rnd(N, D, 11)
    mask = np.ones((2, 4), dtype=bool)
    mask[1] = False
    o = so.attend_head(q, k, v, mask, False)
    assert np.all(o[128:] == 0)
    assert np.abs(o[:128] - sdpa64(q[:128], k, v)).max() < 1e-12


def test_single_kept_block_is_softmax_over_that_block():
    N, D = 256, 64
    q, k, v = rnd(N, D, 5)
    mask = np.zeros((2, 4), dtype=bool)
    mask[0, 3] = True
    mask[1, 1] = True
    o = so.attend_head(q, k, v, mask, False)
    assert np.abs(o[:128] - sdpa64(q[:128], k[192:256], v[192:256])).max() < 1e-12
    assert np.abs(o[128:] - sdpa64(q[128:], k[64:128], v[64:128])).max() < 1e-12


def test_causal_rows_ignore_future():
    N, D = 300, 64
    q, k, v = rnd(N, D, 9)
    mask = so.block_valid(N, True)
    o1 = so.attend_head(q, k, v, mask, True)
    k2, v2 = k.copy(), v.copy()
    k2[200:] += 5.0
    v2[200:] -= 3.0
    o2 = so.attend_head(q, k2, v2, mask, True)
    assert np.array_equal(o1[:200], o2[:200])
    assert not np.allclose(o1[200:], o2[200:])


def test_brute_force_tiny():
    N, D = 70, 8
    q, k, v = rnd(N, D, 13)
    r = np.random.default_rng(2)
    mask = r.random((1, 2)) < 2  # all ones
    mask[0, 1] = False
    o = so.attend_head(q, k, v, mask, True, scale=0.3)
    for t in range(N):
        keys = [s for s in range(N) if s <= t and s < 64]
        w = [math.exp(0.3 * sum(q[t, c] * k[s, c] for c in range(D))) for s in keys]
        tot = sum(w)
        for c in range(D):
            ref = sum(wi * v[s, c] for wi, s in zip(w, keys)) / tot
            assert abs(o[t, c] - ref) < 1e-12


# ------------------------------------------------------------- stage 1: predictor

def test_selfsim_closed_form_matches_cosine_matrix():
    r = np.random.default_rng(0)
    for n, D in ((64, 64), (128, 128), (17, 32), (1, 8)):
        x = r.standard_normal((n, D)) + r.standard_normal(D) * r.random()
        x[n // 2] = 0.0 if n > 2 else x[n // 2]
        _, _, sims = so.block_stats(x, n)
        X = torch.from_numpy(x)
        cs = F.cosine_similarity(X[:, None, :], X[None, :, :], dim=-1, eps=1e-300)
        nz = torch.from_numpy(np.linalg.norm(x, axis=1) > 0)
        cs = cs * nz[:, None] * nz[None, :]
        assert abs(sims[0] - cs.mean().item()) < 1e-12


def test_selfsim_special_cases():
    D = 64
    row = np.random.default_rng(1).standard_normal(D)
    _, _, s = so.block_stats(np.tile(row, (64, 1)), 64)
    assert abs(s[0] - 1.0) < 1e-12
    _, _, s = so.block_stats(np.eye(64)[:, :D] * 3.0, 64)
    assert abs(s[0] - 1.0 / 64) < 1e-15
    x = np.tile(row, (64, 1))
    x[:32] = 0
    _, _, s = so.block_stats(x, 64)
    assert abs(s[0] - 0.25) < 1e-12          # 32 equal unit vectors over n=64
    m = np.vstack([np.tile(row, (32, 1)), np.tile(-row, (32, 1))])
    _, _, s = so.block_stats(m, 64)
    assert abs(s[0]) < 1e-12


def test_block_sums_and_ragged_counts():
    x = np.arange(200 * 4, dtype=np.float64).reshape(200, 4)
    sums, counts, _ = so.block_stats(x, 64)
    assert counts.tolist() == [64, 64, 64, 8]
    assert np.array_equal(sums[3], x[192:].sum(axis=0))


def test_keep_count_rounding():
    assert so.keep_count(10, 0.3) == 3          # 0.3*10 = 3.0000000000000004 must not become 4
    assert so.keep_count(7, 0.5) == 4
    assert so.keep_count(5, 1.0) == 5
    assert so.keep_count(1000, 1e-6) == 1
    assert so.keep_count(0, 0.5) == 0
    assert so.keep_count(3, 0.34) == 2
    for C in range(1, 200):
        for tk in (0.1, 0.25, 0.3, 0.5, 0.7, 0.9, 1.0):
            kk = so.keep_count(C, tk)
            assert 1 <= kk <= C
            assert kk >= tk * C - 1e-6 and (kk - 1) < tk * C + 1e-6


def test_select_brute_force_with_ties():
    r = np.random.default_rng(4)
    for trial in range(300):
        n = int(r.integers(1, 11))
        s = np.round(r.standard_normal(n), 1)        # many exact ties
        cand = r.random(n) < 0.8
        k = int(r.integers(0, cand.sum() + 1))
        sel = set(so.select_row(s, cand, k).tolist())
        js = [j for j in range(n) if cand[j]]
        found = []
        for sub in itertools.combinations(js, k):
            S = set(sub)
            ok = all((s[a] > s[b]) or (s[a] == s[b] and a < b)
                     for a in S for b in js if b not in S)
            if ok:
                found.append(S)
        assert len(found) == 1
        assert sel == found[0]


def test_topk_on_softmax_equals_topk_on_logits():
    r = np.random.default_rng(5)
    for _ in range(50):
        s = r.standard_normal(40) * 3
        cand = r.random(40) < 0.7
        p = so.row_softmax(s, cand)
        for k in (1, 5, int(cand.sum())):
            a = so.select_row(s, cand, k)
            b = so.select_row(p, cand, k)
            assert np.array_equal(a, b)
        assert abs(p[cand].sum() - 1) < 1e-12


def test_cdf_keep_count_brute_force():
    # the kept count is the smallest size of ANY candidate subset whose softmax mass
    # reaches tau (the best blocks reach it first), found by enumeration
    r = np.random.default_rng(41)
    for trial in range(300):
        n = int(r.integers(1, 10))
        s = r.standard_normal(n) * 2
        cand = r.random(n) < 0.8
        if not cand.any():
            assert so.cdf_keep_count(s, cand, 0.5) == 0
            continue
        tau = float(r.uniform(0.05, 1.0))
        js = np.flatnonzero(cand)
        w = np.exp(s[js] - s[js].max())
        w /= w.sum()
        best = None
        for kk in range(1, js.size + 1):
            if max(sum(c) for c in itertools.combinations(w, kk)) >= tau - 1e-12:
                best = kk
                break
        best = js.size if best is None else best
        got = so.cdf_keep_count(s, cand, tau)
        near = np.abs(np.cumsum(np.sort(w)[::-1]) - tau).min() < 1e-9
        assert got == best or near


def test_cdf_keep_count_closed_forms():
    cand = np.ones(10, dtype=bool)
    s = np.zeros(10)                                   # uniform: p = 0.1 each
    for tau, want in ((0.05, 1), (0.25, 3), (0.55, 6), (0.99, 10), (1.0, 10)):
        assert so.cdf_keep_count(s, cand, tau) == want
    s2 = np.array([math.log(9.0), 0, 0, 0, 0, 0, 0, 0, 0, 0])   # p = (0.5, 1/18 x 9)
    assert so.cdf_keep_count(s2, cand, 0.4) == 1
    assert so.cdf_keep_count(s2, cand, 0.5 + 1.5 / 18) == 3
    assert so.cdf_keep_count(s2, ~cand, 0.5) == 0
    r = np.random.default_rng(42)
    s3 = r.standard_normal(50)
    ks = [so.cdf_keep_count(s3, np.ones(50, bool), t) for t in np.linspace(0.01, 1.0, 60)]
    assert ks[0] >= 1 and ks[-1] == 50 and all(a <= b for a, b in zip(ks, ks[1:]))


def test_cdf_mask_keeps_the_ranked_prefix():
    N, D = 1000, 64
    q, k, _ = _drift_head(N, D, 43)
    for causal in (False, True):
        for tau in (0.3, 0.9):
            mask, info = so.predict_mask(q, k, so.OracleParams(cdf=tau, causal=causal, theta=0.05))
            S, valid, simk, simq = info["scores"], info["valid"], info["simk"], info["simq"]
            for i in range(mask.shape[0]):
                cand = valid[i] & simk
                if not cand.any() or not simq[i]:
                    continue
                kept = np.flatnonzero(mask[i] & cand)
                p = so.row_softmax(S[i], cand)
                assert p[kept].sum() >= tau - 1e-12                 # the mass is reached
                assert kept.size == info["kcount"][i]
                rest = np.flatnonzero(cand & ~mask[i])
                if rest.size:                                      # ... by the best blocks
                    assert S[i][kept].min() >= S[i][rest].max()
                    drop = p[kept].sum() - p[kept].min()
                    assert drop < tau + 1e-12                      # and no block is spare


def test_planted_cdf_off_by_one_is_caught(monkeypatch):
    orig = so.cdf_keep_count

    def bad(scores_row, cand, tau):
        return max(0, orig(scores_row, cand, tau) - 1)
    monkeypatch.setattr(so, "cdf_keep_count", bad)
    with pytest.raises(AssertionError):
        test_cdf_keep_count_closed_forms()


def _drift_head(N, D, seed):
    r = np.random.default_rng(seed)
    nb = (N + 63) // 64
    mu = np.cumsum(r.standard_normal((nb, D)) * 0.3, axis=0)
    return [np.repeat(mu, 64, axis=0)[:N] + r.standard_normal((N, D)) for _ in range(3)]


@pytest.mark.parametrize("causal", [False, True])
def test_topk1_filter_off_equals_sdpa(causal):
    N, D = 450, 64
    q, k, v = _drift_head(N, D, 2)
    p = so.OracleParams(topk=1.0, causal=causal)
    mask, _ = so.predict_mask(q, k, p)
    assert np.array_equal(mask, so.block_valid(N, causal))
    o = so.attend_head(q, k, v, mask, causal)
    assert np.abs(o - sdpa64(q, k, v, causal=causal)).max() < 1e-12


def test_mask_counting_invariant_and_monotone():
    N, D = 1000, 64
    q, k, v = _drift_head(N, D, 8)
    for causal in (False, True):
        prev = None
        for tk in (0.1, 0.3, 0.5, 0.8, 1.0):
            p = so.OracleParams(topk=tk, causal=causal, theta=0.05)
            mask, info = so.predict_mask(q, k, p)
            valid = info["valid"]
            assert not (mask & ~valid).any()
            forced = valid & (~info["simq"][:, None] | ~info["simk"][None, :])
            cand = valid & info["simk"][None, :]
            for i in range(mask.shape[0]):
                if not info["simq"][i]:
                    assert np.array_equal(mask[i], valid[i])
                else:
                    # forced columns plus exactly k_i of the candidates
                    assert (mask[i] & cand[i]).sum() == info["kcount"][i]
                    assert (mask[i] & forced[i]).sum() == forced[i].sum()
            if prev is not None:
                assert not (prev & ~mask).any()      # larger topk never drops a block
            prev = mask


def test_similarity_gate_is_live_on_structured_and_noise_blocks():
    r = np.random.default_rng(0)
    noise = r.standard_normal((128, 64))
    _, _, s = so.block_stats(noise, 64)
    assert (s < 0.1).all()                     # i.i.d. blocks sit near 1/n
    struct = noise * 0.3 + r.standard_normal(64)
    _, _, s = so.block_stats(struct, 64)
    assert (s > 0.5).all()


# --------------------------------------------------------------------- the filter

def _filter_case():
    # rows see one strong early block, later blocks are 20 logits lower except the last
    N, D = 128, 16
    r = np.random.default_rng(1)
    q = np.zeros((N, D))
    q[:, 0] = 1.0
    k = r.standard_normal((N, D)) * 0.01
    k[:64, 0] = 30.0       # block 0: logits ~30/4
    k[64:, 0] = -50.0      # block 1: logits ~-12.5, i.e. ~20 below block 0
    v = r.standard_normal((N, D))
    return q, k, v


def test_filter_off_equals_lambda_minus_inf_and_skips_only_negligible():
    q, k, v = _filter_case()
    mask = np.ones((1, 2), dtype=bool)
    o0 = so.attend_head(q, k, v, mask, False)
    oi = so.attend_head(q, k, v, mask, False, lam=-np.inf)
    assert np.array_equal(o0, oi)
    of, skips = so.attend_head(q, k, v, mask, False, lam=-10.0, return_skips=True)
    assert all(sk == [1] for sk in skips.values())
    # with block 1 skipped the output is the softmax over block 0 alone
    assert np.abs(of - sdpa64(q, k[:64], v[:64], scale=0.25)).max() < 1e-12
    # and differs from the unfiltered output by less than the bound 2*max|v|*64*e^lam
    assert np.abs(of - o0).max() <= 2 * np.abs(v).max() * 64 * math.exp(-10.0)
    o5, skips5 = so.attend_head(q, k, v, mask, False, lam=-25.0, return_skips=True)
    assert all(sk == [] for sk in skips5.values())
    assert np.array_equal(o5, o0)


def test_filter_first_block_never_skipped_and_later_max_not_skipped():
    q, k, v = _filter_case()
    k2 = k.copy()
    k2[:64, 0], k2[64:, 0] = -50.0, 30.0      # the strong block comes second
    mask = np.ones((1, 2), dtype=bool)
    of, skips = so.attend_head(q, k2, v, mask, False, lam=-10.0, return_skips=True)
    assert all(sk == [] for sk in skips.values())


def test_filter_matches_sequential_scalar_simulation():
    N, D = 600, 32
    r = np.random.default_rng(12)
    q = r.standard_normal((N, D)) * 2
    k = r.standard_normal((N, D)) * 2
    v = r.standard_normal((N, D))
    mask = so.block_valid(N, True)
    lam = -4.0
    _, skips = so.attend_head(q, k, v, mask, True, lam=lam, return_skips=True)
    # independent scalar walk: per row, per block, compare with explicit loops
    for (i, g), sk in skips.items():
        t0 = 128 * i + 32 * g
        t1 = min(N, t0 + 32, 128 * i + 128)
        m = [-math.inf] * (t1 - t0)
        exp_sk = []
        for j in np.flatnonzero(mask[i]):
            best = -math.inf
            mloc = []
            for t in range(t0, t1):
                mx = -math.inf
                for s in range(64 * j, min(N, 64 * j + 64)):
                    if s <= t:
                        mx = max(mx, float(q[t] @ k[s]) / math.sqrt(D))
                mloc.append(mx)
            fin = [x for x in mloc if x > -math.inf]
            if not fin:
                exp_sk.append(int(j))
                continue
            d = max(mloc[r_] - max(m[r_], mloc[r_]) for r_ in range(t1 - t0) if mloc[r_] > -math.inf)
            if d < lam:
                exp_sk.append(int(j))
            else:
                m = [max(a, b) for a, b in zip(m, mloc)]
        assert sk == exp_sk
    assert sum(len(s) for s in skips.values()) > 0


# -------------------------------------------------------------------- int8 option

def test_quantize_exact_grid_round_trip():
    r = np.random.default_rng(3)
    c = r.integers(-127, 128, size=(64, 32))
    c[5, 7] = 127
    x = (c * 2.0 ** -5).astype(np.float32)
    codes, d = so.quantize_blocks(x, 64)
    assert np.array_equal(codes.astype(np.int64), c)
    assert d[0] == np.float32(2.0 ** -5)


def test_quantize_error_bound_and_range():
    r = np.random.default_rng(4)
    x = (r.standard_normal((300, 64)) * 3).astype(np.float32)
    x[128:192] = 0.0
    codes, d = so.quantize_blocks(x, 64)
    assert codes.min() >= -127 and codes.max() <= 127
    assert d[2] == 0 and not codes[128:192].any()
    for b in range(5):
        xb = x[64 * b: 64 * b + 64].astype(np.float64)
        err = np.abs(xb - codes[64 * b: 64 * b + 64] * np.float64(d[b])).max()
        assert err <= 0.5 * d[b] * (1 + 1e-5) + 1e-30
        if d[b] > 0:
            assert np.abs(codes[64 * b: 64 * b + 64]).max() == 127


def test_k_smoothing_leaves_exact_attention_unchanged():
    N, D = 320, 64
    q, k, v = _drift_head(N, D, 6)
    ks, kmean = so.smooth_k(k.astype(np.float32))
    assert np.abs(ks.astype(np.float64).mean(axis=0)).max() < 1e-5
    mask = so.block_valid(N, True)
    o1 = so.attend_head(q, k, v, mask, True)
    o2 = so.attend_head(q, k - kmean.astype(np.float64), v, mask, True)
    assert np.abs(o1 - o2).max() < 1e-12


def test_int8_simulation_close_to_fp64():
    N, D = 512, 64
    q, k, v = _drift_head(N, D, 7)
    mask = so.block_valid(N, True)
    o = so.attend_head(q, k, v, mask, True)
    oi = so.attend_head_int8_sim(q.astype(np.float32), k.astype(np.float32), v, mask, True, q_rows=32)
    assert np.abs(o - oi).max() < 5e-2


# ------------------------------------------------------------------------ Hilbert

@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_hilbert_cube_properties(m):
    from oracle.hilbert_ref import cube_order
    c = cube_order(m)
    side = 1 << m
    lin = (c[:, 0] * side + c[:, 1]) * side + c[:, 2]
    assert np.array_equal(np.sort(lin), np.arange(side ** 3))      # bijection
    assert (c[0] == 0).all()                                          # starts at the origin
    assert (np.abs(np.diff(c, axis=0)).sum(axis=1) == 1).all()        # unit steps
    for lvl in range(1, m):                                           # aligned sub-cubes
        sub = 1 << lvl
        blocks = c.reshape(-1, sub ** 3, 3) // sub
        assert (blocks == blocks[:, :1]).all()


def test_hilbert_grid_order_is_permutation():
    from oracle.hilbert_ref import hilbert_cell_order
    for shp in ((13, 30, 45), (1, 1, 1), (2, 3, 5), (8, 8, 8)):
        p = hilbert_cell_order(*shp)
        assert np.array_equal(np.sort(p), np.arange(np.prod(shp)))


def test_hilbert_reorder_equivariance_of_dense_attention():
    from oracle.hilbert_ref import hilbert_cell_order
    T, Hh, W, text = 2, 5, 7, 9
    N, D = text + T * Hh * W, 16
    q, k, v = rnd(N, D, 21)
    perm = np.concatenate([np.arange(text), text + hilbert_cell_order(T, Hh, W)])
    mask = so.block_valid(N, False)
    o = so.attend_head(q, k, v, mask, False)
    op = so.attend_head(q[perm], k[perm], v[perm], mask, False)
    back = np.empty_like(op)
    back[perm] = op
    assert np.abs(back - o).max() < 1e-12


# ------------------------------------------------- planted mistakes are caught

def test_planted_causal_off_by_one_is_caught(monkeypatch):
    def bad(qg, t0, k, j, causal, scale, N):
        s0, s1 = 64 * j, min(N, 64 * j + 64)
        z = scale * (qg @ k[s0:s1].T)
        if causal:
            t = t0 + np.arange(qg.shape[0])[:, None]
            s = np.arange(s0, s1)[None, :]
            z = np.where(s < t, z, -np.inf)
        return z, s0, s1
    monkeypatch.setattr(so, "_block_logits", bad)
    N, D = 200, 32
    q, k, v = rnd(N, D, 1)
    o = so.attend_head(q, k, v, so.block_valid(N, True), True)
    assert np.abs(o[1:] - sdpa64(q, k, v, causal=True)[1:]).max() > 1e-6


def test_planted_tie_break_is_caught(monkeypatch):
    def bad(scores, cand, k):
        js = np.flatnonzero(cand)
        if k == 0 or js.size == 0:
            return np.zeros(0, dtype=np.int64)
        order = np.lexsort((-js, -scores[js]))      # ties to the HIGHER index
        return np.sort(js[order[:k]])
    monkeypatch.setattr(so, "select_row", bad)
    with pytest.raises(AssertionError):
        test_select_brute_force_with_ties()


def test_planted_selfsim_normalisation_is_caught(monkeypatch):
    orig = so.block_stats

    def bad(x, rows):
        s, c, sims = orig(x, rows)
        return s, c, sims * c / np.maximum(c - 1, 1)   # off-diagonal mean instead
    monkeypatch.setattr(so, "block_stats", bad)
    with pytest.raises(AssertionError):
        test_selfsim_special_cases()


def test_planted_missing_normaliser_is_caught(monkeypatch):
    orig = so.attend_group

    def bad(*a, **kw):
        o, sk = orig(*a, **kw)
        return o * 1.01, sk
    monkeypatch.setattr(so, "attend_group", bad)
    N, D = 128, 16
    q, k, v = rnd(N, D, 4)
    o = so.attend_head(q, k, v, np.ones((1, 2), dtype=bool), False)
    assert np.abs(o - sdpa64(q, k, v)).max() > 1e-6


def test_block_smoothing_with_compensation_is_exact_in_fp64():
    # q.k'' + q.kbar_j == q.k: the block smoothing changes no logit once compensated
    N, D = 300, 64
    q, k, v = _drift_head(N, D, 3)
    k32 = k.astype(np.float32)
    ks, kbar = so.smooth_k_blocks(k32)
    jb = np.arange(N) // 64
    assert np.abs(ks.astype(np.float64) + kbar[jb].astype(np.float64) - k32.astype(np.float64)).max() < 1e-5
    for j in range(kbar.shape[0]):
        blk = ks[64 * j: 64 * j + 64].astype(np.float64)
        assert np.abs(blk.mean(axis=0)).max() < 1e-5          # each block is centred
    z_direct = q @ k32.astype(np.float64).T
    z_split = q @ ks.astype(np.float64).T + (q @ kbar.astype(np.float64).T)[:, jb]
    assert np.abs(z_direct - z_split).max() < 1e-4 * np.abs(z_direct).max()


def test_int8_codes_are_integer_decisions_in_fp32():
    r = np.random.default_rng(9)
    q = (r.standard_normal((96, 64)) * 2).astype(np.float32)
    k = (r.standard_normal((130, 64)) + 3).astype(np.float32)
    qc, qd, kc, kd, kbar = so.int8_qk_inputs(q, k, 32)
    assert qd.shape == (3,) and kd.shape == (3,) and kbar.shape == (3, 64)
    for g in range(3):
        blk = q[32 * g: 32 * g + 32]
        assert np.abs(qc[32 * g: 32 * g + 32]).max() == 127
        assert qd[g] == np.float32(np.abs(blk).max()) / np.float32(127)


# ------------------------------------------------------------------ fp8 P.V option

def _e4m3_table():
    """Every finite non-negative OCP E4M3 value, decoded from its bit fields (bias 7,
    3 fraction bits, exponent field 0 = subnormal, code 0x7f = NaN); index = code."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


def test_e4m3_fixed_points_and_range():
    t = _e4m3_table()
    assert len(t) == 127 and np.all(np.diff(t) > 0)
    assert t[-1] == 448.0 and t[1] == 2.0 ** -9 and t[8] == 2.0 ** -6
    assert np.array_equal(so.e4m3_round(t), t)
    assert np.array_equal(so.e4m3_round(-t), -t)
    assert so.e4m3_round(np.array([463.9]))[0] == 448.0      # below the 448/512 midpoint
    with pytest.raises(ValueError):
        so.e4m3_round(np.array([465.0]))


def test_e4m3_nearest_with_ties_to_even_code():
    t = _e4m3_table()
    mids = (t[:-1] + t[1:]) / 2
    want = np.where(np.arange(len(mids)) % 2 == 0, t[:-1], t[1:])   # even code wins
    assert np.array_equal(so.e4m3_round(mids), want)
    gap = t[1:] - t[:-1]
    assert np.array_equal(so.e4m3_round(mids - 1e-3 * gap), t[:-1])
    assert np.array_equal(so.e4m3_round(mids + 1e-3 * gap), t[1:])
    r = np.random.default_rng(11)
    x = np.concatenate([r.uniform(0, 448, 3000), np.exp2(r.uniform(-12, 8.8, 3000))])
    x = x[x < 448]
    near = t[np.abs(x[:, None] - t[None, :]).argmin(axis=1)]     # brute force
    assert np.array_equal(so.e4m3_round(x), near)


def test_e4m3_matches_torch_float8():
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch has no float8_e4m3fn")
    r = np.random.default_rng(12)
    x = np.exp2(r.uniform(-12, 8.8, 20000)) * r.choice([-1.0, 1.0], 20000)
    x = np.concatenate([x[np.abs(x) < 448], (_e4m3_table()[:-1] + _e4m3_table()[1:]) / 2])
    x32 = x.astype(np.float32)
    lib = torch.from_numpy(x32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(so.e4m3_round(x32.astype(np.float64)), lib)


def test_fp8_v_quant_grid_zero_channel_and_error_bound():
    t = _e4m3_table()
    r = np.random.default_rng(13)
    codes = r.choice(t[8:], size=(200, 16)) * r.choice([-1.0, 1.0], size=(200, 16))
    codes[7, :] = 448.0                                  # every channel reaches the max
    v = codes * 0.125                                    # max |v| = 56 -> inv = 8 exactly
    v[:, 3] = 0.0
    c, s = so.fp8_v_quant(v)
    assert s.dtype == np.float32 and s[3] == 0 and not c[:, 3].any()
    keep = np.arange(16) != 3
    assert np.all(s[keep] == np.float32(0.125))
    assert np.array_equal(c[:, keep], codes[:, keep])
    x = (r.standard_normal((500, 8)) * np.array([1e-3, 0.1, 1, 3, 10, 100, 1e4, 0.5])).astype(np.float32)
    c, s = so.fp8_v_quant(x)
    assert np.all(np.abs(c).max(axis=0) == 448.0)
    y = x.astype(np.float64) * (np.float64(448.0) / np.abs(x.astype(np.float64)).max(axis=0))
    # half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute below 2^-6
    assert np.all(np.abs(c - y) <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10) * (1 + 1e-5))


def _pow2_logit_head(N, D, seed):
    """q, k with scale-1 logits z = n ln 2 for integers n in [-6, 2] (so every
    2^(z log2 e - M) is an exact E4M3 value) and V on the E4M3 grid times 1/8 with
    every channel's max |v| = 56."""
    r = np.random.default_rng(seed)
    q = np.zeros((N, D))
    q[:, 0] = math.log(2.0)
    k = np.zeros((N, D))
    k[:, 0] = r.integers(-6, 3, size=N)
    t = _e4m3_table()
    v = r.choice(t[8:], size=(N, D)) * r.choice([-1.0, 1.0], size=(N, D)) * 0.125
    v[r.integers(0, N), :] = 56.0
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_pv8_exact_when_p_and_v_are_representable(causal):
    N, D = 300, 16
    q, k, v = _pow2_logit_head(N, D, 14 + causal)
    mask = so.block_valid(N, causal)
    o8 = so.attend_head_pv8_sim(q, k, v, mask, causal, scale=1.0)
    assert np.abs(o8 - sdpa64(q, k, v, causal=causal, scale=1.0)).max() < 1e-12
    # the filter with lambda = -inf changes nothing
    o8f = so.attend_head_pv8_sim(q, k, v, mask, causal, scale=1.0, lam=-np.inf)
    assert np.array_equal(o8, o8f)


def test_pv8_rounded_weights_closed_form():
    # two keys with P = (1, 1.0625) relative to the max: 2^(z log2 e - 1) = (0.5, 0.53125),
    # and 0.53125 is the midpoint of 0.5 and 0.5625, so E4M3 gives (0.5, 0.5) and
    # O = (v0 + v1) / 2 exactly (normaliser over the rounded weights)
    D = 8
    q = np.zeros((2, D))
    q[:, 0] = 1.0
    k = np.zeros((2, D))
    k[1, 0] = math.log(1.0625)
    v = np.zeros((2, D))
    v[0, :] = 56.0
    v[1, :] = np.linspace(-56, 56, D) * 0.5
    v[1, 0] = -56.0
    o = so.attend_head_pv8_sim(q, k, v, np.ones((1, 1), bool), False, scale=1.0)
    c, s = so.fp8_v_quant(v)
    want = (c[0] + c[1]) * s.astype(np.float64) / 2
    assert np.abs(o[0] - want).max() < 1e-12 and np.abs(o[1] - want).max() < 1e-12


def test_pv8_close_to_exact_and_int8_variant():
    N, D = 512, 64
    q, k, v = _drift_head(N, D, 15)
    mask = so.block_valid(N, True)
    o = so.attend_head(q, k, v, mask, True)
    o8 = so.attend_head_pv8_sim(q, k, v, mask, True)
    o8i = so.attend_head_pv8_sim(q, k, v, mask, True, qk="int8")
    vmax = np.abs(v).max()
    c, s = so.fp8_v_quant(v)
    verr = np.abs(c * s - v).max()
    # a sanity bound: each value moves by at most verr and each normal weight by at
    # most 2^-4 of itself (subnormal weights, below 2^-6 of the row max, by 2^-10)
    assert 1e-4 < np.abs(o - o8).max() <= verr + 2 * 2.0 ** -4 / (1 - 2.0 ** -4) * 2 * vmax
    assert np.abs(o8 - o8i).max() < 0.05 * vmax
    # rows with many keys average the rounding errors out
    assert np.abs(o - o8)[256:].mean() < 2e-3 * vmax


def test_planted_unrounded_p_is_caught(monkeypatch):
    monkeypatch.setattr(so, "e4m3_round", lambda x: np.asarray(x, dtype=np.float64))
    with pytest.raises(AssertionError):
        test_pv8_rounded_weights_closed_form()
