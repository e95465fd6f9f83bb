"""Pins of the oracle's stage-1 predictor that do not read the oracle's own values.

Two kinds of pin:

* closed forms: inputs built so that every block mean, self-similarity and pooled
  score is known by construction (blocks of identical tokens, alternating tokens,
  blocks padded with zero rows, ragged tails), with the expected mask written out
  by hand from the method's definition ([chapterpal] method paragraph: non-similar
  blocks are always computed, the others compete through a compressed attention
  map; [topgit] FAQ: ``topk`` is the kept fraction; the threshold variant keeps the
  smallest prefix reaching a softmax mass);
* brute force: the whole mask recomputed from the definitions with explicit loops
  and enumeration (block means as explicit token sums, self-similarity as the mean
  of the explicit n x n cosine matrix, validity from the token-level causal matrix,
  the kept set as the best subset over all subsets of the right size), compared
  with ``predict_mask`` at ragged lengths, causal and not, for top-k and the
  threshold selection.

A last group plants three plausible mistakes in the oracle (the pooled-score scale
dropped, ragged tail means divided by the full block size, the similarity gate
ignored) and checks that a pin fails for each.
"""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import sparge_oracle as so


# ------------------------------------------------------------------ brute force

def _bf_block_stats(x, rows):
    """Per block: mean (explicit token sum over its count) and the mean of the
    explicit n x n cosine matrix (zero rows contribute zero cosines)."""
    N, D = x.shape
    X = torch.from_numpy(np.asarray(x, np.float64))
    means, sims = [], []
    for b0 in range(0, N, rows):
        blk = X[b0:min(N, b0 + rows)]
        n = blk.shape[0]
        tot = torch.zeros(D, dtype=torch.float64)
        for r in range(n):
            tot += blk[r]
        means.append((tot / n).numpy())
        cs = F.cosine_similarity(blk[:, None, :], blk[None, :, :], dim=-1, eps=1e-300)
        nz = blk.norm(dim=1) > 0
        cs = cs * nz[:, None] * nz[None, :]
        sims.append(float(cs.sum()) / (n * n))
    return np.stack(means), np.array(sims)


def _bf_valid(N, causal):
    nQ, nK = (N + 127) // 128, (N + 63) // 64
    tok = np.tril(np.ones((N, N), dtype=bool)) if causal else np.ones((N, N), dtype=bool)
    V = np.zeros((nQ, nK), dtype=bool)
    for i in range(nQ):
        for j in range(nK):
            V[i, j] = tok[128 * i:min(N, 128 * i + 128), 64 * j:min(N, 64 * j + 64)].any()
    return V


def _bf_subsets(m):
    """Every subset of range(m) as a (2^m, m) 0/1 matrix."""
    return ((np.arange(1 << m)[:, None] >> np.arange(m)[None, :]) & 1).astype(bool)


def _bf_best_subset(s, size):
    """The subset of the given size with the largest score sum, by enumeration over
    all subsets of that size (ties would make it ambiguous: asserted absent)."""
    idx = np.array(list(itertools.combinations(range(len(s)), size)))
    tot = s[idx].sum(axis=1)
    best = np.flatnonzero(tot == tot.max())
    assert best.size == 1, "exact tie between subsets"
    return set(idx[best[0]].tolist())


def bf_mask(q, k, causal, theta=0.1, topk=None, cdf=None, scale=None):
    """The predicted mask from the definitions, for one head; returns (mask, margin)
    where margin is the smallest distance of a similarity from theta and of a
    cumulative softmax mass from tau (decisions that close are not asserted)."""
    N, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    qm, qs = _bf_block_stats(q, 128)
    km, ks = _bf_block_stats(k, 64)
    valid = _bf_valid(N, causal)
    margin = float(np.abs(np.concatenate([qs, ks]) - theta).min())
    nQ, nK = valid.shape
    M = np.zeros((nQ, nK), dtype=bool)
    for i in range(nQ):
        for j in range(nK):
            if valid[i, j] and (qs[i] < theta or ks[j] < theta):
                M[i, j] = True
        cand = [j for j in range(nK) if valid[i, j] and ks[j] >= theta]
        if not cand:
            continue
        s = np.array([scale * sum(qm[i, c] * km[j, c] for c in range(D)) for j in cand])
        if cdf is None:
            size = next(m for m in range(1, len(cand) + 1) if m >= topk * len(cand) - 1e-9)
            keep = _bf_best_subset(s, size)
        else:
            w = np.exp(s - s.max())
            p = w / w.sum()
            sub = _bf_subsets(len(cand))
            mass = sub.astype(np.float64) @ p
            size = sub.sum(axis=1)
            best = np.array([mass[size == m].max() for m in range(1, len(cand) + 1)])
            margin = min(margin, float(np.abs(best - cdf).min()))
            m_min = 1 + int(np.flatnonzero(best >= cdf)[0])
            keep = _bf_best_subset(s, m_min)
        for a in keep:
            M[i, cand[a]] = True
    return M, margin


def _drift_head(N, D, seed, step=0.3):
    """Q and K around a random-walk mean that starts at zero (so the first blocks
    are noise, hence non-similar) and steps once per 64 tokens."""
    r = np.random.default_rng(seed)
    nb = (N + 63) // 64
    mu = np.concatenate([np.zeros((1, D)), np.cumsum(r.standard_normal((nb - 1, D)) * step, axis=0)])
    return [np.repeat(mu, 64, axis=0)[:N] + r.standard_normal((N, D)) for _ in range(2)]


BRUTE_CASES = [(N, causal, sel) for N in (65, 200, 333, 1000) for causal in (False, True)
               for sel in (("topk", 0.3), ("topk", 0.5), ("cdf", 0.6), ("cdf", 0.9))]


@pytest.mark.parametrize("N,causal,sel", BRUTE_CASES)
def test_whole_mask_brute_force(N, causal, sel):
    D = 16
    q, k = _drift_head(N, D, seed=N + 7 * causal)
    kind, val = sel
    bm, margin = bf_mask(q, k, causal, topk=val if kind == "topk" else None,
                         cdf=val if kind == "cdf" else None)
    p = so.OracleParams(topk=val if kind == "topk" else 0.5, cdf=val if kind == "cdf" else None,
                        causal=causal)
    om, _ = so.predict_mask(q, k, p)
    assert margin > 1e-9
    assert np.array_equal(om, bm)


def test_brute_force_inputs_exercise_every_branch():
    """The brute-force inputs hold similar and non-similar blocks on both axes and
    rows with more candidates than they keep (so gate, forcing and selection are
    all decided somewhere)."""
    q, k = _drift_head(1000, 16, seed=1000)
    _, qs = _bf_block_stats(q, 128)
    _, ks = _bf_block_stats(k, 64)
    assert (qs < 0.1).any() and (qs >= 0.1).any()
    assert (ks < 0.1).any() and (ks >= 0.1).any()
    bm, _ = bf_mask(q, k, False, topk=0.3)
    assert 0 < bm.mean() < 1


# ----------------------------------------------------------------- closed forms

def _const_blocks(vals, rows, N):
    """Tokens such that every block of ``rows`` tokens holds copies of one vector."""
    x = np.zeros((N, vals.shape[1]))
    for b in range(vals.shape[0]):
        x[rows * b:min(N, rows * b + rows)] = vals[b]
    return x


def test_pooled_scale_and_cdf_prefix_closed_form():
    """One Q vector (1, 0, 0, 0) everywhere; K block 0 is copies of (2 ln 9, 1, 0, 0),
    blocks 1..9 copies of (0, 1, 0, 0).  Every block is similar (identical tokens:
    similarity 1).  With D = 4 the pooled scores are (1/2) q . k: ln 9 for block 0 and
    0 for the rest, so the row softmax is 1/2 for block 0 and 1/18 for each other
    block.  Mass 0.6 needs 0.5 + 2/18 = 0.611: blocks {0, 1, 2} (ties to the lower
    index); mass 0.45 is reached by block 0 alone; mass 0.55 needs one more block
    (0.5 + 1/18 = 0.5556); mass 0.99 needs all ten."""
    N, D = 640, 4
    q = np.zeros((N, D))
    q[:, 0] = 1.0
    kv = np.zeros((10, D))
    kv[:, 1] = 1.0
    kv[0, 0] = 2.0 * math.log(9.0)
    k = _const_blocks(kv, 64, N)
    for tau, want in ((0.6, [0, 1, 2]), (0.45, [0]), (0.55, [0, 1]), (0.99, list(range(10)))):
        m, _ = so.predict_mask(q, k, so.OracleParams(cdf=tau))
        for i in range(5):
            assert np.flatnonzero(m[i]).tolist() == want, (tau, i)
    # top-k keeps the fraction of the candidates whatever the scale: 0.25 of 10 -> 3
    m, _ = so.predict_mask(q, k, so.OracleParams(topk=0.25))
    assert all(np.flatnonzero(m[i]).tolist() == [0, 1, 2] for i in range(5))


def test_ragged_tail_means_closed_form():
    """N = 200: K blocks 0..2 hold 64 copies of (a_j, 1, 0, 0) with a = 1, 2, 3; the
    ragged last block holds 8 copies of (4, 1, 0, 0).  Its mean is (4, 1, 0, 0) (a
    mean over its own 8 rows), so with Q = (1, 0, 0, 0) it has the largest score and
    top-k 0.25 (one of four candidates) keeps it.  The ragged Q tail (72 rows) holds
    copies of (3, 0, 0, 0), so its mean is (3, 0, 0, 0) and its pooled scores are
    (1/2) 3 a_j; the masses of the ranked prefixes follow from those scores, and the
    thresholds below sit between them."""
    N, D = 200, 4
    q = np.zeros((N, D))
    q[:128, 0] = 1.0
    q[128:, 0] = 3.0
    kv = np.zeros((4, D))
    kv[:, 1] = 1.0
    kv[:, 0] = [1.0, 2.0, 3.0, 4.0]
    k = _const_blocks(kv, 64, N)
    m, _ = so.predict_mask(q, k, so.OracleParams(topk=0.25))
    assert np.flatnonzero(m[0]).tolist() == [3]
    assert np.flatnonzero(m[1]).tolist() == [3]
    # threshold selection on the ragged Q row: scores (3/2) a_j = 1.5, 3, 4.5, 6
    s = 1.5 * np.array([1.0, 2.0, 3.0, 4.0])
    p = np.exp(s) / np.exp(s).sum()
    # ranked masses p3, p3 + p2, p3 + p2 + p1 = 0.779, 0.953, 0.991
    assert p[3] < 0.88 < p[3] + p[2] < 0.97 < p[3] + p[2] + p[1]
    m, _ = so.predict_mask(q, k, so.OracleParams(cdf=0.88))
    assert np.flatnonzero(m[1]).tolist() == [2, 3]
    m, _ = so.predict_mask(q, k, so.OracleParams(cdf=0.97))
    assert np.flatnonzero(m[1]).tolist() == [1, 2, 3]


def test_similarity_gate_forced_rows_and_columns_closed_form():
    """Q blocks: 0 = copies of e0 (similarity 1), 1 = alternating +e0 / -e0
    (similarity 0: non-similar).  K blocks: 0 = copies of 2 e0, 1 = alternating
    +e1 / -e1 (similarity 0), 2 = 32 copies of e0 then 32 zero rows (similarity
    exactly (32/64)^2 = 0.25), 3 = copies of 3 e0, 4 = copies of -e0.  Non-causal,
    top-k 0.25.

    theta = 0.25 (block 2 similar, since sim >= theta): row 0's candidates are
    K blocks {0, 2, 3, 4} with scores (1/2)(2, 0.5, 3, -1) (block 2's mean is e0/2):
    it keeps one, block 3, plus the forced non-similar column 1.  Row 1 is non-similar:
    every block.  theta just above 0.25: block 2 is forced too."""
    N, D = 320, 4
    e0, e1 = np.eye(D)[0], np.eye(D)[1]
    q = np.zeros((N, D))
    q[:128] = e0
    q[128:256] = np.where((np.arange(128) % 2 == 0)[:, None], e0, -e0)
    q[256:] = e0
    k = np.zeros((N, D))
    k[0:64] = 2 * e0
    k[64:128] = np.where((np.arange(64) % 2 == 0)[:, None], e1, -e1)
    k[128:160] = e0
    k[192:256] = 3 * e0
    k[256:320] = -e0
    m, _ = so.predict_mask(q, k, so.OracleParams(topk=0.25, theta=0.25))
    assert np.flatnonzero(m[0]).tolist() == [1, 3]
    assert m[1].all()
    # the last Q block (64 copies of e0, similar) behaves like row 0
    assert np.flatnonzero(m[2]).tolist() == [1, 3]
    m2, _ = so.predict_mask(q, k, so.OracleParams(topk=0.25, theta=0.25 + 1e-12))
    assert np.flatnonzero(m2[0]).tolist() == [1, 2, 3]
    assert m2[1].all()
    # theta <= 0 makes every block similar: row 1 competes too (one of five kept:
    # ceil(0.25 * 5) = 2 blocks; row 1's mean is 0, so all its scores tie at 0 and
    # the two lowest indices win)
    m3, _ = so.predict_mask(q, k, so.OracleParams(topk=0.25, theta=0.0))
    assert np.flatnonzero(m3[0]).tolist() == [0, 3]
    assert np.flatnonzero(m3[1]).tolist() == [0, 1]


def test_causal_validity_drops_future_blocks_from_candidates_closed_form():
    """Causal, N = 256, every token of Q = e0, K blocks 0..3 copies of (1, 2, 3, 4) e0:
    Q block 0 sees K blocks 0 and 1 only, so top-k 0.5 keeps block 1 (score 2/2 vs
    1/2); Q block 1 sees all four and keeps the best two, {2, 3}."""
    N, D = 256, 4
    e0 = np.eye(D)[0]
    q = np.tile(e0, (N, 1))
    k = _const_blocks(np.outer([1.0, 2.0, 3.0, 4.0], e0), 64, N)
    m, _ = so.predict_mask(q, k, so.OracleParams(topk=0.5, causal=True))
    assert np.flatnonzero(m[0]).tolist() == [1]
    assert np.flatnonzero(m[1]).tolist() == [2, 3]


# ------------------------------------------------------------ planted mistakes

def test_planted_dropped_pooled_scale_is_caught(monkeypatch):
    monkeypatch.setattr(so, "pooled_scores", lambda qm, km, scale: qm @ km.T)
    with pytest.raises(AssertionError):
        test_pooled_scale_and_cdf_prefix_closed_form()
    with pytest.raises(AssertionError):
        test_whole_mask_brute_force(1000, False, ("cdf", 0.6))


def test_planted_tail_mean_over_full_block_is_caught(monkeypatch):
    orig = so.block_stats

    def bad(x, rows):
        s, c, sims = orig(x, rows)
        return s, np.full_like(c, float(rows)), sims    # every block divided by its full size
    monkeypatch.setattr(so, "block_stats", bad)
    with pytest.raises(AssertionError):
        test_ragged_tail_means_closed_form()


def test_planted_ignored_similarity_gate_is_caught(monkeypatch):
    orig = so.block_stats

    def bad(x, rows):
        s, c, sims = orig(x, rows)
        return s, c, np.ones_like(sims)                 # every block counted as similar
    monkeypatch.setattr(so, "block_stats", bad)
    with pytest.raises(AssertionError):
        test_similarity_gate_forced_rows_and_columns_closed_form()
    with pytest.raises(AssertionError):
        test_whole_mask_brute_force(1000, True, ("topk", 0.3))


def test_planted_strict_theta_comparison_is_caught(monkeypatch):
    """sim > theta instead of sim >= theta: only the exact-threshold block notices."""
    orig = so.block_stats

    def bad(x, rows):
        s, c, sims = orig(x, rows)
        return s, c, np.where(sims == 0.25, np.nextafter(0.25, 0.0), sims)
    monkeypatch.setattr(so, "block_stats", bad)
    with pytest.raises(AssertionError):
        test_similarity_gate_forced_rows_and_columns_closed_form()
