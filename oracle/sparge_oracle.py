"""SpargeAttn, step by step, in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg
may import this module.  It shares no code with the GPU library.

Every function works on ONE attention head: tensors of shape (N, D), read as their
exact stored values widened to float64.  Page legend (see ``oracle/__init__``):
[topgit], [readme], [chapterpal], [gittools], [abstract].

What the method computes (the two-stage online filter, [abstract]; [chapterpal]
method paragraph):
  stage 1  predict a block mask from block-compressed Q and K: blocks whose tokens
           are not similar to each other are always computed, the rest compete
           through a compressed (pooled) attention map, of which each block row
           keeps its top fraction ``topk`` ([topgit] "Using the plug-and-play API"
           and FAQ on ``topk``; [gittools] recommended-API section);
  stage 2  block-sparse attention over the kept 128x64 blocks ([topgit] "Key
           features"; [gittools] custom block-sparse mask section), with an online
           softmax-aware filter that drops updates whose weight is negligible for
           a whole wavefront's rows ([chapterpal] method paragraph; [abstract]);
  option   8-bit quantized Q K^T with K mean smoothing, as in the SageAttention
           base the library builds on ([topgit] "Key features" and "Strengths";
           [readme] "Avalible API").

Where the pages leave a step open, the reading taken is stated at the step.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# 128 query rows x 64 key rows per mask block, fixed ([topgit] "Key features" and
# "Known limitations"; [gittools] custom block-sparse mask section).
BQ = 128
BK = 64


@dataclass
class OracleParams:
    """Knobs of the method.  Defaults are the readings where the pages are silent."""

    topk: float = 0.5            # fraction of candidate blocks kept per block row
    cdf: Optional[float] = None  # when set: keep by softmax mass instead (cdf_keep_count)
    causal: bool = False
    theta: float = 0.1           # self-similarity threshold (reading; not on the pages)
    lam: Optional[float] = None  # filter threshold in natural-log logit units; None = off
    group: int = 32              # rows sharing one filter decision (one wavefront's rows)
    scale: Optional[float] = None  # None -> 1/sqrt(D), the SDPA default


def num_blocks(N: int) -> Tuple[int, int]:
    """(ceil(N/128), ceil(N/64)).

    Reading: the mask shape printed in [gittools] (custom block-sparse mask section)
    mixes a ceiling and a floor division; a ceiling on both axes is taken so that a
    ragged tail block exists on both axes.
    """
    return (N + BQ - 1) // BQ, (N + BK - 1) // BK


def block_valid(N: int, causal: bool) -> np.ndarray:
    """(nQ, nK) bool: block (i, j) holds at least one allowed (query, key) pair.

    Causal follows SDPA's convention for equal query/key lengths: query t sees keys
    s <= t ([topgit] "Using the plug-and-play API": ``is_causal`` as for standard
    attention).  Reading: a block is valid when any of its pairs is allowed.
    """
    nQ, nK = num_blocks(N)
    if not causal:
        return np.ones((nQ, nK), dtype=bool)
    i = np.arange(nQ)[:, None]
    j = np.arange(nK)[None, :]
    last_query = np.minimum(BQ * i + BQ - 1, N - 1)
    return BK * j <= last_query


def block_stats(x: np.ndarray, rows: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per block of ``rows`` tokens: channel sums, token counts, self-similarity.

    Self-similarity ([chapterpal] method paragraph: blocks with high internal
    similarity are compressed, non-similar blocks are fully computed).  Reading:
    the mean of the block's full n x n cosine-similarity matrix, diagonal included,
        sim = || sum_r x_r / ||x_r|| ||^2 / n^2,
    with a zero row contributing a zero unit vector.  The unit vector is formed as
    x_r * (1 / ||x_r||) in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    N, D = x.shape
    nb = (N + rows - 1) // rows
    sums = np.zeros((nb, D))
    counts = np.zeros(nb)
    sims = np.zeros(nb)
    for b in range(nb):
        xb = x[b * rows: min(N, (b + 1) * rows)]
        n = xb.shape[0]
        sums[b] = xb.sum(axis=0)
        counts[b] = n
        norms = np.sqrt(np.einsum("rc,rc->r", xb, xb))
        inv = np.zeros(n)
        nz = norms > 0
        inv[nz] = 1.0 / norms[nz]
        unit_sum = (xb * inv[:, None]).sum(axis=0)
        sims[b] = float(unit_sum @ unit_sum) / float(n * n)
    return sums, counts, sims


def pooled_scores(qmean: np.ndarray, kmean: np.ndarray, scale: float) -> np.ndarray:
    """Compressed attention logits between block means: s_ij = scale * qbar_i . kbar_j."""
    return scale * (qmean @ kmean.T)


def keep_count(C: int, topk: float) -> int:
    """How many of C candidate blocks a row keeps.

    Reading: ``topk`` is the kept fraction of the row's candidates ([topgit] FAQ:
    values in (0, 1], lower is sparser; [gittools] quick-start comment: 0.5 keeps
    the top half), rounded up with a 1e-9 guard against fp noise, at least one when
    there is any candidate, and never more than C.
    """
    if C == 0:
        return 0
    return int(min(C, max(1, math.ceil(topk * C - 1e-9))))


def cdf_keep_count(scores_row: np.ndarray, cand: np.ndarray, tau: float) -> int:
    """How many candidates a row keeps under the threshold (non-top-k) selection.

    The pages name threshold-driven variants of the predictor next to the top-k one
    ([readme] "Avalible API" and [gittools] API list: the ``meansim`` calls without
    ``topk``) and advise calibrating the thresholds per layer and head ([chapterpal]
    recommendations), but give no formula.  Reading: rank the candidates as
    ``select_row`` does (score descending, block index ascending), take the row
    softmax p of the compressed map over the candidates (fp64), and keep the
    shortest prefix of the ranking whose cumulative p, summed in ranking order,
    reaches tau: k = 1 + #{m : p_(0) + ... + p_(m) < tau}, at most C.
    """
    js = np.flatnonzero(cand)
    if js.size == 0:
        return 0
    s = scores_row[js]
    order = np.lexsort((js, -s))
    e = np.exp(s[order] - s.max())
    cum = np.cumsum(e / e.sum())
    return int(min(js.size, 1 + int((cum < tau).sum())))


def select_row(scores: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """The k best candidates by (score descending, block index ascending).

    Top-k of the row softmax equals top-k of the logits (softmax is monotone), so
    the logits are ranked.  Reading: exact ties go to the lower block index.
    """
    js = np.flatnonzero(cand)
    if k == 0 or js.size == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((js, -scores[js]))
    return np.sort(js[order[:k]])


def predict_mask(q: np.ndarray, k: np.ndarray, p: OracleParams) -> Tuple[np.ndarray, Dict]:
    """Stage-1 block mask for one head: (nQ, nK) bool plus intermediate values.

    M[i, j] = valid(i, j) and (Q block i not similar, or K block j not similar, or
    j among the top-k candidates of row i), candidates being the valid, similar K
    blocks of the row; with ``p.cdf`` set, k comes from ``cdf_keep_count``.  Q and K
    enter raw (no smoothing) for every precision option.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, D = q.shape
    scale = p.scale if p.scale is not None else 1.0 / math.sqrt(D)
    qs, qn, qsim = block_stats(q, BQ)
    ks, kn, ksim = block_stats(k, BK)
    qmean = qs / qn[:, None]
    kmean = ks / kn[:, None]
    valid = block_valid(N, p.causal)
    simq = qsim >= p.theta
    simk = ksim >= p.theta
    S = pooled_scores(qmean, kmean, scale)
    nQ, nK = valid.shape
    mask = np.zeros((nQ, nK), dtype=bool)
    kcount = np.zeros(nQ, dtype=np.int64)
    ccount = np.zeros(nQ, dtype=np.int64)
    for i in range(nQ):
        cand = valid[i] & simk
        C = int(cand.sum())
        kk = keep_count(C, p.topk) if p.cdf is None else cdf_keep_count(S[i], cand, p.cdf)
        sel = select_row(S[i], cand, kk)
        row = valid[i] & (~simq[i] | ~simk)
        row[sel] = True
        mask[i] = row
        kcount[i] = kk
        ccount[i] = C
    info = dict(qsim=qsim, ksim=ksim, simq=simq, simk=simk, scores=S, valid=valid,
                kcount=kcount, ccount=ccount, qmean=qmean, kmean=kmean, scale=scale)
    return mask, info


def row_softmax(scores_row: np.ndarray, cand: np.ndarray) -> np.ndarray:
    """Row softmax of the compressed map over the candidates (reporting only)."""
    out = np.zeros_like(scores_row)
    if cand.any():
        s = scores_row[cand]
        e = np.exp(s - s.max())
        out[cand] = e / e.sum()
    return out


def predict_mask_all(q: np.ndarray, k: np.ndarray, p: OracleParams) -> np.ndarray:
    """(B, H, nQ, nK) bool mask for (B, H, N, D) inputs."""
    B, H = q.shape[:2]
    out = None
    for b in range(B):
        for h in range(H):
            m, _ = predict_mask(q[b, h], k[b, h], p)
            if out is None:
                out = np.zeros((B, H) + m.shape, dtype=bool)
            out[b, h] = m
    return out


def kept_lists(mask_bh: np.ndarray) -> List[np.ndarray]:
    """Per block row, the kept K-block indices in ascending order."""
    return [np.flatnonzero(r) for r in mask_bh]


def _block_logits(qg: np.ndarray, t0: int, k: np.ndarray, j: int, causal: bool,
                  scale: float, N: int) -> Tuple[np.ndarray, int, int]:
    s0, s1 = BK * j, min(N, BK * j + BK)
    z = scale * (qg @ k[s0:s1].T)
    if causal:
        t = t0 + np.arange(qg.shape[0])[:, None]
        s = np.arange(s0, s1)[None, :]
        z = np.where(s <= t, z, -np.inf)
    return z, s0, s1


def attend_group(q: np.ndarray, k: np.ndarray, v: np.ndarray, t0: int, t1: int,
                 js: Sequence[int], causal: bool, scale: float,
                 lam: Optional[float]) -> Tuple[np.ndarray, List[int]]:
    """Attention output of query rows [t0, t1) over the kept K blocks ``js``.

    With ``lam`` set, the online softmax-aware filter runs first ([chapterpal]
    method paragraph; [abstract]).  Reading: the rows [t0, t1) are one filter group
    (one wavefront's rows); the kept blocks are visited in ascending order with a
    running row max m (initially -inf).  For block j, m_loc is each row's max over
    its allowed logits in the block and m_new = max(m, m_loc).  The block is
    skipped for the whole group when every row with a finite m_loc has
    m_loc - m_new < lam (or no row has one); a skipped block leaves both the
    numerator and the normaliser of those rows, and m is only advanced by blocks
    that are not skipped.

    Output: softmax-weighted sum of V over the remaining allowed keys, each row
    normalised over its own keys.  Reading: a row with no allowed key outputs 0.
    Returns (O rows in fp64, list of skipped block indices).
    """
    N, D = q.shape
    qg = np.asarray(q[t0:t1], dtype=np.float64)
    G = t1 - t0
    blocks = []
    for j in js:
        z, s0, s1 = _block_logits(qg, t0, k, int(j), causal, scale, N)
        blocks.append((int(j), z, s0, s1))
    skipped: List[int] = []
    if lam is not None:
        m_run = np.full(G, -np.inf)
        kept = []
        for (j, z, s0, s1) in blocks:
            m_loc = z.max(axis=1) if z.shape[1] else np.full(G, -np.inf)
            m_new = np.maximum(m_run, m_loc)
            fin = np.isfinite(m_loc)
            if not fin.any():
                skip = True
            else:
                skip = bool((m_loc[fin] - m_new[fin]).max() < lam)
            if skip:
                skipped.append(j)
            else:
                m_run = m_new
                kept.append((j, z, s0, s1))
        blocks = kept
    if not blocks:
        return np.zeros((G, D)), skipped
    Z = np.concatenate([b[1] for b in blocks], axis=1)
    Vk = np.concatenate([np.asarray(v[b[2]:b[3]], dtype=np.float64) for b in blocks], axis=0)
    m = Z.max(axis=1)
    has = np.isfinite(m)
    msafe = np.where(has, m, 0.0)
    P = np.exp(Z - msafe[:, None])          # exp(-inf) = 0 for disallowed keys
    l = P.sum(axis=1)
    O = P @ Vk
    out = np.zeros((G, D))
    nz = l > 0
    out[nz] = O[nz] / l[nz, None]
    return out, skipped


def attend_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask_bh: np.ndarray,
                causal: bool, scale: Optional[float] = None, lam: Optional[float] = None,
                group: int = 32, return_skips: bool = False):
    """Block-sparse attention for one head under a (nQ, nK) block mask (stage 2)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, D = q.shape
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    out = np.zeros((N, D))
    skips: Dict[Tuple[int, int], List[int]] = {}
    for i, js in enumerate(kept_lists(mask_bh)):
        r0, r1 = BQ * i, min(N, BQ * i + BQ)
        for g0 in range(r0, r1, group):
            g1 = min(r1, g0 + group)
            o, sk = attend_group(q, k, v, g0, g1, js, causal, scale, lam)
            out[g0:g1] = o
            skips[(i, (g0 - r0) // group)] = sk
    return (out, skips) if return_skips else out


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask_bh: np.ndarray,
                groups: Sequence[Tuple[int, int]], causal: bool,
                scale: Optional[float] = None, lam: Optional[float] = None,
                group: int = 32) -> Dict[Tuple[int, int], np.ndarray]:
    """Like ``attend_head`` but only for the listed (block row i, group g) pairs."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    N, D = q.shape
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    res = {}
    for (i, g) in groups:
        js = np.flatnonzero(mask_bh[i])
        g0 = BQ * i + group * g
        g1 = min(N, g0 + group, BQ * i + BQ)
        if g0 >= g1:
            continue
        res[(i, g)], _ = attend_group(q, k, v, g0, g1, js, causal, scale, lam)
    return res


# ---------------------------------------------------------------------------------
# 8-bit Q K^T option (SageAttention base: 8-bit quantization with outlier smoothing,
# [topgit] "Key features"; [readme] "Avalible API").  Readings, all in IEEE float32
# so that both sides take every integer decision in the same precision:
#   * symmetric int8, round half to even, clamp to +-127, one fp32 step
#     delta = max|x| / 127 per quantization block;
#   * Q: one step per 32 query rows (one wavefront's rows);
#   * K: mean smoothing per 64-row K block: k'' = fp32(k) - kbar_j with
#     kbar_j = fp32(sum of the block's rows in fp64 / rows), quantized per block;
#     the smoothing is undone exactly by adding q . kbar_j (unquantized q) to every
#     logit of block j, so the logits are
#         z = scale * (dq * dk_j * (q_code . k''_code) + q . kbar_j).
#     (Per-sequence smoothing, the textbook form, leaves a Q-error x K-drift term
#     that grows along a drifting sequence; per-block smoothing removes it.)
# ---------------------------------------------------------------------------------

Q_QUANT_ROWS = 32


def smooth_k(k32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-sequence K mean smoothing (textbook SageAttention form, used in pins).

    k' = fp32(k) - kmean, kmean = fp32(sum_s k_s / N) with an fp64 sum.
    """
    k32 = np.asarray(k32, dtype=np.float32)
    N = k32.shape[0]
    ksum = k32.astype(np.float64).sum(axis=0)
    kmean = (ksum / np.float64(N)).astype(np.float32)
    return (k32 - kmean).astype(np.float32), kmean


def k_block_means(k32: np.ndarray) -> np.ndarray:
    """kbar_j = fp32(fp64 sum of K block j's rows / its row count), shape (nK, D)."""
    k64 = np.asarray(k32, dtype=np.float32).astype(np.float64)
    N = k64.shape[0]
    nK = (N + BK - 1) // BK
    out = np.zeros((nK, k64.shape[1]), dtype=np.float32)
    for j in range(nK):
        blk = k64[BK * j: min(N, BK * j + BK)]
        out[j] = (blk.sum(axis=0) / np.float64(blk.shape[0])).astype(np.float32)
    return out


def smooth_k_blocks(k32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """(k'' = fp32(k) - kbar_j row by row, kbar) for the int8 option."""
    k32 = np.asarray(k32, dtype=np.float32)
    kbar = k_block_means(k32)
    rows_block = np.arange(k32.shape[0]) // BK
    return (k32 - kbar[rows_block]).astype(np.float32), kbar


def quantize_blocks(x32: np.ndarray, rows: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per block of ``rows`` tokens: int8 codes and the fp32 step delta = max|x|/127.

    code = clamp(rint(x * (127 / max|x|)), -127, 127) in float32; an all-zero block
    has codes 0 and delta 0.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    N, D = x32.shape
    nb = (N + rows - 1) // rows
    codes = np.zeros((N, D), dtype=np.int8)
    deltas = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        xb = x32[b * rows: min(N, (b + 1) * rows)]
        a = np.float32(np.abs(xb).max())
        if a == 0:
            continue
        inv = np.float32(127.0) / a
        c = np.rint((xb * inv).astype(np.float32))
        codes[b * rows: b * rows + xb.shape[0]] = np.clip(c, -127, 127).astype(np.int8)
        deltas[b] = a / np.float32(127.0)
    return codes, deltas


def int8_qk_inputs(q32: np.ndarray, k32: np.ndarray, q_rows: int = Q_QUANT_ROWS):
    """Quantized operands of the int8 Q K^T option for one head.

    Returns (q_codes, q_deltas, k_codes, k_deltas, kbar): Q codes with one step per
    ``q_rows`` rows, block-smoothed K codes with one step per 64-row block, and the
    fp32 K block means that the smoothing removed.
    """
    ks, kbar = smooth_k_blocks(k32)
    qc, qd = quantize_blocks(q32, q_rows)
    kc, kd = quantize_blocks(ks, BK)
    return qc, qd, kc, kd, kbar


def _round_half(x: np.ndarray, kind: Optional[str]) -> np.ndarray:
    """Round fp64 values to fp16 or bfloat16 (RNE) and widen back; None = no rounding."""
    if kind is None:
        return x
    if kind == "fp16":
        return x.astype(np.float16).astype(np.float64)
    import torch  # bfloat16 rounding only; numpy has no bfloat16
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(torch.float64).numpy()


def attend_head_int8_sim(q32, k32, v, mask_bh, causal, q_rows=Q_QUANT_ROWS, scale=None,
                         lam=None, group=32, pv_round: Optional[str] = "fp16"):
    """Diagnostic: stage 2 with the int8 logits and half-precision P and V.

    z = scale * (dq * dk_j * (q_code . k''_code) + q . kbar_j) in fp64 (the integer
    product is exact), softmax in fp64, P and V rounded to ``pv_round`` ("fp16",
    "bf16" or None) for the P.V product, normaliser summed from unrounded P.  Not a
    parity gate: it measures what the quantization spec alone costs against fp64.
    """
    q32 = np.asarray(q32, dtype=np.float32)
    N, D = q32.shape
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    qc, qd, kc, kd, kbar = int8_qk_inputs(q32, k32, q_rows)
    qi = qc.astype(np.int64)
    ki = kc.astype(np.int64)
    q64 = q32.astype(np.float64)
    corr = q64 @ kbar.astype(np.float64).T            # (N, nK): q . kbar_j
    vv = _round_half(np.asarray(v, dtype=np.float64), pv_round)
    out = np.zeros((N, D))
    for i, js in enumerate(kept_lists(mask_bh)):
        r0, r1 = BQ * i, min(N, BQ * i + BQ)
        for g0 in range(r0, r1, group):
            g1 = min(r1, g0 + group)
            t = np.arange(g0, g1)
            dq = qd[t // q_rows].astype(np.float64)
            zs, vs = [], []
            m_run = np.full(g1 - g0, -np.inf)
            for j in js:
                s0, s1 = BK * j, min(N, BK * j + BK)
                z = scale * (dq[:, None] * np.float64(kd[j]) * (qi[g0:g1] @ ki[s0:s1].T).astype(np.float64)
                             + corr[g0:g1, j][:, None])
                if causal:
                    z = np.where(np.arange(s0, s1)[None, :] <= t[:, None], z, -np.inf)
                if lam is not None:
                    m_loc = z.max(axis=1)
                    m_new = np.maximum(m_run, m_loc)
                    fin = np.isfinite(m_loc)
                    if (not fin.any()) or (m_loc[fin] - m_new[fin]).max() < lam:
                        continue
                    m_run = m_new
                zs.append(z)
                vs.append(vv[s0:s1])
            if not zs:
                continue
            Z = np.concatenate(zs, axis=1)
            V = np.concatenate(vs, axis=0)
            m = Z.max(axis=1)
            ok = np.isfinite(m)
            P = np.exp(Z - np.where(ok, m, 0.0)[:, None])
            l = P.sum(axis=1)
            Pr = _round_half(P, pv_round)
            o = Pr @ V
            nz = l > 0
            o[nz] /= l[nz, None]
            o[~nz] = 0
            out[g0:g1] = o
    return out


# ---------------------------------------------------------------------------------
# fp8 P.V option (the SageAttention2 base the pages name runs P.V in 8-bit floating
# point; [readme] "Installation" lists fp8 support; [topgit] "Key features").
# Readings (the pages give no formula):
#   * format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
#     subnormals down to 2^-9, largest finite 448, no infinities); rounding to
#     nearest, ties to even;
#   * V: one fp32 scale per (head, channel) over the whole sequence,
#     s_d = fp32(max_n |v_nd| / 448), and codes e4m3(fp32(v_nd * fp32(448 / max)));
#     a channel that is all zero gets scale 0 and zero codes;
#   * P, online as in flash attention: the kept blocks are visited in ascending
#     order; before block j each row's reference M moves to ceil(running max of
#     z log2(e)) over the blocks so far, the accumulators are rescaled by the
#     (exact) power of two 2^(M_old - M), and the block's numerators are
#     e4m3(2^(z log2(e) - M + 8)): the largest lies in (2^7, 2^8], near the top of
#     the E4M3 range, so long rows keep their small weights (E4M3 spans only 2^-9
#     to 448);
#   * the normaliser is the sum of the ROUNDED numerators, so the weights of a row
#     still sum to one; O = (sum P~ code) * s_d / sum P~, accumulated in fp64.
# ---------------------------------------------------------------------------------

E4M3_MAX = 448.0
LOG2E = 1.0 / math.log(2.0)


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest OCP FP8 E4M3 value of each fp64 x (ties to even), as fp64.

    Normal values have 3 fraction bits, so one unit in the last place is
    2^(e - 3) for x in [2^e, 2^(e+1)); below 2^-6 the spacing stays 2^-9
    (subnormals).  |x| above the largest finite value is outside the format; the
    callers keep |x| <= 448, and this function raises rather than saturate."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e2 = np.frexp(a)                          # a = f * 2^e2, f in [0.5, 1)
    ulp = np.ldexp(1.0, np.maximum(e2 - 4, -9))  # 2^(floor(log2 a) - 3), at least 2^-9
    r = np.rint(a / ulp) * ulp                   # a / ulp < 16: exact; rint is ties-to-even
    if np.any(r > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    return np.copysign(r, x)


def fp8_v_quant(v32: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-channel E4M3 codes of V (as fp64 values) and the fp32 channel scales."""
    v32 = np.asarray(v32, dtype=np.float32)
    vmax = np.abs(v32).max(axis=0)                                     # exact
    with np.errstate(divide="ignore"):
        inv = np.where(vmax > 0, np.float32(E4M3_MAX) / vmax, np.float32(0)).astype(np.float32)
    scale = (vmax / np.float32(E4M3_MAX)).astype(np.float32)
    codes = e4m3_round((v32 * inv[None, :]).astype(np.float32).astype(np.float64))
    return codes, scale


def _pv8_group(z_blocks, c_blocks, sv, G, D):
    """O rows of one filter group from its logit blocks (in visiting order) and their
    E4M3 V code blocks, with the online integer reference of the fp8 reading."""
    O = np.zeros((G, D))
    l = np.zeros(G)
    M = np.full(G, -np.inf)
    for z, C in zip(z_blocks, c_blocks):
        x = z * LOG2E
        mloc = x.max(axis=1)
        M_new = np.where(np.isfinite(mloc), np.maximum(M, np.ceil(mloc)), M)
        f = np.where(np.isfinite(M), np.exp2(np.where(np.isfinite(M), M - M_new, 0.0)), 1.0)
        O *= f[:, None]
        l *= f
        M = M_new
        ok = np.isfinite(M)
        P = e4m3_round(np.exp2(x - np.where(ok, M, 0.0)[:, None] + 8.0) * ok[:, None])
        O += P @ C
        l += P.sum(axis=1)
    out = np.zeros((G, D))
    nz = l > 0
    out[nz] = O[nz] * sv.astype(np.float64)[None, :] / l[nz, None]
    return out


def attend_rows_pv8(q, k, v, mask_bh, groups, causal, scale=None, lam=None, group=32,
                    qk: str = "exact", q_rows=Q_QUANT_ROWS) -> Dict[Tuple[int, int], np.ndarray]:
    """Stage 2 with the fp8 P.V for the listed (block row i, group g) pairs.

    V: per-channel E4M3 codes over the whole head (``fp8_v_quant``).  Logits: the
    exact fp64 ones (qk="exact") or the int8 ones of ``attend_head_int8_sim``
    (qk="int8").  The filter, when ``lam`` is set, runs on those logits as in
    ``attend_group``.  The remaining blocks then enter ``_pv8_group`` in visiting
    order (online integer reference, numerators at 2^8 scale, rounded to E4M3).
    Returns O rows in fp64."""
    q32 = np.asarray(q, dtype=np.float32)
    k32 = np.asarray(k, dtype=np.float32)
    N, D = q32.shape
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    codes, sv = fp8_v_quant(v)
    q64, k64 = q32.astype(np.float64), k32.astype(np.float64)
    if qk == "int8":
        qc, qd, kc, kd, kbar = int8_qk_inputs(q32, k32, q_rows)
        qi, ki = qc.astype(np.int64), kc.astype(np.int64)
        kbar64 = kbar.astype(np.float64)
    res = {}
    for (i, g) in groups:
        g0 = BQ * i + group * g
        g1 = min(N, g0 + group, BQ * i + BQ)
        if g0 >= g1:
            continue
        t = np.arange(g0, g1)
        zs, cs = [], []
        m_run = np.full(g1 - g0, -np.inf)
        for j in np.flatnonzero(mask_bh[i]):
            s0, s1 = BK * j, min(N, BK * j + BK)
            if qk == "int8":
                dq = qd[t // q_rows].astype(np.float64)
                z = scale * (dq[:, None] * np.float64(kd[j]) * (qi[g0:g1] @ ki[s0:s1].T).astype(np.float64)
                             + (q64[g0:g1] @ kbar64[j])[:, None])
            else:
                z = scale * (q64[g0:g1] @ k64[s0:s1].T)
            if causal:
                z = np.where(np.arange(s0, s1)[None, :] <= t[:, None], z, -np.inf)
            if lam is not None:
                m_loc = z.max(axis=1)
                m_new = np.maximum(m_run, m_loc)
                fin = np.isfinite(m_loc)
                if (not fin.any()) or (m_loc[fin] - m_new[fin]).max() < lam:
                    continue
                m_run = m_new
            zs.append(z)
            cs.append(codes[s0:s1])
        res[(i, g)] = _pv8_group(zs, cs, sv, g1 - g0, D)
    return res


def attend_head_pv8_sim(q, k, v, mask_bh, causal, scale=None, lam=None, group=32,
                        qk: str = "exact", q_rows=Q_QUANT_ROWS):
    """``attend_rows_pv8`` over every row group of one head, as an (N, D) array."""
    N = np.asarray(q).shape[0]
    nQ = mask_bh.shape[0]
    groups = [(i, g) for i in range(nQ) for g in range((BQ + group - 1) // group)]
    res = attend_rows_pv8(q, k, v, mask_bh, groups, causal, scale, lam, group, qk, q_rows)
    out = np.zeros((N, np.asarray(q).shape[1]))
    for (i, g), o in res.items():
        g0 = BQ * i + group * g
        out[g0:g0 + o.shape[0]] = o
    return out
