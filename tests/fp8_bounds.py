"""Elementwise error bounds for the tests' output comparisons (test helper, no GPU).

fp8 (E4M3) P.V.  The fp8 reading rounds every softmax numerator P and every scaled
value v / s_c to E4M3 and normalises by the sum of the rounded numerators.  Against
exact attention on the same logits, its output moves by at most, per (row t,
channel c), to first order in the rounding errors,

    B_tc = [ sum_s e(P_ts) |v_sc - O_tc|  +  sum_s (P_ts + e(P_ts)) u_sc ]
           / (sum_s P_ts - sum_s e(P_ts))

where P_ts = 2^(z_ts log2 e - M_t + 8) with M_t the ceiling of the row's largest
z log2 e (the reference the reading ends with: numerators rounded earlier against
a smaller reference carry an error no larger, once rescaled), u_sc = s_c e(|v_sc| / s_c)
with s_c = max_s |v_sc| / 448, and e(y) the largest distance from y in [0, 448] to its
nearest E4M3 value: 2^-4 y where E4M3 is normal (y >= 2^-6, 3 fraction bits), 2^-10
in the subnormal range (spacing 2^-9), and y itself below 2^-10 (y rounds to 0).
The first term is the change of the weights (numerator and normaliser move
together: sum_s (P~_s - P_s)(v_s - O) / sum P~), the second the change of the values.
A further 1e-4 P_ts per numerator covers logits that differ from the reference's by
up to 1e-4 log2 units (the int8 path's q . kbar term, fp32 arithmetic), the output's
rounding to its storage type adds half an ulp, and 1e-4 + 1e-5 |O| covers fp32
accumulation.

16-bit outputs.  Storing an fp32 result in bfloat16 (fp16) moves it by at most half
an ulp: 2^-8 |x| (2^-11 |x|) for normal x.
"""
from __future__ import annotations

import math

import numpy as np

LOG2E = 1.0 / math.log(2.0)
E4M3_MAX = 448.0


def e4m3_half_step(y):
    """Largest |e4m3(y) - y| for y in [0, 448], elementwise."""
    y = np.asarray(y, dtype=np.float64)
    return np.maximum(2.0 ** -4 * y, np.minimum(y, 2.0 ** -10))


def half_ulp(x, dtype: str):
    """Half an ulp of the 16-bit storage type at |x| (normal range; 0 for x = 0)."""
    frac = {"bf16": 8, "fp16": 11, "fp32": 24}[dtype]
    a = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - frac), 0.0)


def group_logits(q, k, js, t0, t1, causal, scale, lam=None, int8=None):
    """(G, N) fp64 logits of query rows [t0, t1) over every key; -inf where a key is
    not attended: outside the kept blocks ``js``, in the causal future, or in a block
    that the online filter drops for this row group (kept blocks in ascending order,
    a running row max m; block j is dropped when every row with a visible key has
    max_block(z) - max(m, max_block(z)) < lam, or no row has one; m advances only on
    kept blocks).  ``int8`` = (q_codes, q_steps, k_codes, k_steps, kbar) gives the int8
    option's logits scale (dq dk (q_code . k_code) + q . kbar_j) instead of scale q . k."""
    N = q.shape[0]
    G = t1 - t0
    Z = np.full((G, N), -np.inf)
    rows = np.arange(t0, t1)
    m = np.full(G, -np.inf)
    for j in sorted(int(x) for x in js):
        s0, s1 = 64 * j, min(N, 64 * j + 64)
        if int8 is None:
            z = scale * (q[t0:t1] @ k[s0:s1].T)
        else:
            qc, qd, kc, kd, kbar = int8
            dq = qd[rows // 32].astype(np.float64)
            z = scale * (dq[:, None] * np.float64(kd[j]) *
                         (qc[t0:t1].astype(np.int64) @ kc[s0:s1].astype(np.int64).T).astype(np.float64)
                         + (q[t0:t1] @ kbar[j].astype(np.float64))[:, None])
        if causal:
            z = np.where(np.arange(s0, s1)[None, :] <= rows[:, None], z, -np.inf)
        if lam is not None:
            mloc = z.max(axis=1)
            mnew = np.maximum(m, mloc)
            fin = np.isfinite(mloc)
            if not fin.any() or (mloc[fin] - mnew[fin]).max() < lam:
                continue
            m = mnew
        Z[:, s0:s1] = z
    return Z


def exact_attention(Z, V):
    """O = softmax(Z) V in fp64 (rows with no finite logit give 0)."""
    mx = Z.max(axis=1)
    ok = np.isfinite(mx)
    P = np.exp(Z - np.where(ok, mx, 0.0)[:, None])
    l = P.sum(axis=1)
    O = np.zeros((Z.shape[0], V.shape[1]))
    O[ok] = (P[ok] @ V) / l[ok, None]
    return O


def fp8_bound(Z, V, vmax, out_dtype="bf16", logit_slack=1e-4):
    """(O, B): exact attention O on logits Z (G, N) and values V (N, D), and the
    elementwise bound B on |O_fp8 - O| of the fp8 P.V reading; vmax (D,) is the
    per-channel max |v| over the whole head (it fixes the channel scales)."""
    G, D = Z.shape[0], V.shape[1]
    O = exact_attention(Z, V)
    B = np.zeros((G, D))
    keys = np.flatnonzero(np.isfinite(Z).any(axis=0))
    if keys.size == 0:
        return O, B
    x = Z[:, keys] * LOG2E
    Vk = V[keys]
    top = x.max(axis=1)
    ok = np.isfinite(top)
    M = np.ceil(np.where(ok, top, 0.0))
    P = np.where(np.isfinite(x), np.exp2(x - M[:, None] + 8.0), 0.0)
    P[~ok] = 0.0
    e = e4m3_half_step(P) + logit_slack * P
    den = P.sum(axis=1) - e.sum(axis=1)
    sc = np.asarray(vmax, dtype=np.float64) / E4M3_MAX
    with np.errstate(divide="ignore", invalid="ignore"):
        u = np.where(sc > 0, sc * e4m3_half_step(np.abs(Vk) / np.where(sc > 0, sc, 1.0)), 0.0)
    for t in np.flatnonzero(ok):
        bp = e[t] @ np.abs(Vk - O[t])
        bv = (P[t] + e[t]) @ u
        B[t] = (bp + bv) / den[t]
    B += half_ulp(np.abs(O) + B, out_dtype) + 1e-4 + 1e-5 * np.abs(O)
    return O, B


def qkbar_two_level(q32, kbar, rows=32):
    """q . kbar_j as the int8 Q.K^T path forms it, (N, nK): q ~= dq (q8 + r8 / 256)
    with one step dq = max|q| / 127 per ``rows``-row group, kbar ~= sk (c1 + c2 / 256)
    with one step sk = max|kbar| / 127 per head (codes: round half to even, clamp to
    +-127, in fp32), and the product dq sk (q8 . c1 + (q8 . c2 + r8 . c1) / 256), the
    r8 . c2 term left out.  Used to size the logit slack of the int8 comparisons."""
    q32 = np.asarray(q32, dtype=np.float32)
    kb = np.asarray(kbar, dtype=np.float32)

    def two_level(x, amax):
        amax = np.float32(amax)
        if amax == 0:
            z = np.zeros(x.shape)
            return z, z
        y = (x * (np.float32(127.0) / amax)).astype(np.float32)
        c1 = np.clip(np.rint(y), -127, 127).astype(np.float32)
        c2 = np.clip(np.rint(((y - c1).astype(np.float32) * np.float32(256.0)).astype(np.float32)), -127, 127)
        return c1.astype(np.float64), c2.astype(np.float64)

    N = q32.shape[0]
    c1, c2 = two_level(kb, np.abs(kb).max())
    sk = np.float64(np.float32(np.abs(kb).max()) / np.float32(127.0))
    out = np.zeros((N, kb.shape[0]))
    for g0 in range(0, N, rows):
        blk = q32[g0:g0 + rows]
        a = np.abs(blk).max()
        q8, r8 = two_level(blk, a)
        dq = np.float64(np.float32(a) / np.float32(127.0))
        out[g0:g0 + rows] = dq * sk * (q8 @ c1.T + (q8 @ c2.T + r8 @ c1.T) / 256.0)
    return out


def int8_logit_slack(q32, kbar, scale, rows=32):
    """Largest |q . kbar_j - its two-level form| over all (row, block), in log2 units
    of the scaled logits, as a relative change of each P (exp2 of it minus one)."""
    exact = np.asarray(q32, dtype=np.float32).astype(np.float64) @ np.asarray(kbar, np.float32).astype(np.float64).T
    d = scale * LOG2E * np.abs(exact - qkbar_two_level(q32, kbar, rows)).max()
    return float(np.exp2(d) - 1.0)
