#!/usr/bin/env python3
"""One-GPU benchmark of the SpargeAttn hot path on MI355X; prints ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-extras]

A step is one pass of the whole path over one batch of synthetic input that is
already resident in HBM:
  llm128k (default; B=1 H=32 N=131072 D=128, causal, topk=0.5): stage-1 predictor
      (block stats, pooled scores, top-k select), block-smoothed int8 K
      quantization, stage-2 sparse attention (int8 Q K^T, fp16 P.V, filter on);
  llm8k: the same recipe at N=8192 with 16-bit Q K^T and P.V;
  video: Hilbert gather of Q/K/V, the same path (topk=0.3, non-causal, D=64),
      scatter of O back to token order;
  image: block_sparse_attn under a seeded Bernoulli(0.3) block mask.
`value` is dense-equivalent TOPS of the whole step: 4*B*H*N^2*D (halved when
causal) per step / step time.  `roofline` covers the attention kernel alone,
timed with HIP events recorded around its launch on the stream it runs on.
"""

from __future__ import annotations

import argparse
import ctypes
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dense-equiv TOPS & latency of sparse attn at N=8K..128K, topk=0.5; MFMA util"
PEAK_BF16 = 2.5e15      # dense bf16/fp16 MFMA, FLOP/s (MI355X published)
PEAK_INT8 = 5.0e15      # dense int8 MFMA, OP/s
PEAK_FP8 = 5.0e15       # dense fp8 (E4M3) MFMA, MI355X published
BK, BQ, G = 64, 128, 32


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles from the HIP runtime instance torch and libsparge share."""

    def __init__(self):
        import torch  # noqa: F401  (loads the runtime)
        maps = open("/proc/self/maps").read()
        paths = sorted(set(re.findall(r"(\S*libamdhip64\.so\S*)", maps)))
        self.hip = ctypes.CDLL(paths[0] if paths else "libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        self.hip.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)


def dense_equiv_ops(B, H, N, D, causal):
    ops = 4.0 * B * H * N * N * D
    return ops / 2 if causal else ops


class Path:
    """The hot path of one workload with preallocated outputs and workspace."""

    def __init__(self, wl, dev, qk_int8=None, pv_fp16=None, inputs=None, pv_fp8=None, cdf=None,
                 filter_lambda=-10.0):
        import torch

        import block_sparse_quantized_amd as bsq
        from block_sparse_quantized_amd import synth
        self.bsq, self.wl, self.dev = bsq, wl, dev
        self.qk_int8 = wl.qk_int8 if qk_int8 is None else qk_int8
        self.pv_fp16 = wl.pv_fp16 if pv_fp16 is None else pv_fp16
        self.pv_fp8 = wl.pv_fp8 if pv_fp8 is None else pv_fp8
        self.cdf = cdf   # softmax-mass threshold of the threshold selection, or None (top-k)
        self.lam = filter_lambda
        t0 = time.time()
        if inputs is None:
            self.q, self.k, self.v = synth.make_qkv(wl, device=dev)
            self.mask = synth.make_block_mask(wl, device=dev) if wl.api == "block_sparse" else None
            torch.cuda.synchronize()
            log(f"[bench] generated {wl.name} inputs on {dev} in {time.time() - t0:.1f}s")
        else:
            self.q, self.k, self.v, self.mask = inputs
        self.out = torch.empty_like(self.q)
        self.ws = torch.empty(bsq.sparge_workspace_bytes(*self.q.shape, self.q.dtype),
                              dtype=torch.uint8, device=dev)
        if wl.hilbert:
            self.cells = 1
            for s in wl.grid:
                self.cells *= s
            self.perm = bsq.sparge_hilbert_perm3d(*wl.grid).to(dev)
            self.qr, self.kr, self.vr, self.orr = (torch.empty_like(self.q) for _ in range(4))

    def step(self, prof=None, stats=False):
        bsq, wl = self.bsq, self.wl
        q, k, v, out = self.q, self.k, self.v, self.out
        if wl.hilbert:
            bsq.sparge_reorder(q, self.perm, wl.text, self.cells, out=self.qr)
            bsq.sparge_reorder(k, self.perm, wl.text, self.cells, out=self.kr)
            bsq.sparge_reorder(v, self.perm, wl.text, self.cells, out=self.vr)
            q, k, v, out = self.qr, self.kr, self.vr, self.orr
        if wl.api == "block_sparse":
            r = bsq.block_sparse_attn(q, k, v, self.mask, filter_on=wl.filter_on,
                                      filter_lambda=self.lam, qk_int8=self.qk_int8, pv_fp16=self.pv_fp16,
                                      pv_fp8=self.pv_fp8, stats=stats, out=out, workspace=self.ws,
                                      prof=prof)
        elif self.cdf is not None:
            r = bsq.sparge_cdf_attn(q, k, v, self.cdf, wl.causal, filter_on=wl.filter_on,
                                    filter_lambda=self.lam, qk_int8=self.qk_int8, pv_fp16=self.pv_fp16,
                                    pv_fp8=self.pv_fp8, stats=stats, out=out, workspace=self.ws,
                                    prof=prof)
        else:
            r = bsq.sparge_topk_attn(q, k, v, wl.topk, wl.causal, filter_on=wl.filter_on,
                                     filter_lambda=self.lam, qk_int8=self.qk_int8, pv_fp16=self.pv_fp16,
                                     pv_fp8=self.pv_fp8, stats=stats, out=out, workspace=self.ws,
                                     prof=prof)
        if wl.hilbert:
            bsq.sparge_reorder(self.orr, self.perm, wl.text, self.cells, inverse=True, out=self.out)
        return r


def graph_replay(path, steps):
    """The same step captured once in a HIP graph (the library allocates nothing and
    does not synchronise without stats) and replayed: per-step time without the
    host-side launch gaps, or None when capture is unavailable."""
    import torch
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            path.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            path.step()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    except Exception as e:  # capture not supported by this runtime / build
        log(f"[bench] graph replay unavailable: {e}")
        return None


def time_path(path, ev, steps, warmup):
    """Whole-step wall time (synchronised) and per-launch attention-kernel time."""
    import torch
    for _ in range(warmup):
        path.step()
    torch.cuda.synchronize()
    evs = [(ev.create(), ev.create(), ev.create()) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        path.step(prof=evs[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    attn = [ev.elapsed_ms(e[1], e[2]) for e in evs]
    pre = [ev.elapsed_ms(e[0], e[1]) for e in evs]
    return (t1 - t0) * 1e3 / steps, sum(attn) / steps, sum(pre) / steps


def algorithmic_work(stats, D, qk_int8):
    """(QK ops, PV flops) the attention kernel executes per launch on computed tiles.

    Per visited (32-row group, kept 64-key block): Q K^T 2*32*64*D; P.V 2*32*64*D
    unless the filter dropped the update."""
    per = 2.0 * G * BK * D
    qk = stats["group_updates"] * per
    pv = (stats["group_updates"] - stats["skipped_updates"]) * per
    return qk, pv


def roofline(stats, D, qk_int8, attn_ms, traffic, pv_fp8=False):
    qk, pv = algorithmic_work(stats, D, qk_int8)
    t = attn_ms * 1e-3
    # mixed roofline: Q K^T at the peak of its type (int8 or bf16) plus P.V at the
    # peak of its type (fp8, or bf16/fp16); the effective peak is the work over that
    # minimum time
    qk_peak = PEAK_INT8 if qk_int8 else PEAK_BF16
    pv_peak = PEAK_FP8 if pv_fp8 else PEAK_BF16
    peak = (qk + pv) / (qk / qk_peak + pv / pv_peak)
    achieved = (qk + pv) / t
    return {"bound": "mfma", "achieved": round(achieved / 1e12, 2), "peak": round(peak / 1e12, 1),
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": traffic,
            "frac_of_bf16_peak": round(achieved / PEAK_BF16, 4),
            "kernel": "sparse_attn_kernel", "ms_per_launch": round(attn_ms, 4),
            "work_per_launch": {"qk_ops": qk, "pv_flops": pv}}


def path_dtype(qk_int8, pv_fp16, pv_fp8):
    """Arithmetic types of the Q.K^T and P.V products, as reported in the JSON line."""
    pv = "fp8-pv" if pv_fp8 else ("f16-pv" if pv_fp16 else None)
    if qk_int8:
        return f"i8-qk/{pv or 'bf16-pv'}"
    return f"{pv}/bf16-qk" if pv else "bf16"


def committed_traffic(wl_name, kernel_src, dtype):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary of this
    workload and path (profiles/sparse_attn_<workload>*_traffic.json), if it was
    taken on the current kernel source; else None."""
    try:
        sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
        for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"sparse_attn_{wl_name}*_traffic.json"))):
            rec = json.load(open(path))
            if rec.get("path") == dtype and rec.get("kernel_source_sha256") == sha:
                return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None
    return None


# ---- CPU baseline: the oracle in a pool of worker processes -------------------------
# The workers are forked at start-up, before this process touches the GPU, and hold no
# GPU state.  Each draws head (0, 0) of the workload on the CPU (the seeded generator's
# CPU stream: the same recipe and shapes as the GPU draw), predicts its block mask with
# the oracle once, and then computes the oracle's stage-2 output for the block rows it
# is handed, one at a time, with BLAS held to one thread.

_W = {}


def _cpu_worker_init(name):
    # one BLAS thread per worker: through the environment for a BLAS library loaded
    # after this point, and through threadpoolctl for one already loaded
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    import torch
    torch.set_num_threads(1)
    from block_sparse_quantized_amd import synth
    from oracle import sparge_oracle as so
    wl = synth.workload(name, B=1, H=1)
    q, k, v = (t[0, 0].double().numpy() for t in synth.make_qkv(wl, device="cpu"))
    if wl.api == "block_sparse":
        mask = synth.make_block_mask(wl, device="cpu")[0, 0].numpy().astype(bool)
    else:
        mask, _ = so.predict_mask(q, k, so.OracleParams(topk=wl.topk, causal=wl.causal))
    _W.update(wl=wl, q=q, k=k, v=v, mask=mask)


def _cpu_worker_rows(i):
    """The oracle's output for block row i of head (0, 0): (dense-equivalent ops, rows)."""
    from oracle import sparge_oracle as so
    wl, q, k, v, mask = _W["wl"], _W["q"], _W["k"], _W["v"], _W["mask"]
    N, D = q.shape
    lam = -10.0 if wl.filter_on else None
    groups = [(i, g) for g in range(4) if BQ * i + G * g < N]
    so.attend_rows(q, k, v, mask, groups, wl.causal, lam=lam)
    ops, rows = 0.0, 0
    for (_, g) in groups:
        r0 = BQ * i + G * g
        r1 = min(N, r0 + G, BQ * i + BQ)
        keys = (sum(range(r0 + 1, r1 + 1))) if wl.causal else (r1 - r0) * N
        ops += 4.0 * D * keys
        rows += r1 - r0
    return ops, rows


def cpu_pool(name, workers=None):
    """The forked worker pool (call before any GPU work)."""
    import multiprocessing
    n = workers or min(16, len(os.sched_getaffinity(0)))
    return multiprocessing.get_context("fork").Pool(n, initializer=_cpu_worker_init, initargs=(name,)), n


def cpu_baseline(wl, pool, nworkers, budget_s=20.0):
    """The CPU oracle (fp64 numpy) on a bounded sample of the workload: block rows of
    head (0, 0), spread over the sequence (longest first), one per worker at a time,
    handed out until the budget is spent."""
    import multiprocessing  # noqa: F401
    nQ = (wl.N + BQ - 1) // BQ
    order = []
    for stride in (max(1, nQ // 8), max(1, nQ // 64), 1):
        order += [i for i in range(nQ - 1, -1, -stride) if i not in order]
    # every worker has drawn its inputs and predicted its mask (its initializer, run
    # at start-up while the GPU part ran) before the clock starts
    warm = [pool.apply_async(os.getpid) for _ in range(4 * nworkers)]
    [w.get() for w in warm]
    t0 = time.perf_counter()
    c0 = time.process_time()
    pending, nxt, ops, rows, done_rows = [], 0, 0.0, 0, []
    while nxt < len(order) and len(pending) < nworkers:
        pending.append((order[nxt], pool.apply_async(_cpu_worker_rows, (order[nxt],))))
        nxt += 1
    while pending:
        i, r = pending.pop(0)
        o, n = r.get()
        ops += o
        rows += n
        done_rows.append(i)
        if nxt < len(order) and time.perf_counter() - t0 < budget_s:
            pending.append((order[nxt], pool.apply_async(_cpu_worker_rows, (order[nxt],))))
            nxt += 1
    t = time.perf_counter() - t0
    pool.close()
    pool.join()
    return {"value": round(ops / t / 1e12, 8), "unit": "TOPS (dense-equivalent)",
            "cores": nworkers, "kind": "oracle",
            "sample": (f"head (0,0) of {wl.name} drawn on the CPU: stage-2 fp64 oracle attention"
                       f"{' with the filter' if wl.filter_on else ''} of {len(done_rows)} block rows "
                       f"({rows} query rows, spread over the sequence, longest first) in {t:.2f}s, in "
                       f"{nworkers} worker processes (one BLAS thread each, each having drawn the "
                       f"head and predicted its mask with the oracle before the clock started); "
                       f"value = dense-equivalent ops of those rows / wall time"),
            "host": host_info()}


def host_info():
    """CPU model, usable cores, numpy and its BLAS."""
    import numpy as np
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{d.get('internal_api')} {d.get('version')}" for d in threadpool_info()
                if d.get("user_api") == "blas"]
        blas = ", ".join(sorted(set(libs))) or blas
    except Exception:
        pass
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas}


def sdpa_baseline(q, k, v, causal, steps=3):
    """torch SDPA in bf16 at the same shape, each fused backend on its own (flash, then
    memory-efficient); returns {backend: ms per call} for those that run."""
    import torch
    import torch.nn.functional as F
    res = {}
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
    except Exception as e:
        log(f"[bench] torch SDPA backends unavailable: {e}")
        return res
    qb, kb, vb = (t.to(torch.bfloat16) for t in (q, k, v))
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                F.scaled_dot_product_attention(qb, kb, vb, is_causal=causal)
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(steps):
                    F.scaled_dot_product_attention(qb, kb, vb, is_causal=causal)
                torch.cuda.synchronize()
            res[name] = (time.perf_counter() - t0) * 1e3 / steps
        except Exception as e:  # this backend does not take the shape
            log(f"[bench] torch SDPA {name} backend unavailable: {e}")
    return res


SWEEP_N = (8192, 16384, 32768, 65536, 131072)


def sweep(wl, dev, ev, main_path, steps=3):
    """Dense-equivalent TOPS and latency over N = 8K..128K (the LLM generator, causal,
    topk 0.5, filter on), for the int8 Q.K^T path with fp16 or fp8 P.V and the bf16
    path."""
    from block_sparse_quantized_amd import synth
    out = []
    for n in SWEEP_N:
        wn = synth.workload("llm8k", N=n)
        inputs = None
        if n == main_path.wl.N and wl.B == main_path.wl.B and wl.H == main_path.wl.H:
            inputs = (main_path.q, main_path.k, main_path.v, main_path.mask)
        for qk8, pv16, pv8 in ((True, True, False), (True, False, True), (False, False, False)):
            pth = Path(wn, dev, qk_int8=qk8, pv_fp16=pv16, inputs=inputs, pv_fp8=pv8)
            inputs = (pth.q, pth.k, pth.v, pth.mask)
            _, st = pth.step(stats=True)
            s_ms, a_ms, _ = time_path(pth, ev, steps, 1)
            dense = dense_equiv_ops(wn.B, wn.H, n, wn.D, wn.causal)
            rf = roofline(st, wn.D, qk8, a_ms, None, pv8)
            out.append({"N": n, "path": path_dtype(qk8, pv16, pv8),
                        "ms_per_step": round(s_ms, 4), "attention_ms": round(a_ms, 4),
                        "tops_dense_equiv": round(dense / (s_ms * 1e-3) / 1e12, 2),
                        "attention_frac": rf["frac"], "attention_frac_of_bf16_peak": rf["frac_of_bf16_peak"],
                        "kept_block_density": round(st["kept_blocks"] / max(1, st["valid_blocks"]), 4)})
            log(f"[bench] sweep N={n} {out[-1]['path']}: {out[-1]['tops_dense_equiv']} TOPS, "
                f"{s_ms:.3f} ms/step")
            del pth
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llm128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--pv-fp8", action="store_true",
                    help="time the int8 Q.K^T / fp8 P.V path of the workload instead of its own")
    ap.add_argument("--bf16", action="store_true",
                    help="time the 16-bit path (bf16 Q.K^T and P.V) of the workload instead of its own")
    ap.add_argument("--cdf", type=float, default=None, metavar="TAU",
                    help="time the threshold selection (softmax mass TAU) instead of top-k")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the path shards over (batch, head) with no "
              f"communication, and this benchmark does not run several GPUs; got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    from block_sparse_quantized_amd import synth
    wl = synth.WORKLOADS[args.workload]
    pool = None
    if not args.no_cpu_baseline:
        pool, nworkers = cpu_pool(wl.name)   # forked before anything touches the GPU

    import torch

    dev = torch.device("cuda:0")
    ev = HipEvents()
    log(f"[bench] workload {wl.name}: B={wl.B} H={wl.H} N={wl.N} D={wl.D} steps={args.steps} "
        f"warmup={args.warmup}")

    if args.pv_fp8:
        path = Path(wl, dev, qk_int8=True, pv_fp16=False, pv_fp8=True, cdf=args.cdf)
    elif args.bf16:
        path = Path(wl, dev, qk_int8=False, pv_fp16=False, pv_fp8=False, cdf=args.cdf)
    else:
        path = Path(wl, dev, cdf=args.cdf)
    _, stats = path.step(stats=True)
    torch.cuda.synchronize()
    ms_step, ms_attn, ms_pre = time_path(path, ev, args.steps, args.warmup)
    log(f"[bench] step {ms_step:.3f} ms, attention kernel {ms_attn:.3f} ms, before-attention {ms_pre:.3f} ms")
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    dense = dense_equiv_ops(B, H, N, D, wl.causal)
    value = dense / (ms_step * 1e-3) / 1e12
    kernel_src = os.path.join(ROOT, "block_sparse_quantized_amd", "csrc", "attn.hip")
    roof = roofline(stats, D, path.qk_int8, ms_attn,
                    committed_traffic(wl.name, kernel_src, path_dtype(path.qk_int8, path.pv_fp16,
                                                                      path.pv_fp8)),
                    path.pv_fp8)

    extras = {}
    if not args.no_extras:
        gr = graph_replay(path, args.steps)
        if gr is not None:
            extras["graph_replay"] = {"ms_per_step": round(gr, 4),
                                      "tops_dense_equiv": round(dense / (gr * 1e-3) / 1e12, 2)}
        if path.qk_int8 or path.pv_fp16:
            p16 = Path(wl, dev, qk_int8=False, pv_fp16=False,
                       inputs=(path.q, path.k, path.v, path.mask))
            _, st16 = p16.step(stats=True)
            s16, a16, _ = time_path(p16, ev, max(3, args.steps // 2), 1)
            extras["bf16_variant"] = {"ms_per_step": round(s16, 3),
                                      "tops_dense_equiv": round(dense / (s16 * 1e-3) / 1e12, 2),
                                      "roofline": roofline(st16, D, False, a16,
                                                           committed_traffic(wl.name, kernel_src, "bf16"))}
            del p16
        if wl.dtype != torch.float32 and not path.pv_fp8:   # fp8 P.V takes 16-bit inputs
            p8 = Path(wl, dev, qk_int8=True, pv_fp16=False, pv_fp8=True,
                      inputs=(path.q, path.k, path.v, path.mask))
            _, st8 = p8.step(stats=True)
            s8, a8, _ = time_path(p8, ev, max(3, args.steps // 2), 1)
            extras["i8qk_fp8pv_variant"] = {
                "ms_per_step": round(s8, 3), "tops_dense_equiv": round(dense / (s8 * 1e-3) / 1e12, 2),
                "roofline": roofline(st8, D, True, a8,
                                     committed_traffic(wl.name, kernel_src, "i8-qk/fp8-pv"), True)}
            del p8
        if wl.api != "block_sparse":
            # the threshold selection (softmax mass 0.95) on the same inputs and path
            pc = Path(wl, dev, inputs=(path.q, path.k, path.v, path.mask), cdf=0.95)
            _, stc = pc.step(stats=True)
            sc, ac, prc = time_path(pc, ev, max(3, args.steps // 2), 1)
            extras["cdf_select_variant"] = {
                "cdf_threshold": 0.95, "ms_per_step": round(sc, 3),
                "before_attention_ms": round(prc, 4), "attention_ms": round(ac, 4),
                "tops_dense_equiv": round(dense / (sc * 1e-3) / 1e12, 2),
                "kept_block_density": round(stc["kept_blocks"] / max(1, stc["valid_blocks"]), 4)}
            del pc
        if wl.filter_on:
            # what the softmax-aware filter buys on these inputs: the same step with the
            # filter off and with looser thresholds (lambda in natural-log logit units)
            fe = []
            for lam in (None, -10.0, -6.0, -3.0):
                wf = synth.workload(wl.name, filter_on=lam is not None)
                pf = Path(wf, dev, qk_int8=path.qk_int8, pv_fp16=path.pv_fp16, pv_fp8=path.pv_fp8,
                          inputs=(path.q, path.k, path.v, path.mask),
                          filter_lambda=-10.0 if lam is None else lam)
                _, stf = pf.step(stats=True)
                sf, af, _ = time_path(pf, ev, max(3, args.steps // 2), 1)
                fe.append({"filter_lambda": lam, "ms_per_step": round(sf, 4), "attention_ms": round(af, 4),
                           "skipped_update_frac": round(stf["skipped_updates"] / max(1, stf["group_updates"]), 5)})
                log(f"[bench] filter lambda={lam}: {sf:.3f} ms/step, skipped {fe[-1]['skipped_update_frac']}")
                del pf
            extras["filter_effect"] = fe
        if wl.api != "block_sparse" and not wl.hilbert:
            pd = Path(synth.workload(wl.name, topk=1.0, filter_on=False), dev, qk_int8=False,
                      pv_fp16=False, inputs=(path.q, path.k, path.v, path.mask))
            sd, _, _ = time_path(pd, ev, 3, 1)
            extras["dense_ours_bf16"] = {"ms_per_step": round(sd, 3),
                                         "tops_dense_equiv": round(dense / (sd * 1e-3) / 1e12, 2)}
            del pd
        if wl.name in ("llm8k", "llm128k"):
            extras["sweep"] = sweep(wl, dev, ev, path)
        sd = sdpa_baseline(path.q, path.k, path.v, wl.causal)
        if sd:
            best = min(sd, key=sd.get)
            extras["dense_torch_sdpa_bf16"] = {
                "backend": best, "ms_per_step": round(sd[best], 3),
                "tops_dense_equiv": round(dense / (sd[best] * 1e-3) / 1e12, 2),
                "per_backend_ms": {b: round(t, 3) for b, t in sd.items()},
                "torch": torch.__version__}
    cpu = None
    if not args.no_cpu_baseline:
        t0 = time.time()
        cpu = cpu_baseline(wl, pool, nworkers)
        log(f"[bench] cpu baseline took {time.time() - t0:.1f}s")

    density = stats["kept_blocks"] / max(1, stats["valid_blocks"])
    dtype = path_dtype(path.qk_int8, path.pv_fp16, path.pv_fp8)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS (dense-equivalent)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded torch generators on the GPU; see block_sparse_quantized_amd/synth.py)",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "D": D, "causal": wl.causal,
                   "topk": wl.topk if wl.api != "block_sparse" else None, "api": wl.api,
                   "filter_on": wl.filter_on, "qk_int8": path.qk_int8, "pv_fp16": path.pv_fp16,
                   "pv_fp8": path.pv_fp8, "cdf_threshold": path.cdf,
                   "hilbert": wl.hilbert},
        "roofline": roof,
        "cpu_baseline": cpu,
        "latency_ms": {"step": round(ms_step, 4), "attention_kernel": round(ms_attn, 4),
                       "before_attention": round(ms_pre, 4)},
        "sparsity": {"kept_block_density": round(density, 4),
                     "filter_skip_frac": round(stats["skipped_updates"] / max(1, stats["group_updates"]), 5),
                     **stats},
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
