"""A pool of CPU worker processes for whole-tensor oracle references (test helper).

The pool is forked when pytest starts (tests/conftest.py), before any test touches
the GPU, so the workers hold no GPU state; they only run the numpy oracle, one head
per task, with BLAS held to one thread each.
"""
import multiprocessing
import os


def _init_worker():
    # one BLAS thread per worker: through the environment for a BLAS library loaded
    # after this point, and through threadpoolctl for one already loaded
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy  # noqa: F401  (loads the BLAS library now, so the limit below reaches it)
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def head_reference(args):
    """The oracle's stage-2 output for one head: (q, k, v, mask, causal, lam) -> (N, D)."""
    from oracle import sparge_oracle as so
    qn, kn, vn, mask, causal, lam = args
    return so.attend_head(qn, kn, vn, mask, causal, lam=lam)


def make_pool():
    n = min(16, len(os.sched_getaffinity(0)))
    if n < 2:
        return None
    return multiprocessing.get_context("fork").Pool(n, initializer=_init_worker)
