"""Run the fp64 oracle on many (batch, head) pairs at once, in worker processes.

Test infrastructure only.  numpy's elementwise work (exp, masks, sums) runs on one core,
so full-size oracle runs take minutes in one process; this spreads the pairs over a pool
of spawned worker processes (no GPU use in them: they import only the oracle and numpy),
each with single-threaded BLAS.  Inputs travel as float32 (exact for bf16 values); the
oracle upcasts them to float64 as usual.
"""

from __future__ import annotations

import os
import sys
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def workers() -> int:
    """Pool size: the CPUs this process may use, at most 16 (a GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _init():
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)


def _forward(args):
    import oracle
    q, k, v, scale, causal, rows = args
    return oracle.head_forward(q, k, v, scale, causal, rows=rows)


def _backward(args):
    import oracle
    q, k, v, do, scale, causal = args
    return oracle.head_backward(q, k, v, do, scale, causal)


class Pool:
    """Context manager: ``forward(tasks)`` / ``backward(tasks)`` map oracle.head_forward /
    oracle.head_backward over argument tuples and return the results in order."""

    def __enter__(self):
        # Workers are spawned on demand and read the thread settings when they start, so
        # the single-thread setting stays in the environment while the pool exists.
        self._saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        self._ex = ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"), initializer=_init)
        return self

    def __exit__(self, *exc):
        self._ex.shutdown(wait=True, cancel_futures=True)
        for k, v in self._saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        return False

    def forward(self, tasks):
        return list(self._ex.map(_forward, tasks))

    def backward(self, tasks):
        return list(self._ex.map(_backward, tasks))


def f32(t) -> np.ndarray:
    """A torch tensor (bf16 on any device) as a float32 numpy array, exactly."""
    return t.detach().float().cpu().numpy()
