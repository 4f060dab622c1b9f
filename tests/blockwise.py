"""Runs an oracle call over row blocks of a large batch on a thread pool (numpy's
matrix products and ufuncs release the GIL), so that full-size parity checks finish in
seconds.  Each block's BLAS calls run on one thread, so the blocks themselves are the
parallelism.  Only the mapping lives here; every block result is the oracle's own."""
from __future__ import annotations

import concurrent.futures as cf
import os


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def map_blocks(fn, n_rows: int, block: int):
    """[fn(r0, r1) for consecutive blocks [r0, r1) covering n_rows rows], in order."""
    from threadpoolctl import threadpool_limits
    starts = list(range(0, n_rows, block))
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(workers()) as ex:
            return list(ex.map(lambda r0: fn(r0, min(n_rows, r0 + block)), starts))
