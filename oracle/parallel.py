"""Row-block thread pool for the fp64 oracle.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the test suite, the
smoke check and the benchmark's CPU-baseline leg may use it, the product path
never.

It holds none of the method's arithmetic.  It only cuts a row range into
consecutive blocks, hands each block to an oracle function in a thread pool
and puts the per-row results back in row order.  Rows of the selected
logprob are independent, so this gives exactly the values of one call over
all rows.  numpy releases the interpreter lock inside its array kernels
(decoding, exp, sums, BLAS products), so the threads run in parallel.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np


def host_threads():
    """Threads to use: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except (AttributeError, OSError):
        return max(1, os.cpu_count() or 1)


def map_row_blocks(fn, n_rows, block_rows=64, workers=None):
    """Call ``fn(r0, r1)`` for consecutive blocks [r0, r1) covering
    [0, n_rows) and concatenate the returned per-row arrays (or tuples of
    arrays) in row order."""
    workers = host_threads() if workers is None else max(1, int(workers))
    spans = [(r0, min(n_rows, r0 + block_rows)) for r0 in range(0, n_rows, block_rows)]
    if not spans:
        return None
    if workers == 1 or len(spans) == 1:
        parts = [fn(r0, r1) for r0, r1 in spans]
    else:
        with ThreadPoolExecutor(max_workers=min(workers, len(spans))) as ex:
            parts = list(ex.map(lambda s: fn(*s), spans))
    if isinstance(parts[0], tuple):
        return tuple(np.concatenate([p[k] for p in parts]) for k in range(len(parts[0])))
    return np.concatenate(parts)
