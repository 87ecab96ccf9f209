"""The unchanged float64 oracle run over consecutive chunks of samples.

y[b] and dx[b] depend only on sample b (token mixing permutes within a
sample), and every parameter gradient is a sum over samples, so running the
oracle on chunks and adding the chunks' parameter gradients in float64 gives
the whole-batch result up to the order of the float64 sums.  Lets the tests
compare every output of the largest workloads without holding the whole
batch's float64 intermediates at once."""
from __future__ import annotations

import numpy as np

import oracle


def oracle_by_chunks(x, p, dy, chunk, visit):
    """Call visit(b0, b1, y_chunk, dx_chunk) for each chunk of samples [b0, b1);
    return the 14 parameter gradients summed over all chunks."""
    B = x.shape[0]
    sums = {}
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        y_c, cache = oracle.forward(x[b0:b1], p)
        g_c = oracle.backward(dy[b0:b1], cache, p)
        del cache
        visit(b0, b1, y_c, g_c.pop("dx"))
        for key, v in g_c.items():
            if key in sums:
                sums[key] += v
            else:
                sums[key] = v
    return sums
