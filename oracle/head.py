"""CPU reference for the verify head's greedy token and its probability.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library and never calls it.

"[Engine] perf(hip): optimize MTP draft, shared expert, and verify/sampler head
kernels on RDNA4" (Problem and result item 1; Summary item 1; Verification &
Parity Evidence) describes the two operations that consume the verifier's
logits -- T rows of 248,320 fp32 logits -- and checks them on ties, NaN and
-inf entries for 1 to 8 rows.  The pages name the operations (greedy argmax
per row, the row's top probability) but state no rule for those cases; the
readings taken here, per row x[0 .. V-1]:

* token = the smallest index i with x[i] = max over the non-NaN entries
  (ties go to the smallest index; -inf is an ordinary value, so a row of -inf
  gives index 0); a row with no non-NaN entry gives -1;
* top_prob = softmax(x)[token] = 1 / sum_i exp(x[i] - x[token]) over the
  non-NaN entries (a -inf entry contributes 0); NaN when the row has no
  finite maximum (every entry NaN or -inf), where the softmax is undefined.

+inf entries are outside the contract.  The sum is taken in fp64 over the
exact fp32 inputs, in index order.
"""

from __future__ import annotations

import math

import numpy as np


def greedy_head(logits: np.ndarray):
    """logits fp32 [rows][V] -> (token int64 [rows], top_prob fp64 [rows])."""
    x = np.asarray(logits)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("logits must be a float32 [rows][V] array")
    rows, V = x.shape
    token = np.full(rows, -1, dtype=np.int64)
    top = np.full(rows, np.nan)
    for r in range(rows):
        row = x[r].astype(np.float64)
        valid = ~np.isnan(row)
        if not valid.any():
            continue
        m = row[valid].max()
        token[r] = int(np.flatnonzero(valid & (row == m))[0])
        if m == -math.inf:
            continue
        terms = np.exp(row[valid] - m)  # exp(-inf) = 0
        top[r] = 1.0 / terms.sum()
    return token, top
