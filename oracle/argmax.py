"""The target model's greedy prediction at every tree node.

DARTree paper, Preliminaries > Speculative Sampling: at temperature 0 the
verifier compares each draft token with the target's greedy prediction, i.e.
the arg-max of the target logits at that position. Ties go to the lowest
vocabulary index (a reading: the pages do not discuss ties). Rows are assumed
finite; a row holding NaN has no defined answer.
"""

import numpy as np


def argmax_rows(logits):
    """numpy's arg-max per row (first occurrence of the row maximum)."""
    return np.argmax(np.asarray(logits), axis=1).astype(np.int64)


def argmax_rows_loop(logits):
    """The same, as an explicit Python scan (for small inputs): keep the first
    index whose value is strictly greater than every earlier one."""
    out = []
    for row in np.asarray(logits):
        best, best_j = row[0], 0
        for j in range(1, len(row)):
            if row[j] > best:
                best, best_j = row[j], j
        out.append(best_j)
    return np.array(out, dtype=np.int64)
