"""Plain CPU oracle for the offline top-K cache writer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module: only the tests and ``bench.py``'s ``cpu_baseline`` leg use
it.  It shares no code, constant or helper with the HIP library.

What it computes.  The teacher is run once and only its K most likely
predictions per position are kept ("A New Trick Slashes the Cost of Shrinking
Giant AI Models", section "What did the researchers change?": the top 100
predictions per position are saved to disk; "Making Knowledge Distillation
Cheap Enough to Run at Scale" (elseif.net), offline-cache paragraph).  Per
row of teacher logits that is the K largest logits with their token ids.
The pages do not say how equal logits are ordered; the reading taken is the
plain stable one: by value descending, equal values by id ascending, so the
result is unique.  Values compare as real numbers (-0.0 equals +0.0); NaN is
outside the supported inputs.

The definition is written out with a library sort as its only step: a stable
sort of each row by its negated value keeps equal values in id order.

Pins (tests/test_topk_oracle.py): a pure-Python sort on small rows, heapq,
argmax for K = 1, a full sort for K = V, all-equal rows, signed zeros,
infinities, and the selection invariants on bf16 rows with many ties.
"""

from __future__ import annotations

import numpy as np

__all__ = ["topk_rows"]


def topk_rows(logits, K):
    """ids int32 [N, K] and values float32 [N, K] of the K largest logits per row,
    by value descending, equal values by id ascending."""
    x = np.asarray(logits, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("logits must be [N, V]")
    N, V = x.shape
    if not 1 <= K <= V:
        raise ValueError("need 1 <= K <= V")
    # -x: the largest value first; +0.0 for -0.0 so that signed zeros are equal
    order = np.argsort(-x + 0.0, axis=1, kind="stable")[:, :K]
    vals = np.take_along_axis(x, order, axis=1)
    return order.astype(np.int32), vals.astype(np.float32)
