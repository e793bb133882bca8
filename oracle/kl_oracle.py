"""Plain CPU oracle for the fused chunked KL distillation loss.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constant or
helper with the HIP library.

What it computes (all arithmetic in float64, from the exact input values:
bf16 and fp32 inputs upcast exactly):

* Teacher distribution.  The teacher is run once offline and only its top-K
  logits per position are kept ("A New Trick Slashes the Cost of Shrinking
  Giant AI Models", section "What did the researchers change?": the top 100
  predictions per position are cached; "Making Knowledge Distillation Cheap
  Enough to Run at Scale" (elseif.net), offline-cache and limitations
  paragraphs: the probabilities of the remaining tokens are dropped).  Reading:
  p_T is the softmax over the K cached logits alone, renormalised, with no
  tail bucket and temperature 1.
* Student distribution.  log p_S is the log-softmax over the full vocabulary of
  z = H_r . W^T: the vocabulary x sequence grid the pages say the dense loss
  builds ("A New Trick...", section "Why is this so hard to do cheaply?").
* Loss.  Per position KL(p_T || p_S) = sum_k p_T,k (log p_T,k - log p_S,id_k),
  averaged over valid (mask = 1) positions; 0 if no position is valid.  The
  fused chunked loss is stated to be mathematically equivalent to the dense
  one ("Model compression is a distraction...", introduction), so the oracle
  is the dense definition itself.
* Gradient.  dL/dz_r = w_r (softmax(z_r) - scatter(p_T,r)), w_r = mask_r / n,
  then dH = G W and dW = G^T H (chain rule through z = H W^T).

Rows are independent, so ``kl_dense`` walks row blocks only to bound host
memory; the block size does not enter the arithmetic of any single row, and
dW is the plain sum of the per-block contributions.

Pins (tests/test_oracle.py): finite differences, Gibbs' inequality, the
K = V zero case, block invariance, the K = 1 cross-entropy special case, the
W = 0 closed form, gradient row sums, shift and permutation invariances, mask
compaction, a pure-Python brute force and hand-computed golden values.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "teacher_log_probs",
    "student_log_softmax",
    "row_terms",
    "logit_grad",
    "loss_from_logits",
    "kl_dense",
    "kl_rows",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def teacher_log_probs(tlogit):
    """log p_T over the K cached teacher logits of each row.

    Softmax restricted to the cached top-K (renormalised); the rest of the
    vocabulary carries no teacher mass.  Computed as T - (tau + log sum
    exp(T - tau)) with tau the row maximum.
    """
    t = _f64(tlogit)
    tau = t.max(axis=1, keepdims=True)
    lse_t = tau + np.log(np.exp(t - tau).sum(axis=1, keepdims=True))
    return t - lse_t


def student_log_softmax(z):
    """Full-vocabulary log-softmax of the student logits; returns (log p_S, lse)."""
    z = _f64(z)
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    return z - lse, lse[:, 0]


def row_terms(z, idx, tlogit):
    """Per-row KL(p_T || p_S), student lse and the gathered logits z[r, idx[r, k]].

    z: [R, V] student logits; idx: [R, K] int teacher ids; tlogit: [R, K].
    The gather is a plain index copy, so zg is exactly z at those positions.
    """
    z = _f64(z)
    idx = np.asarray(idx, dtype=np.int64)
    logp_t = teacher_log_probs(tlogit)
    p_t = np.exp(logp_t)
    _, lse = student_log_softmax(z)
    rows = np.arange(z.shape[0])[:, None]
    zg = z[rows, idx]
    logp_s_at = zg - lse[:, None]
    kl = (p_t * (logp_t - logp_s_at)).sum(axis=1)
    return kl, lse, zg


def logit_grad(z, idx, tlogit, weight):
    """G = dL/dz = weight_r * (softmax(z_r) - scatter_add(p_T,r)).

    ``weight`` is mask_r / n_valid per row.  Scatter-add, so duplicate ids in
    a row (outside the supported inputs) would add their teacher mass.
    """
    z = _f64(z)
    idx = np.asarray(idx, dtype=np.int64)
    p_t = np.exp(teacher_log_probs(tlogit))
    logp_s, _ = student_log_softmax(z)
    g = np.exp(logp_s)
    rows = np.broadcast_to(np.arange(z.shape[0])[:, None], idx.shape)
    np.subtract.at(g, (rows, idx), p_t)
    return g * _f64(weight)[:, None]


def _weights(mask, n_rows):
    if mask is None:
        m = np.ones(n_rows, dtype=np.float64)
    else:
        m = (np.asarray(mask) != 0).astype(np.float64)
    n_valid = int(m.sum())
    scale = 1.0 / n_valid if n_valid > 0 else 0.0
    return m, n_valid, scale


def loss_from_logits(z, idx, tlogit, mask=None):
    """Mean over valid rows of KL(p_T || p_S), from student logits directly."""
    m, _, scale = _weights(mask, np.shape(z)[0])
    kl, _, _ = row_terms(z, idx, tlogit)
    return float(scale * (m * kl).sum())


def kl_dense(H, W, idx, tlogit, mask=None, block=None, want_rows=False):
    """Dense KL loss and its gradients with respect to H and W.

    H: [N, d], W: [V, d], idx: [N, K] int, tlogit: [N, K], mask: [N] or None.
    Returns a dict with ``loss`` (float), ``dH`` [N, d], ``dW`` [V, d] (float64)
    and, if ``want_rows``, per-row ``kl``, ``lse`` and ``zg`` [N, K].
    """
    H = _f64(H)
    W = _f64(W)
    N = H.shape[0]
    block = max(N, 1) if not block else int(block)  # N = 0: no rows, no blocks
    m, n_valid, scale = _weights(mask, N)
    weight = m * scale
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    kl_all = np.zeros(N)
    lse_all = np.zeros(N)
    zg_all = np.zeros(np.shape(idx), dtype=np.float64)
    loss = 0.0
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        z = H[r0:r1] @ W.T
        kl, lse, zg = row_terms(z, idx[r0:r1], tlogit[r0:r1])
        kl = np.where(m[r0:r1] > 0, kl, 0.0)
        loss += float((weight[r0:r1] * kl).sum())
        g = logit_grad(z, idx[r0:r1], tlogit[r0:r1], weight[r0:r1])
        dH[r0:r1] = g @ W
        dW += g.T @ H[r0:r1]
        kl_all[r0:r1] = kl
        lse_all[r0:r1] = lse
        zg_all[r0:r1] = zg
    out = {"loss": loss, "dH": dH, "dW": dW, "n_valid": n_valid}
    if want_rows:
        out.update(kl=kl_all, lse=lse_all, zg=zg_all)
    return out


def kl_rows(H_rows, W, idx_rows, tlogit_rows, weight_rows):
    """Per-row quantities for a sample of rows of a larger problem.

    Each row's KL, lse and dH row depend only on that row and on W, plus the
    row weight mask_r / n_valid of the whole problem, so a sample of rows is
    checked exactly without forming the rest.  Returns kl, lse, zg, dH rows.
    """
    H_rows = _f64(H_rows)
    W = _f64(W)
    z = H_rows @ W.T
    kl, lse, zg = row_terms(z, idx_rows, tlogit_rows)
    g = logit_grad(z, idx_rows, tlogit_rows, weight_rows)
    return {"kl": kl, "lse": lse, "zg": zg, "dH": g @ W}
