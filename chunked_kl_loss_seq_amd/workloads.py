"""Seeded synthetic inputs for the fused chunked KL loss.

This module only draws inputs: it holds none of the loss arithmetic and
imports neither the HIP binding nor the oracle, so both sides can be fed the
same arrays.  No public dataset or benchmark suite stands behind the five
workloads; the pages give the vocabulary (201,088, gpt-oss-120b) and K = 100
("A New Trick Slashes the Cost of Shrinking Giant AI Models", sections "Why is
this so hard to do cheaply?" and "What did the researchers change?"), the rest
of each shape is the workload's own specification.

Conventions
* Every array comes from ``numpy.random.default_rng`` children of
  ``SeedSequence(seed)`` spawned in the fixed order [W, H, ids, logits, mask].
  The default seed of a named workload is its number (1..5).
* Normals are drawn in fp32 with the stated standard deviation and, for bf16
  workloads, rounded to bf16 with round-to-nearest-even; the arrays returned
  are float32 holding bf16-exact values, so the device copy and the oracle's
  float64 copy are the same numbers.
* Teacher logits are sorted descending along k and paired with the ids in the
  order they were drawn.
* H and W are drawn in blocks of 4096 rows, block b from the b-th child of
  its stream; everything else row-major in row order.  So the first R rows of
  a workload generated with ``rows=R`` equal the first R rows of the full one.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make", "make_custom", "round_bf16", "bf16_bits", "teacher_logits"]


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    d: int
    V: int
    K: int
    dtype: str  # "bf16" or "f32": type of H, W and dH
    chunk: int  # 0 = chosen by the chunk planner
    ids: str  # "uniform", "overlap50" or "zipf"
    tstd: float  # teacher logit standard deviation
    mask: str  # "none", "random5" or "tailpad"
    seq_len: int = 0  # sequence length for "tailpad" masks
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload("tiny-fp32", 256, 256, 4096, 16, "f32", 64, "uniform", 2.0, "none"),
    2: Workload("bf16-32k-vocab", 4096, 2048, 32000, 100, "bf16", 1024, "overlap50", 3.0, "none"),
    3: Workload("llama3-3b-head", 8192, 3072, 128256, 100, "bf16", 1024, "overlap50", 3.0, "random5"),
    4: Workload("gpt-oss-head-32k", 32768, 2880, 201088, 100, "bf16", 0, "zipf", 3.0, "none"),
    5: Workload("gpt-oss-head-4x32k", 131072, 2880, 201088, 100, "bf16", 0, "zipf", 3.0, "tailpad",
                seq_len=32768),
    # one 256K-token sequence: the pages' long-context point (memory stays
    # nearly constant as the input grows), at the gpt-oss head's shape
    6: Workload("gpt-oss-head-256k", 262144, 2880, 201088, 100, "bf16", 0, "zipf", 3.0, "none"),
}


def round_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    bias = ((b >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) & np.uint32(0xFFFF0000)).view(np.float32)


def bf16_bits(x):
    """uint16 bit patterns of bf16-exact float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _normal(ss, shape, std, bf16, block_rows=4096):
    """Normal(0, std) array drawn in blocks of ``block_rows`` rows.

    Block b comes from the b-th child of SeedSequence ``ss``, so blocks can be
    filled by several threads and the result does not depend on their number.
    """
    out = np.empty(shape, dtype=np.float32)
    n_blocks = (shape[0] + block_rows - 1) // block_rows
    children = ss.spawn(n_blocks)

    def fill(b):
        r0 = b * block_rows
        r1 = min(shape[0], r0 + block_rows)
        blk = np.random.default_rng(children[b]).standard_normal(
            (r1 - r0,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[r0:r1] = round_bf16(blk) if bf16 else blk

    workers = max(1, min(16, os.cpu_count() or 1, n_blocks))
    if workers == 1:
        for b in range(n_blocks):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_blocks)))
    return out


def _first_distinct(draws, K, forbid=None):
    """First K distinct values of each row of ``draws`` in order of first appearance.

    Entries for which ``forbid`` is True are skipped.  Returns (sel [R,K], ok [R]);
    rows with fewer than K admissible distinct values have ok = False.
    """
    R, B = draws.shape
    order = np.argsort(draws, axis=1, kind="stable")
    sd = np.take_along_axis(draws, order, axis=1)
    first = np.ones(sd.shape, dtype=bool)
    first[:, 1:] = sd[:, 1:] != sd[:, :-1]
    if forbid is not None:
        first &= ~np.take_along_axis(forbid, order, axis=1)
    pos = np.where(first, order, B)
    pos.sort(axis=1)
    ok = pos[:, K - 1] < B
    sel = np.take_along_axis(draws, np.minimum(pos[:, :K], B - 1), axis=1)
    return sel, ok


def _zipf_cdf(V, a):
    w = np.arange(1, V + 1, dtype=np.float64) ** (-a)
    c = np.cumsum(w)
    return c / c[-1]


def _distinct_rows(ss, N, K, V, sampler, batch, forbid_fn=None, block_rows=8192):
    """K distinct ids per row by draw-with-replacement-and-discard.

    ``sampler(u)`` maps uniforms in [0,1) to ids.  Each row first gets ``batch``
    uniforms from the stream of SeedSequence ``ss`` (row-major, so row prefixes
    are stable).  A row that has not reached K distinct admissible ids after
    that is continued from its own stream (a child of ``ss`` keyed by the row),
    which keeps the draw order defined without touching other rows.
    """
    rng = np.random.default_rng(ss)
    out = np.empty((N, K), dtype=np.int64)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        draws = sampler(rng.random((r1 - r0, batch)))
        forbid = forbid_fn(r0, r1, draws) if forbid_fn else None
        sel, ok = _first_distinct(draws, K, forbid)
        out[r0:r1] = sel
        for i in np.nonzero(~ok)[0]:
            r = r0 + int(i)
            rrng = np.random.default_rng(
                np.random.SeedSequence(ss.entropy, spawn_key=tuple(ss.spawn_key) + (1 << 20, r)))
            row = draws[i]
            while True:
                row = np.concatenate([row, sampler(rrng.random(4 * batch))])
                f = forbid_fn(r, r + 1, row[None, :]) if forbid_fn else None
                s, k_ok = _first_distinct(row[None, :], K, f)
                if k_ok[0]:
                    out[r] = s[0]
                    break
    return out


def _student_top(H, W, top, block_rows=1024):
    """Student's own top-``top`` ids per row, by fp32 scores H W^T; ties -> lower id.

    Used only to choose which teacher ids overlap with the student's favourites.
    """
    N = H.shape[0]
    res = np.empty((N, top), dtype=np.int64)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        s = H[r0:r1] @ W.T
        part = np.argpartition(-s, top - 1, axis=1)[:, :top]
        ps = np.take_along_axis(s, part, axis=1)
        # lexicographic: score descending, then id ascending
        order = np.lexsort((part, -ps), axis=1)
        res[r0:r1] = np.take_along_axis(part, order, axis=1)
    return res


def _ids(ss, wl, N, H, W):
    V, K = wl.V, wl.K
    uniform = lambda u: np.minimum((u * V).astype(np.int64), V - 1)  # noqa: E731
    if wl.ids == "uniform":
        return _distinct_rows(ss, N, K, V, uniform, batch=max(4 * K, 64))
    if wl.ids == "zipf":
        cdf = _zipf_cdf(V, 1.1)
        return _distinct_rows(ss, N, K, V,
                              lambda u: np.minimum(np.searchsorted(cdf, u, side="right"), V - 1),
                              batch=256)
    if wl.ids == "overlap50":
        half = K // 2
        s_pick, s_rest, s_perm = ss.spawn(3)
        top = _student_top(H, W, K)
        # half of the ids: a random subset of the student's own top-K
        keys = np.random.default_rng(s_pick).random((N, K))
        pick = np.take_along_axis(top, np.argsort(keys, axis=1)[:, :half], axis=1)

        # the other half: distinct uniform ids outside the student's top-K
        def forbid(r0, r1, draws):
            return (draws[:, :, None] == top[r0:r1][:, None, :]).any(axis=2)

        rest = _distinct_rows(s_rest, N, K - half, V, uniform, batch=4 * K,
                              forbid_fn=forbid, block_rows=1024)
        both = np.concatenate([pick, rest], axis=1)
        perm = np.argsort(np.random.default_rng(s_perm).random((N, K)), axis=1)
        return np.take_along_axis(both, perm, axis=1)
    raise ValueError(wl.ids)


def _mask(rng, wl, N):
    if wl.mask == "none":
        return np.ones(N, dtype=np.uint8)
    if wl.mask == "random5":
        m = np.ones(N, dtype=np.uint8)
        n_off = int(round(0.05 * N))
        m[rng.permutation(N)[:n_off]] = 0
        return m
    if wl.mask == "tailpad":
        T = wl.seq_len
        B = (N + T - 1) // T
        u = rng.uniform(0.0, 0.2, size=B)
        m = np.ones(B * T, dtype=np.uint8)
        for b in range(B):
            pad = int(np.floor(u[b] * T))
            if pad:
                m[b * T + T - pad:(b + 1) * T] = 0
        return m[:N]
    raise ValueError(wl.mask)


def make_custom(wl, seed, rows=None):
    """Inputs for workload ``wl`` with the given seed (optionally the first ``rows`` rows).

    Returns a dict: H [R,d] f32, W [V,d] f32 (bf16-exact for bf16 workloads),
    ids [R,K] int32, tlogit [R,K] f32, mask [R] uint8, plus the workload.
    """
    N = wl.N if rows is None else min(int(rows), wl.N)
    bf16 = wl.dtype == "bf16"
    s_w, s_h, s_ids, s_t, s_m = np.random.SeedSequence(seed).spawn(5)
    W = _normal(s_w, (wl.V, wl.d), 0.02, bf16)
    H = _normal(s_h, (N, wl.d), 1.0, bf16)
    ids = _ids(s_ids, wl, N, H, W).astype(np.int32)
    t = np.random.default_rng(s_t).standard_normal((N, wl.K), dtype=np.float32) * np.float32(wl.tstd)
    t = -np.sort(-t, axis=1)
    # masks are drawn for the whole workload and then cut, so prefixes agree
    mask = _mask(np.random.default_rng(s_m), wl, wl.N)[:N]
    return {"H": H, "W": W, "ids": ids, "tlogit": np.ascontiguousarray(t, dtype=np.float32),
            "mask": mask, "wl": wl, "seed": seed, "N": N}


def make(number, rows=None, seed=None):
    """Inputs of named workload ``number`` (1..5); default seed = the number."""
    wl = WORKLOADS[number]
    return make_custom(wl, number if seed is None else seed, rows=rows)


def small(N, d, V, K, dtype="bf16", ids="uniform", tstd=3.0, mask="none", seed=0, seq_len=0):
    """An ad-hoc workload of any shape, drawn by the same recipe."""
    wl = Workload(f"custom-{N}x{d}x{V}x{K}", N, d, V, K, dtype, 0, ids, tstd, mask, seq_len=seq_len)
    return make_custom(wl, seed)


def teacher_logits(N, V, std=3.0, seed=0, bf16=True, rows=None):
    """Full-vocabulary teacher logit rows [N, V] for the top-K cache writer:
    N(0, std) drawn in fp32 (rounded RNE to bf16 when ``bf16``), in blocks of
    256 rows from the children of SeedSequence(seed), so the first ``rows``
    rows do not depend on N.  bf16 rounding leaves many equal values, which
    exercises the tie order."""
    n = N if rows is None else min(rows, N)
    ss = np.random.SeedSequence(seed)
    if n == N:
        return _normal(ss, (N, V), std, bf16, block_rows=256)
    # the first blocks only: same children, same draws
    full_blocks = (N + 255) // 256
    kids = ss.spawn(full_blocks)
    need = (n + 255) // 256
    out = np.empty((need * 256, V), dtype=np.float32)
    for b in range(need):
        r1 = min(N, (b + 1) * 256)
        blk = np.random.default_rng(kids[b]).standard_normal((r1 - b * 256, V), dtype=np.float32)
        if std != 1.0:
            blk *= np.float32(std)
        out[b * 256:r1] = round_bf16(blk) if bf16 else blk
    return out[:n]
