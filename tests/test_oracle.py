"""Pins of the CPU oracle against facts fixed by the mathematics.

The pages print no worked numeric example, so every pin here is a closed
form, an identity, a special case that reduces to a library routine, finite
differences, or a brute-force evaluation of the definition.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import kl_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(rng, N, d, V, K, tstd=3.0, wstd=0.5, masked=()):
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d)) * wstd
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int64)
    T = np.sort(rng.standard_normal((N, K)) * tstd, axis=1)[:, ::-1]
    mask = np.ones(N, dtype=np.uint8)
    mask[list(masked)] = 0
    return H, W, ids, np.ascontiguousarray(T), mask


# ---------------------------------------------------------------- golden
def test_closed_form_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "closed_forms.json")))["cases"]
    for c in cases:
        z = np.array(c["z"])
        ids = np.array(c["ids"])
        t = np.array(c["tlogit"])
        mask = np.array(c["mask"])
        loss = O.loss_from_logits(z, ids, t, mask)
        assert loss == pytest.approx(c["loss"], rel=1e-14, abs=1e-15), c["name"]
        n = int(mask.sum())
        w = mask / n if n else np.zeros(len(mask))
        G = O.logit_grad(z, ids, t, w)
        np.testing.assert_allclose(G, np.array(c["G"]), rtol=1e-13, atol=1e-15, err_msg=c["name"])


# ---------------------------------------------------------------- P1 finite differences
def test_finite_differences_H_W_Z():
    rng = np.random.default_rng(11)
    N, d, V, K = 3, 5, 11, 4
    H, W, ids, T, mask = rand_problem(rng, N, d, V, K, masked=(1,))
    out = O.kl_dense(H, W, ids, T, mask)

    def L(Hx, Wx):
        return O.kl_dense(Hx, Wx, ids, T, mask)["loss"]

    h = 1e-6
    num_dH = np.zeros_like(H)
    for i in range(N):
        for j in range(d):
            Hp, Hm = H.copy(), H.copy()
            Hp[i, j] += h
            Hm[i, j] -= h
            num_dH[i, j] = (L(Hp, W) - L(Hm, W)) / (2 * h)
    num_dW = np.zeros_like(W)
    for i in range(V):
        for j in range(d):
            Wp, Wm = W.copy(), W.copy()
            Wp[i, j] += h
            Wm[i, j] -= h
            num_dW[i, j] = (L(H, Wp) - L(H, Wm)) / (2 * h)
    scale = max(np.abs(out["dH"]).max(), np.abs(out["dW"]).max())
    np.testing.assert_allclose(out["dH"], num_dH, atol=1e-7 * scale, rtol=1e-6)
    np.testing.assert_allclose(out["dW"], num_dW, atol=1e-7 * scale, rtol=1e-6)
    assert np.all(out["dH"][1] == 0.0)  # masked row

    # logit-level gradient
    z = H @ W.T
    G = O.logit_grad(z, ids, T, mask / mask.sum())
    num_G = np.zeros_like(z)
    for i in range(N):
        for j in range(V):
            zp, zm = z.copy(), z.copy()
            zp[i, j] += h
            zm[i, j] -= h
            num_G[i, j] = (O.loss_from_logits(zp, ids, T, mask) - O.loss_from_logits(zm, ids, T, mask)) / (2 * h)
    np.testing.assert_allclose(G, num_G, atol=1e-8, rtol=1e-6)


# ---------------------------------------------------------------- P2 Gibbs
@pytest.mark.parametrize("K", [1, 2, 7, 32])
def test_kl_nonnegative(K):
    rng = np.random.default_rng(100 + K)
    for _ in range(5):
        H, W, ids, T, mask = rand_problem(rng, 16, 8, 32, K, tstd=4.0, wstd=1.0)
        kl, _, _ = O.row_terms(H @ W.T, ids, T)
        assert np.all(kl >= -1e-12)


# ---------------------------------------------------------------- P3 zero case
def test_zero_when_teacher_equals_student_full_vocab():
    rng = np.random.default_rng(3)
    N, d, V = 6, 4, 9
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    z = H @ W.T
    ids = np.stack([rng.permutation(V) for _ in range(N)])
    T = np.take_along_axis(z, ids, axis=1)
    out = O.kl_dense(H, W, ids, T, None, want_rows=True)
    assert np.all(np.abs(out["kl"]) <= 1e-12)
    assert abs(out["loss"]) <= 1e-12
    assert np.abs(out["dH"]).max() <= 1e-14 * max(1, np.abs(W).max() * V)
    assert np.abs(out["dW"]).max() <= 1e-14 * max(1, np.abs(H).max() * N)


# ---------------------------------------------------------------- P4 block invariance
def test_block_invariance():
    rng = np.random.default_rng(4)
    H, W, ids, T, mask = rand_problem(rng, 70, 12, 40, 6, masked=(3, 50))
    ref = O.kl_dense(H, W, ids, T, mask, block=None, want_rows=True)
    for b in (1, 3, 64, 70):
        o = O.kl_dense(H, W, ids, T, mask, block=b, want_rows=True)
        assert o["loss"] == pytest.approx(ref["loss"], rel=1e-13)
        np.testing.assert_allclose(o["dH"], ref["dH"], rtol=0, atol=1e-13 * np.abs(ref["dH"]).max())
        np.testing.assert_allclose(o["dW"], ref["dW"], rtol=0, atol=1e-13 * np.abs(ref["dW"]).max())
        # z itself comes from BLAS, whose rounding depends on the block shape
        np.testing.assert_allclose(o["zg"], ref["zg"], rtol=0, atol=1e-14 * np.abs(ref["zg"]).max())


# ---------------------------------------------------------------- P5 K = 1 cross-entropy
def test_k1_is_cross_entropy():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    N, d, V = 20, 6, 33
    H = rng.standard_normal((N, d))
    W = rng.standard_normal((V, d))
    y = rng.integers(0, V, size=(N, 1))
    T = rng.standard_normal((N, 1))
    out = O.kl_dense(H, W, y, T, None)
    Ht = torch.tensor(H, requires_grad=True)
    Wt = torch.tensor(W, requires_grad=True)
    ce = torch.nn.functional.cross_entropy(Ht @ Wt.T, torch.tensor(y[:, 0]))
    ce.backward()
    assert out["loss"] == pytest.approx(ce.item(), rel=1e-13)
    np.testing.assert_allclose(out["dH"], Ht.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(out["dW"], Wt.grad.numpy(), rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P6 W = 0 closed form
def test_zero_weight_closed_form():
    rng = np.random.default_rng(6)
    N, d, V, K = 9, 5, 17, 5
    H, _, ids, T, mask = rand_problem(rng, N, d, V, K, masked=(2,))
    W = np.zeros((V, d))
    out = O.kl_dense(H, W, ids, T, mask, want_rows=True)
    pT = np.exp(T - T.max(1, keepdims=True))
    pT /= pT.sum(1, keepdims=True)
    ent = -(pT * np.log(pT)).sum(1)
    kl_expect = np.log(V) - ent
    valid = mask == 1
    np.testing.assert_allclose(out["kl"][valid], kl_expect[valid], rtol=1e-13)
    assert out["loss"] == pytest.approx(kl_expect[valid].mean(), rel=1e-13)
    assert np.all(out["dH"] == 0.0)
    G = np.full((N, V), 1.0 / V)
    for r in range(N):
        for k in range(K):
            G[r, ids[r, k]] -= pT[r, k]
    G *= (mask / mask.sum())[:, None]
    np.testing.assert_allclose(out["dW"], G.T @ H, rtol=1e-12, atol=1e-16)


# ---------------------------------------------------------------- P7 row sums
def test_gradient_row_and_column_sums_vanish():
    rng = np.random.default_rng(7)
    H, W, ids, T, mask = rand_problem(rng, 30, 7, 50, 8, masked=(0, 29))
    z = H @ W.T
    G = O.logit_grad(z, ids, T, mask / mask.sum())
    assert np.abs(G.sum(1)).max() <= 1e-15
    out = O.kl_dense(H, W, ids, T, mask)
    assert np.abs(out["dW"].sum(0)).max() <= 1e-13 * np.abs(out["dW"]).max() * 50


# ---------------------------------------------------------------- P8 invariances
def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(8)
    N, d, V, K = 12, 6, 25, 5
    H, W, ids, T, mask = rand_problem(rng, N, d, V, K, masked=(4,))
    ref = O.kl_dense(H, W, ids, T, mask)
    # teacher logits + per-row constant
    o1 = O.kl_dense(H, W, ids, T + rng.standard_normal((N, 1)) * 10, mask)
    # W + 1 c^T: every logit of row r moves by H_r . c
    c = rng.standard_normal(d)
    o2 = O.kl_dense(H, W + c[None, :], ids, T, mask)
    # permute the (id, logit) pairs of each row
    perm = np.stack([rng.permutation(K) for _ in range(N)])
    o3 = O.kl_dense(H, W, np.take_along_axis(ids, perm, 1), np.take_along_axis(T, perm, 1), mask)
    for o in (o1, o2, o3):
        assert o["loss"] == pytest.approx(ref["loss"], rel=1e-12)
        np.testing.assert_allclose(o["dH"], ref["dH"], rtol=1e-10, atol=1e-14)
        np.testing.assert_allclose(o["dW"], ref["dW"], rtol=1e-10, atol=1e-14)


# ---------------------------------------------------------------- P9 mask compaction
def test_mask_equals_compaction():
    rng = np.random.default_rng(9)
    N, d, V, K = 40, 6, 30, 4
    masked = (0, 5, 6, 39)
    H, W, ids, T, mask = rand_problem(rng, N, d, V, K, masked=masked)
    full = O.kl_dense(H, W, ids, T, mask)
    keep = mask == 1
    comp = O.kl_dense(H[keep], W, ids[keep], T[keep], None)
    assert full["loss"] == pytest.approx(comp["loss"], rel=1e-13)
    np.testing.assert_allclose(full["dW"], comp["dW"], rtol=1e-12, atol=1e-16)
    np.testing.assert_allclose(full["dH"][keep], comp["dH"], rtol=1e-13)
    assert np.all(full["dH"][~keep] == 0.0)
    assert full["n_valid"] == N - len(masked)


def test_all_masked_is_zero():
    rng = np.random.default_rng(10)
    H, W, ids, T, _ = rand_problem(rng, 5, 4, 10, 3)
    out = O.kl_dense(H, W, ids, T, np.zeros(5, dtype=np.uint8))
    assert out["loss"] == 0.0 and np.all(out["dH"] == 0) and np.all(out["dW"] == 0)


def test_empty_batch_is_an_all_masked_one():
    # no positions at all: the same reading as no valid position (loss 0, no
    # gradient), whatever the block size
    rng = np.random.default_rng(11)
    H, W, ids, T, _ = rand_problem(rng, 5, 4, 10, 3)
    masked = O.kl_dense(H, W, ids, T, np.zeros(5, dtype=np.uint8), want_rows=True)
    for block in (None, 1, 4):
        out = O.kl_dense(H[:0], W, ids[:0], T[:0], np.zeros(0, dtype=np.uint8), block=block, want_rows=True)
        assert out["loss"] == masked["loss"] == 0.0 and out["n_valid"] == 0
        assert out["dH"].shape == (0, 4) and out["kl"].shape == (0,) and out["lse"].shape == (0,)
        assert np.array_equal(out["dW"], masked["dW"])


# ---------------------------------------------------------------- P10 exact gather
def test_gather_is_exact_copy_with_one_hot_rows():
    rng = np.random.default_rng(12)
    N, d, V, K = 10, 8, 20, 5
    W = rng.integers(-8, 9, size=(V, d)).astype(np.float64)
    cols = rng.integers(0, d, size=N)
    H = np.zeros((N, d))
    H[np.arange(N), cols] = 1.0
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)])
    T = rng.standard_normal((N, K))
    out = O.kl_dense(H, W, ids, T, None, want_rows=True)
    expect = W[ids, cols[:, None]]
    np.testing.assert_array_equal(out["zg"], expect)


# ---------------------------------------------------------------- P11 brute force
def brute(H, W, ids, T, mask):
    N, d = len(H), len(H[0])
    V, K = len(W), len(ids[0])
    n = sum(1 for m in mask if m)
    s = 1.0 / n if n else 0.0
    loss = 0.0
    dH = [[0.0] * d for _ in range(N)]
    dW = [[0.0] * d for _ in range(V)]
    for r in range(N):
        if not mask[r]:
            continue
        z = [sum(H[r][c] * W[v][c] for c in range(d)) for v in range(V)]
        zmax = max(z)
        lse = zmax + math.log(sum(math.exp(x - zmax) for x in z))
        tmax = max(T[r])
        lset = tmax + math.log(sum(math.exp(x - tmax) for x in T[r]))
        g = [math.exp(z[v] - lse) for v in range(V)]
        for k in range(K):
            lpt = T[r][k] - lset
            pt = math.exp(lpt)
            loss += s * pt * (lpt - (z[ids[r][k]] - lse))
            g[ids[r][k]] -= pt
        for v in range(V):
            for c in range(d):
                dH[r][c] += s * g[v] * W[v][c]
                dW[v][c] += s * g[v] * H[r][c]
    return loss, dH, dW


def test_brute_force_tiny():
    rng = np.random.default_rng(13)
    for (N, d, V, K) in [(1, 1, 2, 1), (3, 2, 5, 2), (4, 4, 16, 3), (4, 3, 16, 16)]:
        H, W, ids, T, mask = rand_problem(rng, N, d, V, K, masked=(0,) if N > 2 else ())
        bl, bdH, bdW = brute(H.tolist(), W.tolist(), ids.tolist(), T.tolist(), mask.tolist())
        out = O.kl_dense(H, W, ids, T, mask)
        assert out["loss"] == pytest.approx(bl, rel=1e-12, abs=1e-14)
        np.testing.assert_allclose(out["dH"], np.array(bdH), rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(out["dW"], np.array(bdW), rtol=1e-11, atol=1e-14)


def test_kl_rows_matches_dense_on_sample():
    rng = np.random.default_rng(14)
    H, W, ids, T, mask = rand_problem(rng, 25, 6, 30, 5, masked=(7,))
    full = O.kl_dense(H, W, ids, T, mask, want_rows=True)
    rows = np.array([0, 7, 13, 24])
    w = mask / mask.sum()
    part = O.kl_rows(H[rows], W, ids[rows], T[rows], w[rows])
    np.testing.assert_allclose(part["dH"], full["dH"][rows], rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(part["lse"], full["lse"][rows], rtol=1e-14)
    np.testing.assert_array_equal(part["zg"], full["zg"][rows])
