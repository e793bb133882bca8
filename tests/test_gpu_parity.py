"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: fp32 path 1e-5 relative on the loss and relative Frobenius on dH
and dW; bf16 paths 2e-3 relative on the loss and 1e-2 relative Frobenius on
dH and dW.  Index work (gather, scatter ids) is compared bit for bit.
"""
import os
import sys

import numpy as np
import pytest

from chunked_kl_loss_seq_amd import workloads as WL
from oracle import kl_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the parity tests")
    from chunked_kl_loss_seq_amd import binding

    binding.lib()  # raises if libckl.so is missing
    return binding


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def to_dev(inp, dtype):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H = torch.from_numpy(inp["H"]).to(dev).to(tdt).contiguous()
    W = torch.from_numpy(inp["W"]).to(dev).to(tdt).contiguous()
    ids = torch.from_numpy(inp["ids"]).to(dev).contiguous()
    T = torch.from_numpy(inp["tlogit"]).to(dev).contiguous()
    mask = torch.from_numpy(inp["mask"]).to(dev).contiguous()
    return H, W, ids, T, mask


def run_gpu(binding, inp, dtype, chunk, use_mask=True, rows=False):
    H, W, ids, T, mask = to_dev(inp, dtype)
    N = H.shape[0]
    kw = {}
    if rows:
        kw["row_kl"] = torch.empty(N, dtype=torch.float32, device=H.device)
        kw["row_lse"] = torch.empty(N, dtype=torch.float32, device=H.device)
    loss, dH, dW = binding.fwd_bwd(H, W, ids, T, mask if use_mask else None, chunk=chunk, **kw)
    torch.cuda.synchronize()
    out = {"loss": float(loss.item()), "dH": dH.float().cpu().numpy(), "dW": dW.cpu().numpy()}
    if rows:
        out["kl"] = kw["row_kl"].cpu().numpy()
        out["lse"] = kw["row_lse"].cpu().numpy()
    return out


def check(g, o, dtype, what=""):
    tl, tg = (1e-5, 1e-5) if dtype == "f32" else (2e-3, 1e-2)
    el = abs(g["loss"] - o["loss"]) / max(abs(o["loss"]), 1e-30)
    eh = rel_fro(g["dH"], o["dH"])
    ew = rel_fro(g["dW"], o["dW"])
    say(f"[parity {what}] loss {g['loss']:.7g} vs {o['loss']:.7g} rel {el:.2e}; dH {eh:.2e}; dW {ew:.2e}")
    assert el <= tl, (what, el)
    assert eh <= tg, (what, eh)
    assert ew <= tg, (what, ew)


def _fp32_slack(s_at, T, w):
    """Absolute fp32 rounding allowance of w (exp(z - lse) - p_T) at the cached
    ids: a few units of 2^-24 of each of its two terms (they may cancel)."""
    pt = np.exp(O.teacher_log_probs(T)) * np.asarray(w, np.float64)[:, None]
    return 3e-6 * (np.abs(s_at) + pt) + 1e-30


# ------------------------------------------------------------------ row pass alone
@pytest.mark.parametrize("g_bf16", [True, False])
def test_row_pass_gather_scatter_and_gradient(g_bf16):
    binding = _need_gpu()
    say(f"[case] row pass g_bf16={g_bf16}")
    rng = np.random.default_rng(21)
    R, V, K = 37, 5003, 64
    Z = (rng.standard_normal((R, V)) * 2.0).astype(np.float32)
    ids = np.stack([rng.permutation(V)[:K] for _ in range(R)]).astype(np.int32)
    T = np.sort(rng.standard_normal((R, K)).astype(np.float32) * 3, axis=1)[:, ::-1].copy()
    mask = np.ones(R, dtype=np.uint8)
    mask[[3, 30]] = 0
    scale = 1.0 / 35
    dev = torch.device("cuda:0")
    out = binding.debug_rows(torch.from_numpy(Z).to(dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(T).to(dev), torch.from_numpy(mask).to(dev), scale, g_bf16)
    # index work: the scatter ids are the cached ids, and the gathered logits
    # are Z at those ids, bit for bit
    np.testing.assert_array_equal(out["sid"].cpu().numpy(), ids)
    zg = out["zg"].cpu().numpy()
    np.testing.assert_array_equal(zg.view(np.uint32), Z[np.arange(R)[:, None], ids].view(np.uint32))
    kl_o, lse_o, _ = O.row_terms(Z, ids, T)
    w = mask * scale
    G_o = O.logit_grad(Z, ids, T, w)
    S_o = np.exp(Z.astype(np.float64) - lse_o[:, None]) * w[:, None]  # dense part w softmax(z)
    G = out["G"].float().cpu().numpy()
    valid = mask == 1
    # masked rows report a log-normaliser of 0
    np.testing.assert_allclose(out["lse"].cpu().numpy()[valid], lse_o[valid], rtol=1e-6)
    assert np.all(out["lse"].cpu().numpy()[~valid] == 0)
    # exact gathered logits and fp32 slice sums: the KL is fp32-accurate in
    # both gradient types
    np.testing.assert_allclose(out["kl"].cpu().numpy()[valid], kl_o[valid], rtol=2e-5, atol=1e-6)
    assert np.all(out["kl"].cpu().numpy()[~valid] == 0)
    assert np.all(G[~valid] == 0)
    if g_bf16:
        # away from the ids: p rounded to bf16, then f p rounded to bf16 (each
        # at most 2^-8 relative); at the ids: the fp32 value w (exp(z - lse) -
        # p_T) rounded once
        assert np.all(np.abs(G - G_o) <= 2.0**-7 * S_o + 2.0**-8 * np.abs(G_o) + 1e-12)
        rows = np.arange(R)[:, None]
        at, at_o = G[rows, ids].astype(np.float64), G_o[rows, ids]
        assert np.all(np.abs(at - at_o) <= 2.0**-8 * np.abs(at_o) + _fp32_slack(S_o[rows, ids], T, w))
    else:
        assert rel_fro(G, G_o) <= 1e-5
    # row sums of the gradient vanish
    assert np.abs(G_o.sum(1)).max() < 1e-15


@pytest.mark.parametrize("g_bf16", [True, False])
def test_row_pass_cached_logit_far_below_its_slice_max(g_bf16):
    """Cached ids whose logit lies 100, 150 and 300 below the largest logit of
    their 128-id slice: exp(z - max) underflows in bf16 and fp32 alike, yet the
    gathered logit, the KL and the gradient at the id are those of the
    definition (p_S there is far below any float, so G at the id is -w p_T)."""
    binding = _need_gpu()
    say(f"[case] row pass far-below-max cached logits g_bf16={g_bf16}")
    rng = np.random.default_rng(31)
    R, V, K = 9, 1000, 12
    Z = rng.standard_normal((R, V)).astype(np.float32)
    ids = np.stack([rng.permutation(V)[:K] for _ in range(R)]).astype(np.int32)
    for r in range(R):
        for k, drop in ((0, 100.0), (3, 150.0), (7, 300.0)):
            v = ids[r, k]
            s0 = (v // 128) * 128
            Z[r, v] = np.float32(Z[r, s0:s0 + 128].max() - drop)
    T = np.sort(rng.standard_normal((R, K)).astype(np.float32) * 2, axis=1)[:, ::-1].copy()
    dev = torch.device("cuda:0")
    out = binding.debug_rows(torch.from_numpy(Z).to(dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(T).to(dev), None, 1.0 / R, g_bf16)
    zg = out["zg"].cpu().numpy()
    np.testing.assert_array_equal(zg.view(np.uint32), Z[np.arange(R)[:, None], ids].view(np.uint32))
    kl_o, lse_o, _ = O.row_terms(Z, ids, T)
    np.testing.assert_allclose(out["kl"].cpu().numpy(), kl_o, rtol=2e-5, atol=1e-6)
    w = np.full(R, 1.0 / R)
    G_o = O.logit_grad(Z, ids, T, w)
    S_o = np.exp(Z.astype(np.float64) - lse_o[:, None]) * w[:, None]
    G = out["G"].float().cpu().numpy().astype(np.float64)
    rows = np.arange(R)[:, None]
    at, at_o = G[rows, ids], G_o[rows, ids]
    tol = 2.0**-8 if g_bf16 else 0.0
    assert np.all(np.abs(at - at_o) <= tol * np.abs(at_o) + _fp32_slack(S_o[rows, ids], T, w))


def test_row_pass_gathers_the_requested_columns():
    """Logits that differ by 0.01 from column to column: the fp32 path's gathered
    value is within 1e-3 of the true logit, so it names its column exactly."""
    binding = _need_gpu()
    say("[case] row pass gather addressing")
    rng = np.random.default_rng(22)
    R, V, K = 19, 3001, 50
    col = np.arange(V, dtype=np.float64)
    Z = np.stack([(rng.permutation(V) - V / 2) * 0.01 for _ in range(R)]).astype(np.float32)
    ids = np.stack([rng.permutation(V)[:K] for _ in range(R)]).astype(np.int32)
    T = rng.standard_normal((R, K)).astype(np.float32)
    dev = torch.device("cuda:0")
    out = binding.debug_rows(torch.from_numpy(Z).to(dev), torch.from_numpy(ids).to(dev),
                             torch.from_numpy(T).to(dev), None, 1.0 / R, False)
    zg = out["zg"].cpu().numpy().astype(np.float64)
    found = np.argmin(np.abs(Z[:, None, :].astype(np.float64) - zg[:, :, None]), axis=2)
    np.testing.assert_array_equal(found, ids)
    assert col.size == V


# ------------------------------------------------------------------ fp32 tiny workload
def test_tiny_fp32_workload_full():
    binding = _need_gpu()
    say("[case] tiny fp32 workload, chunk 64")
    inp = WL.make(1)
    g = run_gpu(binding, inp, "f32", chunk=64)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    check(g, o, "f32", "tiny-fp32")


# ------------------------------------------------------------------ ragged small shapes
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(600, 200, 1003, 37, 256), (1000, 512, 5000, 100, 384), (77, 64, 300, 300, 0)])
def test_small_ragged_shapes(dtype, shape):
    binding = _need_gpu()
    N, d, V, K, chunk = shape
    say(f"[case] ragged {dtype} N={N} d={d} V={V} K={K} chunk={chunk}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5", seed=N + d)
    g = run_gpu(binding, inp, dtype, chunk=chunk, rows=True)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
    check(g, o, dtype, f"ragged {shape}")
    valid = inp["mask"] == 1
    assert np.all(g["dH"][~valid] == 0)
    assert np.all(g["kl"][~valid] == 0)
    tol = 1e-5 if dtype == "f32" else 3e-3
    np.testing.assert_allclose(g["lse"][valid], o["lse"][valid], rtol=tol, atol=tol)
    assert np.all(g["lse"][~valid] == 0)
    assert rel_fro(g["kl"][valid], o["kl"][valid]) <= (1e-5 if dtype == "f32" else 5e-3)


# ------------------------------------------------------------------ vocabulary slice and tile edges
# The logits epilogue keeps a (max, sum) pair per 128-id slice and stores exp
# values per 64 x 64 tile: vocabularies shorter than one slice, one or two ids
# past a slice, and token counts that end one row into a tile or a chunk.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(45, 64, 72, 8, 0), (300, 96, 130, 20, 0), (513, 128, 257, 50, 256),
                                   (129, 32, 383, 383, 0)])
def test_vocabulary_slice_edges(dtype, shape):
    binding = _need_gpu()
    N, d, V, K, chunk = shape
    say(f"[case] slice edges {dtype} N={N} d={d} V={V} K={K} chunk={chunk}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5", seed=7 * N + V)
    g = run_gpu(binding, inp, dtype, chunk=chunk, rows=True)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
    check(g, o, dtype, f"slice edges {shape}")
    valid = inp["mask"] == 1
    tol = 1e-5 if dtype == "f32" else 3e-3
    np.testing.assert_allclose(g["lse"][valid], o["lse"][valid], rtol=tol, atol=tol)
    assert np.all(g["lse"][~valid] == 0)
    assert np.all(g["dH"][~valid] == 0)


# ------------------------------------------------------------------ chunk invariance, determinism
def test_chunk_invariance_and_determinism():
    binding = _need_gpu()
    say("[case] chunk invariance bf16 N=256")
    inp = WL.small(256, 256, 4096, 100, dtype="bf16", ids="zipf", mask="random5", seed=7)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    res = {}
    for c in (64, 96, 128, 256, 0):
        res[c] = run_gpu(binding, inp, "bf16", chunk=c)
        check(res[c], o, "bf16", f"chunk {c}")
    for c in (64, 96, 128, 0):
        # per-row work does not depend on the chunking; the loss sums rows in a fixed order
        assert abs(res[c]["loss"] - res[256]["loss"]) <= 1e-6 * abs(res[256]["loss"])
        assert rel_fro(res[c]["dH"], res[256]["dH"]) <= 1e-5
        assert rel_fro(res[c]["dW"], res[256]["dW"]) <= 1e-5
    again = run_gpu(binding, inp, "bf16", chunk=96)
    assert again["loss"] == res[96]["loss"]
    np.testing.assert_array_equal(again["dH"], res[96]["dH"])
    np.testing.assert_array_equal(again["dW"], res[96]["dW"])


# ------------------------------------------------------------------ degenerate cases
def test_all_masked_gives_zero():
    binding = _need_gpu()
    say("[case] all positions masked")
    inp = WL.small(130, 64, 500, 10, dtype="bf16", seed=3)
    inp["mask"][:] = 0
    g = run_gpu(binding, inp, "bf16", chunk=64)
    assert g["loss"] == 0.0
    assert np.all(g["dH"] == 0) and np.all(g["dW"] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_batch_gives_zero(dtype):
    # N = 0: every loss call writes the oracle's no-valid-position result
    # (loss 0, dW 0) over outputs that held NaN, and reads no row
    binding = _need_gpu()
    say(f"[case] empty batch {dtype}")
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d, V, K = 64, 500, 10
    inp = WL.small(1, d, V, K, dtype=dtype, seed=4)
    W = torch.from_numpy(inp["W"]).to(dev).to(tdt).contiguous()
    H = torch.empty((0, d), dtype=tdt, device=dev)
    ids = torch.empty((0, K), dtype=torch.int32, device=dev)
    T = torch.empty((0, K), dtype=torch.float32, device=dev)
    o = O.kl_dense(inp["H"][:0], inp["W"], inp["ids"][:0], inp["tlogit"][:0], inp["mask"][:0])
    nan = float("nan")
    for noalloc in (False, True):
        loss = torch.full((), nan, dtype=torch.float32, device=dev)
        dW = torch.full((V, d), nan, dtype=torch.float32, device=dev)
        loss, dH, dW = binding.fwd_bwd(H, W, ids, T, None, out_loss=loss, dW=dW, noalloc=noalloc)
        torch.cuda.synchronize()
        assert loss.item() == o["loss"] == 0.0 and dH.shape == (0, d)
        assert np.array_equal(dW.cpu().numpy(), o["dW"])
    loss = torch.full((), nan, dtype=torch.float32, device=dev)
    loss, lse = binding.fwd(H, W, ids, T, torch.empty(0, dtype=torch.uint8, device=dev), out_loss=loss)
    dW = torch.full((V, d), nan, dtype=torch.float32, device=dev)
    dH, dW = binding.bwd(H, W, ids, T, lse, dW=dW)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and lse.shape == (0,) and dH.shape == (0, d)
    assert np.array_equal(dW.cpu().numpy(), o["dW"])
    ids_k, vals_k = binding.topk(torch.empty((0, V), dtype=tdt, device=dev), K)
    assert ids_k.shape == (0, K) and vals_k.shape == (0, K)


def test_teacher_equals_student_full_vocab_fp32():
    binding = _need_gpu()
    say("[case] K = V, teacher = student")
    rng = np.random.default_rng(5)
    N, d, V = 64, 32, 96
    inp = WL.small(N, d, V, V, dtype="f32", seed=9)
    z = inp["H"].astype(np.float64) @ inp["W"].astype(np.float64).T
    ids = np.stack([rng.permutation(V) for _ in range(N)]).astype(np.int32)
    inp["ids"] = ids
    inp["tlogit"] = np.take_along_axis(z, ids, axis=1).astype(np.float32)
    g = run_gpu(binding, inp, "f32", chunk=0)
    assert abs(g["loss"]) <= 1e-5


def test_one_hot_rows_exact_logits():
    binding = _need_gpu()
    say("[case] one-hot H rows, small-integer W")
    rng = np.random.default_rng(8)
    N, d, V, K = 200, 64, 3000, 50
    W = rng.integers(-4, 5, size=(V, d)).astype(np.float32) * 0.25
    cols = rng.integers(0, d, size=N)
    H = np.zeros((N, d), dtype=np.float32)
    H[np.arange(N), cols] = 1.0
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    T = np.sort(rng.standard_normal((N, K)).astype(np.float32) * 3, axis=1)[:, ::-1].copy()
    inp = {"H": H, "W": W, "ids": ids, "tlogit": T, "mask": np.ones(N, dtype=np.uint8)}
    g = run_gpu(binding, inp, "bf16", chunk=64, rows=True)
    o = O.kl_dense(H, W, ids, T, None, want_rows=True)
    # the logits are exact on both sides (one product per sum), so the
    # gathered logits are bit-identical and only the fp32 arithmetic of the
    # row pass (lse from the fp32 slice sums, the KL sum) separates the rows
    np.testing.assert_allclose(g["lse"], o["lse"], rtol=2e-6)
    np.testing.assert_allclose(g["kl"], o["kl"], rtol=2e-5, atol=2e-6)
    check(g, o, "bf16", "one-hot")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cached_logit_far_below_its_slice_max_end_to_end(dtype):
    """One-hot H rows and small-integer W, with some cached ids' weight rows
    at -100 or -160: their logits lie 100+ below the largest logit of their
    128-id slice, where exp(z - max) underflows, and are exact on both sides.
    The KL of every row, the loss and the gradients follow the definition."""
    binding = _need_gpu()
    say(f"[case] end to end, cached logits 100+ below the slice max, {dtype}")
    rng = np.random.default_rng(33)
    N, d, V, K = 150, 32, 1500, 20
    W = rng.integers(-4, 5, size=(V, d)).astype(np.float32) * 0.25
    cols = rng.integers(0, d, size=N)
    H = np.zeros((N, d), dtype=np.float32)
    H[np.arange(N), cols] = 1.0
    ids = np.stack([rng.permutation(V)[:K] for _ in range(N)]).astype(np.int32)
    low = np.unique(ids[:, :3])
    W[low[: len(low) // 2]] = -100.0
    W[low[len(low) // 2:]] = -160.0
    T = np.sort(rng.standard_normal((N, K)).astype(np.float32) * 2, axis=1)[:, ::-1].copy()
    inp = {"H": H, "W": W, "ids": ids, "tlogit": T, "mask": np.ones(N, dtype=np.uint8)}
    g = run_gpu(binding, inp, dtype, chunk=64, rows=True)
    o = O.kl_dense(H, W, ids, T, None, want_rows=True)
    np.testing.assert_allclose(g["lse"], o["lse"], rtol=2e-6)
    np.testing.assert_allclose(g["kl"], o["kl"], rtol=2e-5, atol=2e-6)
    check(g, o, dtype, f"far below slice max {dtype}")


@pytest.mark.parametrize("debug", [False, True])
def test_ids_outside_the_vocabulary_or_repeated_are_left_out_and_flagged(debug):
    """Cached ids outside [0, V) or repeated within a row are outside the
    supported inputs.  No kernel reads or writes at them: every other row's KL
    and dH row are those of the definition.  With CKL_DEBUG=1 the call reports
    them as CKL_EINVAL."""
    binding = _need_gpu()
    say(f"[case] ids out of range / repeated, CKL_DEBUG={int(debug)}")
    N, d, V, K = 200, 64, 1100, 16
    inp = WL.small(N, d, V, K, dtype="f32", seed=41)
    ids = inp["ids"].copy()
    bad = {3: V, 50: -1, 77: 2**31 - 1, 120: None, 199: V + 127}
    for r, v in bad.items():
        ids[r, 5] = ids[r, 2] if v is None else v  # None: a repeat of another cached id
    H, W, idt, T, mask = to_dev(dict(inp, ids=ids), "f32")
    kl = torch.empty(N, dtype=torch.float32, device=H.device)
    old = os.environ.get("CKL_DEBUG")
    os.environ["CKL_DEBUG"] = "1" if debug else "0"
    try:
        if debug:
            with pytest.raises(binding.CklError) as e:
                binding.fwd_bwd(H, W, idt, T, None, chunk=64, row_kl=kl)
            assert e.value.status == -1
        else:
            binding.fwd_bwd(H, W, idt, T, None, chunk=64, row_kl=kl)
    finally:
        if old is None:
            del os.environ["CKL_DEBUG"]
        else:
            os.environ["CKL_DEBUG"] = old
    torch.cuda.synchronize()
    loss, dH, _ = binding.fwd_bwd(H, W, idt, T, None, chunk=64, row_kl=kl)
    torch.cuda.synchronize()
    good = np.array([r not in bad for r in range(N)])
    o = O.kl_rows(inp["H"][good], inp["W"], inp["ids"][good], inp["tlogit"][good], np.full(good.sum(), 1.0 / N))
    np.testing.assert_allclose(kl.cpu().numpy()[good], o["kl"], rtol=2e-5, atol=1e-6)
    assert rel_fro(dH.cpu().numpy()[good], o["dH"]) <= 1e-5
    assert np.all(np.isfinite(dH.cpu().numpy())) and np.isfinite(loss.item())


# ------------------------------------------------------------------ named workloads
def test_bf16_32k_vocab_workload_full():
    binding = _need_gpu()
    say("[case] bf16 32k-vocab workload (N=4096, d=2048, V=32000), chunk 1024")
    inp = WL.make(2)
    g = run_gpu(binding, inp, "bf16", chunk=1024)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], block=1024)
    check(g, o, "bf16", "bf16-32k")


def _sampled_full_size(binding, number, n_sample=48):
    wl = WL.WORKLOADS[number]
    say(f"[case] full-size {wl.name}: generating inputs")
    inp = WL.make(number)
    N = wl.N
    say(f"[case] full-size {wl.name}: GPU call (planner chunk)")
    g = run_gpu(binding, inp, wl.dtype, chunk=wl.chunk, rows=True)
    n_valid = int(inp["mask"].sum())
    rng = np.random.default_rng(1234 + number)
    rows = np.unique(np.concatenate([[0, N - 1], rng.choice(N, n_sample, replace=False)]))
    w = inp["mask"][rows] / n_valid
    say(f"[case] full-size {wl.name}: oracle on {len(rows)} sampled rows")
    o = O.kl_rows(inp["H"][rows], inp["W"], inp["ids"][rows], inp["tlogit"][rows], w)
    valid = inp["mask"][rows] == 1
    e_kl = rel_fro(g["kl"][rows][valid], o["kl"][valid])
    e_dh = rel_fro(g["dH"][rows], o["dH"])
    e_lse = float(np.max(np.abs(g["lse"][rows][valid] - o["lse"][valid])))
    assert np.all(g["lse"][rows][~valid] == 0)
    say(f"[parity {wl.name} sampled] kl {e_kl:.2e} dH rows {e_dh:.2e} lse max abs {e_lse:.2e}")
    assert e_kl <= 2e-3 and e_dh <= 1e-2 and e_lse <= 1e-3
    # the loss is the mean of the per-row KL over valid rows
    mean_kl = float(np.sum(g["kl"].astype(np.float64)) / n_valid)
    assert abs(g["loss"] - mean_kl) <= 1e-5 * abs(mean_kl)
    # dW properties that hold at any size: columns of G sum to zero per row,
    # so the rows of dW sum to zero; and W^T dW = dH^T H (both equal W^T G^T H)
    # (exact for the oracle; for the GPU, 1^T dW = 1^T (dW - dW_oracle), whose
    # norm is about ||dW - dW_oracle||_F when the rounding errors are independent,
    # so the dW tolerance bounds it by 1e-2 ||dW||_F)
    dW = g["dW"].astype(np.float64)
    col = np.linalg.norm(dW.sum(0)) / np.linalg.norm(dW)
    say(f"[parity {wl.name}] ||sum_v dW[v,:]|| / ||dW||_F = {col:.2e}")
    assert col <= 1e-2
    U = rng.standard_normal((wl.d, 4))
    lhs = inp["W"].astype(np.float64).T @ (dW @ U)
    rhs = g["dH"].astype(np.float64).T @ (inp["H"].astype(np.float64) @ U)
    e_id = rel_fro(lhs, rhs)
    say(f"[parity {wl.name}] W^T dW u vs dH^T H u rel {e_id:.2e}")
    assert e_id <= 1e-2
    assert np.all(g["dH"][inp["mask"] == 0] == 0)


def test_llama3_head_workload_full_oracle():
    # 8192 positions (410 masked), d = 3072, V = 128,256: every output against
    # the dense oracle, at 1024-row chunks and at the planner's chunk
    binding = _need_gpu()
    say("[case] llama3 head full size: generating inputs")
    inp = WL.make(3)
    say("[case] llama3 head full size: oracle (8192 positions)")
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], block=1024, want_rows=True)
    valid = inp["mask"] == 1
    for chunk in (1024, 0):
        say(f"[case] llama3 head full size: GPU, chunk {chunk}")
        g = run_gpu(binding, inp, "bf16", chunk=chunk, rows=True)
        check(g, o, "bf16", f"llama3 head full, chunk {chunk}")
        assert rel_fro(g["kl"][valid], o["kl"][valid]) <= 2e-3
        assert np.all(g["dH"][~valid] == 0) and np.all(g["kl"][~valid] == 0)


@pytest.mark.parametrize("number", [4, 5])
def test_gpt_oss_head_4096_row_slice_full_oracle(number):
    # the first 4096 positions at full d = 2880 and V = 201,088: all of dW
    # (the half-full last 256-id tile, the quarter-full last 256-column tile)
    # and dH against the dense oracle, at the planner's chunk and at 1024 rows
    binding = _need_gpu()
    say(f"[case] workload {number}, 4096-row slice: generating inputs")
    inp = WL.make(number, rows=4096)
    say(f"[case] workload {number}, 4096-row slice: oracle")
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], block=512, want_rows=True)
    for chunk in (0, 1024):
        say(f"[case] workload {number}, 4096-row slice: GPU, chunk {chunk}")
        g = run_gpu(binding, inp, "bf16", chunk=chunk, rows=True)
        check(g, o, "bf16", f"workload {number} slice, chunk {chunk}")
        assert rel_fro(g["kl"], o["kl"]) <= 2e-3
        V = inp["W"].shape[0]
        tail = slice(V - 128, V)  # the half-full last tile of 256 ids
        assert rel_fro(g["dW"][tail], o["dW"][tail]) <= 1e-2
        assert rel_fro(g["dW"][:, 2816:], o["dW"][:, 2816:]) <= 1e-2  # the last 64 columns


def test_llama3_head_workload_sampled():
    binding = _need_gpu()
    _sampled_full_size(binding, 3)


def test_gpt_oss_head_workload_sampled():
    binding = _need_gpu()
    _sampled_full_size(binding, 4)


def test_gpt_oss_head_long_batch_workload_sampled():
    binding = _need_gpu()
    _sampled_full_size(binding, 5)


def test_gpt_oss_head_256k_sequence_workload_sampled():
    # one 262,144-token sequence: 32 chunks under the same 6 GiB workspace
    binding = _need_gpu()
    _sampled_full_size(binding, 6)


# ------------------------------------------------------------------ limits of the supported shapes
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    (1, 64, 500, 20, 0),        # one position
    (40, 8, 3000, 2048, 0),     # the largest K, and the smallest d
    (33, 16, 2048, 2048, 16),   # K = V at the largest K: every id of every slice cached
])
def test_shape_limits(shape, dtype):
    binding = _need_gpu()
    N, d, V, K, chunk = shape
    say(f"[case] shape limit {dtype} N={N} d={d} V={V} K={K} chunk={chunk}")
    inp = WL.small(N, d, V, K, dtype=dtype, seed=N * 7 + K)
    g = run_gpu(binding, inp, dtype, chunk=chunk, rows=True)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
    check(g, o, dtype, f"limit {dtype} {shape}")
    # the logits at the cached ids are the contraction's own: the KL per row
    # is fp32-accurate even on the bf16 path
    np.testing.assert_allclose(g["kl"], o["kl"], rtol=2e-5 if dtype == "f32" else 1e-4, atol=1e-5)


def test_single_valid_position():
    binding = _need_gpu()
    say("[case] one valid position among 300")
    inp = WL.small(300, 64, 2000, 30, dtype="bf16", seed=12)
    inp["mask"][:] = 0
    inp["mask"][137] = 1
    g = run_gpu(binding, inp, "bf16", chunk=128)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    check(g, o, "bf16", "one valid position")
    rows = np.arange(300) != 137
    assert np.all(g["dH"][rows] == 0)


# ------------------------------------------------------------------ seeded random sweep
def _sweep_cases(n=14, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 3 == 0 else "bf16"
        K = int(rng.integers(1, 300))
        V = int(rng.integers(max(2 * K, 64), 7000))
        d = 8 * int(rng.integers(1, 49))
        N = int(rng.integers(1, 900))
        chunk = [0, N, 64 * int(rng.integers(1, 9))][int(rng.integers(0, 3))]
        kinds = ["uniform", "overlap50"] + (["zipf"] if K <= V // 4 else [])
        ids = kinds[int(rng.integers(0, len(kinds)))]
        mask = ["none", "random5"][int(rng.integers(0, 2))]
        cases.append((dtype, N, d, V, K, chunk, ids, mask))
    return cases


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "-".join(str(x) for x in c))
def test_seeded_random_shapes(case):
    # shapes, chunk sizes, id distributions and masks drawn from a fixed seed:
    # ragged in every dimension, d from 8 to 384, K from 1 to 299
    binding = _need_gpu()
    dtype, N, d, V, K, chunk, ids, mask = case
    say(f"[case] sweep {case}")
    inp = WL.small(N, d, V, K, dtype=dtype, ids=ids, mask=mask, seed=N * 7 + V)
    g = run_gpu(binding, inp, dtype, chunk=chunk)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    check(g, o, dtype, f"sweep {case}")
    valid = inp["mask"] == 1
    assert np.all(g["dH"][~valid] == 0)


# ------------------------------------------------------------------ masked tails
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_row_chunks(dtype):
    # the finest chunking: 37 chunks of one row (and 13 of three), each a
    # single partial tile in every contraction, with dH split far along V;
    # the per-row results equal the one-chunk call's, and all match the oracle
    binding = _need_gpu()
    N, d, V, K = 37, 96, 1500, 20
    say(f"[case] one-row chunks {dtype}")
    inp = WL.small(N, d, V, K, dtype=dtype, ids="zipf", mask="random5", seed=41)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
    res = {c: run_gpu(binding, inp, dtype, chunk=c, rows=True) for c in (1, 3, N)}
    for c, g in res.items():
        check(g, o, dtype, f"chunk {c}")
        # KL and log-normaliser per row do not depend on the chunking
        assert np.array_equal(g["kl"], res[N]["kl"]) and np.array_equal(g["lse"], res[N]["lse"])
        assert abs(g["loss"] - res[N]["loss"]) <= 1e-6 * abs(res[N]["loss"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_chunk_tails_are_skipped_and_exact(dtype):
    # right-padded sequences: the rows after each chunk's last valid row are
    # skipped by every kernel (whole logits and dH tiles, dW k-steps); one
    # chunk is all padding and one has no padding.  Results must still match
    # the oracle, masked dH rows are +0, masked rows report KL 0 and lse 0.
    binding = _need_gpu()
    N, d, V, K, chunk = 1536, 192, 3000, 40, 512
    say(f"[case] masked chunk tails {dtype}")
    inp = WL.small(N, d, V, K, dtype=dtype, ids="uniform", seed=99)
    m = np.ones(N, dtype=np.uint8)
    m[512 - 300:512] = 0      # chunk 0: valid rows 0..211, then 300 padded (a whole 256-row tile)
    m[512:1024] = 0           # chunk 1: all padding
    m[1024 + 7] = 0           # chunk 2: one masked row inside, valid to the end
    inp["mask"] = m
    for c in (chunk, 256, 0):
        g = run_gpu(binding, inp, dtype, chunk=c, rows=True)
        o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
        check(g, o, dtype, f"masked tails chunk {c}")
        valid = m == 1
        assert np.all(g["dH"][~valid] == 0) and not np.any(np.signbit(g["dH"][~valid]))
        assert np.all(g["kl"][~valid] == 0) and np.all(g["lse"][~valid] == 0)
        tol = 1e-5 if dtype == "f32" else 3e-3
        np.testing.assert_allclose(g["lse"][valid], o["lse"][valid], rtol=tol, atol=tol)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_heavily_masked_chunks_compact_exactly(dtype):
    # half the positions masked at random, and chunks whose only valid rows
    # sit at their very end: the compacted rows come from anywhere in the
    # chunk, and the compacted row count is far below the chunk's rows
    binding = _need_gpu()
    N, d, V, K = 1100, 136, 2500, 33
    say(f"[case] heavily masked chunks {dtype}")
    inp = WL.small(N, d, V, K, dtype=dtype, ids="uniform", seed=123)
    rng = np.random.default_rng(5)
    m = (rng.random(N) < 0.5).astype(np.uint8)
    m[300:600] = 0
    m[590:600] = 1      # chunk 300..599 (with chunk 300): only its last 10 rows are valid
    inp["mask"] = m
    for c in (300, 128, 0):
        g = run_gpu(binding, inp, dtype, chunk=c, rows=True)
        o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
        check(g, o, dtype, f"heavily masked chunk {c}")
        valid = m == 1
        assert np.all(g["dH"][~valid] == 0) and np.all(g["kl"][~valid] == 0) and np.all(g["lse"][~valid] == 0)
        tol = 1e-5 if dtype == "f32" else 3e-3
        np.testing.assert_allclose(g["lse"][valid], o["lse"][valid], rtol=tol, atol=tol)


def test_workspace_allocation_failure_returns_enomem_and_leaves_outputs():
    # CKL_TEST_FAIL_ALLOC=1 makes the workspace allocation fail: the call
    # returns CKL_ENOMEM before enqueuing anything, so the outputs keep their
    # contents, and a later call without it works
    binding = _need_gpu()
    say("[case] workspace allocation failure")
    inp = WL.small(300, 64, 2000, 20, dtype="bf16", mask="random5", seed=2)
    H, W, ids, T, mask = to_dev(inp, "bf16")
    loss = torch.full((), 7.0, dtype=torch.float32, device=H.device)
    dH = torch.full_like(H, 3.0)
    dW = torch.full((W.shape[0], W.shape[1]), 5.0, dtype=torch.float32, device=H.device)
    lse = torch.full((H.shape[0],), 9.0, dtype=torch.float32, device=H.device)
    binding.release_workspace()  # the cache is empty: the next call must allocate
    assert binding.workspace_bytes_held() == 0
    os.environ["CKL_TEST_FAIL_ALLOC"] = "1"
    try:
        with pytest.raises(binding.CklError) as e:
            binding.fwd_bwd(H, W, ids, T, mask, chunk=128, out_loss=loss, dH=dH, dW=dW)
        assert e.value.status == -2
        with pytest.raises(binding.CklError) as e:
            binding.fwd(H, W, ids, T, mask, chunk=128, out_loss=loss, row_lse=lse)
        assert e.value.status == -2
    finally:
        del os.environ["CKL_TEST_FAIL_ALLOC"]
    torch.cuda.synchronize()
    assert loss.item() == 7.0 and torch.all(dH == 3.0) and torch.all(dW == 5.0) and torch.all(lse == 9.0)
    assert binding.workspace_bytes_held() == 0
    g = run_gpu(binding, inp, "bf16", chunk=128)
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    check(g, o, "bf16", "after a failed allocation")


def test_trace_ranges_leave_results_unchanged():
    # CKL_TRACE=1 wraps every call and chunk in roctx ranges (host side only):
    # the results are bitwise those of an untraced call
    binding = _need_gpu()
    say("[case] CKL_TRACE=1")
    inp = WL.small(500, 128, 3000, 40, dtype="bf16", mask="random5", seed=44)
    base = run_gpu(binding, inp, "bf16", chunk=128)
    os.environ["CKL_TRACE"] = "1"
    try:
        traced = run_gpu(binding, inp, "bf16", chunk=128)
    finally:
        del os.environ["CKL_TRACE"]
    assert traced["loss"] == base["loss"]
    np.testing.assert_array_equal(traced["dH"], base["dH"])
    np.testing.assert_array_equal(traced["dW"], base["dW"])
