"""The top-K cache writer (ckl_topk) through the C ABI, against the CPU oracle.

Index work is compared bit for bit: the ids and their order are unique (value
descending, equal values by id ascending), and the values are the inputs'
own, so they must match exactly too.
"""
import sys

import numpy as np
import pytest

from chunked_kl_loss_seq_amd import workloads as WL
from oracle import topk_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for these tests")
    from chunked_kl_loss_seq_amd import binding

    binding.lib()  # raises if libckl.so is missing
    return binding


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run(binding, x, K, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()
    ids, vals = binding.topk(t, K)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), vals.cpu().numpy()


def check_exact(binding, x, K, dtype, what):
    ids, vals = run(binding, x, K, dtype)
    oi, ov = topk_rows(x, K)
    bad = int(np.sum(np.any(ids != oi, axis=1)))
    say(f"[topk {what}] rows {x.shape[0]} V {x.shape[1]} K {K}: rows differing {bad}")
    np.testing.assert_array_equal(ids, oi)
    np.testing.assert_array_equal(vals.view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(300, 50000, 100), (64, 1003, 37), (200, 77, 1), (40, 300, 300), (16, 5000, 1000)])
def test_random_rows_match_oracle(dtype, shape):
    # (40, 300, 300): K = V; (16, 5000, 1000): K above the thread count, exact path
    binding = _need_gpu()
    N, V, K = shape
    x = WL.teacher_logits(N, V, seed=N + V, bf16=dtype == "bf16")
    check_exact(binding, x, K, dtype, f"{dtype} random")


def test_tie_heavy_rows_take_both_paths():
    binding = _need_gpu()
    rng = np.random.default_rng(7)
    N, V, K = 24, 60000, 100
    # few distinct values: the largest one is held by about 6,000 ids (more
    # than the candidate store holds, so the exact path runs) ...
    x = rng.integers(0, 10, size=(N, V)).astype(np.float32)
    # ... and rows where only a few hundred ids reach the threshold (fast path)
    x[N // 2:] = rng.integers(0, 200, size=(N - N // 2, V)).astype(np.float32)
    check_exact(binding, x, K, "bf16", "ties")
    check_exact(binding, x, K, "f32", "ties")


def test_all_equal_signed_zeros_and_infinities():
    binding = _need_gpu()
    x = np.full((3, 9000), 1.5, dtype=np.float32)
    x[1] = 0.0
    x[1, ::3] = -0.0
    x[2] = -np.inf
    x[2, 4000] = np.inf
    x[2, 17] = -0.0
    x[2, 8999] = 0.0
    for dtype in ("bf16", "f32"):
        check_exact(binding, x, 50, dtype, f"{dtype} degenerate")
        ids, _ = run(binding, x, 50, dtype)
        assert ids[0].tolist() == list(range(50))
        assert ids[1].tolist() == list(range(50))  # -0 equals +0: id order
        assert ids[2, :3].tolist() == [4000, 17, 8999]


def test_full_vocabulary_rows():
    # V = 201,088 (the gpt-oss vocabulary), K = 100, 8192 rows of N(0, 3) bf16
    # logits: 256 sampled rows exactly against the oracle, and on every row
    # the properties that pin a top-K selection
    binding = _need_gpu()
    N, V, K = 8192, 201088, 100
    say(f"[case] top-K full vocabulary: generating {N} x {V} bf16 logits")
    x = WL.teacher_logits(N, V, seed=1)
    say("[case] top-K full vocabulary: GPU")
    ids, vals = run(binding, x, K, "bf16")
    rows = np.random.default_rng(11).choice(N, 256, replace=False)
    say("[case] top-K full vocabulary: oracle on 256 rows")
    oi, ov = topk_rows(x[rows], K)
    np.testing.assert_array_equal(ids[rows], oi)
    np.testing.assert_array_equal(vals[rows], ov)
    say("[case] top-K full vocabulary: properties of all rows")
    np.testing.assert_array_equal(vals, np.take_along_axis(x, ids.astype(np.int64), axis=1))
    assert np.all(np.diff(vals, axis=1) <= 0)
    s = np.sort(ids, axis=1)
    assert np.all(np.diff(s, axis=1) > 0) and s.min() >= 0 and s.max() < V
    kth = vals[:, -1:]
    assert np.all((x > kth).sum(axis=1) < K) and np.all((x >= kth).sum(axis=1) >= K)


@pytest.mark.parametrize("dtype,V", [("bf16", 262144), ("bf16", 262152), ("bf16", 300000), ("f32", 262144),
                                     ("f32", 262148)])
def test_long_rows_around_the_kept_maxima_limit(dtype, V):
    # the first pass keeps, per thread, the maximum of every 16-byte chunk of a
    # bf16 row (up to 262,144 elements) or of every 8 chunks of an fp32 row (up
    # to 262,144 elements); longer rows are scanned again whole
    binding = _need_gpu()
    x = WL.teacher_logits(6, V, seed=V, bf16=dtype == "bf16")
    check_exact(binding, x, 100, dtype, f"{dtype} V={V}")
