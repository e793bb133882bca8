"""The forward / recomputing-backward pair (ckl_fwd, ckl_bwd) through the C ABI.

Two kinds of check:
  * against the fused call on the same inputs and chunk: the loss, the
    per-position log-normaliser and KL, dH and dW must be bitwise equal (the
    backward recomputes the same logits with the same kernels and reads the
    forward's log-normaliser instead of merging it again);
  * against the CPU oracle, with an upstream gradient other than 1, to the
    tolerances of the fused path (fp32: 1e-5; bf16: loss 2e-3, dH and dW 1e-2
    relative Frobenius).
"""
import sys

import numpy as np
import pytest

from chunked_kl_loss_seq_amd import workloads as WL
from oracle import kl_oracle as O

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


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def to_dev(inp, dtype):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return (torch.from_numpy(inp["H"]).to(dev).to(tdt).contiguous(),
            torch.from_numpy(inp["W"]).to(dev).to(tdt).contiguous(),
            torch.from_numpy(inp["ids"]).to(dev).contiguous(),
            torch.from_numpy(inp["tlogit"]).to(dev).contiguous(),
            torch.from_numpy(inp["mask"]).to(dev).contiguous())


def fused_and_two_pass(binding, inp, dtype, chunk, fwd_chunk=None, masked=True):
    H, W, ids, T, mask = to_dev(inp, dtype)
    if not masked:
        mask = None
    N = H.shape[0]
    kl_f = torch.empty(N, dtype=torch.float32, device=H.device)
    lse_f = torch.empty_like(kl_f)
    loss_f, dH_f, dW_f = binding.fwd_bwd(H, W, ids, T, mask, chunk=chunk, row_kl=kl_f, row_lse=lse_f)
    kl_1 = torch.empty_like(kl_f)
    loss_1, lse_1 = binding.fwd(H, W, ids, T, mask, chunk=chunk if fwd_chunk is None else fwd_chunk, row_kl=kl_1)
    dH_2, dW_2 = binding.bwd(H, W, ids, T, lse_1, mask, chunk=chunk)
    torch.cuda.synchronize()
    return (loss_f, dH_f, dW_f, kl_f, lse_f), (loss_1, lse_1, kl_1), (dH_2, dW_2)


def assert_bitwise(fused, fwd, bwd):
    loss_f, dH_f, dW_f, kl_f, lse_f = fused
    loss_1, lse_1, kl_1 = fwd
    dH_2, dW_2 = bwd
    assert torch.equal(loss_1, loss_f), (loss_1.item(), loss_f.item())
    assert torch.equal(lse_1, lse_f)
    assert torch.equal(kl_1, kl_f)
    assert torch.equal(dH_2, dH_f)
    assert torch.equal(dW_2, dW_f)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(600, 200, 1003, 37, 256), (1000, 512, 5000, 100, 384)])
def test_two_pass_bitwise_equals_fused(dtype, shape):
    binding = _need_gpu()
    N, d, V, K, chunk = shape
    say(f"[case] two-pass vs fused {dtype} N={N} d={d} V={V} K={K} chunk={chunk}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5", seed=3 * N + d)
    assert_bitwise(*fused_and_two_pass(binding, inp, dtype, chunk))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_pass_bitwise_equals_fused_without_mask(dtype):
    # every row counts: the chunks are not compacted, so the backward's
    # gradient epilogue indexes the saved log-normaliser by chunk row directly
    binding = _need_gpu()
    N, d, V, K, chunk = 700, 256, 2111, 64, 320
    say(f"[case] two-pass vs fused, no mask, {dtype} N={N} d={d} V={V} K={K} chunk={chunk}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5", seed=23)
    assert_bitwise(*fused_and_two_pass(binding, inp, dtype, chunk, masked=False))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_pass_unit_upstream_gradient_is_bitwise_neutral(dtype):
    # w = (1 / n_valid) x 1.0 is the same fp32 number as 1 / n_valid, so an
    # upstream gradient of exactly 1 read from the device changes no bit
    binding = _need_gpu()
    N, d, V, K, chunk = 500, 192, 1500, 40, 256
    say(f"[case] two-pass grad_loss = 1 vs none {dtype} N={N} d={d} V={V} K={K}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5", seed=29)
    H, W, ids, T, mask = to_dev(inp, dtype)
    _, lse = binding.fwd(H, W, ids, T, mask, chunk=chunk)
    dH_a, dW_a = binding.bwd(H, W, ids, T, lse, mask, chunk=chunk)
    one = torch.ones((), dtype=torch.float32, device=H.device)
    dH_b, dW_b = binding.bwd(H, W, ids, T, lse, mask, grad_loss=one, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(dH_a, dH_b) and torch.equal(dW_a, dW_b)


def _random_cases(n_cases, seed):
    rng = np.random.default_rng(seed)
    cases = [(1, 8, 1, 1, 0, "f32", "none"), (1, 64, 300, 7, 0, "bf16", "random5"),
             (257, 8, 129, 129, 64, "bf16", "none")]
    while len(cases) < n_cases:
        N = int(rng.integers(1, 900))
        d = 8 * int(rng.integers(1, 65))
        V = int(rng.integers(1, 5000))
        K = int(rng.integers(1, min(V, 160) + 1))
        chunk = 0 if rng.random() < 0.4 else int(rng.integers(1, N + 64))
        dtype = "bf16" if rng.random() < 0.6 else "f32"
        mask = "random5" if rng.random() < 0.5 else "none"
        cases.append((N, d, V, K, chunk, dtype, mask))
    return cases


@pytest.mark.parametrize("case", _random_cases(16, 2024), ids=lambda c: "x".join(map(str, c)))
def test_two_pass_bitwise_equals_fused_random_shapes(case):
    # seeded random small shapes and edge sizes (one row, one id, V below one
    # slice, K past a 64-id lane group), both element types, with and without
    # a mask, at the planner's chunk (the forward then plans its own) or a
    # given one
    binding = _need_gpu()
    N, d, V, K, chunk, dtype, mask = case
    say(f"[case] two-pass vs fused random shape N={N} d={d} V={V} K={K} chunk={chunk} {dtype} mask={mask}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5" if mask != "none" else "none", seed=N * 7 + V)
    assert_bitwise(*fused_and_two_pass(binding, inp, dtype, chunk, fwd_chunk=0 if chunk == 0 else None,
                                       masked=mask != "none"))


def test_forward_is_chunk_invariant_bitwise():
    # per-row logits, their slice statistics and the loss's fixed-order sum do
    # not depend on the chunking, so a forward with other chunks gives the
    # fused call's loss, KL and log-normaliser bit for bit
    binding = _need_gpu()
    say("[case] forward chunk invariance bf16 N=1000")
    inp = WL.small(1000, 256, 4096, 100, dtype="bf16", ids="zipf", mask="random5", seed=11)
    fused, fwd, bwd = fused_and_two_pass(binding, inp, "bf16", chunk=256, fwd_chunk=384)
    loss_f, _, _, kl_f, lse_f = fused
    loss_1, lse_1, kl_1 = fwd
    assert torch.equal(lse_1, lse_f) and torch.equal(kl_1, kl_f) and torch.equal(loss_1, loss_f)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_two_pass_with_upstream_gradient_matches_oracle(dtype):
    binding = _need_gpu()
    N, d, V, K = 700, 128, 3001, 64
    g = 2.5
    say(f"[case] two-pass with grad_loss={g} {dtype} N={N} d={d} V={V} K={K}")
    inp = WL.small(N, d, V, K, dtype=dtype, mask="random5", seed=17)
    H, W, ids, T, mask = to_dev(inp, dtype)
    loss, lse = binding.fwd(H, W, ids, T, mask, chunk=256)
    gl = torch.tensor(g, dtype=torch.float32, device=H.device)
    dH, dW = binding.bwd(H, W, ids, T, lse, mask, grad_loss=gl, chunk=256)
    torch.cuda.synchronize()
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"], want_rows=True)
    tl, tg = (1e-5, 1e-5) if dtype == "f32" else (2e-3, 1e-2)
    el = abs(loss.item() - o["loss"]) / abs(o["loss"])
    eh = rel_fro(dH.float().cpu().numpy(), g * o["dH"])
    ew = rel_fro(dW.cpu().numpy(), g * o["dW"])
    say(f"[parity two-pass {dtype}] loss rel {el:.2e}; dH {eh:.2e}; dW {ew:.2e}")
    assert el <= tl and eh <= tg and ew <= tg
    tol = 1e-5 if dtype == "f32" else 3e-3
    valid = inp["mask"] == 1
    np.testing.assert_allclose(lse.cpu().numpy()[valid], o["lse"][valid], rtol=tol, atol=tol)
    assert np.all(lse.cpu().numpy()[~valid] == 0)  # masked rows report 0
    assert np.all(dH.float().cpu().numpy()[~valid] == 0)


def test_two_pass_all_masked_and_zero_upstream_gradient():
    binding = _need_gpu()
    say("[case] two-pass degenerate: all masked; zero upstream gradient")
    inp = WL.small(130, 64, 500, 10, dtype="bf16", seed=3)
    H, W, ids, T, mask = to_dev(inp, "bf16")
    zero = torch.zeros_like(mask)
    loss, lse = binding.fwd(H, W, ids, T, zero, chunk=64)
    dH, dW = binding.bwd(H, W, ids, T, lse, zero, chunk=64)
    torch.cuda.synchronize()
    assert loss.item() == 0.0
    assert torch.count_nonzero(dH).item() == 0 and torch.count_nonzero(dW).item() == 0
    loss, lse = binding.fwd(H, W, ids, T, mask, chunk=64)
    dH, dW = binding.bwd(H, W, ids, T, lse, mask, grad_loss=torch.zeros((), device=H.device), chunk=64)
    torch.cuda.synchronize()
    assert loss.item() > 0
    assert torch.count_nonzero(dH).item() == 0 and torch.count_nonzero(dW).item() == 0


def test_autograd_wrappers_agree():
    binding = _need_gpu()
    say("[case] autograd: recompute_kl vs fused_kl, upstream gradient 3")
    inp = WL.small(300, 128, 2000, 50, dtype="f32", mask="random5", seed=5)
    grads = {}
    for name, fn in (("fused", binding.fused_kl), ("recompute", binding.recompute_kl)):
        H, W, ids, T, mask = to_dev(inp, "f32")
        H.requires_grad_(True)
        W.requires_grad_(True)
        loss = fn(H, W, ids, T, mask, 128)
        (3.0 * loss).backward()
        torch.cuda.synchronize()
        grads[name] = (loss.item(), H.grad.cpu().numpy(), W.grad.cpu().numpy())
    assert grads["fused"][0] == grads["recompute"][0]
    # the fused wrapper scales its stored gradients by 3 after the GEMMs, the
    # recomputing backward folds 3 into the gradient weight before them: the
    # two differ by fp32 rounding only, bounded by the fp32 tolerance
    assert rel_fro(grads["recompute"][1], grads["fused"][1]) <= 1e-5
    assert rel_fro(grads["recompute"][2], grads["fused"][2]) <= 1e-5
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
    assert rel_fro(grads["recompute"][1], 3.0 * o["dH"]) <= 1e-5
    assert rel_fro(grads["recompute"][2], 3.0 * o["dW"]) <= 1e-5


def test_two_pass_llama3_head_workload_bitwise():
    # full size (N = 8192, d = 3072, V = 128,256, 5 % masked) in the fused
    # path's chunking; the fused path's own parity with the oracle is tested
    # on the same workload in the fused parity tests
    binding = _need_gpu()
    wl = WL.WORKLOADS[3]
    say(f"[case] two-pass vs fused, full-size {wl.name}: generating inputs")
    inp = WL.make(3)
    say(f"[case] two-pass vs fused, full-size {wl.name}: GPU calls, chunk {wl.chunk}")
    assert_bitwise(*fused_and_two_pass(binding, inp, "bf16", chunk=wl.chunk))


def test_two_pass_gpt_oss_head_planner_chunks_bitwise():
    # N = 32,768, d = 2880, V = 201,088 with every call at its own planner
    # chunk: the forward alone keeps neither exp values nor dH slabs and takes
    # the whole sequence as one chunk (32,768 x 1,571 slice pairs, id tables
    # of 0.9 GB), the backward the fused call's 8192-row chunks.  The
    # forward's outputs are chunk-invariant, so all must be bitwise equal.
    binding = _need_gpu()
    wl = WL.WORKLOADS[4]
    c_fused, _ = binding.plan(wl.N, wl.d, wl.V, wl.K)
    c_fwd, ws_fwd = binding.plan(wl.N, wl.d, wl.V, wl.K, pass_="fwd")
    c_bwd, _ = binding.plan(wl.N, wl.d, wl.V, wl.K, pass_="bwd")
    assert c_fwd == wl.N and c_fused == c_bwd < wl.N
    say(f"[case] two-pass vs fused, full-size {wl.name}: fwd chunk {c_fwd} ({ws_fwd / 2**30:.2f} GiB), "
        f"fused/bwd chunk {c_fused}; generating inputs")
    inp = WL.make(4)
    say(f"[case] two-pass vs fused, full-size {wl.name}: GPU calls")
    assert_bitwise(*fused_and_two_pass(binding, inp, "bf16", chunk=0, fwd_chunk=0))


def test_forward_on_the_256k_sequence_at_its_planner_chunk_bitwise():
    # N = 262,144: the forward alone plans 87,552-row chunks, whose cached-id
    # masks (786 vocabulary pairs x 87,552 rows x 32 B) pass 2 GiB; its loss,
    # log-normalisers and KL must still be bitwise the fused call's
    binding = _need_gpu()
    wl = WL.WORKLOADS[6]
    c_fused, _ = binding.plan(wl.N, wl.d, wl.V, wl.K)
    c_fwd, ws_fwd = binding.plan(wl.N, wl.d, wl.V, wl.K, pass_="fwd")
    pairs = -(-wl.V // 256)
    assert pairs * (-(-c_fwd // 256) * 256) * 32 > 2**31 and c_fwd > c_fused
    say(f"[case] forward at its planner chunk, {wl.name}: fwd chunk {c_fwd} ({ws_fwd / 2**30:.2f} GiB), "
        f"fused chunk {c_fused}; generating inputs")
    inp = WL.make(6)
    H, W, ids, T, mask = to_dev(inp, "bf16")
    kl_f = torch.empty(wl.N, dtype=torch.float32, device=H.device)
    lse_f = torch.empty_like(kl_f)
    say(f"[case] forward at its planner chunk, {wl.name}: fused call")
    loss_f, dH, dW = binding.fwd_bwd(H, W, ids, T, mask, row_kl=kl_f, row_lse=lse_f)
    del dH, dW
    kl_1 = torch.empty_like(kl_f)
    say(f"[case] forward at its planner chunk, {wl.name}: forward call")
    loss_1, lse_1 = binding.fwd(H, W, ids, T, mask, row_kl=kl_1)
    torch.cuda.synchronize()
    assert torch.equal(loss_1, loss_f), (loss_1.item(), loss_f.item())
    assert torch.equal(lse_1, lse_f) and torch.equal(kl_1, kl_f)


def test_fused_wrapper_scales_in_place_and_refuses_a_second_backward():
    # the fused wrapper's gradients were computed in the forward call; its
    # backward scales them in place by the upstream gradient, once
    binding = _need_gpu()
    say("[case] autograd: fused_kl backward twice")
    inp = WL.small(200, 64, 1500, 30, dtype="f32", seed=6)
    H, W, ids, T, _ = to_dev(inp, "f32")
    H.requires_grad_(True)
    W.requires_grad_(True)
    loss = binding.fused_kl(H, W, ids, T, None, 64)
    (2.0 * loss).backward(retain_graph=True)
    torch.cuda.synchronize()
    o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], None)
    assert rel_fro(H.grad.cpu().numpy(), 2.0 * o["dH"]) <= 1e-5
    assert rel_fro(W.grad.cpu().numpy(), 2.0 * o["dW"]) <= 1e-5
    with pytest.raises(RuntimeError, match="second backward"):
        loss.backward()
