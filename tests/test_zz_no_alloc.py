"""ckl_fwd_bwd_noalloc: the fused call in the library's fixed device array.

Two calls in a row, the second on a smaller input, each checked bit for bit
against ckl_fwd_bwd_ex on the same inputs and chunk (they share every kernel;
only the workspace differs), and against the CPU oracle to the path's
tolerances (fp32: 1e-5; bf16: loss 2e-3, dH and dW 1e-2 relative Frobenius).
"""
import sys

import numpy as np
import pytest

from chunked_kl_loss_seq_amd import workloads as WL
from oracle import kl_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def _both(binding, inp, dtype, chunk):
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H = torch.from_numpy(inp["H"]).to(dev).to(tdt).contiguous()
    W = torch.from_numpy(inp["W"]).to(dev).to(tdt).contiguous()
    ids = torch.from_numpy(inp["ids"]).to(dev).contiguous()
    T = torch.from_numpy(inp["tlogit"]).to(dev).contiguous()
    mask = torch.from_numpy(inp["mask"]).to(dev).contiguous()
    N = H.shape[0]
    out = []
    for noalloc in (True, False):
        kl = torch.empty(N, dtype=torch.float32, device=dev)
        lse = torch.empty(N, dtype=torch.float32, device=dev)
        loss, dH, dW = binding.fwd_bwd(H, W, ids, T, mask, chunk=chunk, row_kl=kl, row_lse=lse, noalloc=noalloc)
        out.append((loss, dH, dW, kl, lse))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_fused_call_twice_second_smaller(dtype):
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required")
    from chunked_kl_loss_seq_amd import binding

    binding.lib()
    cases = [((1000, 512, 5000, 100), 384, 11), ((300, 128, 2000, 50), 0, 12)]
    for (N, d, V, K), chunk, seed in cases:
        say(f"[case] noalloc {dtype} N={N} d={d} V={V} K={K} chunk={chunk}")
        inp = WL.small(N, d, V, K, dtype=dtype, ids="zipf", mask="random5", seed=seed)
        (a, b) = _both(binding, inp, dtype, chunk)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        o = O.kl_dense(inp["H"], inp["W"], inp["ids"], inp["tlogit"], inp["mask"])
        tl, tg = (1e-5, 1e-5) if dtype == "f32" else (2e-3, 1e-2)
        loss = float(a[0].item())
        el = abs(loss - o["loss"]) / abs(o["loss"])
        eh = rel_fro(a[1].float().cpu().numpy(), o["dH"])
        ew = rel_fro(a[2].cpu().numpy(), o["dW"])
        say(f"[noalloc {dtype} N={N}] loss rel {el:.2e} dH {eh:.2e} dW {ew:.2e}")
        assert el <= tl and eh <= tg and ew <= tg
