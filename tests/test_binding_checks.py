"""Host-side argument checks of the Python binding (no GPU needed): every shape
the kernels index by must agree, or the call raises before reaching the library."""
import pytest

torch = pytest.importorskip("torch")

from chunked_kl_loss_seq_amd import binding as B  # noqa: E402


def inputs(N=4, d=8, V=10, K=3, dtype=torch.bfloat16):
    return (torch.zeros(N, d, dtype=dtype), torch.zeros(V, d, dtype=dtype),
            torch.zeros(N, K, dtype=torch.int32), torch.zeros(N, K, dtype=torch.float32))


def check(*a, mask=None):
    return B._check_inputs(torch, *a, "test", mask, need_gpu=False)


def test_consistent_inputs_pass():
    assert check(*inputs()) == B.DTYPE_BF16
    assert check(*inputs(dtype=torch.float32), mask=torch.ones(4, dtype=torch.uint8)) == B.DTYPE_F32


@pytest.mark.parametrize("bad", ["W_d", "ids_rows", "tlogit_K", "mask_len", "dtypes", "ids_dtype", "noncontig"])
def test_inconsistent_inputs_raise(bad):
    H, W, ids, T = inputs()
    mask = None
    if bad == "W_d":
        W = torch.zeros(10, 16, dtype=torch.bfloat16)
    elif bad == "ids_rows":
        ids = torch.zeros(5, 3, dtype=torch.int32)
    elif bad == "tlogit_K":
        T = torch.zeros(4, 4)
    elif bad == "mask_len":
        mask = torch.ones(5, dtype=torch.uint8)
    elif bad == "dtypes":
        W = W.float()
    elif bad == "ids_dtype":
        ids = ids.long()
    elif bad == "noncontig":
        H = torch.zeros(8, 4, dtype=torch.bfloat16).t()
    with pytest.raises(ValueError):
        check(H, W, ids, T, mask=mask)


def test_output_tensor_checks():
    B._check_out(torch, None, (4, 8), torch.float32, torch.device("cpu"), "x")
    B._check_out(torch, torch.zeros(4, 8), (4, 8), torch.float32, torch.device("cpu"), "x")
    for t in (torch.zeros(4, 9), torch.zeros(4, 8, dtype=torch.float64), torch.zeros(8, 4).t()):
        with pytest.raises(ValueError):
            B._check_out(torch, t, (4, 8), torch.float32, torch.device("cpu"), "x")


def test_gpu_calls_refuse_cpu_tensors():
    H, W, ids, T = inputs()
    with pytest.raises(ValueError):
        B.fwd_bwd(H, W, ids, T)
    with pytest.raises(ValueError):
        B.fwd(H, W, ids, T)
    with pytest.raises(ValueError):
        B.topk(torch.zeros(4, 10, dtype=torch.bfloat16), 3)
