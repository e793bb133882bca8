"""Thin ctypes binding of libckl.so (argument marshalling only).

Every step of the loss runs in the library's HIP kernels; PyTorch only
supplies device memory and the current stream.  There is no fallback: if the
library is missing, or the tensors are not on a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libckl.so")

CKL_OK = 0
DTYPE_BF16 = 0
DTYPE_F32 = 1
PASSES = {"fused": 0, "fwd": 1, "bwd": 2}
TIMING_KINDS = {"logits": 0, "rows": 1, "dh": 2, "dh_reduce": 3, "dw": 4, "other": 5, "topk": 6}

_lib = None


class CklError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} ({status})")


def lib():
    """Load libckl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m chunked_kl_loss_seq_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i64, u64, vp, f32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_float
    L.ckl_fwd_bwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp]
    L.ckl_fwd_bwd.restype = ctypes.c_int
    L.ckl_fwd_bwd_f32.argtypes = L.ckl_fwd_bwd.argtypes
    L.ckl_fwd_bwd_f32.restype = ctypes.c_int
    L.ckl_fwd_bwd_ex.argtypes = [ctypes.c_int] + L.ckl_fwd_bwd.argtypes[:-1] + [vp, vp, vp]
    L.ckl_fwd_bwd_ex.restype = ctypes.c_int
    L.ckl_fwd_bwd_noalloc.argtypes = L.ckl_fwd_bwd_ex.argtypes
    L.ckl_fwd_bwd_noalloc.restype = ctypes.c_int
    L.ckl_plan.argtypes = [i64, i64, i64, i64, ctypes.c_int, u64, ctypes.POINTER(i64), ctypes.POINTER(u64)]
    L.ckl_plan.restype = ctypes.c_int
    L.ckl_plan_pass.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int, i64, u64, ctypes.POINTER(i64),
                                ctypes.POINTER(u64)]
    L.ckl_plan_pass.restype = ctypes.c_int
    L.ckl_fwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp, vp]
    L.ckl_fwd.restype = ctypes.c_int
    L.ckl_bwd.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp]
    L.ckl_bwd.restype = ctypes.c_int
    L.ckl_topk.argtypes = [ctypes.c_int, vp, i64, i64, i64, vp, vp, vp]
    L.ckl_topk.restype = ctypes.c_int
    L.ckl_release_workspace.argtypes = []
    L.ckl_release_workspace.restype = None
    L.ckl_workspace_bytes_held.argtypes = []
    L.ckl_workspace_bytes_held.restype = u64
    L.ckl_strerror.argtypes = [ctypes.c_int]
    L.ckl_strerror.restype = ctypes.c_char_p
    L.ckl_debug_rows.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, ctypes.c_int, vp, vp, vp, vp, vp, vp]
    L.ckl_debug_rows.restype = ctypes.c_int
    L.ckl_timing_enable.argtypes = [ctypes.c_int]
    L.ckl_timing_enable.restype = ctypes.c_int
    L.ckl_timing_query.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.ckl_timing_query.restype = ctypes.c_int
    _lib = L
    return L


def strerror(status):
    return lib().ckl_strerror(int(status)).decode()


def _check(st, what):
    if st != CKL_OK:
        raise CklError(st, what)


def plan(N, d, V, K, dtype="bf16", chunk=0, budget_bytes=0, pass_="fused"):
    """(chunk rows, workspace bytes) the library will use for this shape and call
    (``pass_`` = "fused", "fwd" or "bwd")."""
    c = ctypes.c_int64(0)
    b = ctypes.c_uint64(0)
    dt = DTYPE_BF16 if dtype == "bf16" else DTYPE_F32
    _check(lib().ckl_plan_pass(PASSES[pass_], N, d, V, K, dt, chunk, budget_bytes, ctypes.byref(c),
                               ctypes.byref(b)), "ckl_plan_pass")
    return int(c.value), int(b.value)


def release_workspace():
    lib().ckl_release_workspace()


def workspace_bytes_held():
    return int(lib().ckl_workspace_bytes_held())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(torch, device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


NOALLOC_MAX_BYTES = 256 << 20  # CKL_NOALLOC_MAX_BYTES


def fwd_bwd(H, W, ids, tlogit, mask=None, chunk=0, out_loss=None, dH=None, dW=None, row_kl=None,
            row_lse=None, noalloc=False):
    """Loss, dH and dW of the fused chunked KL loss; tensors on one GPU.

    H [N,d] and W [V,d] are both bfloat16 or both float32; ids int32 [N,K];
    tlogit float32 [N,K]; mask uint8/bool [N] or None.  Returns
    (loss 0-dim float32, dH like H, dW float32 [V,d]), all enqueued on the
    current stream.  ``row_kl`` / ``row_lse`` (float32 [N] tensors) receive
    the per-position KL and student logsumexp when given (both 0 for masked
    positions).  ``noalloc`` calls ckl_fwd_bwd_noalloc, whose workspace is the
    library's fixed device array (the outputs are still allocated here unless
    given).
    """
    import torch

    _check_inputs(torch, H, W, ids, tlogit, "fwd_bwd", mask)
    N, d = H.shape
    V = W.shape[0]
    K = ids.shape[1]
    if mask is not None:
        mask = mask.to(torch.uint8).contiguous()
    dev = H.device
    _check_out(torch, out_loss, (), torch.float32, dev, "out_loss")
    _check_out(torch, dH, (N, d), H.dtype, dev, "dH")
    _check_out(torch, dW, (V, d), torch.float32, dev, "dW")
    _check_out(torch, row_kl, (N,), torch.float32, dev, "row_kl")
    _check_out(torch, row_lse, (N,), torch.float32, dev, "row_lse")
    if out_loss is None:
        out_loss = torch.empty((), dtype=torch.float32, device=dev)
    if dH is None:
        dH = torch.empty_like(H)
    if dW is None:
        dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    st_dev = _stream(torch, dev)
    if noalloc:
        dt = DTYPE_BF16 if H.dtype == torch.bfloat16 else DTYPE_F32
        st = lib().ckl_fwd_bwd_noalloc(dt, _ptr(H), _ptr(W), _ptr(ids), _ptr(tlogit), _ptr(mask), N, d, V, K,
                                       int(chunk), _ptr(out_loss), _ptr(dH), _ptr(dW), _ptr(row_kl),
                                       _ptr(row_lse), st_dev)
        _check(st, "ckl_fwd_bwd_noalloc")
        return out_loss, dH, dW
    if row_kl is None and row_lse is None:
        fn = lib().ckl_fwd_bwd if H.dtype == torch.bfloat16 else lib().ckl_fwd_bwd_f32
        st = fn(_ptr(H), _ptr(W), _ptr(ids), _ptr(tlogit), _ptr(mask), N, d, V, K, int(chunk),
                _ptr(out_loss), _ptr(dH), _ptr(dW), st_dev)
    else:
        dt = DTYPE_BF16 if H.dtype == torch.bfloat16 else DTYPE_F32
        st = lib().ckl_fwd_bwd_ex(dt, _ptr(H), _ptr(W), _ptr(ids), _ptr(tlogit), _ptr(mask), N, d, V, K,
                                  int(chunk), _ptr(out_loss), _ptr(dH), _ptr(dW), _ptr(row_kl), _ptr(row_lse),
                                  st_dev)
    _check(st, "ckl_fwd_bwd")
    return out_loss, dH, dW


def _check_inputs(torch, H, W, ids, tlogit, what, mask=None, need_gpu=True):
    """Dtypes, contiguity, one device and consistent shapes: the kernels index
    every array by N, d, V and K, so a mismatch would read out of bounds."""
    if need_gpu and not H.is_cuda:
        raise ValueError(f"{what} needs GPU tensors")
    for name, t in (("H", H), ("W", W), ("ids", ids), ("tlogit", tlogit)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != H.device:
            raise ValueError(f"{name} must be on {H.device}")
    if ids.dtype != torch.int32 or tlogit.dtype != torch.float32:
        raise ValueError("ids must be int32 and tlogit float32")
    if H.dtype != W.dtype or H.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("H and W must both be bfloat16 or both float32")
    if H.dim() != 2 or W.dim() != 2 or H.shape[1] != W.shape[1]:
        raise ValueError("H must be [N, d] and W [V, d]")
    N = H.shape[0]
    if ids.dim() != 2 or ids.shape[0] != N or tuple(tlogit.shape) != tuple(ids.shape):
        raise ValueError("ids and tlogit must both be [N, K]")
    if mask is not None and (tuple(mask.shape) != (N,) or mask.device != H.device):
        raise ValueError(f"mask must be [N] on {H.device}")
    return DTYPE_BF16 if H.dtype == torch.bfloat16 else DTYPE_F32


def _check_out(torch, t, shape, dtype, device, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")


def fwd(H, W, ids, tlogit, mask=None, chunk=0, out_loss=None, row_lse=None, row_kl=None):
    """Forward only: (loss 0-dim float32, row_lse float32 [N], 0 for masked positions); row_kl [N]
    filled when given."""
    import torch

    dt = _check_inputs(torch, H, W, ids, tlogit, "fwd", mask)
    N, d = H.shape
    V, K = W.shape[0], ids.shape[1]
    if mask is not None:
        mask = mask.to(torch.uint8).contiguous()
    _check_out(torch, out_loss, (), torch.float32, H.device, "out_loss")
    _check_out(torch, row_lse, (N,), torch.float32, H.device, "row_lse")
    _check_out(torch, row_kl, (N,), torch.float32, H.device, "row_kl")
    if out_loss is None:
        out_loss = torch.empty((), dtype=torch.float32, device=H.device)
    if row_lse is None:
        row_lse = torch.empty((N,), dtype=torch.float32, device=H.device)
    st = lib().ckl_fwd(dt, _ptr(H), _ptr(W), _ptr(ids), _ptr(tlogit), _ptr(mask), N, d, V, K, int(chunk),
                       _ptr(out_loss), _ptr(row_lse), _ptr(row_kl), _stream(torch, H.device))
    _check(st, "ckl_fwd")
    return out_loss, row_lse


def bwd(H, W, ids, tlogit, row_lse, mask=None, grad_loss=None, chunk=0, dH=None, dW=None):
    """Backward that recomputes the logits: (dH like H, dW float32 [V,d]) of
    grad_loss x loss; grad_loss is a float32 device scalar tensor or None (1)."""
    import torch

    dt = _check_inputs(torch, H, W, ids, tlogit, "bwd", mask)
    if row_lse is None:
        raise ValueError("bwd needs the row_lse that fwd returned")
    N, d = H.shape
    V, K = W.shape[0], ids.shape[1]
    if mask is not None:
        mask = mask.to(torch.uint8).contiguous()
    _check_out(torch, row_lse, (N,), torch.float32, H.device, "row_lse")
    _check_out(torch, dH, (N, d), H.dtype, H.device, "dH")
    _check_out(torch, dW, (V, d), torch.float32, H.device, "dW")
    if grad_loss is not None:
        grad_loss = grad_loss.to(device=H.device, dtype=torch.float32).contiguous()
    if dH is None:
        dH = torch.empty_like(H)
    if dW is None:
        dW = torch.empty((V, d), dtype=torch.float32, device=H.device)
    st = lib().ckl_bwd(dt, _ptr(H), _ptr(W), _ptr(ids), _ptr(tlogit), _ptr(mask), _ptr(row_lse),
                       _ptr(grad_loss), N, d, V, K, int(chunk), _ptr(dH), _ptr(dW), _stream(torch, H.device))
    _check(st, "ckl_bwd")
    return dH, dW


def topk(logits, K, ids_out=None, vals_out=None):
    """Teacher cache writer: (ids int32 [N,K], values float32 [N,K]) of the K largest
    logits per row of a contiguous bf16 or fp32 GPU tensor [N,V], by value
    descending, equal values by id ascending."""
    import torch

    if not logits.is_cuda or not logits.is_contiguous() or logits.dim() != 2:
        raise ValueError("topk needs a contiguous 2-D GPU tensor")
    if logits.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("logits must be bfloat16 or float32")
    N, V = logits.shape
    dt = DTYPE_BF16 if logits.dtype == torch.bfloat16 else DTYPE_F32
    _check_out(torch, ids_out, (N, K), torch.int32, logits.device, "ids_out")
    _check_out(torch, vals_out, (N, K), torch.float32, logits.device, "vals_out")
    if ids_out is None:
        ids_out = torch.empty((N, K), dtype=torch.int32, device=logits.device)
    if vals_out is None:
        vals_out = torch.empty((N, K), dtype=torch.float32, device=logits.device)
    st = lib().ckl_topk(dt, _ptr(logits), N, V, int(K), _ptr(ids_out), _ptr(vals_out),
                        _stream(torch, logits.device))
    _check(st, "ckl_topk")
    return ids_out, vals_out


def debug_rows(Z, ids, tlogit, mask=None, scale=1.0, g_bf16=True):
    """Row pass alone on caller-given fp32 logits Z [R,V] (synchronises)."""
    import torch

    R, V = Z.shape
    K = ids.shape[1]
    dev = Z.device
    if tuple(ids.shape) != (R, K) or tuple(tlogit.shape) != (R, K) or (mask is not None and tuple(mask.shape) != (R,)):
        raise ValueError("ids and tlogit must be [R, K] and mask [R]")
    if ids.dtype != torch.int32 or tlogit.dtype != torch.float32 or Z.dtype != torch.float32:
        raise ValueError("Z and tlogit must be float32, ids int32")
    zg = torch.empty((R, K), dtype=torch.float32, device=dev)
    sid = torch.empty((R, K), dtype=torch.int32, device=dev)
    G = torch.empty((R, V), dtype=torch.bfloat16 if g_bf16 else torch.float32, device=dev)
    kl = torch.empty((R,), dtype=torch.float32, device=dev)
    lse = torch.empty((R,), dtype=torch.float32, device=dev)
    if mask is not None:
        mask = mask.to(torch.uint8).contiguous()
    st = lib().ckl_debug_rows(_ptr(Z.contiguous()), _ptr(ids), _ptr(tlogit), _ptr(mask), R, V, K,
                              float(scale), 1 if g_bf16 else 0, _ptr(zg), _ptr(sid), _ptr(G), _ptr(kl),
                              _ptr(lse), _stream(torch, dev))
    _check(st, "ckl_debug_rows")
    return {"zg": zg, "sid": sid, "G": G, "kl": kl, "lse": lse}


def timing_enable(on=True):
    _check(lib().ckl_timing_enable(1 if on else 0), "ckl_timing_enable")


def timing_query(kind):
    """(total milliseconds, launches) recorded for one kernel kind since enabling."""
    t = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    _check(lib().ckl_timing_query(TIMING_KINDS[kind], ctypes.byref(t), ctypes.byref(n)), "ckl_timing_query")
    return float(t.value), int(n.value)


class _FusedKL:
    """torch.autograd.Function wrapper, created lazily so importing needs no torch."""

    _fn = None

    @classmethod
    def get(cls):
        if cls._fn is None:
            import torch

            class FusedKL(torch.autograd.Function):
                @staticmethod
                def forward(ctx, H, W, ids, tlogit, mask, chunk):
                    loss, dH, dW = fwd_bwd(H.contiguous(), W.contiguous(), ids, tlogit, mask, chunk)
                    # kept as plain attributes (not saved tensors): backward
                    # scales them in place, once
                    ctx.grads = (dH, dW)
                    ctx.w_dtype = W.dtype
                    return loss

                @staticmethod
                def backward(ctx, g):
                    if ctx.grads is None:
                        raise RuntimeError("fused_kl: its gradients were computed once, in the forward call, "
                                           "and have been used; a second backward needs a new forward call")
                    dH, dW = ctx.grads
                    ctx.grads = None
                    # in place: no second copy of the fp32 [V, d] gradient (a
                    # bf16 W still gets a bf16 gradient, as autograd requires)
                    g = g.to(torch.float32)
                    dH.mul_(g)
                    dW.mul_(g)
                    return dH, dW if ctx.w_dtype == torch.float32 else dW.to(ctx.w_dtype), None, None, None, None

            cls._fn = FusedKL
        return cls._fn


def fused_kl(H, W, ids, tlogit, mask=None, chunk=0):
    """Loss as a differentiable torch scalar: gradients were computed in the forward pass."""
    return _FusedKL.get().apply(H, W, ids, tlogit, mask, chunk)


class _RecomputeKL:
    """Two-pass autograd wrapper: the forward keeps the per-position log-normaliser,
    the backward recomputes the logits (ckl_fwd / ckl_bwd)."""

    _fn = None

    @classmethod
    def get(cls):
        if cls._fn is None:
            import torch

            class RecomputeKL(torch.autograd.Function):
                @staticmethod
                def forward(ctx, H, W, ids, tlogit, mask, chunk):
                    H, W = H.contiguous(), W.contiguous()
                    loss, lse = fwd(H, W, ids, tlogit, mask, chunk)
                    ctx.save_for_backward(H, W, ids, tlogit, lse, mask if mask is not None else torch.empty(0))
                    ctx.has_mask = mask is not None
                    ctx.chunk = chunk
                    return loss

                @staticmethod
                def backward(ctx, g):
                    H, W, ids, tlogit, lse, mask = ctx.saved_tensors
                    dH, dW = bwd(H, W, ids, tlogit, lse, mask if ctx.has_mask else None,
                                 grad_loss=g.reshape(()), chunk=ctx.chunk)
                    return dH, dW.to(W.dtype), None, None, None, None

            cls._fn = RecomputeKL
        return cls._fn


def recompute_kl(H, W, ids, tlogit, mask=None, chunk=0):
    """Loss as a differentiable torch scalar whose backward recomputes each chunk's logits."""
    return _RecomputeKL.get().apply(H, W, ids, tlogit, mask, chunk)
