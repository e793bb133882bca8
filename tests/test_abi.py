"""Host-side checks of the C ABI: symbols, planner arithmetic and argument errors (no GPU needed)."""
import ctypes
import os
import re

import pytest

from chunked_kl_loss_seq_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libckl.so not built")


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "ckl.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ckl_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    L = B.lib()
    names = declared_functions()
    assert "ckl_fwd_bwd" in names and "ckl_plan" in names
    for n in names:
        assert hasattr(L, n), n


def test_strerror():
    assert B.strerror(0) == "ok"
    assert "budget" in B.strerror(-3)
    assert B.strerror(12345) == "unknown status"


GiB = 1 << 30


def ws_formula(N, d, V, K, C, splits, esz=2, keep_exp=True):
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    pblk = -(-V // 64) * 4096          # elements between 64-row tile rows of the exp / gradient tiles
    tile_rows = -(-C // 64)
    nsl = -(-V // 128)
    wt = -(-V // 64) * (-(-d // 64) * 4096)  # tiled copy of W
    compact = a(C * d * esz) + 2 * a(C * K * 4) + 2 * a(C * 4)  # masked calls: the compacted chunk
    cpad, pairs = -(-C // 256) * 256, -(-V // 256)
    idtab = a(pairs * cpad * 32) + a(pairs * cpad * 4) + 2 * a(C * K * 4)  # cached-id masks, counts, ranks, logits
    exp_vals = a(tile_rows * pblk * esz) if keep_exp else 0  # the forward alone keeps none
    return (a(wt * esz) + exp_vals + a(C * nsl * 8) + a(C * K * 4) + a(splits * C * d * 4)
            + 2 * a(N * 4) + 256 + compact + idtab)


def test_plan_explicit_chunk_matches_formula():
    for (N, d, V, K, C) in [(256, 256, 4096, 16, 64), (4096, 2048, 32000, 100, 1024), (600, 200, 1003, 37, 256)]:
        c, ws = B.plan(N, d, V, K, chunk=C)
        assert c == min(C, N)
        # the dH split count is 1..32; the bytes must match the formula for one of them
        assert any(ws == ws_formula(N, d, V, K, c, s) for s in range(1, 33)), (N, d, V, ws)
    c, ws = B.plan(256, 256, 4096, 16, dtype="f32", chunk=64)
    assert any(ws == ws_formula(256, 256, 4096, 16, 64, s, esz=4) for s in range(1, 33))
    # one 64-row chunk is a single dH tile: 8 splits cannot fill a wave of 256
    # workgroups, so the split count passes 8 (128 fp32 k-steps of 32 ids, at
    # least 8 per split: at most 16)
    assert any(ws == ws_formula(256, 256, 4096, 16, 64, s, esz=4) for s in range(9, 17))
    # the gpt-oss head fills whole waves with 2 splits
    assert B.plan(32768, 2880, 201088, 100)[1] == ws_formula(32768, 2880, 201088, 100, 8192, 2)


def test_plan_gpt_oss_head_fits_six_gib():
    c, ws = B.plan(32768, 2880, 201088, 100)
    assert ws <= 6 * GiB
    assert c % 256 == 0 and c > 0
    # a chunk one 256-row step larger would not fit, or the chunks were evened out
    nch = -(-32768 // c)
    assert nch * c >= 32768 and (nch - 1) * c < 32768
    # the long batch gets the same chunk: the workspace does not grow with N
    c5, ws5 = B.plan(131072, 2880, 201088, 100)
    assert ws5 <= 6 * GiB
    assert abs(ws5 - ws) < 4 * 131072 * 2 + 1 << 20 or c5 != c


def test_plan_workspace_bounded_in_sequence_length():
    # peak workspace stays under the budget at any N; the chunk count grows instead
    prev_chunks = 0
    for N in (16384, 32768, 65536, 131072, 262144):
        c, ws = B.plan(N, 2880, 201088, 100)
        assert ws <= 6 * GiB
        n_chunks = -(-N // c)
        assert n_chunks >= prev_chunks
        prev_chunks = n_chunks
    assert prev_chunks >= 262144 // 16384


def test_plan_budget_errors():
    with pytest.raises(B.CklError) as e:
        B.plan(32768, 2880, 201088, 100, budget_bytes=100 << 20)
    assert e.value.status == -3
    with pytest.raises(B.CklError) as e:
        B.plan(32768, 2880, 201088, 100, chunk=16384)  # 16384 x 201088 x 2 B + slabs > 6 GiB
    assert e.value.status == -3


@pytest.mark.parametrize("args,status", [
    ((-1, 8, 10, 1), -1), ((4, 0, 10, 1), -1), ((4, 8, 0, 1), -1), ((4, 8, 10, 0), -1),
    ((4, 8, 10, 11), -1), ((4, 12, 10, 2), -5), ((4, 8, 5000, 3000), -5),
])
def test_plan_argument_errors(args, status):
    with pytest.raises(B.CklError) as e:
        B.plan(*args)
    assert e.value.status == status


def test_plan_empty_batch():
    # N = 0: no chunk and no workspace, for every call; the other sizes are
    # still checked
    for pass_ in ("fused", "fwd", "bwd"):
        assert B.plan(0, 2880, 201088, 100, pass_=pass_) == (0, 0)
    assert B.plan(0, 8, 10, 1, dtype="f32") == (0, 0)
    with pytest.raises(B.CklError) as e:
        B.plan(0, 8, 10, 11)
    assert e.value.status == -1


def test_plan_negative_chunk():
    with pytest.raises(B.CklError) as e:
        B.plan(4, 8, 10, 2, chunk=-1)
    assert e.value.status == -1


def test_fwd_bwd_rejects_bad_pointers_before_any_gpu_call():
    L = B.lib()
    vp = ctypes.c_void_p
    good = vp(1 << 20)
    # null H
    st = L.ckl_fwd_bwd(vp(0), good, good, good, vp(0), 4, 8, 10, 2, 0, good, good, good, vp(0))
    assert st == -1
    # misaligned W
    st = L.ckl_fwd_bwd(good, vp((1 << 20) + 2), good, good, vp(0), 4, 8, 10, 2, 0, good, good, good, vp(0))
    assert st == -1
    # K > V
    st = L.ckl_fwd_bwd(good, good, good, good, vp(0), 4, 8, 10, 11, 0, good, good, good, vp(0))
    assert st == -1
    # d not a multiple of 8
    st = L.ckl_fwd_bwd_f32(good, good, good, good, vp(0), 4, 12, 10, 2, 0, good, good, good, vp(0))
    assert st == -5
    # unknown dtype
    st = L.ckl_fwd_bwd_ex(7, good, good, good, good, vp(0), 4, 8, 10, 2, 0, good, good, good, vp(0), vp(0), vp(0))
    assert st == -1


def test_timing_query_argument_check():
    L = B.lib()
    t = ctypes.c_double(0)
    n = ctypes.c_int64(0)
    assert L.ckl_timing_query(99, ctypes.byref(t), ctypes.byref(n)) == -1
    assert B.timing_enable(False) is None


def test_plan_per_pass():
    # the backward needs the same workspace as the fused call; the forward
    # alone keeps neither exp values nor dH split-K slabs, so at equal chunk it
    # is exactly that much smaller, and one chunk covers the 32K-token head
    for (N, d, V, K, C) in [(4096, 2048, 32000, 100, 1024), (600, 200, 1003, 37, 256)]:
        cf, wf = B.plan(N, d, V, K, chunk=C)
        cb, wb = B.plan(N, d, V, K, chunk=C, pass_="bwd")
        c1, w1 = B.plan(N, d, V, K, chunk=C, pass_="fwd")
        assert cf == cb == c1 == min(C, N)
        assert wb == wf
        assert w1 == ws_formula(N, d, V, K, c1, 0, keep_exp=False)
    c_fused, _ = B.plan(32768, 2880, 201088, 100)
    c_fwd, w_fwd = B.plan(32768, 2880, 201088, 100, pass_="fwd")
    assert c_fwd == 32768 and w_fwd == ws_formula(32768, 2880, 201088, 100, c_fwd, 0, keep_exp=False)
    assert w_fwd <= 6 * GiB and c_fwd > c_fused
    L = B.lib()
    c = ctypes.c_int64(0)
    b = ctypes.c_uint64(0)
    assert L.ckl_plan_pass(3, 64, 8, 10, 2, 0, 0, 0, ctypes.byref(c), ctypes.byref(b)) == -1


def test_fwd_and_bwd_reject_bad_arguments_before_any_gpu_call():
    L = B.lib()
    vp = ctypes.c_void_p
    good = vp(1 << 20)
    z = vp(0)
    # forward: row_lse is required, out_loss is required
    assert L.ckl_fwd(0, good, good, good, good, z, 4, 8, 10, 2, 0, good, z, z, z) == -1
    assert L.ckl_fwd(0, good, good, good, good, z, 4, 8, 10, 2, 0, z, good, z, z) == -1
    assert L.ckl_fwd(5, good, good, good, good, z, 4, 8, 10, 2, 0, good, good, z, z) == -1
    assert L.ckl_fwd(0, good, good, good, good, z, 4, 12, 10, 2, 0, good, good, z, z) == -5
    # backward: the saved row_lse, dH and dW are required; a misaligned grad_loss is rejected
    assert L.ckl_bwd(0, good, good, good, good, z, z, z, 4, 8, 10, 2, 0, good, good, z) == -1
    assert L.ckl_bwd(0, good, good, good, good, z, good, z, 4, 8, 10, 2, 0, z, good, z) == -1
    assert L.ckl_bwd(0, good, good, good, good, z, good, vp((1 << 20) + 2), 4, 8, 10, 2, 0, good, good, z) == -1
    assert L.ckl_bwd(0, good, good, good, good, z, good, z, 4, 8, 10, 11, 0, good, good, z) == -1


def test_topk_rejects_bad_arguments_before_any_gpu_call():
    L = B.lib()
    vp = ctypes.c_void_p
    good = vp(1 << 20)
    z = vp(0)
    assert L.ckl_topk(0, z, 4, 10, 2, good, good, z) == -1          # null logits
    assert L.ckl_topk(0, good, 4, 10, 2, z, good, z) == -1          # null ids
    assert L.ckl_topk(1, vp((1 << 20) + 2), 4, 10, 2, good, good, z) == -1  # fp32 logits misaligned
    assert L.ckl_topk(0, good, 4, 10, 11, good, good, z) == -1      # K > V
    assert L.ckl_topk(0, good, 0, 10, 2, good, good, z) == 0        # N = 0: nothing to do
    assert L.ckl_topk(0, z, 0, 10, 2, z, z, z) == 0                  # ... with null buffers
    assert L.ckl_topk(0, good, -1, 10, 2, good, good, z) == -1      # N < 0
    assert L.ckl_topk(0, good, 4, 5000, 3000, good, good, z) == -5  # K > 2048
    assert L.ckl_topk(9, good, 4, 10, 2, good, good, z) == -1       # unknown dtype


def test_noalloc_rejects_shapes_beyond_its_fixed_workspace():
    # the planner runs with the fixed array's size as budget: the gpt-oss head
    # (a 1.16 GB tiled copy of W alone) cannot fit and is refused before any
    # GPU call; a chunk that does not fit is refused too
    L = B.lib()
    vp = ctypes.c_void_p
    good = vp(1 << 20)
    z = vp(0)
    assert L.ckl_fwd_bwd_noalloc(0, good, good, good, good, z, 256, 2880, 201088, 100, 0, good, good, good, z, z,
                                 z) == -3
    assert L.ckl_fwd_bwd_noalloc(0, good, good, good, good, z, 4096, 2048, 32000, 100, 4096, good, good, good, z,
                                 z, z) == -3
    assert L.ckl_fwd_bwd_noalloc(3, good, good, good, good, z, 64, 8, 10, 2, 0, good, good, good, z, z, z) == -1
    assert B.NOALLOC_MAX_BYTES == 256 << 20
    _, ws = B.plan(4096, 2048, 32000, 100, budget_bytes=B.NOALLOC_MAX_BYTES)
    assert ws <= B.NOALLOC_MAX_BYTES


def test_planned_workspace_never_exceeds_the_budget():
    # the dH split count depends on the chunk, so the workspace is not
    # monotonic in it: the chosen chunk itself must fit, for any N and budget
    import numpy as np

    rng = np.random.default_rng(7)
    for _ in range(300):
        N = int(rng.integers(1, 300000))
        budget = int(rng.choice([2, 3, 4, 6, 8, 12])) << 30
        try:
            c, ws = B.plan(N, 2880, 201088, 100, budget_bytes=budget)
        except B.CklError as e:
            assert e.status == -3
            continue
        assert 0 < c <= N and ws <= budget, (N, budget, c, ws)
        assert c == N or c % 256 == 0


def test_plan_signature_budget_then_outputs():
    # ckl_plan(N, d, V, K, dtype, budget, &chunk, &bytes): the planner's own
    # chunk, equal to ckl_plan_pass(fused, ..., chunk = 0, ...)
    L = B.lib()
    c = ctypes.c_int64(0)
    b = ctypes.c_uint64(0)
    assert L.ckl_plan(32768, 2880, 201088, 100, 0, 0, ctypes.byref(c), ctypes.byref(b)) == 0
    assert (c.value, b.value) == B.plan(32768, 2880, 201088, 100)
    assert L.ckl_plan(32768, 2880, 201088, 100, 0, 100 << 20, ctypes.byref(c), ctypes.byref(b)) == -3
    assert L.ckl_plan(32768, 2880, 201088, 100, 0, 3 << 30, None, None) == 0
    assert L.ckl_plan(0, 2880, 201088, 100, 0, 0, ctypes.byref(c), ctypes.byref(b)) == 0  # empty batch
    assert (c.value, b.value) == (0, 0)
    assert L.ckl_plan(-1, 2880, 201088, 100, 0, 0, None, None) == -1
