"""Fused chunked KL distillation loss for MI355X (gfx950): HIP kernels behind a C ABI.

``binding`` loads libckl.so on first use and raises if it is missing;
``workloads`` draws the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    CklError,
    bwd,
    debug_rows,
    fused_kl,
    fwd,
    fwd_bwd,
    plan,
    recompute_kl,
    release_workspace,
    timing_enable,
    topk,
    timing_query,
    workspace_bytes_held,
)
