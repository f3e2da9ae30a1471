"""MI355X (gfx950) row RMSNorm forward: HIP kernels behind a C-ABI library.

``rmsnorm_fwd(x, w, eps, offset)`` computes, per row of a 2-D bf16/fp16 tensor,
``y = x * rsqrt(mean(x^2) + eps) * (offset + w)`` and the per-row fp32 ``rstd``;
``rmsnorm_bwd(x, w, dy, rstd, offset)`` returns its gradients dx and dw
("Rmsnorm Kernel Optimization", Overview; "Why cutile's rmsnorm required full
register", kernel listing).  Every step runs in the hand-written kernels of
``librmsnorm_mi355x.so``; Python only marshals pointers, sizes and the stream.

The binding is imported on first use so that ``workloads`` (input generation
only) can be imported on a machine without the built library.
"""
from __future__ import annotations

__all__ = [
    "rmsnorm_fwd", "rmsnorm_fwd_out", "plan_query", "plan_resources", "kernel_query", "status_string",
    "rmsnorm_bwd", "rmsnorm_bwd_out", "bwd_plan_query", "bwd_workspace_size",
    "library_path", "version", "Plan", "RmsnormError",
    "plan_validate", "set_tuned", "clear_tuned", "tuned_count", "load_tuned",
    "rmsnorm_fwd_ex", "plan_query_ex", "row_layout", "Layout",
    "rmsnorm_bwd_ex", "bwd_plan_query_ex", "bwd_layout", "BwdLayout",
]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
