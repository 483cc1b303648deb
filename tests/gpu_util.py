"""Helpers for the GPU tests: move seeded host inputs to the device and results back (plumbing only)."""
import numpy as np

import synthetic as syn

TOL_O = {"f32": 2e-5, "bf16": 1.6e-2}
TOL_LSE = 1e-3


def to_dev(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()


def to_host64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def inputs(w: syn.Workload):
    """Host storage arrays (f32 or bf16 bits) for q, k, v and their exact float64 values."""
    host = {t: syn.make_tensor(w, t) for t in ("q", "k", "v")}
    f64 = {t: syn.as_f64(host[t], w.dtype) for t in host}
    return host, f64


def host_workers() -> int:
    """Threads for host-side oracle work: the cores this process may use, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_output_floor(ref) -> float:
    """max |ref - bf16(ref)|: the error that rounding the exact output to bf16 (round to nearest even) costs
    by itself, the least any bf16-output kernel can reach on these rows."""
    import torch
    r = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float64))
    return float((r - r.to(torch.bfloat16).to(torch.float64)).abs().max()) if r.numel() else 0.0


def max_err(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    if not np.all(np.isfinite(a)):
        return float("inf")
    return float(np.abs(a - b).max())
