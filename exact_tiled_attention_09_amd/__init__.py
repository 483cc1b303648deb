"""Python binding of libfa: exact tiled attention for MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libfa.so; there is no CPU or PyTorch fallback.  PyTorch provides the
device memory and the stream: tensors are passed by ``data_ptr()`` and work is
enqueued on ``torch.cuda.current_stream()`` (HIP on ROCm) unless a stream is
given.

The C entry points are exposed under their C names (``fa_fwd``, ``fa_decode``,
...), taking torch tensors instead of raw pointers; ``attention`` and ``decode``
are allocation helpers around them.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_DEVICE = range(5)
FA_DTYPE_BF16, FA_DTYPE_F32 = 0, 1

FA_PLAN_FWD, FA_PLAN_FWD_SPLIT, FA_PLAN_DECODE, FA_PLAN_BWD_DQ, FA_PLAN_BWD_DKDV = range(5)
KERNEL_NAMES = {1: "bf16_4wave", 2: "bf16_8wave", 3: "bf16_split", 4: "f32_rows", 5: "f32_keysplit",
                6: "decode_split", 7: "bwd_dq", 8: "bwd_dkdv"}

_lib = None


class PlanInfo(ctypes.Structure):
    """fa_plan_info of include/fa.h."""
    _fields_ = [("kernel", ctypes.c_int), ("waves_per_group", ctypes.c_int), ("rows_per_group", ctypes.c_int),
                ("paired", ctypes.c_int), ("groups", ctypes.c_longlong), ("num_splits", ctypes.c_int)]


class FaError(RuntimeError):
    """A non-OK status returned by libfa."""

    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {status_str(status)}: {detail}")


def lib() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by build.py); raise loudly if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libfa.so is not built at {LIB_PATH}; run `python -m exact_tiled_attention_09_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i]
    L.fa_fwd_bf16.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.fa_fwd_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.fa_decode_num_splits.argtypes = [i, i, i, i, i]
    L.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_decode_workspace_bytes.restype = sz
    L.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp, i]
    L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
    L.fa_decode_split.argtypes = [vp, vp, vp, i, i, i, i, f, i, vp, sz, vp, i]
    L.fa_decode_combine.argtypes = [vp, sz, vp, vp, i, i, i, i, vp, i]
    L.fa_fwd_split_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_fwd_split_workspace_bytes.restype = sz
    L.fa_fwd_split_num_splits.argtypes = [i, i, i, i, i]
    L.fa_fwd_split_num_splits.restype = i
    L.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp, i]
    L.fa_decode_gqa_num_splits.argtypes = [i, i, i, i, i, i]
    L.fa_decode_gqa_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.fa_decode_gqa_workspace_bytes.restype = sz
    L.fa_decode_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp, i]
    L.fa_decode_paged_num_splits.argtypes = [i, i, i, i, i]
    L.fa_decode_paged_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.fa_decode_paged_workspace_bytes.restype = sz
    L.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp, i]
    L.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    L.fa_bwd_workspace_bytes.restype = sz
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp, i]
    L.fa_plan.argtypes = [i, i, i, i, i, i, i, i, i, i, ctypes.POINTER(PlanInfo)]
    L.fa_plan.restype = ctypes.c_int
    L.fa_device_num_cu.argtypes = []
    L.fa_device_num_cu.restype = ctypes.c_int
    L.fa_probe_read_bandwidth.argtypes = [vp, sz, vp, sz, i, vp]
    L.fa_probe_read_bandwidth.restype = ctypes.c_int
    L.fa_probe_clock.argtypes = [vp, sz, i, i, vp]
    L.fa_probe_clock.restype = ctypes.c_int
    L.fa_status_str.argtypes = [i]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_last_error.argtypes = []
    L.fa_last_error.restype = ctypes.c_char_p
    L.fa_version.restype = ctypes.c_char_p
    for name in ("fa_fwd", "fa_fwd_bf16", "fa_fwd_f32", "fa_decode", "fa_decode_split", "fa_decode_combine",
                 "fa_decode_num_splits", "fa_bwd", "fa_fwd_split", "fa_decode_gqa", "fa_decode_gqa_num_splits",
                 "fa_decode_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_str(s: int) -> str:
    return lib().fa_status_str(s).decode()


def last_error() -> str:
    return lib().fa_last_error().decode()


def version() -> str:
    return lib().fa_version().decode()


def _check(status: int, func: str):
    if status != FA_OK:
        raise FaError(status, func, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _check_tensor(name, t, shape, dtype):
    """Every tensor handed to the library: a contiguous device tensor of the expected shape and dtype (the C
    layer sees only a pointer, so a strided view or a host tensor would be read as something else)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _check_workspace(t):
    """A workspace: a contiguous device tensor of bytes (uint8); returns its size in bytes."""
    import torch
    if not t.is_cuda:
        raise ValueError("workspace must be a device tensor")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if t.dtype != torch.uint8:
        raise ValueError(f"workspace must be a uint8 (byte) tensor, got {t.dtype}")
    return t.numel()


def plan(op: int, B: int, H: int, N_q: int, N_kv: int, d: int, causal: bool = True, dtype: int = FA_DTYPE_BF16,
         num_splits: int = 0, num_cu: int = 0) -> dict:
    """fa_plan: the launch decisions of an entry point for these sizes on a device with num_cu compute units
    (0 = the current device).  Host arithmetic only when num_cu > 0."""
    info = PlanInfo()
    st = lib().fa_plan(op, B, H, N_q, N_kv, d, int(bool(causal)), dtype, num_splits, num_cu, ctypes.byref(info))
    _check(st, "fa_plan")
    return {"kernel": KERNEL_NAMES.get(info.kernel, info.kernel), "waves_per_group": info.waves_per_group,
            "rows_per_group": info.rows_per_group, "paired": bool(info.paired), "groups": info.groups,
            "num_splits": info.num_splits}


def device_num_cu() -> int:
    """Compute units of the current device (0 when none can be queried)."""
    return lib().fa_device_num_cu()


# ----------------------------------------------------------------------------- C entry points, torch arguments

def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None):
    """libfa fa_fwd on torch tensors: q [B,H,N_q,d], k/v [B,H,N_kv,d], o like q, lse [B,H,N_q] fp32 or None."""
    import torch
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    _check_tensor("q", q, (B, H, Nq, d), q.dtype)
    _check_tensor("k", k, (B, H, Nkv, d), q.dtype)
    _check_tensor("v", v, (B, H, Nkv, d), q.dtype)
    _check_tensor("o", o, (B, H, Nq, d), q.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H, Nq), torch.float32)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nkv, d, float(scale), int(bool(causal)),
                      _stream(stream), _dtype_code(q))
    _check(st, "fa_fwd")


def fa_decode_num_splits(B: int, H: int, N_kv: int, d: int, num_splits: int = 0) -> int:
    return lib().fa_decode_num_splits(B, H, N_kv, d, num_splits)


def fa_decode_workspace_bytes(B: int, H: int, N_kv: int, d: int, num_splits: int = 0) -> int:
    return lib().fa_decode_workspace_bytes(B, H, N_kv, d, num_splits)


def fa_decode(q, k, v, o, lse, scale: float, num_splits: int, workspace, stream=None):
    """libfa fa_decode: q [B,H,d], k/v [B,H,N_kv,d] bf16; o [B,H,d] bf16; lse [B,H] fp32 or None;
    workspace a byte (uint8) device tensor of at least fa_decode_workspace_bytes()."""
    import torch
    B, H, Nkv, d = k.shape
    _check_tensor("k", k, (B, H, Nkv, d), k.dtype)
    _check_tensor("q", q, (B, H, d), k.dtype)
    _check_tensor("v", v, (B, H, Nkv, d), k.dtype)
    _check_tensor("o", o, (B, H, d), k.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H), torch.float32)
    nws = _check_workspace(workspace)
    st = lib().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nkv, d, float(scale), int(num_splits),
                         _ptr(workspace), nws, _stream(stream), _dtype_code(k))
    _check(st, "fa_decode")


# Bytes of the scratch array fa_decode_noalloc keeps per GPU (FA_NOALLOC_SCRATCH_BYTES in fa.h).
NOALLOC_SCRATCH_BYTES = 32 << 20


def fa_decode_noalloc(q, k, v, o, lse, scale: float, num_splits: int, stream=None):
    """libfa fa_decode_noalloc: fa_decode with the split partials in the library's built-in per-GPU scratch
    (no workspace, no device allocation).  Calls that overlap in time on one GPU race on that scratch."""
    import torch
    B, H, Nkv, d = k.shape
    _check_tensor("k", k, (B, H, Nkv, d), k.dtype)
    _check_tensor("q", q, (B, H, d), k.dtype)
    _check_tensor("v", v, (B, H, Nkv, d), k.dtype)
    _check_tensor("o", o, (B, H, d), k.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H), torch.float32)
    st = lib().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nkv, d, float(scale),
                                 int(num_splits), _stream(stream), _dtype_code(k))
    _check(st, "fa_decode_noalloc")


def fa_decode_split(q, k, v, scale: float, num_splits: int, workspace, stream=None):
    B, H, Nkv, d = k.shape
    _check_tensor("k", k, (B, H, Nkv, d), k.dtype)
    _check_tensor("q", q, (B, H, d), k.dtype)
    _check_tensor("v", v, (B, H, Nkv, d), k.dtype)
    nws = _check_workspace(workspace)
    st = lib().fa_decode_split(_ptr(q), _ptr(k), _ptr(v), B, H, Nkv, d, float(scale), int(num_splits), _ptr(workspace),
                               nws, _stream(stream), _dtype_code(k))
    _check(st, "fa_decode_split")


def fa_decode_combine(workspace, o, lse, num_splits: int, stream=None):
    import torch
    B, H, d = o.shape
    _check_tensor("o", o, (B, H, d), o.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H), torch.float32)
    nws = _check_workspace(workspace)
    st = lib().fa_decode_combine(_ptr(workspace), nws, _ptr(o), _ptr(lse), B, H, d, int(num_splits), _stream(stream),
                                 _dtype_code(o))
    _check(st, "fa_decode_combine")


def fa_fwd_split_workspace_bytes(B: int, H: int, N_q: int, d: int, num_splits: int) -> int:
    return lib().fa_fwd_split_workspace_bytes(B, H, N_q, d, num_splits)


def fa_fwd_split_num_splits(B: int, H: int, N_q: int, N_kv: int, d: int) -> int:
    return lib().fa_fwd_split_num_splits(B, H, N_q, N_kv, d)


def fa_fwd_split(q, k, v, o, lse, scale: float, causal: bool, num_splits: int, workspace, stream=None):
    """libfa fa_fwd_split: fa_fwd with the keys cut into num_splits ranges (bf16); workspace a byte device
    tensor of at least fa_fwd_split_workspace_bytes()."""
    import torch
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    _check_tensor("q", q, (B, H, Nq, d), q.dtype)
    _check_tensor("k", k, (B, H, Nkv, d), q.dtype)
    _check_tensor("v", v, (B, H, Nkv, d), q.dtype)
    _check_tensor("o", o, (B, H, Nq, d), q.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H, Nq), torch.float32)
    nws = _check_workspace(workspace)
    st = lib().fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Nq, Nkv, d, float(scale),
                            int(bool(causal)), int(num_splits), _ptr(workspace), nws, _stream(stream),
                            _dtype_code(q))
    _check(st, "fa_fwd_split")


def fa_decode_gqa_num_splits(B: int, H: int, H_kv: int, N_kv: int, d: int, num_splits: int = 0) -> int:
    return lib().fa_decode_gqa_num_splits(B, H, H_kv, N_kv, d, num_splits)


def fa_decode_gqa_workspace_bytes(B: int, H: int, H_kv: int, N_kv: int, d: int, num_splits: int = 0) -> int:
    return lib().fa_decode_gqa_workspace_bytes(B, H, H_kv, N_kv, d, num_splits)


def fa_decode_gqa(q, k, v, o, lse, scale: float, num_splits: int, workspace, stream=None):
    """libfa fa_decode_gqa: q [B,H,d], k/v [B,H_kv,N_kv,d] (bf16, H a multiple of H_kv); o [B,H,d];
    lse [B,H] fp32 or None; workspace of at least fa_decode_gqa_workspace_bytes()."""
    import torch
    B, H, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    _check_tensor("k", k, (B, Hkv, Nkv, d), k.dtype)
    _check_tensor("q", q, (B, H, d), k.dtype)
    _check_tensor("v", v, (B, Hkv, Nkv, d), k.dtype)
    _check_tensor("o", o, (B, H, d), k.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H), torch.float32)
    nws = _check_workspace(workspace)
    st = lib().fa_decode_gqa(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nkv, d, float(scale),
                             int(num_splits), _ptr(workspace), nws, _stream(stream), _dtype_code(k))
    _check(st, "fa_decode_gqa")


def fa_decode_paged_num_splits(B: int, H_kv: int, max_seq_len: int, d: int, num_splits: int = 0) -> int:
    return lib().fa_decode_paged_num_splits(B, H_kv, max_seq_len, d, num_splits)


def fa_decode_paged_workspace_bytes(B: int, H: int, H_kv: int, max_seq_len: int, d: int, num_splits: int = 0) -> int:
    return lib().fa_decode_paged_workspace_bytes(B, H, H_kv, max_seq_len, d, num_splits)


def fa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, o, lse, scale: float, num_splits: int, workspace,
                    stream=None):
    """libfa fa_decode_paged: q [B,H,d]; k_pages/v_pages [num_pages,H_kv,page_size,d] (bf16); block_table
    [B,max_blocks] and seq_lens [B] int32 device tensors; o [B,H,d]; lse [B,H] fp32 or None; workspace of at
    least fa_decode_paged_workspace_bytes(B, H, H_kv, max_blocks * page_size, d, num_splits)."""
    import torch
    B, H, d = q.shape
    n_pages, Hkv, P = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_blocks = block_table.shape[1] if block_table.dim() == 2 else -1
    _check_tensor("q", q, (B, H, d), k_pages.dtype)
    _check_tensor("k_pages", k_pages, (n_pages, Hkv, P, d), k_pages.dtype)
    _check_tensor("v_pages", v_pages, (n_pages, Hkv, P, d), k_pages.dtype)
    _check_tensor("block_table", block_table, (B, max_blocks), torch.int32)
    _check_tensor("seq_lens", seq_lens, (B,), torch.int32)
    _check_tensor("o", o, (B, H, d), k_pages.dtype)
    if lse is not None:
        _check_tensor("lse", lse, (B, H), torch.float32)
    nws = _check_workspace(workspace)
    st = lib().fa_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seq_lens), _ptr(o),
                               _ptr(lse), B, H, Hkv, n_pages, P, max_blocks, d, float(scale), int(num_splits),
                               _ptr(workspace), nws, _stream(stream), _dtype_code(k_pages))
    _check(st, "fa_decode_paged")


def fa_bwd_workspace_bytes(B: int, H: int, N_q: int) -> int:
    return lib().fa_bwd_workspace_bytes(B, H, N_q)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale: float, causal: bool, workspace, stream=None):
    """libfa fa_bwd: q, o, dout, dq [B,H,N_q,d]; k, v, dk, dv [B,H,N_kv,d] (bf16); lse [B,H,N_q] fp32 as
    fa_fwd wrote it; workspace a byte device tensor of at least fa_bwd_workspace_bytes()."""
    import torch
    B, H, Nq, d = q.shape
    Nkv = k.shape[2]
    for name, t, n in (("q", q, Nq), ("o", o, Nq), ("dout", dout, Nq), ("dq", dq, Nq), ("k", k, Nkv),
                       ("v", v, Nkv), ("dk", dk, Nkv), ("dv", dv, Nkv)):
        _check_tensor(name, t, (B, H, n, d), q.dtype)
    _check_tensor("lse", lse, (B, H, Nq), torch.float32)
    nws = _check_workspace(workspace)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, H, Nq, Nkv, d, float(scale), int(bool(causal)), _ptr(workspace), nws, _stream(stream),
                      _dtype_code(q))
    _check(st, "fa_bwd")


# ----------------------------------------------------------------------------- measurement probes (fa_probe.h)

def probe_read_bandwidth(buf, sink, groups: int, stream=None):
    """fa_probe_read_bandwidth: one non-temporal streaming read of the byte tensor buf; sink is a device
    tensor of at least groups * 512 int32 words."""
    _check_workspace(buf)
    if not sink.is_cuda or not sink.is_contiguous():
        raise ValueError("sink must be a contiguous device tensor")
    st = lib().fa_probe_read_bandwidth(_ptr(buf), buf.numel(), _ptr(sink), sink.numel() * sink.element_size(),
                                       int(groups), _stream(stream))
    if st != 0:
        raise FaError(FA_ERR_INVALID_ARG if st == 1 else FA_ERR_DEVICE, "fa_probe_read_bandwidth", f"status {st}")


def probe_clock(out, groups: int, iters: int, stream=None):
    """fa_probe_clock: out is an int64 device tensor of at least 5 * groups words."""
    import torch
    if not out.is_cuda or not out.is_contiguous() or out.dtype != torch.int64:
        raise ValueError("out must be a contiguous int64 device tensor")
    st = lib().fa_probe_clock(_ptr(out), out.numel(), int(groups), int(iters), _stream(stream))
    if st != 0:
        raise FaError(FA_ERR_INVALID_ARG if st == 1 else FA_ERR_DEVICE, "fa_probe_clock", f"status {st}")


# ----------------------------------------------------------------------------- allocation helpers

def attention(q, k, v, scale: float | None = None, causal: bool = False, stream=None):
    """Allocate o and lse and run fa_fwd; returns (o, lse)."""
    import torch
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, causal, stream)
    return o, lse


def decode_workspace(B, H, N_kv, d, num_splits=0, device="cuda"):
    import torch
    n = fa_decode_workspace_bytes(B, H, N_kv, d, num_splits)
    if n == 0:
        raise FaError(FA_ERR_INVALID_ARG, "fa_decode_workspace_bytes", last_error())
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode(q, k, v, scale: float | None = None, num_splits: int = 0, workspace=None, stream=None):
    """Allocate o, lse (and the workspace if not given) and run fa_decode; returns (o, lse)."""
    import torch
    B, H, Nkv, d = k.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if workspace is None:
        workspace = decode_workspace(B, H, Nkv, d, num_splits, q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    fa_decode(q, k, v, o, lse, scale, num_splits, workspace, stream)
    return o, lse


def attention_backward(q, k, v, o, lse, dout, scale: float | None = None, causal: bool = False, stream=None):
    """Allocate dq, dk, dv and the workspace and run fa_bwd; returns (dq, dk, dv)."""
    import torch
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    B, H, Nq, _ = q.shape
    ws = torch.empty(fa_bwd_workspace_bytes(B, H, Nq), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, scale, causal, ws, stream)
    return dq, dk, dv


def attention_split(q, k, v, num_splits: int, scale: float | None = None, causal: bool = False, stream=None):
    """Allocate o, lse and the workspace and run fa_fwd_split; returns (o, lse)."""
    import torch
    B, H, Nq, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    ws = torch.empty(fa_fwd_split_workspace_bytes(B, H, Nq, d, num_splits), dtype=torch.uint8, device=q.device)
    fa_fwd_split(q, k, v, o, lse, scale, causal, num_splits, ws, stream)
    return o, lse


def decode_gqa(q, k, v, scale: float | None = None, num_splits: int = 0, stream=None):
    """Allocate o, lse and the workspace and run fa_decode_gqa; returns (o, lse)."""
    import torch
    B, H, d = q.shape
    Hkv, Nkv = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    n = fa_decode_gqa_workspace_bytes(B, H, Hkv, Nkv, d, num_splits)
    if n == 0:
        raise FaError(FA_ERR_INVALID_ARG, "fa_decode_gqa_workspace_bytes", last_error())
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    fa_decode_gqa(q, k, v, o, lse, scale, num_splits, ws, stream)
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale: float | None = None, num_splits: int = 0,
                 stream=None):
    """Allocate o, lse and the workspace and run fa_decode_paged; returns (o, lse)."""
    import torch
    B, H, d = q.shape
    Hkv, P = k_pages.shape[1], k_pages.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    n = fa_decode_paged_workspace_bytes(B, H, Hkv, block_table.shape[-1] * P, d, num_splits)
    if n == 0:
        raise FaError(FA_ERR_INVALID_ARG, "fa_decode_paged_workspace_bytes", last_error())
    ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    fa_decode_paged(q, k_pages, v_pages, block_table, seq_lens, o, lse, scale, num_splits, ws, stream)
    return o, lse
