"""Python binding of libds4idx, the Lightning Indexer (score + top-k) for MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/ds4idx.h``. PyTorch provides device
memory and the current stream. There is no CPU fallback: if the library is
not built, every call raises.

    idx, vals = select(q, k, k_scale, w, causal_offset, topk=512)

q [B,T,H,D] bf16/fp32, k [B,S,D] bf16/fp32 or uint8 OCP E4M3 codes (or
torch.float8_e4m3fn), k_scale [B,S] fp32 for fp8 keys, w [B,T,H] fp32.

    k_cache_write(k_new, cache, cache_scale, slots=None)

quantises new keys [n,D] (bf16/fp32) into E4M3 cache rows with one scale each.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libds4idx.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 32 << 20
F32, BF16, FP8_E4M3 = 0, 1, 2
OP_SCORE, OP_TOPK, OP_SELECT = 0, 1, 2
IMPL_AUTO, IMPL_REF, IMPL_OPT = 0, 1, 2
MAX_TOPK = 2048
K_CACHE_MAX_D = 512
ABI_VERSION = 1

# Every symbol include/ds4idx.h declares.
EXPORTS = ("ds4idx_abi_version", "ds4idx_status_string", "ds4idx_set_impl", "ds4idx_get_impl",
           "ds4idx_workspace_bytes", "ds4idx_score", "ds4idx_topk", "ds4idx_select",
           "ds4idx_k_cache_write", "ds4idx_varlen_workspace_bytes", "ds4idx_select_varlen",
           "ds4idx_sparse_attention", "ds4idx_select_qfp8", "ds4idx_select_noalloc", "ds4idx_set_split",
           "ds4idx_get_split", "ds4idx_set_prefill_split", "ds4idx_get_prefill_split")
SPLIT_LENS = (8192, 12288, 16384)


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("S", ctypes.c_int32),
                ("H", ctypes.c_int32), ("D", ctypes.c_int32), ("causal_offset", ctypes.c_int64),
                ("q_dtype", ctypes.c_int32), ("k_dtype", ctypes.c_int32)]


class VarlenProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int64),
                ("max_k", ctypes.c_int32), ("H", ctypes.c_int32),
                ("D", ctypes.c_int32), ("q_dtype", ctypes.c_int32), ("k_dtype", ctypes.c_int32)]


class AttnProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("S", ctypes.c_int32), ("H", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class Ds4idxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_token_lightning_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, vp, i32, sz = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.ds4idx_abi_version.argtypes = []
        L.ds4idx_abi_version.restype = ctypes.c_int
        L.ds4idx_status_string.argtypes = [ctypes.c_int]
        L.ds4idx_status_string.restype = ctypes.c_char_p
        L.ds4idx_set_impl.argtypes = [ctypes.c_int]
        L.ds4idx_set_impl.restype = ctypes.c_int
        L.ds4idx_get_impl.argtypes = []
        L.ds4idx_get_impl.restype = ctypes.c_int
        L.ds4idx_set_split.argtypes = [ctypes.c_int]
        L.ds4idx_set_split.restype = ctypes.c_int
        L.ds4idx_get_split.argtypes = []
        L.ds4idx_get_split.restype = ctypes.c_int
        L.ds4idx_set_prefill_split.argtypes = [ctypes.c_int]
        L.ds4idx_set_prefill_split.restype = ctypes.c_int
        L.ds4idx_get_prefill_split.argtypes = []
        L.ds4idx_get_prefill_split.restype = ctypes.c_int
        L.ds4idx_workspace_bytes.argtypes = [P, i32, i32]
        L.ds4idx_workspace_bytes.restype = sz
        L.ds4idx_score.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.ds4idx_score.restype = ctypes.c_int
        L.ds4idx_topk.argtypes = [P, vp, i32, vp, vp, vp, sz, vp]
        L.ds4idx_topk.restype = ctypes.c_int
        L.ds4idx_select.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.ds4idx_select.restype = ctypes.c_int
        L.ds4idx_select_noalloc.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp]
        L.ds4idx_select_noalloc.restype = ctypes.c_int
        L.ds4idx_k_cache_write.argtypes = [vp, i32, ctypes.c_int64, i32, vp, vp, vp,
                                           ctypes.c_int64, vp]
        L.ds4idx_k_cache_write.restype = ctypes.c_int
        VP = ctypes.POINTER(VarlenProblem)
        L.ds4idx_varlen_workspace_bytes.argtypes = [VP, i32]
        L.ds4idx_varlen_workspace_bytes.restype = sz
        L.ds4idx_select_varlen.argtypes = [VP, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        L.ds4idx_select_varlen.restype = ctypes.c_int
        L.ds4idx_sparse_attention.argtypes = [ctypes.POINTER(AttnProblem), vp, vp, vp, vp, vp, vp]
        L.ds4idx_sparse_attention.restype = ctypes.c_int
        L.ds4idx_select_qfp8.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp]
        L.ds4idx_select_qfp8.restype = ctypes.c_int
        if L.ds4idx_abi_version() != ABI_VERSION:
            raise RuntimeError("libds4idx ABI version mismatch; rebuild the library")
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ds4idx_status_string(int(status)).decode()


def set_impl(impl) -> int:
    """Select the kernel family ('auto', 'ref', 'opt' or IMPL_*); returns the previous one."""
    if isinstance(impl, str):
        impl = {"auto": IMPL_AUTO, "ref": IMPL_REF, "opt": IMPL_OPT}[impl]
    prev = lib().ds4idx_set_impl(int(impl))
    if prev < 0:
        raise ValueError(f"unknown kernel family {impl}")
    return prev


def get_impl() -> int:
    return lib().ds4idx_get_impl()


def set_split(keys: int) -> int:
    """Fix the split-key kernel's partition length (8192, 12288 or 16384 keys;
    0 = automatic) for later calls; returns the previous value. Workspaces are
    sized for the length in force when they are created."""
    prev = lib().ds4idx_set_split(int(keys))
    if prev < 0:
        raise ValueError(f"unsupported partition length {keys}; use 0 or one of {SPLIT_LENS}")
    return prev


def get_split() -> int:
    return lib().ds4idx_get_split()


def set_prefill_split(keys: int) -> int:
    """Key parts for ragged prefill batches: 0 automatic, -1 never, or a part
    length in keys; returns the previous value. Workspaces are sized for the
    setting in force when they are created."""
    return lib().ds4idx_set_prefill_split(int(keys))


def get_prefill_split() -> int:
    return lib().ds4idx_get_prefill_split()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor, key: bool) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if key and t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return FP8_E4M3
    raise TypeError(f"unsupported {'key' if key else 'query'} dtype {t.dtype}")


def make_problem(q: torch.Tensor, k: torch.Tensor, causal_offset: int) -> Problem:
    if q.dim() != 4 or k.dim() != 3:
        raise ValueError("q must be [B,T,H,D] and k [B,S,D]")
    B, T, H, D = q.shape
    if k.shape[0] != B or k.shape[2] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    return Problem(B, T, k.shape[1], H, D, int(causal_offset), _dtype_code(q, False),
                   _dtype_code(k, True))


def _check_inputs(q, k, k_scale, w):
    for name, t in (("q", q), ("k", k), ("w", w)) + ((("k_scale", k_scale),) if k_scale is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    B, T, H, _ = q.shape
    if w.dtype != torch.float32 or tuple(w.shape) != (B, T, H):
        raise ValueError("w must be float32 [B,T,H]")
    if k_scale is not None and (k_scale.dtype != torch.float32 or tuple(k_scale.shape) != tuple(k.shape[:2])):
        raise ValueError("k_scale must be float32 [B,S]")


def _check_out(t: Optional[torch.Tensor], name: str, shape, dtype, device) -> None:
    """A caller-supplied output must have exactly the shape and dtype the
    kernels write, live on the inputs' device and be contiguous: the kernels
    write shape-many elements through its pointer."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")


def _check_workspace(ws: Optional[torch.Tensor], device) -> int:
    """Byte size of a caller-supplied workspace (the library checks it against
    what the call needs)."""
    if ws is None:
        return 0
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_cuda or ws.device != device \
            or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous 1-D uint8 tensor on {device}")
    return ws.numel()


def _zeros_on(n: int, device, stream) -> torch.Tensor:
    """n zero bytes allocated and cleared on `stream` (the stream the kernel
    that reads them is launched on), so the fill is ordered before it."""
    s = stream if stream is not None else torch.cuda.current_stream(device)
    if not isinstance(s, torch.cuda.Stream):
        s = torch.cuda.ExternalStream(int(s), device=device)
    with torch.cuda.stream(s):
        return torch.zeros(n, dtype=torch.uint8, device=device)


def workspace_bytes(problem: Problem, k: int, op: int = OP_SELECT) -> int:
    n = lib().ds4idx_workspace_bytes(ctypes.byref(problem), int(k), int(op))
    if n == ctypes.c_size_t(-1).value:
        raise Ds4idxError(ERR_INVALID_ARG, "ds4idx_workspace_bytes")
    return n


def new_workspace(problem: Problem, k: int, device=None, stream=None) -> Optional[torch.Tensor]:
    """A device workspace big enough for ds4idx_select (or None), zero-filled
    on `stream` (default: the current stream), the stream of the calls that
    will use it."""
    n = workspace_bytes(problem, k, OP_SELECT)
    if n == 0:
        return None
    return _zeros_on(n, torch.device(device or "cuda"), stream)


def score(q, k, k_scale, w, causal_offset: int, out: Optional[torch.Tensor] = None,
          stream=None) -> torch.Tensor:
    """scores [B,T,S] fp32: the indexer score of every visible key, -inf elsewhere."""
    _check_inputs(q, k, k_scale, w)
    p = make_problem(q, k, causal_offset)
    _check_out(out, "out", (p.B, p.T, p.S), torch.float32, q.device)
    if out is None:
        out = torch.empty((p.B, p.T, p.S), dtype=torch.float32, device=q.device)
    st = lib().ds4idx_score(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(k_scale), _ptr(w), _ptr(out),
                            _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_score")
    return out


def topk(scores: torch.Tensor, k: int, causal_offset: int, idx: Optional[torch.Tensor] = None,
         vals: Optional[torch.Tensor] = None, with_vals: bool = True,
         stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Top-k (ascending indices, -1 padded) of materialised scores [B,T,S]."""
    if scores.dtype != torch.float32 or scores.dim() != 3 or not scores.is_contiguous():
        raise ValueError("scores must be contiguous float32 [B,T,S]")
    B, T, S = scores.shape
    if not scores.is_cuda:
        raise ValueError("scores must be a device tensor")
    p = Problem(B, T, S, 1, 1, int(causal_offset), F32, F32)
    _check_out(idx, "idx", (B, T, k), torch.int32, scores.device)
    _check_out(vals, "vals", (B, T, k), torch.float32, scores.device)
    if idx is None:
        idx = torch.empty((B, T, k), dtype=torch.int32, device=scores.device)
    if vals is None and with_vals:
        vals = torch.empty((B, T, k), dtype=torch.float32, device=scores.device)
    st = lib().ds4idx_topk(ctypes.byref(p), _ptr(scores), int(k), _ptr(idx), _ptr(vals), None, 0,
                           _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_topk")
    return idx, vals


def select(q, k, k_scale, w, causal_offset: int, topk: int = 512,
           idx: Optional[torch.Tensor] = None, vals: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, with_vals: bool = True,
           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused indexer: (idx [B,T,topk] int32 ascending/-1 padded, vals fp32 or None)."""
    _check_inputs(q, k, k_scale, w)
    p = make_problem(q, k, causal_offset)
    _check_out(idx, "idx", (p.B, p.T, topk), torch.int32, q.device)
    _check_out(vals, "vals", (p.B, p.T, topk), torch.float32, q.device)
    if idx is None:
        idx = torch.empty((p.B, p.T, topk), dtype=torch.int32, device=q.device)
    if vals is None and with_vals:
        vals = torch.empty((p.B, p.T, topk), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_workspace(p, topk, q.device, stream)
    ws_bytes = _check_workspace(workspace, q.device)
    st = lib().ds4idx_select(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(k_scale), _ptr(w), int(topk),
                             _ptr(idx), _ptr(vals), _ptr(workspace), ws_bytes, _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_select")
    return idx, vals


def select_noalloc(q, k, k_scale, w, causal_offset: int, idx: torch.Tensor,
                   vals: Optional[torch.Tensor] = None, stream=None) -> None:
    """ds4idx_select without a workspace and without allocating: writes the
    caller's idx [B,T,topk] int32 (topk = idx.shape[-1]) and optional vals.
    The library's fixed per-GPU scratch array stands in for the workspace, so
    calls whose executions overlap on one GPU must not be made."""
    _check_inputs(q, k, k_scale, w)
    p = make_problem(q, k, causal_offset)
    if idx is None or idx.dim() != 3:
        raise ValueError("idx must be a preallocated [B,T,topk] int32 tensor")
    topk = idx.shape[-1]
    _check_out(idx, "idx", (p.B, p.T, topk), torch.int32, q.device)
    _check_out(vals, "vals", (p.B, p.T, topk), torch.float32, q.device)
    st = lib().ds4idx_select_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(k_scale), _ptr(w), int(topk),
                                     _ptr(idx), _ptr(vals), _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_select_noalloc")


def make_varlen_problem(q, k, cu_q, cu_k, max_k: int) -> VarlenProblem:
    if q.dim() != 3 or k.dim() != 2:
        raise ValueError("ragged q must be [total_q,H,D] and k [total_k,D]")
    total_q, H, D = q.shape
    if k.shape[1] != D:
        raise ValueError(f"k shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if cu_q.dim() != 1 or cu_k.dim() != 1 or cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_q and cu_k must be [B+1] prefix sums")
    return VarlenProblem(cu_q.numel() - 1, total_q, k.shape[0], int(max_k), H, D,
                         _dtype_code(q, False), _dtype_code(k, True))


def varlen_workspace_bytes(problem: VarlenProblem, k: int) -> int:
    n = lib().ds4idx_varlen_workspace_bytes(ctypes.byref(problem), int(k))
    if n == ctypes.c_size_t(-1).value:
        raise Ds4idxError(ERR_INVALID_ARG, "ds4idx_varlen_workspace_bytes")
    return n


def new_varlen_workspace(problem: VarlenProblem, k: int, device=None, stream=None) -> Optional[torch.Tensor]:
    """A device workspace big enough for ds4idx_select_varlen (or None),
    zero-filled on `stream` (default: the current stream)."""
    n = varlen_workspace_bytes(problem, k)
    return None if n == 0 else _zeros_on(n, torch.device(device or "cuda"), stream)


def select_varlen(q, k, k_scale, w, cu_q, cu_k, max_k: int, topk: int = 512,
                  idx: Optional[torch.Tensor] = None, vals: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, with_vals: bool = True,
                  stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Fused indexer over a ragged batch. q [total_q,H,D], k [total_k,D],
    k_scale [total_k] (fp8 keys), w [total_q,H]; cu_q int32 / cu_k int64 device
    prefix sums [B+1]; stream b's query t sees its keys s <= S_b - T_b + t.
    Returns (idx [total_q,topk] int32, stream-local, ascending, -1 padded; vals)."""
    for name, t in (("q", q), ("k", k), ("w", w), ("cu_q", cu_q), ("cu_k", cu_k)) + \
            ((("k_scale", k_scale),) if k_scale is not None else ()):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if cu_q.dtype != torch.int32 or cu_k.dtype != torch.int64:
        raise ValueError("cu_q must be int32 and cu_k int64")
    p = make_varlen_problem(q, k, cu_q, cu_k, max_k)
    if w.dtype != torch.float32 or tuple(w.shape) != (p.total_q, p.H):
        raise ValueError("w must be float32 [total_q,H]")
    if k_scale is not None and (k_scale.dtype != torch.float32 or tuple(k_scale.shape) != (p.total_k,)):
        raise ValueError("k_scale must be float32 [total_k]")
    for name, t in (("k", k), ("w", w), ("cu_q", cu_q), ("cu_k", cu_k)) + \
            ((("k_scale", k_scale),) if k_scale is not None else ()):
        if t.device != q.device:
            raise ValueError(f"{name} must be on {q.device}")
    _check_out(idx, "idx", (p.total_q, topk), torch.int32, q.device)
    _check_out(vals, "vals", (p.total_q, topk), torch.float32, q.device)
    if idx is None:
        idx = torch.empty((p.total_q, topk), dtype=torch.int32, device=q.device)
    if vals is None and with_vals:
        vals = torch.empty((p.total_q, topk), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = new_varlen_workspace(p, topk, q.device, stream)
    ws_bytes = _check_workspace(workspace, q.device)
    st = lib().ds4idx_select_varlen(ctypes.byref(p), _ptr(cu_q), _ptr(cu_k), _ptr(q), _ptr(k),
                                    _ptr(k_scale), _ptr(w), int(topk), _ptr(idx), _ptr(vals),
                                    _ptr(workspace), ws_bytes, _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_select_varlen")
    return idx, vals


def select_qfp8(q8, q_scale, k, k_scale, w, causal_offset: int, topk: int = 512,
                idx: Optional[torch.Tensor] = None, vals: Optional[torch.Tensor] = None,
                with_vals: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """fp8 x fp8 indexer: q8 [B,T,H,D] E4M3 codes (uint8 / float8_e4m3fn) with
    q_scale [B,T,H] fp32, k [B,S,D] E4M3 with k_scale [B,S], w [B,T,H] fp32."""
    for name, t in (("q8", q8), ("q_scale", q_scale), ("k", k), ("k_scale", k_scale), ("w", w)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if q8.dtype not in (torch.uint8, torch.float8_e4m3fn) or k.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError("q8 and k must hold E4M3 codes")
    B, T, H, D = q8.shape
    if tuple(q_scale.shape) != (B, T, H) or q_scale.dtype != torch.float32:
        raise ValueError("q_scale must be float32 [B,T,H]")
    if tuple(w.shape) != (B, T, H) or w.dtype != torch.float32:
        raise ValueError("w must be float32 [B,T,H]")
    if k.dim() != 3 or k.shape[0] != B or k.shape[2] != D or tuple(k_scale.shape) != tuple(k.shape[:2]):
        raise ValueError("k must be [B,S,D] with k_scale [B,S]")
    p = Problem(B, T, k.shape[1], H, D, int(causal_offset), FP8_E4M3, FP8_E4M3)
    for name, t in (("q_scale", q_scale), ("k", k), ("k_scale", k_scale), ("w", w)):
        if t.device != q8.device:
            raise ValueError(f"{name} must be on {q8.device}")
    if k_scale.dtype != torch.float32:
        raise ValueError("k_scale must be float32 [B,S]")
    _check_out(idx, "idx", (B, T, topk), torch.int32, q8.device)
    _check_out(vals, "vals", (B, T, topk), torch.float32, q8.device)
    if idx is None:
        idx = torch.empty((B, T, topk), dtype=torch.int32, device=q8.device)
    if vals is None and with_vals:
        vals = torch.empty((B, T, topk), dtype=torch.float32, device=q8.device)
    st = lib().ds4idx_select_qfp8(ctypes.byref(p), _ptr(q8), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w),
                                  int(topk), _ptr(idx), _ptr(vals), _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_select_qfp8")
    return idx, vals


def sparse_attention(q: torch.Tensor, kv: torch.Tensor, idx: torch.Tensor, softmax_scale: float,
                     d_v: int = 512, out: Optional[torch.Tensor] = None, with_lse: bool = True,
                     stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of each query token over its selected cache rows.

    q [B,T,H,d_qk] bf16, kv [B,S,d_qk] bf16 (key = whole row, value = first
    d_v columns), idx [B,T,k] int32 (-1 padding skipped). Returns
    (out [B,T,H,d_v] bf16, lse [B,T,H] fp32 or None)."""
    if q.dim() != 4 or kv.dim() != 3 or idx.dim() != 3:
        raise ValueError("q must be [B,T,H,d_qk], kv [B,S,d_qk] and idx [B,T,k]")
    B, T, H, dqk = q.shape
    if kv.shape[0] != B or kv.shape[2] != dqk or tuple(idx.shape[:2]) != (B, T):
        raise ValueError("q, kv and idx shapes do not match")
    if q.dtype != torch.bfloat16 or kv.dtype != torch.bfloat16 or idx.dtype != torch.int32:
        raise ValueError("q and kv must be bfloat16, idx int32")
    for name, t in (("q", q), ("kv", kv), ("idx", idx)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if kv.device != q.device or idx.device != q.device:
        raise ValueError(f"kv and idx must be on {q.device}")
    _check_out(out, "out", (B, T, H, d_v), torch.bfloat16, q.device)
    if out is None:
        out = torch.empty((B, T, H, d_v), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, T, H), dtype=torch.float32, device=q.device) if with_lse else None
    p = AttnProblem(B, T, kv.shape[1], H, idx.shape[2], dqk, int(d_v), float(softmax_scale))
    st = lib().ds4idx_sparse_attention(ctypes.byref(p), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse),
                                       _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_sparse_attention")
    return out, lse


def k_cache_write(k_new: torch.Tensor, cache: torch.Tensor, cache_scale: torch.Tensor,
                  slots: Optional[torch.Tensor] = None, stream=None) -> None:
    """Quantise k_new [n,D] (bf16/fp32) to E4M3 with one fp32 scale per token
    and store row i into cache[slots[i]] / cache_scale[slots[i]] (rows 0..n-1
    when slots is None). cache [rows,D] uint8 or float8_e4m3fn, cache_scale
    [rows] fp32. Slots outside [0, rows) are skipped."""
    if k_new.dim() != 2 or cache.dim() != 2 or cache_scale.dim() != 1:
        raise ValueError("k_new must be [n,D], cache [rows,D], cache_scale [rows]")
    n, D = k_new.shape
    if cache.shape[1] != D or cache_scale.shape[0] != cache.shape[0]:
        raise ValueError("cache and cache_scale do not match k_new")
    if cache.dtype not in (torch.uint8, torch.float8_e4m3fn) or cache_scale.dtype != torch.float32:
        raise ValueError("cache must be uint8/float8_e4m3fn and cache_scale float32")
    named = (("k_new", k_new), ("cache", cache), ("cache_scale", cache_scale))
    if slots is not None:
        if slots.dtype != torch.int64 or tuple(slots.shape) != (n,):
            raise ValueError("slots must be int64 [n]")
        named += (("slots", slots),)
    for name, t in named:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.device != k_new.device:
            raise ValueError(f"{name} must be on {k_new.device}")
    st = lib().ds4idx_k_cache_write(_ptr(k_new), _dtype_code(k_new, False), int(n), int(D),
                                    _ptr(slots), _ptr(cache), _ptr(cache_scale),
                                    int(cache.shape[0]), _stream(stream))
    if st != OK:
        raise Ds4idxError(st, "ds4idx_k_cache_write")
