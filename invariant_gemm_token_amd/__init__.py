"""Batch-invariant token logprobs on MI355X: Python binding of ``libtig.so``.

The functions named ``tig_*`` mirror the C entry points of ``include/tig.h``
one for one: they check that each tensor lives on the GPU with the dtype and
shape the C call expects, then pass raw device pointers, sizes and the current
HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no fallback: if ``libtig.so`` is missing or fails to load, every call
raises.  PyTorch is used only for device memory and streams.

``tree_gemm``, ``logprob_gather`` and ``moe_tree_gemm_combine`` are
conveniences that allocate the outputs and the workspace with torch and then
call the matching ``tig_*`` function.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "TigError", "load", "lib_path",
    "tig_tree_gemm", "tig_logprob_gather", "tig_logprob_workspace_bytes", "tig_logprob_gather_noalloc",
    "tig_moe_tree_gemm_combine", "tig_moe_workspace_bytes", "tig_moe_route", "tig_topk_positions",
    "tig_expert_gemm_masked", "tig_expert_gemm_contiguous", "tig_expert_workspace_bytes", "tig_silu_mul",
    "tig_fp8_quantize", "tig_fp8_tree_gemm", "tig_fp8_gemm_workspace_bytes", "tig_fp8_dequantize",
    "tig_silu_mul_fp8", "tig_expert_fp8_gemm_masked", "tig_expert_fp8_gemm_contiguous",
    "tig_expert_fp8_workspace_bytes",
    "tig_plan_describe",
    "tig_status_string", "tig_last_error",
    "tree_gemm", "logprob_gather", "moe_tree_gemm_combine", "moe_route", "topk_positions",
    "expert_gemm_masked", "expert_gemm_contiguous", "silu_mul", "fp8_quantize", "fp8_tree_gemm", "fp8_dequantize",
    "silu_mul_fp8", "expert_fp8_gemm_masked", "expert_fp8_gemm_contiguous",
    "TIG_OK", "TIG_ERR_INVALID_ARG", "TIG_ERR_UNSUPPORTED", "TIG_ERR_WORKSPACE", "TIG_ERR_HIP",
    "TIG_OUT_F32", "TIG_OUT_BF16",
]

TIG_OK, TIG_ERR_INVALID_ARG, TIG_ERR_UNSUPPORTED, TIG_ERR_WORKSPACE, TIG_ERR_HIP = range(5)
TIG_OUT_F32, TIG_OUT_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    """The in-tree ``libtig.so``, or the library named by ``$TIG_LIB`` (for example a
    sanitizer build of the host code used by the CPU tests)."""
    return os.environ.get("TIG_LIB") or os.path.join(_HERE, "libtig.so")


class TigError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {tig_status_string(status)} ({status}): {detail}")


class _Plan(ctypes.Structure):
    _fields_ = [
        ("version", ctypes.c_int32), ("leaves", ctypes.c_int32), ("leaf_len", ctypes.c_int32),
        ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("mfma_m", ctypes.c_int32), ("mfma_n", ctypes.c_int32), ("mfma_k", ctypes.c_int32),
        ("tree_id", ctypes.c_int32), ("digest", ctypes.c_uint8 * 32), ("policy", ctypes.c_char * 512),
    ]


_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

_SIGNATURES = {
    "tig_tree_gemm": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i32, _i64, _i64, _i64, _i32, _vp]),
    "tig_logprob_gather": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "tig_logprob_workspace_bytes": (_i32, [_i64, _i64, _i64, _i32, ctypes.POINTER(_sz)]),
    "tig_logprob_gather_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _vp]),
    "tig_moe_tree_gemm_combine": (_i32, [_vp, _vp, _i32, _vp, _vp, _i32, _vp, _i64, _i64, _i64,
                                         _i32, _vp, _sz, _vp]),
    "tig_moe_workspace_bytes": (_i32, [_i64, _i64, _i64, _i32, _i32, ctypes.POINTER(_sz)]),
    "tig_moe_route": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp]),
    "tig_topk_positions": (_i32, [_vp, _i64, _vp, _i64, _i32, _vp, _vp]),
    "tig_expert_gemm_masked": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "tig_expert_gemm_contiguous": (_i32, [_vp, _vp, _i64, _vp, _vp, _i32, _i32, _i64, _i64, _i64, _i32, _vp, _sz,
                                          _vp]),
    "tig_expert_workspace_bytes": (_i32, [_i64, _i32, ctypes.POINTER(_sz)]),
    "tig_silu_mul": (_i32, [_vp, _i64, _vp, _i64, _i64, _i64, _vp]),
    "tig_fp8_quantize": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i32, _vp]),
    "tig_fp8_tree_gemm": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i64, _i64, _i64, _i32, _vp, _sz, _vp]),
    "tig_fp8_gemm_workspace_bytes": (_i32, [_i64, _i64, _i64, ctypes.POINTER(_sz)]),
    "tig_fp8_dequantize": (_i32, [_vp, _vp, _vp, _i64, _i64, _i32, _vp]),
    "tig_silu_mul_fp8": (_i32, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp]),
    "tig_expert_fp8_gemm_masked": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i64, _i32, _vp, _sz,
                                          _vp]),
    "tig_expert_fp8_gemm_contiguous": (_i32, [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i64, _i64, _i64, _i32,
                                              _vp, _sz, _vp]),
    "tig_expert_fp8_workspace_bytes": (_i32, [_i64, _i32, _i64, _i64, ctypes.POINTER(_sz)]),
    "tig_plan_describe": (_i32, [_i64, _i32, ctypes.POINTER(_Plan)]),
    "tig_status_string": (ctypes.c_char_p, [_i32]),
    "tig_last_error": (ctypes.c_char_p, []),
}


def load():
    """Load ``libtig.so`` (once).  Raises if it is missing or does not load."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run `python -m invariant_gemm_token_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def tig_status_string(status: int) -> str:
    return load().tig_status_string(int(status)).decode()


def tig_last_error() -> str:
    return load().tig_last_error().decode()


def _check(status: int, where: str) -> None:
    if status != TIG_OK:
        raise TigError(status, where, tig_last_error())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream) -> int:
    torch = _torch()
    if stream is not None:
        return int(stream.cuda_stream)
    # The current stream's handle without building a Stream object (which costs
    # a few microseconds per call); the public route where that getter is absent.
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return int(raw(torch._C._cuda_getDevice()))
    return int(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")


def _rowmajor(t, name):
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")


def _contig(t, name):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on different devices: {sorted(map(str, devs))}")


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def tig_tree_gemm(A, W, C, leaves: int, stream=None) -> None:
    """``C[M, N] = leaf-tree(A[M, K] W[N, K]^T)``; C is float32 or bfloat16."""
    torch = _torch()
    _need(A, "A", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    if C.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("C must be float32 or bfloat16")
    _need(C, "C", C.dtype, 2)
    _same_device(A, W, C)
    for t, n in ((A, "A"), (W, "W"), (C, "C")):
        _rowmajor(t, n)
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shapes do not match: A {tuple(A.shape)}, W {tuple(W.shape)}, C {tuple(C.shape)}")
    out_dtype = TIG_OUT_F32 if C.dtype == torch.float32 else TIG_OUT_BF16
    # A single row has no row stride of its own: pass the packed one.
    lda = A.stride(0) if M > 1 else K
    ldw = W.stride(0) if N > 1 else K
    ldc = C.stride(0) if M > 1 else N
    st = load().tig_tree_gemm(A.data_ptr(), lda, W.data_ptr(), ldw, C.data_ptr(), ldc, out_dtype,
                              M, N, K, int(leaves), _stream(stream))
    _check(st, "tig_tree_gemm")


def tig_logprob_workspace_bytes(M: int, K: int, n_vocab: int, leaves: int) -> int:
    out = _sz(0)
    _check(load().tig_logprob_workspace_bytes(int(M), int(K), int(n_vocab), int(leaves),
                                              ctypes.byref(out)), "tig_logprob_workspace_bytes")
    return int(out.value)


def tig_logprob_gather(H, W, ids, logprob_out, lse_out, leaves: int, workspace, stream=None) -> None:
    """Logprob of each row's sampled token under softmax(H W^T); see include/tig.h."""
    torch = _torch()
    _need(H, "H", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(ids, "ids", torch.int64, 1)
    _need(logprob_out, "logprob_out", torch.float32, 1)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 1)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(H, W, ids, logprob_out, lse_out, workspace)
    for t, n in ((H, "H"), (W, "W"), (ids, "ids"), (logprob_out, "logprob_out"), (workspace, "workspace")):
        _contig(t, n)
    if lse_out is not None:
        _contig(lse_out, "lse_out")
    M, K = H.shape
    V = W.shape[0]
    if W.shape[1] != K or ids.shape[0] != M or logprob_out.shape[0] != M or (
            lse_out is not None and lse_out.shape[0] != M):
        raise ValueError("shapes do not match")
    st = load().tig_logprob_gather(H.data_ptr(), W.data_ptr(), ids.data_ptr(), logprob_out.data_ptr(),
                                   lse_out.data_ptr() if lse_out is not None else None, M, K, V,
                                   int(leaves), workspace.data_ptr(), workspace.numel(),
                                   _stream(stream))
    _check(st, "tig_logprob_gather")


def tig_logprob_gather_noalloc(H, W, ids, logprob_out, lse_out, leaves: int, stream=None) -> None:
    """tig_logprob_gather on the library's fixed device array instead of a workspace; see include/tig.h."""
    torch = _torch()
    _need(H, "H", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(ids, "ids", torch.int64, 1)
    _need(logprob_out, "logprob_out", torch.float32, 1)
    if lse_out is not None:
        _need(lse_out, "lse_out", torch.float32, 1)
    _same_device(H, W, ids, logprob_out, lse_out)
    for t, n in ((H, "H"), (W, "W"), (ids, "ids"), (logprob_out, "logprob_out")):
        _contig(t, n)
    if lse_out is not None:
        _contig(lse_out, "lse_out")
    M, K = H.shape
    V = W.shape[0]
    if W.shape[1] != K or ids.shape[0] != M or logprob_out.shape[0] != M or (
            lse_out is not None and lse_out.shape[0] != M):
        raise ValueError("shapes do not match")
    st = load().tig_logprob_gather_noalloc(H.data_ptr(), W.data_ptr(), ids.data_ptr(), logprob_out.data_ptr(),
                                           lse_out.data_ptr() if lse_out is not None else None, M, K, V,
                                           int(leaves), _stream(stream))
    _check(st, "tig_logprob_gather_noalloc")


def tig_moe_workspace_bytes(T: int, N: int, K: int, n_experts: int, topk: int) -> int:
    out = _sz(0)
    _check(load().tig_moe_workspace_bytes(int(T), int(N), int(K), int(n_experts), int(topk),
                                          ctypes.byref(out)), "tig_moe_workspace_bytes")
    return int(out.value)


def tig_moe_tree_gemm_combine(H, W_experts, topk_ids, topk_w, out, leaves: int, workspace,
                              stream=None) -> None:
    """MoE-shaped leaf-tree contraction plus ascending-expert-id FP32 combine."""
    torch = _torch()
    _need(H, "H", torch.bfloat16, 2)
    _need(W_experts, "W_experts", torch.bfloat16, 3)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    _need(out, "out", torch.float32, 2)
    _need(workspace, "workspace", torch.uint8, 1)
    _same_device(H, W_experts, topk_ids, topk_w, out, workspace)
    for t, n in ((H, "H"), (W_experts, "W_experts"), (topk_ids, "topk_ids"), (topk_w, "topk_w"),
                 (out, "out"), (workspace, "workspace")):
        _contig(t, n)
    T, K = H.shape
    E, N, K2 = W_experts.shape
    topk = topk_ids.shape[1]
    if K2 != K or tuple(topk_ids.shape) != (T, topk) or tuple(topk_w.shape) != (T, topk) or tuple(
            out.shape) != (T, N):
        raise ValueError("shapes do not match")
    st = load().tig_moe_tree_gemm_combine(H.data_ptr(), W_experts.data_ptr(), E, topk_ids.data_ptr(),
                                          topk_w.data_ptr(), topk, out.data_ptr(), T, N, K, int(leaves),
                                          workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "tig_moe_tree_gemm_combine")


def tig_moe_route(H, Wr, logits, topk_ids, topk_w, leaves: int, stream=None) -> None:
    """MoE router: FP32 leaf-tree logits, top-k (ties to the lower id) and softmax gates."""
    torch = _torch()
    _need(H, "H", torch.bfloat16, 2)
    _need(Wr, "Wr", torch.bfloat16, 2)
    _need(logits, "logits", torch.float32, 2)
    _need(topk_ids, "topk_ids", torch.int32, 2)
    _need(topk_w, "topk_w", torch.float32, 2)
    _same_device(H, Wr, logits, topk_ids, topk_w)
    for t, n in ((H, "H"), (Wr, "Wr"), (logits, "logits"), (topk_ids, "topk_ids"), (topk_w, "topk_w")):
        _contig(t, n)
    T, K = H.shape
    E, K2 = Wr.shape
    topk = topk_ids.shape[1]
    if K2 != K or tuple(logits.shape) != (T, E) or tuple(topk_ids.shape) != (T, topk) or tuple(
            topk_w.shape) != (T, topk):
        raise ValueError("shapes do not match")
    st = load().tig_moe_route(H.data_ptr(), Wr.data_ptr(), logits.data_ptr(), topk_ids.data_ptr(),
                              topk_w.data_ptr(), T, K, E, topk, int(leaves), _stream(stream))
    _check(st, "tig_moe_route")


def tig_expert_workspace_bytes(rows: int, n_experts: int) -> int:
    out = _sz(0)
    _check(load().tig_expert_workspace_bytes(int(rows), int(n_experts), ctypes.byref(out)),
           "tig_expert_workspace_bytes")
    return int(out.value)


def _expert_args(X, counts, W, Y):
    torch = _torch()
    _need(X, "X", torch.bfloat16, X.dim())
    _need(W, "W", torch.bfloat16, 3)
    _need(counts, "counts", torch.int32, 1)
    if Y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("Y must be float32 or bfloat16")
    _same_device(X, W, counts, Y)
    for t, n in ((X, "X"), (W, "W"), (counts, "counts"), (Y, "Y")):
        _contig(t, n)
    E, N, K = W.shape
    if counts.shape[0] != E:
        raise ValueError("counts must have one entry per expert")
    if X.shape[-1] != K or Y.shape[-1] != N or X.shape[:-1] != Y.shape[:-1]:
        raise ValueError(f"shapes do not match: X {tuple(X.shape)}, W {tuple(W.shape)}, Y {tuple(Y.shape)}")
    return E, N, K, (TIG_OUT_F32 if Y.dtype == torch.float32 else TIG_OUT_BF16)


def tig_expert_gemm_masked(X, counts, W, Y, leaves: int, workspace, stream=None) -> None:
    """Masked layout: X ``[E, cap, K]``, Y ``[E, cap, N]``; expert e's first counts[e] rows of its block."""
    if X.dim() != 3:
        raise ValueError("X must be [n_experts, cap, K]")
    E, N, K, od = _expert_args(X, counts, W, Y)
    if X.shape[0] != E:
        raise ValueError("X must have one block per expert")
    st = load().tig_expert_gemm_masked(X.data_ptr(), counts.data_ptr(), W.data_ptr(), Y.data_ptr(), od, E,
                                       X.shape[1], N, K, int(leaves), workspace.data_ptr(), workspace.numel(),
                                       _stream(stream))
    _check(st, "tig_expert_gemm_masked")


def tig_expert_gemm_contiguous(X, counts, W, Y, align: int, leaves: int, workspace, stream=None) -> None:
    """Contiguous layout: X ``[M, K]``, Y ``[M, N]``; experts packed in order, segments aligned to ``align``."""
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    E, N, K, od = _expert_args(X, counts, W, Y)
    st = load().tig_expert_gemm_contiguous(X.data_ptr(), counts.data_ptr(), int(align), W.data_ptr(),
                                           Y.data_ptr(), od, E, X.shape[0], N, K, int(leaves),
                                           workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "tig_expert_gemm_contiguous")


def tig_silu_mul(GU, out, stream=None) -> None:
    """``out[r, i] = bf16(SiLU(GU[r, i]) * GU[r, I + i])`` computed in FP32, one rounding."""
    torch = _torch()
    _need(GU, "GU", torch.float32, 2)
    _need(out, "out", torch.bfloat16, 2)
    _same_device(GU, out)
    _rowmajor(GU, "GU")
    _rowmajor(out, "out")
    rows, I = out.shape
    if GU.shape[0] != rows or GU.shape[1] != 2 * I:
        raise ValueError("GU must be [rows, 2 I] for out [rows, I]")
    ldgu = GU.stride(0) if rows > 1 else 2 * I
    ldo = out.stride(0) if rows > 1 else I
    st = load().tig_silu_mul(GU.data_ptr(), ldgu, out.data_ptr(), ldo, rows, I, _stream(stream))
    _check(st, "tig_silu_mul")


def tig_expert_fp8_workspace_bytes(rows: int, n_experts: int, N: int, K: int) -> int:
    out = _sz(0)
    _check(load().tig_expert_fp8_workspace_bytes(int(rows), int(n_experts), int(N), int(K), ctypes.byref(out)),
           "tig_expert_fp8_workspace_bytes")
    return int(out.value)


def _expert_fp8_args(QX, SX, counts, QW, SW, Y):
    torch = _torch()
    for t, n in ((QX, "QX"), (SX, "SX"), (QW, "QW"), (SW, "SW")):
        _need(t, n, torch.uint8, t.dim())
        _contig(t, n)
    _need(counts, "counts", torch.int32, 1)
    if Y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("Y must be float32 or bfloat16")
    _same_device(QX, SX, counts, QW, SW, Y)
    _contig(counts, "counts")
    _contig(Y, "Y")
    if QW.dim() != 3 or SW.dim() != 3:
        raise ValueError("QW must be [E, N, K] and SW [E, ceil(N/128), K/128]")
    E, N, K = QW.shape
    if counts.shape[0] != E or tuple(SW.shape) != (E, -(-N // 128), -(-K // 128)):
        raise ValueError("counts, QW and SW do not match")
    if QX.shape[-1] != K or SX.shape[-1] != -(-K // 128) or Y.shape[-1] != N or QX.shape[:-1] != Y.shape[:-1] or \
            SX.shape[:-1] != QX.shape[:-1]:
        raise ValueError("QX, SX and Y do not match")
    return E, N, K, (TIG_OUT_F32 if Y.dtype == torch.float32 else TIG_OUT_BF16)


def tig_expert_fp8_gemm_masked(QX, SX, counts, QW, SW, Y, leaves: int, workspace, stream=None) -> None:
    """Masked layout in block FP8: QX ``[E, cap, K]``, SX ``[E, cap, K/128]``, Y ``[E, cap, N]``."""
    if QX.dim() != 3:
        raise ValueError("QX must be [n_experts, cap, K]")
    E, N, K, od = _expert_fp8_args(QX, SX, counts, QW, SW, Y)
    st = load().tig_expert_fp8_gemm_masked(QX.data_ptr(), SX.data_ptr(), counts.data_ptr(), QW.data_ptr(),
                                           SW.data_ptr(), Y.data_ptr(), od, E, QX.shape[1], N, K, int(leaves),
                                           workspace.data_ptr(), workspace.numel(), _stream(stream))
    _check(st, "tig_expert_fp8_gemm_masked")


def tig_expert_fp8_gemm_contiguous(QX, SX, counts, QW, SW, Y, align: int, leaves: int, workspace,
                                   stream=None) -> None:
    """Contiguous layout in block FP8: QX ``[M, K]``, SX ``[M, K/128]``, Y ``[M, N]``."""
    if QX.dim() != 2:
        raise ValueError("QX must be [M, K]")
    E, N, K, od = _expert_fp8_args(QX, SX, counts, QW, SW, Y)
    st = load().tig_expert_fp8_gemm_contiguous(QX.data_ptr(), SX.data_ptr(), counts.data_ptr(), int(align),
                                               QW.data_ptr(), SW.data_ptr(), Y.data_ptr(), od, E, QX.shape[0], N, K,
                                               int(leaves), workspace.data_ptr(), workspace.numel(),
                                               _stream(stream))
    _check(st, "tig_expert_fp8_gemm_contiguous")


def tig_silu_mul_fp8(GU, Q, scales, stream=None) -> None:
    """``bf16(SiLU(g) u)`` (one rounding), then block FP8 in 1 x 128 blocks per row."""
    torch = _torch()
    _need(GU, "GU", torch.float32, 2)
    _need(Q, "Q", torch.uint8, 2)
    _need(scales, "scales", torch.uint8, 2)
    _same_device(GU, Q, scales)
    _rowmajor(GU, "GU")
    _rowmajor(Q, "Q")
    _contig(scales, "scales")
    rows, I = Q.shape
    if GU.shape[0] != rows or GU.shape[1] != 2 * I or tuple(scales.shape) != (rows, -(-I // 128)):
        raise ValueError("GU must be [rows, 2 I], Q [rows, I] and scales [rows, ceil(I/128)]")
    ldgu = GU.stride(0) if rows > 1 else 2 * I
    ldq = Q.stride(0) if rows > 1 else I
    st = load().tig_silu_mul_fp8(GU.data_ptr(), ldgu, Q.data_ptr(), ldq, scales.data_ptr(), rows, I,
                                 _stream(stream))
    _check(st, "tig_silu_mul_fp8")


def tig_fp8_quantize(X, Q, scales, block_rows: int, stream=None) -> None:
    """Block FP8 (E4M3, power-of-two block scales as E8M0 bytes) of bf16 ``X [R, C]``."""
    torch = _torch()
    _need(X, "X", torch.bfloat16, 2)
    _need(Q, "Q", torch.uint8, 2)
    _need(scales, "scales", torch.uint8, 2)
    _same_device(X, Q, scales)
    _rowmajor(X, "X")
    _rowmajor(Q, "Q")
    _contig(scales, "scales")
    R, C = X.shape
    br = int(block_rows)
    if tuple(Q.shape) != (R, C) or tuple(scales.shape) != (-(-R // br) if br > 0 else 0, -(-C // 128)):
        raise ValueError("Q must be [R, C] and scales [ceil(R/block_rows), ceil(C/128)]")
    ldx = X.stride(0) if R > 1 else C
    ldq = Q.stride(0) if R > 1 else C
    st = load().tig_fp8_quantize(X.data_ptr(), ldx, Q.data_ptr(), ldq, scales.data_ptr(), R, C, br,
                                 _stream(stream))
    _check(st, "tig_fp8_quantize")


def tig_fp8_dequantize(Q, scales, out, block_rows: int, stream=None) -> None:
    """``out`` (bf16) = the E4M3 values of ``Q`` times their blocks' scales (exact)."""
    torch = _torch()
    _need(Q, "Q", torch.uint8, 2)
    _need(scales, "scales", torch.uint8, 2)
    _need(out, "out", torch.bfloat16, 2)
    _same_device(Q, scales, out)
    for t, n in ((Q, "Q"), (scales, "scales"), (out, "out")):
        _contig(t, n)
    R, C = Q.shape
    if tuple(out.shape) != (R, C):
        raise ValueError("out must have Q's shape")
    st = load().tig_fp8_dequantize(Q.data_ptr(), scales.data_ptr(), out.data_ptr(), R, C, int(block_rows),
                                   _stream(stream))
    _check(st, "tig_fp8_dequantize")


def tig_fp8_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    out = _sz(0)
    _check(load().tig_fp8_gemm_workspace_bytes(int(M), int(N), int(K), ctypes.byref(out)),
           "tig_fp8_gemm_workspace_bytes")
    return int(out.value)


def tig_fp8_tree_gemm(QA, SA, QW, SW, C, leaves: int, workspace, stream=None) -> None:
    """``C = leaf-tree(dequant(A) dequant(W)^T)`` (W8A8 block FP8)."""
    torch = _torch()
    for t, n in ((QA, "QA"), (SA, "SA"), (QW, "QW"), (SW, "SW")):
        _need(t, n, torch.uint8, 2)
        _contig(t, n)
    if C.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("C must be float32 or bfloat16")
    _need(C, "C", C.dtype, 2)
    _rowmajor(C, "C")
    _same_device(QA, SA, QW, SW, C)
    M, K = QA.shape
    N = QW.shape[0]
    if QW.shape[1] != K or tuple(C.shape) != (M, N) or tuple(SA.shape) != (M, -(-K // 128)) or \
            tuple(SW.shape) != (-(-N // 128), -(-K // 128)):
        raise ValueError("shapes do not match")
    od = TIG_OUT_F32 if C.dtype == torch.float32 else TIG_OUT_BF16
    ldc = C.stride(0) if M > 1 else N
    st = load().tig_fp8_tree_gemm(QA.data_ptr(), SA.data_ptr(), QW.data_ptr(), SW.data_ptr(), C.data_ptr(), ldc,
                                  od, M, N, K, int(leaves), workspace.data_ptr(), workspace.numel(),
                                  _stream(stream))
    _check(st, "tig_fp8_tree_gemm")


def tig_topk_positions(scores, lengths, out, stream=None) -> None:
    """Top-k positions per row by (score, position), listed by descending position, -1 padded."""
    torch = _torch()
    _need(scores, "scores", torch.float32, 2)
    _need(lengths, "lengths", torch.int32, 1)
    _need(out, "out", torch.int32, 2)
    _same_device(scores, lengths, out)
    _contig(scores, "scores")
    _contig(lengths, "lengths")
    _contig(out, "out")
    R, ld = scores.shape
    if lengths.shape[0] != R or out.shape[0] != R:
        raise ValueError("scores, lengths and out must have the same number of rows")
    st = load().tig_topk_positions(scores.data_ptr(), ld, lengths.data_ptr(), R, out.shape[1], out.data_ptr(),
                                   _stream(stream))
    _check(st, "tig_topk_positions")


def tig_plan_describe(K: int, leaves: int) -> dict:
    plan = _Plan()
    _check(load().tig_plan_describe(int(K), int(leaves), ctypes.byref(plan)), "tig_plan_describe")
    d = {f: getattr(plan, f) for f, _ in _Plan._fields_ if f not in ("digest", "policy")}
    d["digest"] = bytes(plan.digest).hex()
    d["policy"] = plan.policy.decode()
    return d


# ---------------------------------------------------------------------------
# conveniences (allocate outputs / workspace with torch, then call the above)
# ---------------------------------------------------------------------------

def tree_gemm(A, W, leaves: int, out_dtype=None, stream=None):
    torch = _torch()
    C = torch.empty((A.shape[0], W.shape[0]), dtype=out_dtype or torch.float32, device=A.device)
    tig_tree_gemm(A, W, C, leaves, stream)
    return C


def logprob_gather(H, W, ids, leaves: int, workspace=None, with_lse: bool = True, stream=None):
    torch = _torch()
    M, K = H.shape
    need = tig_logprob_workspace_bytes(M, K, W.shape[0], leaves)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    lp = torch.empty(M, dtype=torch.float32, device=H.device)
    lse = torch.empty(M, dtype=torch.float32, device=H.device) if with_lse else None
    tig_logprob_gather(H, W, ids, lp, lse, leaves, workspace, stream)
    return lp, lse


def moe_route(H, Wr, topk: int, leaves: int, stream=None):
    """Allocate and return (logits, topk_ids, topk_w) of tig_moe_route."""
    torch = _torch()
    T = H.shape[0]
    E = Wr.shape[0]
    logits = torch.empty((T, E), dtype=torch.float32, device=H.device)
    ids = torch.empty((T, topk), dtype=torch.int32, device=H.device)
    w = torch.empty((T, topk), dtype=torch.float32, device=H.device)
    tig_moe_route(H, Wr, logits, ids, w, leaves, stream)
    return logits, ids, w


def moe_tree_gemm_combine(H, W_experts, topk_ids, topk_w, leaves: int, workspace=None, stream=None):
    torch = _torch()
    T, K = H.shape
    E, N, _ = W_experts.shape
    need = tig_moe_workspace_bytes(T, N, K, E, topk_ids.shape[1])
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    out = torch.empty((T, N), dtype=torch.float32, device=H.device)
    tig_moe_tree_gemm_combine(H, W_experts, topk_ids, topk_w, out, leaves, workspace, stream)
    return out


def topk_positions(scores, lengths, k: int, stream=None):
    """Allocate and return the ``[R, k]`` int32 output of tig_topk_positions."""
    torch = _torch()
    out = torch.empty((scores.shape[0], int(k)), dtype=torch.int32, device=scores.device)
    tig_topk_positions(scores, lengths, out, stream)
    return out


def _expert_ws(rows, n_experts, device, workspace):
    torch = _torch()
    need = tig_expert_workspace_bytes(rows, n_experts)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def expert_gemm_masked(X, counts, W, leaves: int, out_dtype=None, workspace=None, stream=None):
    """Allocate and return Y ``[E, cap, N]`` of tig_expert_gemm_masked."""
    torch = _torch()
    E, cap = X.shape[0], X.shape[1]
    Y = torch.empty((E, cap, W.shape[1]), dtype=out_dtype or torch.float32, device=X.device)
    tig_expert_gemm_masked(X, counts, W, Y, leaves, _expert_ws(E * cap, E, X.device, workspace), stream)
    return Y


def expert_gemm_contiguous(X, counts, W, align: int, leaves: int, out_dtype=None, workspace=None, stream=None):
    """Allocate and return Y ``[M, N]`` of tig_expert_gemm_contiguous."""
    torch = _torch()
    Y = torch.empty((X.shape[0], W.shape[1]), dtype=out_dtype or torch.float32, device=X.device)
    tig_expert_gemm_contiguous(X, counts, W, Y, align, leaves,
                               _expert_ws(X.shape[0], W.shape[0], X.device, workspace), stream)
    return Y


def silu_mul(GU, stream=None):
    """Allocate and return the bf16 ``[rows, I]`` output of tig_silu_mul."""
    torch = _torch()
    out = torch.empty((GU.shape[0], GU.shape[1] // 2), dtype=torch.bfloat16, device=GU.device)
    tig_silu_mul(GU, out, stream)
    return out


def fp8_quantize(X, block_rows: int, stream=None):
    """Allocate and return ``(Q, scales)`` of tig_fp8_quantize."""
    torch = _torch()
    R, C = X.shape
    Q = torch.empty((R, C), dtype=torch.uint8, device=X.device)
    S = torch.empty((-(-R // int(block_rows)), -(-C // 128)), dtype=torch.uint8, device=X.device)
    tig_fp8_quantize(X, Q, S, block_rows, stream)
    return Q, S


def fp8_tree_gemm(QA, SA, QW, SW, leaves: int, out_dtype=None, workspace=None, stream=None):
    """Allocate and return C ``[M, N]`` of tig_fp8_tree_gemm."""
    torch = _torch()
    M, K = QA.shape
    N = QW.shape[0]
    need = tig_fp8_gemm_workspace_bytes(M, N, K)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=QA.device)
    C = torch.empty((M, N), dtype=out_dtype or torch.float32, device=QA.device)
    tig_fp8_tree_gemm(QA, SA, QW, SW, C, leaves, workspace, stream)
    return C


def fp8_dequantize(Q, scales, block_rows: int, stream=None):
    """Allocate and return the bf16 output of tig_fp8_dequantize."""
    torch = _torch()
    out = torch.empty(Q.shape, dtype=torch.bfloat16, device=Q.device)
    tig_fp8_dequantize(Q, scales, out, block_rows, stream)
    return out


def silu_mul_fp8(GU, stream=None):
    """Allocate and return ``(Q, scales)`` of tig_silu_mul_fp8."""
    torch = _torch()
    rows, I = GU.shape[0], GU.shape[1] // 2
    Q = torch.empty((rows, I), dtype=torch.uint8, device=GU.device)
    S = torch.empty((rows, -(-I // 128)), dtype=torch.uint8, device=GU.device)
    tig_silu_mul_fp8(GU, Q, S, stream)
    return Q, S


def _expert_fp8_ws(rows, E, N, K, device, workspace):
    torch = _torch()
    need = tig_expert_fp8_workspace_bytes(rows, E, N, K)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return workspace


def expert_fp8_gemm_masked(QX, SX, counts, QW, SW, leaves: int, out_dtype=None, workspace=None, stream=None):
    """Allocate and return Y ``[E, cap, N]`` of tig_expert_fp8_gemm_masked."""
    torch = _torch()
    E, cap, K = QX.shape
    N = QW.shape[1]
    Y = torch.empty((E, cap, N), dtype=out_dtype or torch.float32, device=QX.device)
    tig_expert_fp8_gemm_masked(QX, SX, counts, QW, SW, Y, leaves,
                               _expert_fp8_ws(E * cap, E, N, K, QX.device, workspace), stream)
    return Y


def expert_fp8_gemm_contiguous(QX, SX, counts, QW, SW, align: int, leaves: int, out_dtype=None, workspace=None,
                               stream=None):
    """Allocate and return Y ``[M, N]`` of tig_expert_fp8_gemm_contiguous."""
    torch = _torch()
    M, K = QX.shape
    E, N = QW.shape[0], QW.shape[1]
    Y = torch.empty((M, N), dtype=out_dtype or torch.float32, device=QX.device)
    tig_expert_fp8_gemm_contiguous(QX, SX, counts, QW, SW, Y, align, leaves,
                                   _expert_fp8_ws(M, E, N, K, QX.device, workspace), stream)
    return Y
