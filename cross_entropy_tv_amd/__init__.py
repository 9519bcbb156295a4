"""Fused cross-entropy + total-variation-distance loss for MI355X (gfx950).

Thin Python binding over the C ABI declared in ``include/lx_ce_tvd.h``: every
function here has the name of the C entry point it calls and only marshals
arguments (PyTorch tensors supply device memory and the HIP stream).  All of
the loss is computed by the HIP kernels in ``liblx_ce_tvd.so``; there is no
other code path.  Importing this package fails if the library is not built
(``python cross_entropy_tv_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblx_ce_tvd.so")

LX_OK = 0
LX_ERR_INVALID_ARG = 1
LX_ERR_UNSUPPORTED_DTYPE = 2
LX_ERR_ALIAS = 3
LX_ERR_WORKSPACE = 4
LX_ERR_HIP = 5
LX_ERR_TOO_LARGE = 6
LX_F32 = 0
LX_BF16 = 1
LX_F16 = 2


class LxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = lib.lx_status_string(status).decode()
        extra = f" (hipError {lib.lx_last_hip_error()})" if status == LX_ERR_HIP else ""
        super().__init__(f"{where}: {name}{extra}")


def _load() -> ctypes.CDLL:
    # PyTorch-ROCm ships its own HIP runtime and links it as "libamdhip64.so";
    # the library links "libamdhip64.so.7".  Importing torch first puts torch's
    # runtime in the process under that soname, so the library binds to it.
    # Loading the library first would start a second HIP runtime, whose
    # launches then fail with hipErrorNoDevice.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python cross_entropy_tv_amd/build.py` "
                          "(the HIP library is the only implementation)")
    L = ctypes.CDLL(LIB_PATH)
    p, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    L.lx_status_string.argtypes = [i32]
    L.lx_status_string.restype = ctypes.c_char_p
    L.lx_abi_version.argtypes = []
    L.lx_abi_version.restype = i32
    L.lx_last_hip_error.argtypes = []
    L.lx_last_hip_error.restype = i32
    L.lx_ce_tvd_workspace_bytes.argtypes = [i64, i64, i32, i32]
    L.lx_ce_tvd_workspace_bytes.restype = sz
    L.lx_ce_tvd_forward.argtypes = [p, p, p, i64, i64, i64, p, p, p, p, p, i32, p, sz, p]
    L.lx_ce_tvd_forward.restype = i32
    L.lx_ce_tvd_backward.argtypes = [p, p, p, p, i64, i64, i64, p, p, p, f32, f32, p, i32, p]
    L.lx_ce_tvd_backward.restype = i32
    L.lx_ce_tvd_reduce_mean.argtypes = [p, p, p, i64, i64, p, p, p, p]
    L.lx_ce_tvd_reduce_mean.restype = i32
    L.lx_ce_tvd_forward_backward_workspace_bytes.argtypes = [i64, i64, i32, i32]
    L.lx_ce_tvd_forward_backward_workspace_bytes.restype = sz
    L.lx_ce_tvd_forward_backward.argtypes = [p, p, p, i64, i64, i64, p, p, p, p, p, p, f32, f32, p, i32, p, sz, p]
    L.lx_ce_tvd_forward_backward.restype = i32
    L.lx_ce_tvd_forward_backward_noalloc.argtypes = [p, p, p, i64, i64, i64, p, p, p, p, p, p, f32, f32, p, i32, p]
    L.lx_ce_tvd_forward_backward_noalloc.restype = i32
    L.lx_stream_read.argtypes = [p, i64, p, p]
    L.lx_stream_read.restype = i32
    L.lx_stream_read2_write.argtypes = [p, p, p, i64, p]
    L.lx_stream_read2_write.restype = i32
    L.lx_ce_tvd_count_valid.argtypes = [p, i64, i64, p, p, p]
    L.lx_ce_tvd_count_valid.restype = i32
    L.lx_ce_tvd_vp_stats.argtypes = [p, p, p, i64, i64, i64, i64, i32, p, p]
    L.lx_ce_tvd_vp_stats.restype = i32
    L.lx_ce_tvd_vp_merge_stats.argtypes = [p, i64, p, i64, i64, i64, i32, p, p, p, p]
    L.lx_ce_tvd_vp_merge_stats.restype = i32
    L.lx_ce_tvd_vp_tv.argtypes = [p, p, p, i64, i64, i64, p, p, i32, p, p]
    L.lx_ce_tvd_vp_tv.restype = i32
    L.lx_ce_tvd_vp_merge_tv.argtypes = [p, i64, p, i64, i64, p, p, p]
    L.lx_ce_tvd_vp_merge_tv.restype = i32
    L.lx_ce_tvd_backward_shard.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, p, p, p, f32, f32, p, i32, p]
    L.lx_ce_tvd_backward_shard.restype = i32
    L.lx_ce_tvd_forward_ex.argtypes = [p, i64, p, i64, p, i64, i64, i64, p, p, p, p, p, i32, p, sz, p]
    L.lx_ce_tvd_forward_ex.restype = i32
    L.lx_ce_tvd_backward_ex.argtypes = [p, i64, p, i64, p, i64, p, i64, i64, i64, p, p, p, f32, f32, p, p, p, i32, p]
    L.lx_ce_tvd_backward_ex.restype = i32
    L.lx_ce_tvd_forward_backward_ex.argtypes = [p, i64, p, i64, p, i64, i64, i64, p, p, p, p, p, p, i64, f32, f32,
                                                p, p, p, i32, p, sz, p]
    L.lx_ce_tvd_forward_backward_ex.restype = i32
    L.lx_gemm_bf16.argtypes = [p, i64, i32, p, i64, i32, p, i64, i64, i64, i64, i32, p]
    L.lx_gemm_bf16.restype = i32
    L.lx_ce_tvd_linear_workspace_bytes.argtypes = [i64, i64, i64, i32, i64]
    L.lx_ce_tvd_linear_workspace_bytes.restype = sz
    L.lx_ce_tvd_linear_forward_backward.argtypes = [p, p, i64, p, p, i64, p, i64, i64, i64, p, p, p, p, p, p, p,
                                                    f32, f32, p, i64, p, sz, p]
    L.lx_ce_tvd_linear_forward_backward.restype = i32
    return L


lib = _load()


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t):
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return LX_BF16
    if t.dtype == torch.float32:
        return LX_F32
    if t.dtype == torch.float16:
        return LX_F16
    raise TypeError(f"logits must be bfloat16, float16 or float32, got {t.dtype}")


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _logits2d(t, name):
    if t.dim() != 2 or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous 2-D (BT, V) device tensor")
    return t.shape


def _rows2d(t, name):
    """(BT, V, row stride) of a 2-D device tensor whose rows are contiguous."""
    if t.dim() != 2 or not t.is_cuda or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D (BT, V) device tensor with contiguous rows")
    BT, V = t.shape
    return BT, V, (t.stride(0) if BT > 1 else V)


def _check(status: int, where: str) -> None:
    if status != LX_OK:
        raise LxError(status, where)


# ------------------------------------------------------------------ entry points

def lx_status_string(status: int) -> str:
    return lib.lx_status_string(status).decode()


def lx_abi_version() -> int:
    return lib.lx_abi_version()


def lx_ce_tvd_workspace_bytes(BT: int, V: int, dt: int, has_teacher: bool) -> int:
    return lib.lx_ce_tvd_workspace_bytes(BT, V, dt, int(bool(has_teacher)))


def lx_ce_tvd_forward(student, teacher, target, ignore_index, ce, tvd, lse_s, lse_t, sigma,
                      workspace=None, stream=None) -> None:
    """Forward pass into the caller's float32 [BT] output tensors (tvd, lse_t, sigma
    may be None in CE-only mode, i.e. teacher=None).  ``workspace`` is a uint8
    device tensor of at least lx_ce_tvd_workspace_bytes bytes; when None and the
    shape needs one, it is allocated here with torch."""
    BT, V = _logits2d(student, "student")
    dt = _dtype_code(student)
    if teacher is not None and (teacher.shape != student.shape or teacher.dtype != student.dtype):
        raise ValueError("teacher must match student in shape and dtype")
    need = lx_ce_tvd_workspace_bytes(BT, V, dt, teacher is not None)
    if workspace is None and need:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=student.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lx_ce_tvd_forward(_ptr(student), _ptr(teacher), _ptr(target), BT, V, int(ignore_index),
                                 _ptr(ce), _ptr(tvd), _ptr(lse_s), _ptr(lse_t), _ptr(sigma), dt,
                                 _ptr(workspace), wbytes, _stream(stream)), "lx_ce_tvd_forward")


def lx_ce_tvd_backward(grad, student, teacher, target, ignore_index, lse_s, lse_t, sigma,
                       g_ce: float, g_tvd: float, g_scale=None, stream=None) -> None:
    """Backward pass into ``grad`` (may be ``student`` itself).  ``g_scale`` is an
    optional float32 device tensor of one element multiplying g_ce and g_tvd."""
    BT, V = _logits2d(student, "student")
    dt = _dtype_code(student)
    if grad.shape != student.shape or grad.dtype != student.dtype or not grad.is_contiguous():
        raise ValueError("grad must match student in shape and dtype and be contiguous")
    _check(lib.lx_ce_tvd_backward(_ptr(grad), _ptr(student), _ptr(teacher), _ptr(target), BT, V,
                                  int(ignore_index), _ptr(lse_s), _ptr(lse_t), _ptr(sigma),
                                  float(g_ce), float(g_tvd), _ptr(g_scale), dt, _stream(stream)),
           "lx_ce_tvd_backward")


def lx_ce_tvd_forward_backward_workspace_bytes(BT: int, V: int, dt: int, has_teacher: bool) -> int:
    return lib.lx_ce_tvd_forward_backward_workspace_bytes(BT, V, dt, int(bool(has_teacher)))


def lx_ce_tvd_forward_backward(student, teacher, target, ignore_index, ce, tvd, lse_s, lse_t, sigma, grad,
                               g_ce: float, g_tvd: float, g_scale=None, workspace=None, stream=None) -> None:
    """Forward outputs and the student gradient in one call (``grad`` may be
    ``student``).  ``workspace`` as in lx_ce_tvd_forward, sized by
    lx_ce_tvd_forward_backward_workspace_bytes."""
    BT, V = _logits2d(student, "student")
    dt = _dtype_code(student)
    if teacher is not None and (teacher.shape != student.shape or teacher.dtype != student.dtype):
        raise ValueError("teacher must match student in shape and dtype")
    if grad.shape != student.shape or grad.dtype != student.dtype or not grad.is_contiguous():
        raise ValueError("grad must match student in shape and dtype and be contiguous")
    need = lx_ce_tvd_forward_backward_workspace_bytes(BT, V, dt, teacher is not None)
    if workspace is None and need:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=student.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lx_ce_tvd_forward_backward(_ptr(student), _ptr(teacher), _ptr(target), BT, V, int(ignore_index),
                                          _ptr(ce), _ptr(tvd), _ptr(lse_s), _ptr(lse_t), _ptr(sigma), _ptr(grad),
                                          float(g_ce), float(g_tvd), _ptr(g_scale), dt, _ptr(workspace), wbytes,
                                          _stream(stream)), "lx_ce_tvd_forward_backward")


def lx_ce_tvd_forward_backward_noalloc(student, teacher, target, ignore_index, ce, tvd, lse_s, lse_t, sigma, grad,
                                       g_ce: float, g_tvd: float, g_scale=None, stream=None) -> None:
    """lx_ce_tvd_forward_backward with its scratch memory in the library's static
    device buffer instead of a workspace (nothing is allocated; calls that
    overlap on one device race)."""
    BT, V = _logits2d(student, "student")
    dt = _dtype_code(student)
    if teacher is not None and (teacher.shape != student.shape or teacher.dtype != student.dtype):
        raise ValueError("teacher must match student in shape and dtype")
    if grad.shape != student.shape or grad.dtype != student.dtype or not grad.is_contiguous():
        raise ValueError("grad must match student in shape and dtype and be contiguous")
    _check(lib.lx_ce_tvd_forward_backward_noalloc(_ptr(student), _ptr(teacher), _ptr(target), BT, V,
                                                  int(ignore_index), _ptr(ce), _ptr(tvd), _ptr(lse_s), _ptr(lse_t),
                                                  _ptr(sigma), _ptr(grad), float(g_ce), float(g_tvd), _ptr(g_scale),
                                                  dt, _stream(stream)), "lx_ce_tvd_forward_backward_noalloc")


def lx_ce_tvd_count_valid(target, ignore_index, n_valid=None, inv_n_valid=None, stream=None) -> None:
    """Number of non-ignored rows (int64 [1]) and its reciprocal (float32 [1])."""
    BT = target.shape[0]
    _check(lib.lx_ce_tvd_count_valid(_ptr(target), BT, int(ignore_index), _ptr(n_valid), _ptr(inv_n_valid),
                                     _stream(stream)), "lx_ce_tvd_count_valid")


def lx_ce_tvd_reduce_mean(ce, tvd, target, ignore_index, mean_out, n_valid=None, inv_n_valid=None,
                          stream=None) -> None:
    """Mean of ce (and tvd) over non-ignored rows into mean_out (float32 [2])."""
    BT = target.shape[0]
    _check(lib.lx_ce_tvd_reduce_mean(_ptr(ce), _ptr(tvd), _ptr(target), BT, int(ignore_index),
                                     _ptr(mean_out), _ptr(n_valid), _ptr(inv_n_valid), _stream(stream)),
           "lx_ce_tvd_reduce_mean")


def lx_vp_stats_floats(has_teacher: bool) -> int:
    return 5 if has_teacher else 3


def lx_ce_tvd_vp_stats(student, teacher, target, v0, ignore_index, stats, stream=None) -> None:
    """Step-1 partials of a column shard (student / teacher (BT, V_shard), the shard's
    first column v0) into ``stats``, float32 [BT, 5] (CE-only: [BT, 3])."""
    BT, Vs = _logits2d(student, "student")
    dt = _dtype_code(student)
    if teacher is not None and (teacher.shape != student.shape or teacher.dtype != student.dtype):
        raise ValueError("teacher must match student in shape and dtype")
    _check(lib.lx_ce_tvd_vp_stats(_ptr(student), _ptr(teacher), _ptr(target), BT, Vs, int(v0), int(ignore_index),
                                  dt, _ptr(stats), _stream(stream)), "lx_ce_tvd_vp_stats")


def lx_ce_tvd_vp_merge_stats(stats, target, V, ignore_index, ce, lse_s, lse_t=None, stream=None) -> None:
    """Merge of gathered step-1 partials, ``stats`` float32 [n_shards, BT, 5 or 3]."""
    n, BT, P = stats.shape
    _check(lib.lx_ce_tvd_vp_merge_stats(_ptr(stats), n, _ptr(target), BT, int(V), int(ignore_index), int(P == 5),
                                        _ptr(ce), _ptr(lse_s), _ptr(lse_t), _stream(stream)),
           "lx_ce_tvd_vp_merge_stats")


def lx_ce_tvd_vp_tv(student, teacher, target, ignore_index, lse_s, lse_t, tv, stream=None) -> None:
    """Step-2 partials of a column shard into ``tv``, float32 [BT, 2]."""
    BT, Vs = _logits2d(student, "student")
    dt = _dtype_code(student)
    if teacher is None or teacher.shape != student.shape or teacher.dtype != student.dtype:
        raise ValueError("teacher must be given and match student in shape and dtype")
    _check(lib.lx_ce_tvd_vp_tv(_ptr(student), _ptr(teacher), _ptr(target), BT, Vs, int(ignore_index), _ptr(lse_s),
                               _ptr(lse_t), dt, _ptr(tv), _stream(stream)), "lx_ce_tvd_vp_tv")


def lx_ce_tvd_vp_merge_tv(tv, target, ignore_index, tvd, sigma, stream=None) -> None:
    """Merge of gathered step-2 partials, ``tv`` float32 [n_shards, BT, 2]."""
    n, BT, _ = tv.shape
    _check(lib.lx_ce_tvd_vp_merge_tv(_ptr(tv), n, _ptr(target), BT, int(ignore_index), _ptr(tvd), _ptr(sigma),
                                     _stream(stream)), "lx_ce_tvd_vp_merge_tv")


def lx_ce_tvd_backward_shard(grad, student, teacher, target, v0, V, ignore_index, lse_s, lse_t, sigma,
                             g_ce: float, g_tvd: float, g_scale=None, stream=None) -> None:
    """Backward of a column shard (columns [v0, v0 + V_shard) of rows of V)."""
    BT, Vs = _logits2d(student, "student")
    dt = _dtype_code(student)
    if grad.shape != student.shape or grad.dtype != student.dtype or not grad.is_contiguous():
        raise ValueError("grad must match student in shape and dtype and be contiguous")
    _check(lib.lx_ce_tvd_backward_shard(_ptr(grad), _ptr(student), _ptr(teacher), _ptr(target), BT, Vs, int(v0),
                                        int(V), int(ignore_index), _ptr(lse_s), _ptr(lse_t), _ptr(sigma),
                                        float(g_ce), float(g_tvd), _ptr(g_scale), dt, _stream(stream)),
           "lx_ce_tvd_backward_shard")


def lx_ce_tvd_forward_ex(student, teacher, target, ignore_index, ce, tvd, lse_s, lse_t, sigma,
                         workspace=None, stream=None) -> None:
    """lx_ce_tvd_forward on row-strided views: each of student / teacher may be any
    2-D view with contiguous rows (its stride(0) is passed as the row stride)."""
    BT, V, lds = _rows2d(student, "student")
    dt = _dtype_code(student)
    ldt = V
    if teacher is not None:
        if teacher.shape != student.shape or teacher.dtype != student.dtype:
            raise ValueError("teacher must match student in shape and dtype")
        ldt = _rows2d(teacher, "teacher")[2]
    need = lx_ce_tvd_workspace_bytes(BT, V, dt, teacher is not None)
    if workspace is None and need:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=student.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lx_ce_tvd_forward_ex(_ptr(student), lds, _ptr(teacher), ldt, _ptr(target), BT, V, int(ignore_index),
                                    _ptr(ce), _ptr(tvd), _ptr(lse_s), _ptr(lse_t), _ptr(sigma), dt,
                                    _ptr(workspace), wbytes, _stream(stream)), "lx_ce_tvd_forward_ex")


def lx_ce_tvd_backward_ex(grad, student, teacher, target, ignore_index, lse_s, lse_t, sigma, g_ce: float,
                          g_tvd: float, grad_ce_rows=None, grad_tvd_rows=None, g_scale=None, stream=None) -> None:
    """lx_ce_tvd_backward on row-strided views, with optional per-row factors
    ``grad_ce_rows`` / ``grad_tvd_rows`` (float32 [BT] device tensors)."""
    BT, V, lds = _rows2d(student, "student")
    dt = _dtype_code(student)
    if grad.shape != student.shape or grad.dtype != student.dtype:
        raise ValueError("grad must match student in shape and dtype")
    ldg = _rows2d(grad, "grad")[2]
    ldt = V if teacher is None else _rows2d(teacher, "teacher")[2]
    _check(lib.lx_ce_tvd_backward_ex(_ptr(grad), ldg, _ptr(student), lds, _ptr(teacher), ldt, _ptr(target), BT, V,
                                     int(ignore_index), _ptr(lse_s), _ptr(lse_t), _ptr(sigma), float(g_ce),
                                     float(g_tvd), _ptr(grad_ce_rows), _ptr(grad_tvd_rows), _ptr(g_scale), dt,
                                     _stream(stream)), "lx_ce_tvd_backward_ex")


def lx_ce_tvd_forward_backward_ex(student, teacher, target, ignore_index, ce, tvd, lse_s, lse_t, sigma, grad,
                                  g_ce: float, g_tvd: float, grad_ce_rows=None, grad_tvd_rows=None, g_scale=None,
                                  workspace=None, stream=None) -> None:
    """lx_ce_tvd_forward_backward on row-strided views, with optional per-row factors."""
    BT, V, lds = _rows2d(student, "student")
    dt = _dtype_code(student)
    ldt = V
    if teacher is not None:
        if teacher.shape != student.shape or teacher.dtype != student.dtype:
            raise ValueError("teacher must match student in shape and dtype")
        ldt = _rows2d(teacher, "teacher")[2]
    if grad.shape != student.shape or grad.dtype != student.dtype:
        raise ValueError("grad must match student in shape and dtype")
    ldg = _rows2d(grad, "grad")[2]
    need = lx_ce_tvd_forward_backward_workspace_bytes(BT, V, dt, teacher is not None)
    if workspace is None and need:
        import torch
        workspace = torch.empty(need, dtype=torch.uint8, device=student.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lx_ce_tvd_forward_backward_ex(_ptr(student), lds, _ptr(teacher), ldt, _ptr(target), BT, V,
                                             int(ignore_index), _ptr(ce), _ptr(tvd), _ptr(lse_s), _ptr(lse_t),
                                             _ptr(sigma), _ptr(grad), ldg, float(g_ce), float(g_tvd),
                                             _ptr(grad_ce_rows), _ptr(grad_tvd_rows), _ptr(g_scale), dt,
                                             _ptr(workspace), wbytes, _stream(stream)),
           "lx_ce_tvd_forward_backward_ex")


def lx_gemm_bf16(A, a_k_contiguous: bool, B, b_k_contiguous: bool, C, M: int, N: int, K: int,
                 accumulate: bool = False, stream=None) -> None:
    """C[m][n] (+)= sum_k A(m, k) B(n, k) on bf16 device tensors A, B (2-D, rows contiguous)
    and a float32 2-D C.  A(m, k) is A[m, k] when a_k_contiguous else A[k, m]; likewise B."""
    import torch
    for t, name in ((A, "A"), (B, "B")):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a 2-D bfloat16 tensor with contiguous rows")
    if C.dtype != torch.float32 or C.dim() != 2 or C.stride(1) != 1:
        raise ValueError("C must be a 2-D float32 tensor with contiguous rows")
    _check(lib.lx_gemm_bf16(_ptr(A), A.stride(0), int(bool(a_k_contiguous)), _ptr(B), B.stride(0),
                            int(bool(b_k_contiguous)), _ptr(C), C.stride(0), int(M), int(N), int(K),
                            int(bool(accumulate)), _stream(stream)), "lx_gemm_bf16")


def lx_ce_tvd_linear_workspace_bytes(BT: int, V: int, H_s: int, has_teacher: bool, chunk_rows: int) -> int:
    return lib.lx_ce_tvd_linear_workspace_bytes(BT, V, H_s, int(bool(has_teacher)), chunk_rows)


def lx_ce_tvd_linear_forward_backward(x_s, w_s, x_t, w_t, target, ignore_index, ce, tvd, lse_s, lse_t, sigma,
                                      grad_x_s, grad_w_s, g_ce: float, g_tvd: float, g_scale=None,
                                      chunk_rows: int | None = None, workspace=None, stream=None) -> None:
    """lm_head products and the CE + TVD loss: x_s (BT, H_s), w_s (V, H_s), x_t / w_t (or None)
    contiguous bfloat16; grad_x_s (BT, H_s) / grad_w_s (V, H_s) float32 or None.  The workspace
    (uint8 device tensor) is allocated here with torch when not given."""
    import torch
    BT, H_s = x_s.shape
    V = w_s.shape[0]
    H_t = 0 if x_t is None else x_t.shape[1]
    for t, name in ((x_s, "x_s"), (w_s, "w_s"), (x_t, "x_t"), (w_t, "w_t")):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    chunk = BT if chunk_rows is None else int(chunk_rows)
    need = lx_ce_tvd_linear_workspace_bytes(BT, V, x_s.shape[1], x_t is not None, chunk)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_s.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.lx_ce_tvd_linear_forward_backward(_ptr(x_s), _ptr(w_s), H_s, _ptr(x_t), _ptr(w_t), H_t, _ptr(target),
                                                 BT, V, int(ignore_index), _ptr(ce), _ptr(tvd), _ptr(lse_s),
                                                 _ptr(lse_t), _ptr(sigma), _ptr(grad_x_s), _ptr(grad_w_s),
                                                 float(g_ce), float(g_tvd), _ptr(g_scale), chunk, _ptr(workspace),
                                                 wbytes, _stream(stream)), "lx_ce_tvd_linear_forward_backward")


__all__ = [
    "LxError", "lib", "LIB_PATH", "LX_OK", "LX_ERR_INVALID_ARG", "LX_ERR_UNSUPPORTED_DTYPE", "LX_ERR_ALIAS",
    "LX_ERR_WORKSPACE", "LX_ERR_HIP", "LX_F32", "LX_BF16", "LX_F16", "lx_status_string", "lx_abi_version",
    "lx_ce_tvd_workspace_bytes", "lx_ce_tvd_forward", "lx_ce_tvd_backward", "lx_ce_tvd_reduce_mean",
    "lx_ce_tvd_forward_backward_workspace_bytes", "lx_ce_tvd_forward_backward", "lx_ce_tvd_count_valid",
    "lx_vp_stats_floats", "lx_ce_tvd_vp_stats", "lx_ce_tvd_vp_merge_stats", "lx_ce_tvd_vp_tv", "lx_ce_tvd_vp_merge_tv",
    "lx_ce_tvd_backward_shard", "lx_ce_tvd_forward_ex", "lx_ce_tvd_backward_ex", "lx_ce_tvd_forward_backward_ex",
    "lx_gemm_bf16", "lx_ce_tvd_linear_workspace_bytes", "lx_ce_tvd_linear_forward_backward",
]


def lx_stream_read(src, sink, stream=None) -> None:
    """Reference stream: read every byte of src once (sink: int32/uint32 [1])."""
    _check(lib.lx_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(stream)),
           "lx_stream_read")


def lx_stream_read2_write(a, b, out, stream=None) -> None:
    """Reference stream: out = a XOR b over their bytes (all the same size)."""
    nb = a.numel() * a.element_size()
    if b.numel() * b.element_size() != nb or out.numel() * out.element_size() != nb:
        raise ValueError("a, b and out must have the same number of bytes")
    _check(lib.lx_stream_read2_write(_ptr(a), _ptr(b), _ptr(out), nb, _stream(stream)), "lx_stream_read2_write")
