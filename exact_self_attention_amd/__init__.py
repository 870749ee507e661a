"""Python binding of libattn.so, the gfx950 exact-attention forward library.

Argument marshalling only: every function here checks what ctypes cannot
(tensor dtype, device, contiguity), passes raw device pointers, sizes and the
current HIP stream to the C function of the same name, and turns a non-zero
status into ``AttnError``.  All arithmetic runs in the HIP kernels.  PyTorch
supplies device memory and streams.

Importing this package raises ImportError when libattn.so has not been built
(``python exact_self_attention_amd/build.py``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_F16 = 0
ATTN_BF16 = 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED",
          3: "ATTN_ERR_MISALIGNED", 4: "ATTN_ERR_WORKSPACE", 5: "ATTN_ERR_LAUNCH",
          6: "ATTN_ERR_DEVICE"}
EXPORTS = ["attn_fwd", "attn_fwd_gqa", "attn_fwd_naive", "attn_fwd_naive_workspace_bytes",
           "attn_fwd_splitkv", "attn_fwd_gqa_splitkv", "attn_fwd_gqa_splitkv_static",
           "attn_fwd_splitkv_workspace_bytes",
           "attn_fwd_splitkv_default_splits", "attn_fwd_gqa_splitkv_default_splits",
           "attn_fwd_masked", "attn_fwd_masked_splitkv", "attn_fwd_gqa_kernel_name",
           "attn_status_string", "attn_fwd_kernel_name", "attn_version"]


class AttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({attn_status_string(status)})")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "'python exact_self_attention_amd/build.py' (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    common = [i32, p, p, p, p, p, i64, i64, i64, i64, f32, i32, p]
    lib.attn_fwd.argtypes = common + [p]
    lib.attn_fwd.restype = i32
    general = [i32, p, p, p, p, p, i64, i64, i64, i64, i64, i64, f32, i32, p]
    lib.attn_fwd_gqa.argtypes = general + [p]
    lib.attn_fwd_gqa.restype = i32
    lib.attn_fwd_gqa_splitkv.argtypes = general + [i64, p, ctypes.c_size_t, p]
    lib.attn_fwd_gqa_splitkv.restype = i32
    lib.attn_fwd_gqa_splitkv_static.argtypes = general + [i64, p]
    lib.attn_fwd_gqa_splitkv_static.restype = i32
    lib.attn_fwd_masked.argtypes = general + [p, i64, i64, p]
    lib.attn_fwd_masked.restype = i32
    lib.attn_fwd_masked_splitkv.argtypes = general + [p, i64, i64, i64, p, ctypes.c_size_t, p]
    lib.attn_fwd_masked_splitkv.restype = i32
    lib.attn_fwd_gqa_splitkv_default_splits.argtypes = [i32, i64, i64, i64, i64, i64, i64, i32]
    lib.attn_fwd_gqa_splitkv_default_splits.restype = i64
    lib.attn_fwd_naive.argtypes = common + [p, ctypes.c_size_t, p]
    lib.attn_fwd_naive.restype = i32
    lib.attn_fwd_naive_workspace_bytes.argtypes = [i64, i64, i64]
    lib.attn_fwd_naive_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_splitkv.argtypes = common + [i64, p, ctypes.c_size_t, p]
    lib.attn_fwd_splitkv.restype = i32
    lib.attn_fwd_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    lib.attn_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fwd_splitkv_default_splits.argtypes = [i32, i64, i64, i64, i64, i32]
    lib.attn_fwd_splitkv_default_splits.restype = i64
    lib.attn_status_string.argtypes = [i32]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_fwd_kernel_name.argtypes = [i32, i64, i64, i32, i32, ctypes.c_char_p, ctypes.c_size_t]
    lib.attn_fwd_kernel_name.restype = i32
    lib.attn_fwd_gqa_kernel_name.argtypes = [i32, i64, i64, i64, i64, i64, i32, i32, i64,
                                             ctypes.c_char_p, ctypes.c_size_t]
    lib.attn_fwd_gqa_kernel_name.restype = i32
    lib.attn_version.argtypes = []
    lib.attn_version.restype = i32
    return lib


lib = _load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"dtype {t.dtype} is not float16 or bfloat16")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_tensors(q, k, v, o, lse, key_len):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [B, H, N, d] tensor")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    if not q.is_cuda:
        raise ValueError("tensors must live on a GPU")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) \
                or not lse.is_contiguous() or lse.device != q.device:
            raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    if key_len is not None:
        if key_len.dtype != torch.int32 or tuple(key_len.shape) != (q.shape[0],) \
                or not key_len.is_contiguous() or key_len.device != q.device:
            raise ValueError("key_len must be a contiguous int32 [B] tensor on q's device")


def _check_general(q, k, v, o, lse, key_len):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d tensor")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype and device")
    if o.shape != q.shape:
        raise ValueError("o must have q's shape [B, H, Nq, d]")
    if v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[3] != q.shape[3]:
        raise ValueError("k and v must be [B, Hkv, Nk, d] with q's B and d")
    if not q.is_cuda:
        raise ValueError("tensors must live on a GPU")
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(q.shape[:3]) \
                or not lse.is_contiguous() or lse.device != q.device:
            raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    if key_len is not None:
        if key_len.dtype != torch.int32 or tuple(key_len.shape) != (q.shape[0],) \
                or not key_len.is_contiguous() or key_len.device != q.device:
            raise ValueError("key_len must be a contiguous int32 [B] tensor on q's device")


def attn_fwd_gqa(q, k, v, o, lse=None, *, scale: float, causal: bool = False,
                 key_len=None, stream=None) -> None:
    """Fused forward, general shapes: q, o [B, H, Nq, d]; k, v [B, Hkv, Nk, d]."""
    code = _dtype_code(q)
    _check_general(q, k, v, o, lse, key_len)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    st = lib.attn_fwd_gqa(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                          B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _ptr(key_len),
                          _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_gqa", st)


def attn_fwd_gqa_splitkv(q, k, v, o, lse=None, *, workspace: torch.Tensor, n_splits: int,
                         scale: float, causal: bool = False, key_len=None, stream=None) -> None:
    """attn_fwd_gqa over ``n_splits`` key ranges, merged (see include/attn.h)."""
    code = _dtype_code(q)
    _check_general(q, k, v, o, lse, key_len)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.attn_fwd_gqa_splitkv(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                  _ptr(key_len), int(n_splits), _ptr(workspace), nbytes,
                                  _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_gqa_splitkv", st)


def attn_fwd_gqa_splitkv_static(q, k, v, o, lse=None, *, n_splits: int, scale: float,
                                causal: bool = False, key_len=None, stream=None) -> None:
    """attn_fwd_gqa_splitkv with the library's own scratch: no workspace and
    no allocation (see include/attn.h; calls on one device must not overlap)."""
    code = _dtype_code(q)
    _check_general(q, k, v, o, lse, key_len)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    st = lib.attn_fwd_gqa_splitkv_static(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                         B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                         _ptr(key_len), int(n_splits), _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_gqa_splitkv_static", st)


def _mask_strides(mask, q, k):
    """(stride_b, stride_h) in elements of an fp32 mask tensor of shape
    [Nq, Nk] or [B|1, H|1, Nq, Nk] whose rows are contiguous (broadcast
    views from expand() are accepted: their stride is 0)."""
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    if mask.dtype != torch.float32 or mask.device != q.device:
        raise ValueError("mask must be a float32 tensor on q's device")
    if mask.dim() == 2:
        mask = mask.view(1, 1, *mask.shape)
    if mask.dim() != 4 or tuple(mask.shape[2:]) != (Nq, Nk) or mask.shape[0] not in (1, B) \
            or mask.shape[1] not in (1, H):
        raise ValueError("mask must be [Nq, Nk] or [B|1, H|1, Nq, Nk]")
    if (Nk > 1 and mask.stride(3) != 1) or (Nq > 1 and mask.stride(2) != Nk):
        raise ValueError("mask rows must be contiguous [Nq, Nk] blocks")
    sb = mask.stride(0) if mask.shape[0] == B and B > 1 else 0
    sh = mask.stride(1) if mask.shape[1] == H and H > 1 else 0
    return sb, sh


def attn_fwd_masked(q, k, v, o, lse=None, *, mask: torch.Tensor, scale: float,
                    causal: bool = False, key_len=None, stream=None) -> None:
    """attn_fwd_gqa with an additive fp32 score mask (see include/attn.h)."""
    code = _dtype_code(q)
    _check_general(q, k, v, o, lse, key_len)
    sb, sh = _mask_strides(mask, q, k)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    st = lib.attn_fwd_masked(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                             _ptr(key_len), mask.data_ptr(), sb, sh, _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_masked", st)


def attn_fwd_masked_splitkv(q, k, v, o, lse=None, *, mask: torch.Tensor, workspace: torch.Tensor,
                            n_splits: int, scale: float, causal: bool = False, key_len=None,
                            stream=None) -> None:
    """attn_fwd_masked over ``n_splits`` key ranges, merged."""
    code = _dtype_code(q)
    _check_general(q, k, v, o, lse, key_len)
    sb, sh = _mask_strides(mask, q, k)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.attn_fwd_masked_splitkv(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                     B, H, Hkv, Nq, Nk, d, float(scale), int(bool(causal)),
                                     _ptr(key_len), mask.data_ptr(), sb, sh, int(n_splits),
                                     _ptr(workspace), nbytes, _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_masked_splitkv", st)


def attn_fwd_gqa_splitkv_default_splits(dtype: int, B: int, H: int, Hkv: int, Nq: int, Nk: int,
                                        d: int, causal: bool) -> int:
    return int(lib.attn_fwd_gqa_splitkv_default_splits(dtype, B, H, Hkv, Nq, Nk, d,
                                                       int(bool(causal))))


def attn_fwd(q, k, v, o, lse=None, *, scale: float, causal: bool = False,
             key_len=None, stream=None) -> None:
    """Fused forward: writes o (and lse when given).  See include/attn.h."""
    code = _dtype_code(q)
    _check_tensors(q, k, v, o, lse, key_len)
    B, H, N, d = q.shape
    st = lib.attn_fwd(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                      B, H, N, d, float(scale), int(bool(causal)), _ptr(key_len),
                      _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd", st)


def attn_fwd_naive(q, k, v, o, lse=None, *, workspace: torch.Tensor, scale: float,
                   causal: bool = False, key_len=None, stream=None) -> None:
    """Unfused baseline (materialises S and P in ``workspace``)."""
    code = _dtype_code(q)
    _check_tensors(q, k, v, o, lse, key_len)
    B, H, N, d = q.shape
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.attn_fwd_naive(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                            B, H, N, d, float(scale), int(bool(causal)), _ptr(key_len),
                            _ptr(workspace), nbytes, _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_naive", st)


def attn_fwd_naive_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(lib.attn_fwd_naive_workspace_bytes(B, H, N))


def attn_fwd_splitkv(q, k, v, o, lse=None, *, workspace: torch.Tensor, n_splits: int,
                     scale: float, causal: bool = False, key_len=None, stream=None) -> None:
    """Fused forward over ``n_splits`` key ranges, merged (see include/attn.h)."""
    code = _dtype_code(q)
    _check_tensors(q, k, v, o, lse, key_len)
    B, H, N, d = q.shape
    nbytes = workspace.numel() * workspace.element_size()
    st = lib.attn_fwd_splitkv(code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              B, H, N, d, float(scale), int(bool(causal)), _ptr(key_len),
                              int(n_splits), _ptr(workspace), nbytes, _stream(stream, q.device))
    if st != 0:
        raise AttnError("attn_fwd_splitkv", st)


def attn_fwd_splitkv_workspace_bytes(B: int, H: int, N: int, d: int, n_splits: int) -> int:
    return int(lib.attn_fwd_splitkv_workspace_bytes(B, H, N, d, n_splits))


def attn_fwd_splitkv_default_splits(dtype: int, B: int, H: int, N: int, d: int,
                                    causal: bool) -> int:
    return int(lib.attn_fwd_splitkv_default_splits(dtype, B, H, N, d, int(bool(causal))))


def attn_status_string(status: int) -> str:
    return lib.attn_status_string(int(status)).decode()


def attn_fwd_kernel_name(dtype: int, d: int, N: int, causal: bool, has_key_len: bool) -> str:
    buf = ctypes.create_string_buffer(128)
    st = lib.attn_fwd_kernel_name(dtype, d, N, int(bool(causal)), int(bool(has_key_len)), buf, 128)
    if st != 0:
        raise AttnError("attn_fwd_kernel_name", st)
    return buf.value.decode()


def attn_fwd_gqa_kernel_name(dtype: int, d: int, H: int, Hkv: int, Nq: int, Nk: int,
                             causal: bool, masked: bool = False, n_splits: int = 0) -> str:
    buf = ctypes.create_string_buffer(128)
    st = lib.attn_fwd_gqa_kernel_name(dtype, d, H, Hkv, Nq, Nk, int(bool(causal)), int(bool(masked)),
                                      int(n_splits), buf, 128)
    if st != 0:
        raise AttnError("attn_fwd_gqa_kernel_name", st)
    return buf.value.decode()


def attn_version() -> int:
    return int(lib.attn_version())


def fwd(q, k, v, *, scale: Optional[float] = None, causal: bool = False, key_len=None,
        want_lse: bool = True, stream=None):
    """Allocate O (and LSE) with torch and run attn_fwd; returns (o, lse)."""
    if scale is None:
        scale = float(torch.tensor(1.0 / q.shape[-1] ** 0.5, dtype=torch.float32))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    attn_fwd(q, k, v, o, lse, scale=scale, causal=causal, key_len=key_len, stream=stream)
    return o, lse
