"""TEST INFRASTRUCTURE -- the fp64 CPU oracle for exact attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``exact_self_attention_amd``) and neither imports the other.

The arithmetic lives in ``oracle.c`` (plain C, double precision, OpenMP over
query rows); this module only compiles it with gcc, loads it with ctypes and
marshals numpy arrays.  Inputs are float32 arrays holding the exact widening of
the fp16/bf16 bit patterns the GPU reads; outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
             "-ffp-contract=off", "-fno-fast-math"]

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc into ``out`` (always recompiles)."""
    tmp = f"{out}.{os.getpid()}.tmp"
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str = _LIB, *, build_if_missing: bool = True) -> ctypes.CDLL:
    lib = ctypes.CDLL(path) if os.path.exists(path) else None
    if lib is None:
        if not build_if_missing:
            raise FileNotFoundError(path)
        build(out=path)
        lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_attn_rows.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_double,
                                     ctypes.c_int, p, p, i64, i64, p, i64, p, p]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _get():
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def max_threads(lib: Optional[ctypes.CDLL] = None) -> int:
    return (lib or _get()).oracle_max_threads()


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _mask_arg(mask, B, H, Nq, Nk):
    """(array, stride_b, stride_h) for an additive mask broadcastable to
    ``[B, H, Nq, Nk]``: shape ``[Nq, Nk]``, ``[B or 1, H or 1, Nq, Nk]``."""
    if mask is None:
        return None, 0, 0
    m = np.asarray(mask, dtype=np.float32)
    if m.ndim == 2:
        m = m[None, None]
    if m.ndim != 4 or m.shape[2:] != (Nq, Nk) or m.shape[0] not in (1, B) \
            or m.shape[1] not in (1, H):
        raise ValueError("mask must be [Nq, Nk] or [B|1, H|1, Nq, Nk]")
    m = np.ascontiguousarray(m)
    sb = m.shape[1] * Nq * Nk if m.shape[0] == B and B > 1 else 0
    sh = Nq * Nk if m.shape[1] == H and H > 1 else 0
    return m, sb, sh


def attn_rows(Q, K, V, scale, causal: bool, key_len, sel, *, mask=None, lib=None):
    """Oracle attention on selected rows, general shapes.

    Q: float32 ``[B, H, Nq, d]``; K, V: float32 ``[B, Hkv, Nk, d]`` with H a
    multiple of Hkv (query head h reads key/value head h // (H // Hkv));
    causal visibility is j <= i + Nk - Nq.  ``key_len``: int ``[B]`` or None;
    ``mask``: additive float mask ``[Nq, Nk]`` or ``[B|1, H|1, Nq, Nk]``, or
    None; ``sel``: int64 ``[n, 3]`` of (b, h, i).  Returns (O ``[n, d]``, LSE
    ``[n]``) in float64.
    """
    lib = lib or _get()
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    if Q.ndim != 4 or K.ndim != 4 or V.shape != K.shape:
        raise ValueError("Q must be [B, H, Nq, d] and K, V one [B, Hkv, Nk, d] shape")
    B, H, Nq, d = Q.shape
    Bk, Hkv, Nk, dk = K.shape
    if Bk != B or dk != d or Hkv == 0 or H % Hkv != 0:
        raise ValueError("K/V batch and head size must match Q, and Hkv divide H")
    sel = np.ascontiguousarray(sel, dtype=np.int64).reshape(-1, 3)
    n = sel.shape[0]
    O = np.zeros((n, d), dtype=np.float64)
    LSE = np.zeros((n,), dtype=np.float64)
    kl = None
    if key_len is not None:
        kl = np.ascontiguousarray(key_len, dtype=np.int32)
        if kl.shape != (B,):
            raise ValueError("key_len must have shape [B]")
    m, msb, msh = _mask_arg(mask, B, H, Nq, Nk)
    rc = lib.oracle_attn_rows(_ptr(Q), _ptr(K), _ptr(V), B, H, Hkv, Nq, Nk, d,
                              float(scale), int(bool(causal)),
                              None if kl is None else _ptr(kl),
                              None if m is None else _ptr(m), msb, msh,
                              _ptr(sel), n, _ptr(O), _ptr(LSE))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return O, LSE


def attn(Q, K, V, scale, causal: bool = False, key_len=None, *, mask=None, lib=None):
    """Oracle attention on every row, general shapes: O ``[B,H,Nq,d]`` and
    LSE ``[B,H,Nq]`` (float64)."""
    Q = np.ascontiguousarray(Q, dtype=np.float32)
    B, H, Nq, d = Q.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(Nq), indexing="ij")
    sel = np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1)
    O, LSE = attn_rows(Q, K, V, scale, causal, key_len, sel, mask=mask, lib=lib)
    return O.reshape(B, H, Nq, d), LSE.reshape(B, H, Nq)


def sdpa_rows(Q, K, V, scale, causal: bool, key_len, sel, *, lib=None):
    """Oracle self-attention on selected rows.

    Q, K, V: float32 ``[B, H, N, d]``; ``key_len``: int ``[B]`` or None;
    ``sel``: int64 ``[n, 3]`` of (b, h, i).  Returns (O ``[n, d]``, LSE ``[n]``)
    in float64.
    """
    Q = np.asarray(Q)
    if Q.ndim != 4 or np.shape(K) != Q.shape or np.shape(V) != Q.shape:
        raise ValueError("Q, K, V must share one [B, H, N, d] shape")
    return attn_rows(Q, K, V, scale, causal, key_len, sel, lib=lib)


def sdpa(Q, K, V, scale, causal: bool = False, key_len=None, *, lib=None):
    """Oracle self-attention on every row: O ``[B,H,N,d]`` and LSE ``[B,H,N]`` (float64)."""
    Q = np.asarray(Q)
    if Q.ndim != 4 or np.shape(K) != Q.shape or np.shape(V) != Q.shape:
        raise ValueError("Q, K, V must share one [B, H, N, d] shape")
    return attn(Q, K, V, scale, causal, key_len, lib=lib)
