"""Seeded synthetic inputs for scaled-dot-product attention.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It draws random numbers and rounds them to the 16-bit storage
formats; it performs none of attention's arithmetic (no products, no softmax,
no reductions).

Every tensor is drawn in float32 from ``numpy.random.Generator(PCG64(seed))``
and then rounded to nearest-even into fp16 or bf16.  Both sides of a parity
check read those exact 16-bit patterns: the GPU reads the bits, the oracle
reads their exact widening to float32.

Draw order for a workload: Q, K, V (each ``[B, H, N, d]``), then the per
sequence key lengths, then (long-context only) the sampled query rows per head.

The five workloads follow the shapes the pages measure or describe:

* ``single_head``: B=1 H=1 N=64 d=32 fp16, no mask (a tiny case the oracle
  finishes in milliseconds).
* ``reranker``: B=50 H=12 N=256 d=32 fp16, key-padding mask with valid key
  length uniform in [48, 256] per sequence; the cross-encoder reranker shape
  of "cuda-reranker" (hidden 384 = 12 heads x 32, 50 candidates per query,
  padded sequences), whose real data is absent and stood in for by these draws.
* ``prefill``: B=1 H=32 N=4096 d=128 fp16, causal (the N=4096, d=128 example
  of "Tensor Parallelism with CUDA - Standard Attention" and of the
  naive-attention guide, with 32 heads).
* ``peaky``: B=8 H=16 N=2048 d=64 bf16, non-causal, Q and K drawn with
  standard deviation 3 so that scaled scores have std near 9 and a few keys
  dominate each row.
* ``long_context``: B=1 H=32 N=32768 d=128 bf16, causal (the longest sequence
  of the portfolio page's benchmark table); the oracle checks 256 seeded
  query rows per head.

One more workload measures the split-key forward:

* ``prefill_shard8``: B=1 H=4 N=4096 d=128 fp16, causal: the prefill's
  per-GPU share when its 32 heads are divided among 8 GPUs.

Three measure grouped-query and cross-attention (Q ``[B, H, Nq, d]``, K and
V ``[B, Hkv, N, d]``, N the key length), which "cuda-reranker" lists as
extensions; the pages give no shapes for them, so these reuse theirs:

* ``gqa_prefill``: the prefill with 8 key/value heads for its 32 query heads
  (4 query heads per key/value head), B=1 Nq=N=4096 d=128 fp16, causal.
* ``gqa_decode``: one new query per sequence against a long key/value
  history: B=8 H=32 Hkv=8 Nq=1 N=32768 (the long-context length) d=128
  bf16, causal, valid history length uniform in [16384, 32768] per sequence.
* ``cross``: cross-attention of 2048 queries over 4096 keys, B=4 H=16 d=64
  fp16, no mask.

Draw order for these is Q, K, V with their own shapes, then key lengths.

One measures the additive score mask of "Naive Attention Kernel" (a float
[S, S] mask added to the scaled scores):

* ``masked_prefill``: the prefill (B=1 H=32 N=4096 d=128 fp16, causal) with
  one fp32 [4096, 4096] mask shared by all heads, drawn N(0, 1) after Q, K
  and V (a dense additive bias on top of the causal structure).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F16 = "f16"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    key_padding: bool  # per-sequence valid key length drawn after V
    key_len_lo: int = 0
    key_len_hi: int = 0  # inclusive
    q_sigma: float = 1.0
    k_sigma: float = 1.0
    v_sigma: float = 1.0
    seed: int = 0
    sample_rows: Optional[int] = None  # query rows per head the oracle checks
    Hkv: Optional[int] = None  # key/value heads (None: H)
    Nq: Optional[int] = None   # query rows per head (None: N, the key length)
    mask_sigma: Optional[float] = None  # shared fp32 [Nq, N] additive mask ~ N(0, sigma^2)

    @property
    def scale(self) -> np.float32:
        """The softmax scale 1/sqrt(d), as the float32 both sides receive."""
        return np.float32(1.0 / np.sqrt(np.float64(self.d)))

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv is None else self.Hkv

    @property
    def q_len(self) -> int:
        return self.N if self.Nq is None else self.Nq

    @property
    def general(self) -> bool:
        """Grouped key/value heads or a query length other than the key length."""
        return self.kv_heads != self.H or self.q_len != self.N

    @property
    def shape(self):
        """Q and O shape; K and V are ``kv_shape``."""
        return (self.B, self.H, self.q_len, self.d)

    @property
    def kv_shape(self):
        return (self.B, self.kv_heads, self.N, self.d)


WORKLOADS = {
    "single_head": Workload("single_head", 1, 1, 64, 32, F16, False, False, seed=1001),
    "reranker": Workload("reranker", 50, 12, 256, 32, F16, False, True,
                         key_len_lo=48, key_len_hi=256, seed=1002),
    "prefill": Workload("prefill", 1, 32, 4096, 128, F16, True, False, seed=1003),
    "peaky": Workload("peaky", 8, 16, 2048, 64, BF16, False, False,
                      q_sigma=3.0, k_sigma=3.0, seed=1004),
    "long_context": Workload("long_context", 1, 32, 32768, 128, BF16, True, False,
                             seed=1005, sample_rows=256),
    # The prefill's per-GPU share when its 32 heads are split 8 ways: 4 heads,
    # too few 256-row query tiles (64) to occupy the GPU, the shape the
    # split-key forward is for.
    "prefill_shard8": Workload("prefill_shard8", 1, 4, 4096, 128, F16, True, False, seed=1006),
    # grouped-query and cross-attention shapes
    "gqa_prefill": Workload("gqa_prefill", 1, 32, 4096, 128, F16, True, False, seed=1007, Hkv=8),
    "gqa_decode": Workload("gqa_decode", 8, 32, 32768, 128, BF16, True, True,
                           key_len_lo=16384, key_len_hi=32768, seed=1008, Hkv=8, Nq=1),
    "cross": Workload("cross", 4, 16, 4096, 64, F16, False, False, seed=1009, Nq=2048),
    # additive score mask
    "masked_prefill": Workload("masked_prefill", 1, 32, 4096, 128, F16, True, False, seed=1010,
                               mask_sigma=1.0),
}
WORKLOAD_ORDER = ["single_head", "reranker", "prefill", "peaky", "long_context"]
# workloads beyond the five the pages' configurations describe
EXTRA_WORKLOADS = ["prefill_shard8", "gqa_prefill", "gqa_decode", "cross", "masked_prefill"]


# ---------------------------------------------------------------- rounding
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (nearest-even, numpy's cast); return the bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16, nearest-even on the upper 16 bits; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        r = r.copy()
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of fp16/bf16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(dtype)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(x)
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------- drawing
def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def generate(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw one workload's inputs.

    Returns a dict with uint16 bit arrays ``Q`` (``w.shape``), ``K`` and
    ``V`` (``w.kv_shape``), ``key_len`` (int32 ``[B]`` or None), ``rows``
    (int64 ``[H, R]`` sampled query rows per head, or None), and the scalars
    ``dtype``, ``scale``, ``causal`` and ``seed``.
    """
    seed = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"workload": w.name, "dtype": w.dtype, "scale": w.scale,
           "causal": w.causal, "seed": seed,
           "B": w.B, "H": w.H, "N": w.N, "d": w.d, "Hkv": w.kv_heads, "Nq": w.q_len}
    for name, sigma, shape in (("Q", w.q_sigma, w.shape), ("K", w.k_sigma, w.kv_shape),
                               ("V", w.v_sigma, w.kv_shape)):
        out[name] = round_bits(_normal(rng, shape, sigma), w.dtype)
    out["key_len"] = None
    if w.key_padding:
        out["key_len"] = rng.integers(w.key_len_lo, w.key_len_hi + 1,
                                      size=w.B).astype(np.int32)
    out["mask"] = None
    if w.mask_sigma is not None:
        out["mask"] = _normal(rng, (w.q_len, w.N), w.mask_sigma)
    out["rows"] = None
    if w.sample_rows is not None:
        out["rows"] = np.stack([
            np.sort(rng.choice(w.q_len, size=w.sample_rows, replace=False))
            for _ in range(w.H)]).astype(np.int64)
    return out


def random_case(B: int, H: int, N: int, d: int, dtype: str, *, seed: int,
                sigma: float = 1.0, key_len=None) -> dict:
    """Draw Q, K, V of an arbitrary shape (same recipe as the workloads).

    ``key_len`` may be None, an explicit list, or ``"random"`` (uniform in
    [0, N] per sequence, drawn after V).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"dtype": dtype, "seed": seed, "B": B, "H": H, "N": N, "d": d,
           "scale": np.float32(1.0 / np.sqrt(np.float64(d)))}
    for name in ("Q", "K", "V"):
        out[name] = round_bits(_normal(rng, (B, H, N, d), sigma), dtype)
    if isinstance(key_len, str) and key_len == "random":
        key_len = rng.integers(0, N + 1, size=B)
    out["key_len"] = None if key_len is None else np.asarray(key_len, dtype=np.int32)
    return out


def random_case_general(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, dtype: str, *,
                        seed: int, sigma: float = 1.0, key_len=None) -> dict:
    """Q ``[B, H, Nq, d]`` and K, V ``[B, Hkv, Nk, d]`` drawn as in random_case
    (Q, K, V, then ``key_len``: None, a list, or ``"random"`` uniform in
    [0, Nk])."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"dtype": dtype, "seed": seed, "B": B, "H": H, "Hkv": Hkv, "Nq": Nq, "N": Nk,
           "d": d, "scale": np.float32(1.0 / np.sqrt(np.float64(d)))}
    out["Q"] = round_bits(_normal(rng, (B, H, Nq, d), sigma), dtype)
    for name in ("K", "V"):
        out[name] = round_bits(_normal(rng, (B, Hkv, Nk, d), sigma), dtype)
    if isinstance(key_len, str) and key_len == "random":
        key_len = rng.integers(0, Nk + 1, size=B)
    out["key_len"] = None if key_len is None else np.asarray(key_len, dtype=np.int32)
    return out


def random_mask(shape, *, seed: int, sigma: float = 1.0, neg_inf_frac: float = 0.0,
                empty_rows=()) -> np.ndarray:
    """An fp32 additive mask of the given shape drawn N(0, sigma^2); then a
    fraction ``neg_inf_frac`` of its elements set to -inf, and every element
    of the rows ``empty_rows`` (indices into the second-to-last axis) too."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = _normal(rng, shape, sigma)
    if neg_inf_frac > 0:
        m[rng.random(size=shape) < neg_inf_frac] = -np.inf
    for r in empty_rows:
        m[..., r, :] = -np.inf
    return m


def all_rows_selection(B: int, H: int, N: int) -> np.ndarray:
    """Every (b, h, i) triple, row-major; int64 ``[B*H*N, 3]``."""
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def sampled_rows_selection(rows: np.ndarray, B: int = 1) -> np.ndarray:
    """(b, h, i) triples for per-head row samples ``rows[h, r]`` (every b)."""
    H, R = rows.shape
    out = []
    for b in range(B):
        for h in range(H):
            for i in rows[h]:
                out.append((b, h, int(i)))
    return np.asarray(out, dtype=np.int64)
