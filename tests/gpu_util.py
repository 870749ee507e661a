"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP entry points through the C ABI binding, run the oracle on chosen rows and
compare to the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np
import torch

import attn_inputs as ai
import oracle

# |O_gpu - O_ref| <= atol + rtol |O_ref|, per dtype; |LSE_gpu - LSE_ref| <= LSE_TOL
TOL = {ai.F16: (2e-3, 2e-3), ai.BF16: (1e-2, 1e-2)}
LSE_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device() -> torch.device:
    return torch.device("cuda:0")


def torch_dtype(dtype: str):
    return torch.float16 if dtype == ai.F16 else torch.bfloat16


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device())
    return t.view(torch_dtype(dtype))


def from_dev(t: torch.Tensor, dtype: str) -> np.ndarray:
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return ai.bits_to_f32(bits, dtype)


def dev_inputs(case: dict):
    q = to_dev(case["Q"], case["dtype"])
    k = to_dev(case["K"], case["dtype"])
    v = to_dev(case["V"], case["dtype"])
    kl = None
    if case.get("key_len") is not None:
        kl = torch.from_numpy(np.asarray(case["key_len"], np.int32)).to(device())
    return q, k, v, kl


def run_fused(case: dict, causal: bool, inputs=None):
    import exact_self_attention_amd as attn
    q, k, v, kl = inputs if inputs is not None else dev_inputs(case)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn.attn_fwd(q, k, v, o, lse, scale=float(case["scale"]), causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return from_dev(o, case["dtype"]), lse.cpu().numpy()


def run_naive(case: dict, causal: bool, inputs=None, max_workspace_bytes=None):
    import exact_self_attention_amd as attn
    q, k, v, kl = inputs if inputs is not None else dev_inputs(case)
    B, H, N, _ = q.shape
    nbytes = attn.attn_fwd_naive_workspace_bytes(B, H, N)
    if max_workspace_bytes is not None:
        nbytes = max(min(nbytes, max_workspace_bytes), attn.attn_fwd_naive_workspace_bytes(1, 1, N))
    # NaN-poisoned: the baseline must read only scores it wrote
    ws = torch.full((max(nbytes // 4, 1),), float("nan"), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn.attn_fwd_naive(q, k, v, o, lse, workspace=ws, scale=float(case["scale"]),
                        causal=causal, key_len=kl)
    torch.cuda.synchronize()
    del ws
    return from_dev(o, case["dtype"]), lse.cpu().numpy()


def run_split(case: dict, causal: bool, n_splits=None, inputs=None):
    """attn_fwd_splitkv with n_splits key ranges (None: the library's default)."""
    import exact_self_attention_amd as attn
    q, k, v, kl = inputs if inputs is not None else dev_inputs(case)
    B, H, N, d = q.shape
    if n_splits is None:
        code = attn.ATTN_F16 if case["dtype"] == "f16" else attn.ATTN_BF16
        n_splits = attn.attn_fwd_splitkv_default_splits(code, B, H, N, d, causal)
    nbytes = attn.attn_fwd_splitkv_workspace_bytes(B, H, N, d, n_splits)
    # NaN-poisoned: a split with no visible key for a row writes no partial
    # output for it, and the merge must leave that memory out entirely
    ws = torch.full((max(nbytes // 4, 1),), float("nan"), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn.attn_fwd_splitkv(q, k, v, o, lse, workspace=ws, n_splits=n_splits,
                          scale=float(case["scale"]), causal=causal, key_len=kl)
    torch.cuda.synchronize()
    del ws
    return from_dev(o, case["dtype"]), lse.cpu().numpy(), n_splits


def run_gqa(case: dict, causal: bool, inputs=None):
    """attn_fwd_gqa: q, o [B, H, Nq, d]; k, v [B, Hkv, Nk, d]."""
    import exact_self_attention_amd as attn
    q, k, v, kl = inputs if inputs is not None else dev_inputs(case)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn.attn_fwd_gqa(q, k, v, o, lse, scale=float(case["scale"]), causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return from_dev(o, case["dtype"]), lse.cpu().numpy()


def run_gqa_split(case: dict, causal: bool, n_splits=None, inputs=None):
    """attn_fwd_gqa_splitkv with n_splits key ranges (None: the library's default)."""
    import exact_self_attention_amd as attn
    q, k, v, kl = inputs if inputs is not None else dev_inputs(case)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if n_splits is None:
        code = attn.ATTN_F16 if case["dtype"] == "f16" else attn.ATTN_BF16
        n_splits = attn.attn_fwd_gqa_splitkv_default_splits(code, B, H, Hkv, Nq, Nk, d, causal)
    nbytes = attn.attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits)
    # NaN-poisoned: a split with no visible key for a row writes no partial
    # output for it, and the merge must leave that memory out entirely
    ws = torch.full((max(nbytes // 4, 1),), float("nan"), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    attn.attn_fwd_gqa_splitkv(q, k, v, o, lse, workspace=ws, n_splits=n_splits,
                              scale=float(case["scale"]), causal=causal, key_len=kl)
    torch.cuda.synchronize()
    del ws
    return from_dev(o, case["dtype"]), lse.cpu().numpy(), n_splits


def run_masked(case: dict, causal: bool, mask: np.ndarray, n_splits=None, inputs=None,
               mask_dev=None):
    """attn_fwd_masked (n_splits None) or attn_fwd_masked_splitkv with an fp32
    mask of shape [Nq, Nk] or [B|1, H|1, Nq, Nk]."""
    import exact_self_attention_amd as attn
    q, k, v, kl = inputs if inputs is not None else dev_inputs(case)
    m = mask_dev if mask_dev is not None else torch.from_numpy(np.ascontiguousarray(mask)).to(device())
    # NaN-poisoned, so that a query tile the launch order missed shows up
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    if n_splits is None:
        attn.attn_fwd_masked(q, k, v, o, lse, mask=m, scale=float(case["scale"]), causal=causal,
                             key_len=kl)
    else:
        B, H, Nq, d = q.shape
        nbytes = attn.attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits)
        # NaN-poisoned: a split with no visible key for a row writes no
        # partial output for it, and the merge must leave that memory out
        ws = torch.full((max(nbytes // 4, 1),), float("nan"), dtype=torch.float32, device=q.device)
        attn.attn_fwd_masked_splitkv(q, k, v, o, lse, mask=m, workspace=ws, n_splits=n_splits,
                                     scale=float(case["scale"]), causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return from_dev(o, case["dtype"]), lse.cpu().numpy()


def oracle_rows(case: dict, causal: bool, sel: np.ndarray, mask=None):
    """The oracle on rows sel; K and V may have their own [B, Hkv, Nk, d]
    shape; ``mask`` an additive fp32 mask ([Nq, Nk] or [B|1, H|1, Nq, Nk])."""
    dt = case["dtype"]
    Q = ai.bits_to_f32(case["Q"], dt)
    K = ai.bits_to_f32(case["K"], dt)
    V = ai.bits_to_f32(case["V"], dt)
    return oracle.attn_rows(Q, K, V, float(case["scale"]), causal, case.get("key_len"), sel,
                            mask=mask)


def sample_rows(B: int, H: int, N: int, per_head: int, seed: int) -> np.ndarray:
    """(b, h, i) triples: per (b, h) the first and last rows, the rows on
    both sides of the 32-row wave blocks and of the 128- and 256-row query
    tiles near the start, plus ``per_head`` seeded random rows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513,
             N // 2 - 1, N // 2, N - 257, N - 256, N - 2, N - 1]
    out = []
    for b in range(B):
        for h in range(H):
            rows = set(i for i in fixed if 0 <= i < N)
            rows.update(rng.choice(N, size=min(per_head, N), replace=False).tolist())
            out.extend((b, h, i) for i in sorted(rows))
    return np.asarray(out, dtype=np.int64)


def gather(O: np.ndarray, LSE: np.ndarray, sel: np.ndarray):
    return O[sel[:, 0], sel[:, 1], sel[:, 2]], LSE[sel[:, 0], sel[:, 1], sel[:, 2]]


def assert_close(O, LSE, O_ref, LSE_ref, dtype: str, what: str, sel=None) -> dict:
    atol, rtol = TOL[dtype]
    O = np.asarray(O, np.float64)
    err = np.abs(O - O_ref)
    bound = atol + rtol * np.abs(O_ref)
    bad = ~(err <= bound)  # NaN counts as bad
    ratio = np.where(bound > 0, err / bound, np.inf)
    worst = np.unravel_index(np.nanargmax(np.where(np.isnan(ratio), np.inf, ratio)), ratio.shape)
    fin = np.isfinite(LSE_ref)
    lse_same_inf = np.array_equal(fin, np.isfinite(LSE)) and \
        np.array_equal(LSE_ref[~fin], LSE[~fin])
    lse_err = np.abs(np.asarray(LSE, np.float64)[fin] - LSE_ref[fin])
    stats = {"what": what, "max_abs_err": float(np.nanmax(err)) if err.size else 0.0,
             "max_err_over_bound": float(ratio[worst]) if err.size else 0.0,
             "max_lse_err": float(lse_err.max()) if lse_err.size else 0.0,
             "n_checked": int(O.shape[0])}
    log(f"  {what}: {stats}")
    where = "" if sel is None else f" at (b,h,i)={tuple(sel[worst[0]])}, c={worst[-1]}"
    assert not bad.any(), (f"{what}: {int(bad.sum())} O elements out of tolerance; worst "
                           f"{O[worst]} vs {O_ref[worst]}{where}")
    assert lse_same_inf, f"{what}: -inf LSE rows differ"
    assert not (lse_err > LSE_TOL).any(), f"{what}: LSE error {lse_err.max()}"
    return stats
