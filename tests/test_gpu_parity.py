"""GPU parity: the HIP entry points, called through the C ABI, against the fp64
oracle on the same seeded inputs, and against closed forms at full size."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# Every row is checked except at long_context, whose oracle rows are the
# workload's own seeded sample of 256 rows per head.
ROWS_PER_HEAD = {"single_head": None, "reranker": None, "prefill": None,
                 "peaky": None, "long_context": None}


def _selection(w, case):
    if w.name == "long_context":
        return ai.sampled_rows_selection(case["rows"], w.B)
    if ROWS_PER_HEAD[w.name] is None:
        return ai.all_rows_selection(w.B, w.H, w.N)
    return gu.sample_rows(w.B, w.H, w.N, ROWS_PER_HEAD[w.name], seed=w.seed + 7)


@pytest.fixture(scope="module")
def cases():
    return {}


def _case(cases, name):
    if name not in cases:
        w = ai.WORKLOADS[name]
        gu.log(f"generating {name} {w.shape} {w.dtype} seed={w.seed}")
        cases[name] = ai.generate(w)
    return cases[name]


def _reference(cases, w, case):
    """The workload's checked rows and their oracle values (computed once
    per module: the fused and the unfused tests share them)."""
    key = ("ref", w.name)
    if key not in cases:
        sel = _selection(w, case)
        gu.log(f"oracle {w.name}: {len(sel)} rows")
        cases[key] = (sel, *gu.oracle_rows(case, w.causal, sel))
    return cases[key]


@pytest.mark.parametrize("name", ai.WORKLOAD_ORDER)
def test_fused_matches_oracle_on_workload(cases, name):
    w = ai.WORKLOADS[name]
    case = _case(cases, name)
    gu.log(f"fused parity {name} {w.shape} {w.dtype} causal={w.causal}")
    O, LSE = gu.run_fused(case, w.causal)
    sel, O_ref, LSE_ref = _reference(cases, w, case)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, w.dtype, f"fused/{name}", sel)
    assert np.all(np.isfinite(O))


# The unfused baseline's fp32 scores of a whole workload would not fit at
# long_context (32 heads x 32768^2 x 4 B = 137 GB): it runs one head per
# launch through a one-head workspace (4.3 GB).
NAIVE_MAX_WORKSPACE = {"long_context": 32768 * 32768 * 4}


@pytest.mark.parametrize("name", ai.WORKLOAD_ORDER)
def test_naive_matches_oracle_on_workload(cases, name):
    w = ai.WORKLOADS[name]
    case = _case(cases, name)
    gu.log(f"naive parity {name}")
    O, LSE = gu.run_naive(case, w.causal, max_workspace_bytes=NAIVE_MAX_WORKSPACE.get(name))
    sel, O_ref, LSE_ref = _reference(cases, w, case)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, w.dtype, f"naive/{name}", sel)


def test_naive_in_head_groups_matches_full_workspace(cases):
    w = ai.WORKLOADS["reranker"]
    case = _case(cases, "reranker")
    O1, L1 = gu.run_naive(case, w.causal)
    O2, L2 = gu.run_naive(case, w.causal, max_workspace_bytes=7 * 256 * 256 * 4)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


FUZZ_N = [1, 2, 17, 48, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 1000]
FUZZ = []
for _n in FUZZ_N:
    for _d in (32, 64, 128):
        for _causal in (False, True):
            FUZZ.append((_n, _d, _causal))


@pytest.mark.parametrize("N,d,causal", FUZZ, ids=[f"N{n}-d{d}-{'c' if c else 'f'}" for n, d, c in FUZZ])
def test_fuzz_shapes(N, d, causal):
    dtype = ai.BF16 if (N + d) % 2 else ai.F16
    seed = 10_000 + N * 7 + d * 3 + causal
    # key lengths cover 0, 1, N-1, N and a random value
    B = 5
    kl = [0, 1, max(N - 1, 0), N, int(np.random.default_rng(seed).integers(0, N + 1))]
    case = ai.random_case(B, 2, N, d, dtype, seed=seed, sigma=1.5, key_len=kl)
    gu.log(f"fuzz N={N} d={d} causal={causal} {dtype} key_len={kl}")
    O, LSE = gu.run_fused(case, causal)
    sel = ai.all_rows_selection(B, 2, N)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"fuzz N={N} d={d} causal={causal}", sel)
    # no key-length array: every key visible
    case["key_len"] = None
    O, LSE = gu.run_fused(case, causal)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"fuzz-nomask N={N} d={d}", sel)


@pytest.mark.parametrize("name", ["prefill", "long_context"])
def test_zero_query_gives_prefix_means_every_row(name):
    """Q = 0 under causal masking: O_i is the mean of V_0..V_i and LSE_i = ln(i+1),
    checked on every row at the full workload size."""
    w = ai.WORKLOADS[name]
    gu.log(f"zero-query closed form {name}")
    rng = np.random.Generator(np.random.PCG64(w.seed + 100))
    vbits = ai.round_bits(rng.standard_normal(size=w.shape, dtype=np.float32), w.dtype)
    qbits = np.zeros(w.shape, np.uint16)
    kbits = ai.round_bits(rng.standard_normal(size=w.shape, dtype=np.float32), w.dtype)
    case = {"Q": qbits, "K": kbits, "V": vbits, "dtype": w.dtype, "scale": w.scale, "key_len": None}
    O, LSE = gu.run_fused(case, True)
    del kbits, qbits
    atol, rtol = gu.TOL[w.dtype]
    V = ai.bits_to_f32(vbits, w.dtype)
    n = np.arange(1, w.N + 1, dtype=np.float64)[:, None]
    for h in range(w.H):
        ref = np.cumsum(V[0, h].astype(np.float64), axis=0) / n
        err = np.abs(O[0, h] - ref)
        assert np.all(err <= atol + rtol * np.abs(ref)), (h, float(err.max()))
        assert np.all(np.abs(LSE[0, h] - np.log(n[:, 0])) <= gu.LSE_TOL), h


def test_causal_row_zero_is_exact():
    w = ai.WORKLOADS["prefill"]
    case = ai.generate(w)
    O, LSE = gu.run_fused(case, True)
    V = ai.bits_to_f32(case["V"], w.dtype)
    assert np.array_equal(O[:, :, 0], V[:, :, 0])


def test_padding_rows_are_never_read():
    """NaN in K and V rows at or past each key length leaves O and LSE unchanged."""
    case = ai.random_case(4, 3, 300, 64, ai.F16, seed=77, key_len=[0, 1, 130, 299])
    O1, L1 = gu.run_fused(case, False)
    nan16 = np.uint16(0x7E00)
    for b, L in enumerate(case["key_len"]):
        case["K"][b, :, L:] = nan16
        case["V"][b, :, L:] = nan16
    O2, L2 = gu.run_fused(case, False)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    assert np.all(np.isfinite(O2))
    assert np.all(O2[0] == 0) and np.all(np.isneginf(L2[0]))


def test_key_len_one_returns_first_value_row():
    case = ai.random_case(2, 2, 200, 128, ai.BF16, seed=78, key_len=[1, 1])
    for causal in (False, True):
        O, LSE = gu.run_fused(case, causal)
        V = ai.bits_to_f32(case["V"], ai.BF16)
        for i in (0, 5, 199):
            assert np.array_equal(O[:, :, i], V[:, :, 0])


def test_bitwise_deterministic():
    w = ai.WORKLOADS["peaky"]
    case = ai.generate(w)
    inputs = gu.dev_inputs(case)
    O1, L1 = gu.run_fused(case, w.causal, inputs)
    O2, L2 = gu.run_fused(case, w.causal, inputs)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_slices_are_independent():
    """Changing one (b, h) slice leaves every other slice bitwise equal."""
    case = ai.random_case(2, 3, 257, 32, ai.F16, seed=79)
    O1, L1 = gu.run_fused(case, True)
    case["K"][1, 2] = ai.round_bits(np.full((257, 32), 0.5, np.float32), ai.F16)
    O2, L2 = gu.run_fused(case, True)
    keep = np.ones((2, 3), bool)
    keep[1, 2] = False
    assert np.array_equal(O1[keep], O2[keep]) and np.array_equal(L1[keep], L2[keep])
    assert not np.array_equal(O1[1, 2], O2[1, 2])


def test_output_written_only_inside_bounds():
    """Canaries around O and LSE survive a launch whose N is not a tile multiple."""
    case = ai.random_case(1, 2, 131, 128, ai.F16, seed=80)
    q, k, v, _ = gu.dev_inputs(case)
    import exact_self_attention_amd as attn
    n_o = q.numel()
    buf = torch.full((n_o + 2048,), -7.0, dtype=torch.float16, device=q.device)
    o = buf[1024:1024 + n_o].view(q.shape)
    lbuf = torch.full((2 * 131 + 128,), 3.5, dtype=torch.float32, device=q.device)
    lse = lbuf[64:64 + 2 * 131].view(1, 2, 131)
    attn.attn_fwd(q, k, v, o, lse, scale=float(case["scale"]), causal=False)
    torch.cuda.synchronize()
    assert torch.all(buf[:1024] == -7.0) and torch.all(buf[1024 + n_o:] == -7.0)
    assert torch.all(lbuf[:64] == 3.5) and torch.all(lbuf[64 + 2 * 131:] == 3.5)


# Shapes with many more 256-row query tiles than the GPU holds at once, so
# workgroups of the streaming kernel start as earlier ones retire; key
# lengths mix full, short (padded slices of fewer than 4 tiles), one and
# zero.  Every row is checked.
STREAM_CASES = [
    # (B, H, N, d, causal, dtype)
    (24, 16, 700, 128, True, ai.F16),
    (24, 16, 700, 128, False, ai.BF16),
    (48, 12, 520, 64, False, ai.BF16),
    (48, 12, 520, 64, True, ai.F16),
    (64, 12, 300, 32, False, ai.F16),
]


@pytest.mark.parametrize("B,H,N,d,causal,dtype", STREAM_CASES,
                         ids=[f"B{b}H{h}N{n}d{d}{'c' if c else 'f'}{t}" for b, h, n, d, c, t in STREAM_CASES])
def test_streaming_many_items_per_workgroup(B, H, N, d, causal, dtype):
    seed = 20_000 + B + H + N + d + causal
    rng = np.random.default_rng(seed)
    kl = rng.integers(0, N + 1, size=B)
    kl[:4] = [N, 1, 0, 70]
    case = ai.random_case(B, H, N, d, dtype, seed=seed, sigma=1.5, key_len=[int(x) for x in kl])
    gu.log(f"stream B={B} H={H} N={N} d={d} causal={causal} {dtype}")
    O, LSE = gu.run_fused(case, causal)
    sel = ai.all_rows_selection(B, H, N)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"stream B={B} H={H} N={N} d={d} causal={causal}", sel)


# attn_fwd_splitkv: key ranges computed by separate workgroups and merged.
# Cases cover every d, both dtypes, causal, key lengths 0 / 1 / short / full,
# one split, and more splits than a row has key tiles (empty splits).
SPLIT_CASES = [
    # (B, H, N, d, causal, dtype, n_splits)
    (4, 3, 1000, 128, False, ai.F16, 3),
    (4, 3, 1000, 128, True, ai.BF16, 4),
    (4, 3, 700, 64, False, ai.BF16, 5),
    (4, 3, 700, 64, True, ai.F16, 2),
    (4, 2, 300, 32, False, ai.F16, 3),
    (4, 2, 513, 128, True, ai.F16, 64),
    (4, 2, 200, 64, False, ai.BF16, 1),
]


@pytest.mark.parametrize("B,H,N,d,causal,dtype,S", SPLIT_CASES,
                         ids=[f"B{b}H{h}N{n}d{d}{'c' if c else 'f'}{t}S{s}" for b, h, n, d, c, t, s in SPLIT_CASES])
def test_splitkv_matches_oracle(B, H, N, d, causal, dtype, S):
    seed = 30_000 + B + H + N + d + causal + S
    kl = [N, 1, 0, int(np.random.default_rng(seed).integers(2, N + 1))]
    case = ai.random_case(B, H, N, d, dtype, seed=seed, sigma=1.5, key_len=kl)
    gu.log(f"splitkv B={B} H={H} N={N} d={d} causal={causal} {dtype} S={S} key_len={kl}")
    O, LSE, _ = gu.run_split(case, causal, S)
    sel = ai.all_rows_selection(B, H, N)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"splitkv N={N} d={d} S={S}", sel)


def test_splitkv_default_splits_long_few_heads():
    # few heads, long causal sequence: the default split count fills the GPU
    B, H, N, d = 1, 4, 8192, 128
    case = ai.random_case(B, H, N, d, ai.BF16, seed=31_001, sigma=1.0)
    O, LSE, S = gu.run_split(case, True)
    gu.log(f"splitkv default splits for B={B} H={H} N={N}: {S}")
    assert S > 1
    sel = gu.sample_rows(B, H, N, 48, seed=31_002)
    O_ref, LSE_ref = gu.oracle_rows(case, True, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, ai.BF16, "splitkv default S", sel)


def test_prefill_shard_workload_fused_and_split():
    # the prefill's 8-way head shard: both entry points on the workload's inputs
    w = ai.WORKLOADS["prefill_shard8"]
    case = ai.generate(w)
    sel = gu.sample_rows(w.B, w.H, w.N, 64, seed=w.seed + 7)
    O_ref, LSE_ref = gu.oracle_rows(case, w.causal, sel)
    O, LSE = gu.run_fused(case, w.causal)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, w.dtype, "prefill_shard8 fused", sel)
    O, LSE, S = gu.run_split(case, w.causal)
    gu.log(f"prefill_shard8 default splits: {S}")
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, w.dtype, f"prefill_shard8 split S={S}", sel)


# Grouped-query and cross-attention through attn_fwd_gqa: K and V have Hkv
# heads and Nk rows, Q has H heads of Nq rows.  Cases: both kernels (short:
# Nk <= 256 at d <= 64, <= 128 at d = 128), Nq < Nk and Nq > Nk (rows that
# see no key under the end-aligned causal mask), one key/value head, single
# query rows, slices whose 32-row wave blocks span several heads (Nq = 20,
# 5), key lengths full / 1 / short, and Nk = 0.  Every row is checked.
GQA_CASES = [
    # (B, H, Hkv, Nq, Nk, d, causal, dtype, key_len)
    (2, 8, 2, 300, 1000, 64, True, ai.F16, None),
    (2, 8, 2, 300, 1000, 64, False, ai.BF16, [1000, 517]),
    (1, 6, 1, 700, 300, 128, True, ai.F16, None),
    (3, 16, 4, 1, 2000, 128, True, ai.BF16, [2000, 1, 1234]),
    (2, 12, 3, 20, 700, 32, True, ai.F16, [700, 650]),
    (2, 8, 8, 513, 257, 64, True, ai.BF16, None),
    (2, 6, 3, 77, 200, 32, True, ai.F16, None),
    (2, 4, 2, 5, 128, 128, True, ai.BF16, [128, 60]),
    (1, 4, 4, 33, 250, 64, False, ai.F16, None),
    (2, 6, 2, 300, 64, 64, True, ai.F16, [64, 0]),
    (1, 8, 2, 64, 0, 64, True, ai.F16, None),
    # at most 32 query rows per key/value head (the decode kernel)
    (2, 8, 2, 8, 1500, 64, True, ai.BF16, [1500, 333]),
    (1, 4, 1, 7, 300, 32, True, ai.F16, None),
    (2, 4, 4, 3, 129, 128, True, ai.F16, [129, 64]),
]


def _gqa_id(c):
    B, H, Hkv, Nq, Nk, d, causal, dtype, kl = c
    return f"B{B}H{H}kv{Hkv}q{Nq}k{Nk}d{d}{'c' if causal else 'f'}{dtype}{'' if kl is None else 'L'}"


def _gqa_case(B, H, Hkv, Nq, Nk, d, causal, dtype, kl, salt):
    seed = salt + B + H + Hkv + Nq + Nk + d + causal
    return ai.random_case_general(B, H, Hkv, Nq, Nk, d, dtype, seed=seed, sigma=1.5, key_len=kl)


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,dtype,kl", GQA_CASES, ids=[_gqa_id(c) for c in GQA_CASES])
def test_gqa_matches_oracle(B, H, Hkv, Nq, Nk, d, causal, dtype, kl):
    case = _gqa_case(B, H, Hkv, Nq, Nk, d, causal, dtype, kl, 40_000)
    gu.log(f"gqa {_gqa_id((B, H, Hkv, Nq, Nk, d, causal, dtype, kl))} key_len={kl}")
    O, LSE = gu.run_gqa(case, causal)
    sel = ai.all_rows_selection(B, H, Nq)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"gqa {_gqa_id((B, H, Hkv, Nq, Nk, d, causal, dtype, kl))}", sel)
    if causal and Nq > Nk:  # rows before the first key see nothing
        assert np.all(O[:, :, :Nq - Nk] == 0) and np.all(np.isneginf(LSE[:, :, :Nq - Nk]))


GROWING_SCORE_CASES = [
    # (B, H, N, d, dtype): key tiles whose K rows are scaled up tile after
    # tile, so that later tiles' scores exceed the running max by far more
    # than the exponentials-first bound: the redo with a row max runs
    # (short-sequence kernel at N <= 256, streaming kernel at d = 128 above)
    (2, 3, 256, 32, ai.F16),
    (2, 3, 256, 64, ai.BF16),
    (2, 3, 128, 128, ai.F16),
    (1, 2, 1024, 128, ai.F16),
    (1, 2, 1024, 128, ai.BF16),
]


def _bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == ai.F16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,d,dtype", GROWING_SCORE_CASES,
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{c[4]}" for c in GROWING_SCORE_CASES])
def test_growing_scores_take_the_max_first_path(B, H, N, d, dtype, causal):
    seed = 48_000 + N + d + causal
    case = ai.random_case(B, H, N, d, dtype, seed=seed, sigma=1.5)
    k = _bits_to_f32(case["K"], dtype)
    tile = np.arange(N) // 64
    factor = (1.0 + 4.0 * (tile % 4)).astype(np.float32)  # x1, x5, x9, x13, x1, ...
    case["K"] = ai.round_bits(k * factor[None, None, :, None], dtype)
    gu.log(f"growing scores B={B} H={H} N={N} d={d} {dtype} causal={causal}")
    O, LSE = gu.run_fused(case, causal)
    sel = ai.all_rows_selection(B, H, N)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"growing scores N={N} d={d} causal={causal}", sel)


PADDED_MANY_CASES = [
    # (B, H, Hkv, Nq, Nk, d, dtype): many padded sequences without a causal
    # mask, every tile count among them, on the short-sequence kernel
    (150, 4, 2, 200, 256, 32, ai.F16),
    (70, 2, 2, 128, 200, 64, ai.BF16),
    (65, 1, 1, 100, 128, 128, ai.F16),
    (1030, 1, 1, 40, 64, 32, ai.BF16),
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,dtype", PADDED_MANY_CASES,
                         ids=[f"B{c[0]}H{c[1]}kv{c[2]}q{c[3]}k{c[4]}d{c[5]}{c[6]}" for c in PADDED_MANY_CASES])
def test_padded_many_sequences(B, H, Hkv, Nq, Nk, d, dtype):
    seed = 47_000 + B + Nk + d
    rng = np.random.default_rng(seed)
    kl = rng.integers(0, Nk + 1, size=B)
    edge = [x for x in (0, 1, 63, 64, 65, Nk - 1, Nk) if x <= Nk]  # every tile count, empty and full
    kl[:len(edge)] = edge
    kl = [int(x) for x in rng.permutation(kl)]
    case = ai.random_case_general(B, H, Hkv, Nq, Nk, d, dtype, seed=seed, sigma=1.5, key_len=kl)
    gu.log(f"padded many B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype}")
    O, LSE = gu.run_gqa(case, False)
    sel = ai.all_rows_selection(B, H, Nq)
    O_ref, LSE_ref = gu.oracle_rows(case, False, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"padded many B={B} d={d}", sel)


# The longest sequences, far past the workloads' 32768: positions, tile
# counts and offsets in the hundreds of thousands (and a million keys for
# the split decode), on sampled rows that include the tile boundaries, the
# last rows and a key length that ends inside a tile.
LONG_CASES = [
    # (B, H, N, d, causal, dtype, key_len)
    (1, 2, 262144, 64, True, ai.F16, [262144 - 1000]),
    (1, 1, 131072, 128, False, ai.BF16, [131072 - 33]),
]


@pytest.mark.parametrize("B,H,N,d,causal,dtype,kl", LONG_CASES,
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}{'c' if c[4] else 'f'}{c[5]}" for c in LONG_CASES])
def test_longest_sequences(B, H, N, d, causal, dtype, kl):
    case = ai.random_case(B, H, N, d, dtype, seed=60_000 + N + d, key_len=kl)
    gu.log(f"longest B={B} H={H} N={N} d={d} causal={causal} {dtype}")
    O, LSE = gu.run_fused(case, causal)
    sel = gu.sample_rows(B, H, N, 32, seed=60_100 + N)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"longest N={N}", sel)


def test_million_key_decode_split():
    # one new token of 8 query heads against a history of about 2^20 keys,
    # through the split decode with the library's split count; every row
    B, H, Hkv, Nq, Nk, d = 1, 8, 1, 1, 1 << 20, 128
    case = ai.random_case_general(B, H, Hkv, Nq, Nk, d, ai.BF16, seed=61_000, key_len=[Nk - 77])
    gu.log(f"million-key decode B={B} H={H} Hkv={Hkv} Nk={Nk} d={d}")
    O, LSE, _ = gu.run_gqa_split(case, True)
    sel = ai.all_rows_selection(B, H, Nq)
    O_ref, LSE_ref = gu.oracle_rows(case, True, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, ai.BF16, "million-key decode", sel)


GQA_SPLIT_CASES = [
    # (B, H, Hkv, Nq, Nk, d, causal, dtype, key_len, n_splits)
    (3, 16, 4, 1, 2000, 128, True, ai.BF16, [2000, 1, 1234], 8),
    (2, 8, 2, 300, 1000, 64, True, ai.F16, None, 3),
    (1, 6, 1, 700, 300, 128, True, ai.F16, None, 4),
    (2, 12, 3, 20, 700, 32, True, ai.BF16, [700, 650], 5),
    (2, 8, 8, 1, 600, 64, False, ai.F16, [600, 0], 64),
    (2, 8, 2, 8, 1500, 64, True, ai.BF16, [1500, 333], 5),
    (1, 4, 1, 7, 300, 32, True, ai.F16, None, 2),
    # decode shapes (at most 32 rows per key/value head): many heads of
    # unequal key length with empty ones between them, more splits than
    # tiles, and no visible key at all
    (9, 8, 2, 1, 700, 128, False, ai.F16, [0, 1, 33, 700, 0, 64, 65, 5, 0], 1),
    (9, 8, 2, 4, 700, 64, True, ai.BF16, [0, 1, 33, 700, 0, 64, 65, 5, 0], 3),
    (4, 4, 4, 1, 3000, 32, False, ai.BF16, [3000, 17, 2900, 1], 7),
    (5, 8, 4, 1, 2500, 128, True, ai.BF16, [2500, 1200, 2100, 37, 2499], 4),
    (3, 4, 2, 2, 100, 64, True, ai.F16, [0, 0, 0], 2),
    # the library's default split count (None) on causal shapes whose query
    # tiles see unequal key ranges: most late splits of the early tiles have
    # no work, and query tiles span head boundaries
    (2, 8, 2, 1000, 3000, 128, True, ai.F16, [3000, 1700], None),
    (1, 4, 4, 2500, 2500, 64, True, ai.BF16, None, None),
    (1, 4, 2, 600, 4000, 32, True, ai.F16, [3900], None),
    # more than 64 query tiles per slice (79): a workgroup's search for its
    # tile in the split grid takes two steps of 64 tiles; in the second,
    # query tiles span head boundaries
    (1, 1, 1, 20000, 20000, 64, True, ai.BF16, [19000], 3),
    (1, 4, 1, 5000, 5000, 32, True, ai.F16, None, 2),
    # more query rows than keys under the end-aligned causal mask: the first
    # query tiles see no key at all, get one workgroup each, and that one
    # writes LSE = -inf for every split of their rows
    (1, 2, 2, 1000, 100, 64, True, ai.F16, None, 3),
    (2, 4, 2, 700, 300, 128, True, ai.BF16, [300, 41], 4),
]


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,dtype,kl,S", GQA_SPLIT_CASES,
                         ids=[_gqa_id(c[:9]) + f"S{c[9]}" for c in GQA_SPLIT_CASES])
def test_gqa_splitkv_matches_oracle(B, H, Hkv, Nq, Nk, d, causal, dtype, kl, S):
    case = _gqa_case(B, H, Hkv, Nq, Nk, d, causal, dtype, kl, 50_000)
    gu.log(f"gqa splitkv {_gqa_id((B, H, Hkv, Nq, Nk, d, causal, dtype, kl))} S={S}")
    O, LSE, S = gu.run_gqa_split(case, causal, S)
    gu.log(f"  splits: {S}")
    sel = ai.all_rows_selection(B, H, Nq)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"gqa splitkv S={S}", sel)


def test_gqa_equals_attn_fwd_on_repeated_heads():
    # the same problem through attn_fwd with each key/value head copied to its
    # query heads: bitwise equal (same kernel, same key order per row)
    B, H, Hkv, N, d = 2, 8, 2, 600, 64
    case = ai.random_case_general(B, H, Hkv, N, N, d, ai.F16, seed=41_000, key_len=[600, 333])
    q, k, v, kl = gu.dev_inputs(case)
    O1, L1 = gu.run_gqa(case, True, inputs=(q, k, v, kl))
    kr = torch.repeat_interleave(k, H // Hkv, dim=1).contiguous()
    vr = torch.repeat_interleave(v, H // Hkv, dim=1).contiguous()
    O2, L2 = gu.run_fused(case, True, inputs=(q, kr, vr, kl))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


GQA_ROWS_PER_HEAD = {"gqa_prefill": 32, "gqa_decode": None, "cross": 32}


@pytest.mark.parametrize("name", ["gqa_prefill", "gqa_decode", "cross"])
def test_gqa_workload_matches_oracle(cases, name):
    # the full-size grouped-query / cross-attention workloads, through
    # attn_fwd_gqa and through its split form with the default split count
    w = ai.WORKLOADS[name]
    case = _case(cases, name)
    per_head = GQA_ROWS_PER_HEAD[name]
    sel = ai.all_rows_selection(w.B, w.H, w.q_len) if per_head is None else \
        gu.sample_rows(w.B, w.H, w.q_len, per_head, seed=w.seed + 7)
    O_ref, LSE_ref = gu.oracle_rows(case, w.causal, sel)
    gu.log(f"{name}: fused")
    O, LSE = gu.run_gqa(case, w.causal)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, w.dtype, f"{name} fused", sel)
    O, LSE, S = gu.run_gqa_split(case, w.causal)
    gu.log(f"{name}: default splits {S}")
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, w.dtype, f"{name} split S={S}", sel)


# Additive fp32 mask (attn_fwd_masked): shared [Nq, Nk] masks, per-head and
# per-batch masks, masks with -inf elements and rows that are -inf
# throughout, with and without the causal and key-length masks, every d and
# both dtypes, grouped heads and Nq != Nk, short key lengths (which take the
# streaming kernel when masked).  Every row is checked.
MASK_CASES = [
    # (B, H, Hkv, Nq, Nk, d, causal, dtype, key_len, mask shape kind, -inf fraction)
    (1, 4, 4, 700, 700, 128, True, ai.F16, None, "shared", 0.0),
    (2, 4, 2, 300, 1000, 128, False, ai.BF16, [1000, 421], "per_head", 0.0),
    (2, 6, 3, 257, 257, 64, True, ai.F16, None, "per_batch", 0.3),
    (2, 8, 8, 100, 600, 64, True, ai.BF16, [600, 1], "shared", 0.1),
    (3, 4, 1, 77, 200, 32, False, ai.F16, [200, 0, 150], "per_head", 0.2),
    (1, 4, 2, 513, 130, 32, True, ai.BF16, None, "shared", 0.0),
    (2, 2, 2, 64, 64, 128, False, ai.F16, None, "per_batch", 0.5),
    # masks repeated over the heads take the XCD-blocked launch order; these
    # shapes make it pick each group count (1, 2, 4 and 8 slice groups, and
    # 2 groups inside each batch of a per-batch mask)
    (1, 2, 2, 2048, 2048, 32, True, ai.F16, None, "shared", 0.0),
    (1, 4, 4, 1024, 1024, 128, False, ai.BF16, None, "shared", 0.0),
    (1, 8, 8, 512, 512, 128, True, ai.F16, None, "shared", 0.1),
    (1, 16, 16, 256, 256, 128, True, ai.BF16, None, "shared", 0.0),
    (2, 4, 4, 1024, 1024, 64, True, ai.F16, [1024, 700], "per_batch", 0.0),
]


def _mask_shape(kind, B, H, Nq, Nk):
    return {"shared": (Nq, Nk), "per_head": (B, H, Nq, Nk), "per_batch": (B, 1, Nq, Nk)}[kind]


def _mask_id(c):
    B, H, Hkv, Nq, Nk, d, causal, dtype, kl, kind, frac = c
    return (f"B{B}H{H}kv{Hkv}q{Nq}k{Nk}d{d}{'c' if causal else 'f'}{dtype}"
            f"{'' if kl is None else 'L'}-{kind}-inf{frac}")


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal,dtype,kl,kind,frac", MASK_CASES,
                         ids=[_mask_id(c) for c in MASK_CASES])
def test_masked_matches_oracle(B, H, Hkv, Nq, Nk, d, causal, dtype, kl, kind, frac):
    case = _gqa_case(B, H, Hkv, Nq, Nk, d, causal, dtype, kl, 60_000)
    mask = ai.random_mask(_mask_shape(kind, B, H, Nq, Nk), seed=case["seed"] + 1, sigma=2.0,
                          neg_inf_frac=frac, empty_rows=(min(5, Nq - 1),) if frac > 0 else ())
    gu.log(f"masked {_mask_id((B, H, Hkv, Nq, Nk, d, causal, dtype, kl, kind, frac))}")
    sel = ai.all_rows_selection(B, H, Nq)
    O_ref, LSE_ref = gu.oracle_rows(case, causal, sel, mask=mask)
    O, LSE = gu.run_masked(case, causal, mask)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"masked {kind}", sel)
    O, LSE = gu.run_masked(case, causal, mask, n_splits=3)
    Og, Lg = gu.gather(O, LSE, sel)
    gu.assert_close(Og, Lg, O_ref, LSE_ref, dtype, f"masked split {kind}", sel)


def test_zero_mask_equals_unmasked_and_expand_views():
    # an all-zero mask gives attn_fwd_gqa's result (same tiles, same order:
    # the mask adds exactly 0); a [Nq, Nk] mask expanded to [B, H, Nq, Nk]
    # (stride-0 view) equals the same mask copied out
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 300, 500, 64
    case = ai.random_case_general(B, H, Hkv, Nq, Nk, d, ai.BF16, seed=61_000, key_len=[500, 77])
    inputs = gu.dev_inputs(case)
    zero = np.zeros((Nq, Nk), np.float32)
    O0, L0 = gu.run_masked(case, True, zero, inputs=inputs)
    O1, L1 = gu.run_gqa(case, True, inputs=inputs)
    sel = ai.all_rows_selection(B, H, Nq)
    gu.assert_close(*gu.gather(O0, L0, sel), *[np.asarray(x, np.float64) for x in gu.gather(O1, L1, sel)],
                    ai.BF16, "zero mask vs unmasked", sel)
    m = ai.random_mask((Nq, Nk), seed=61_001)
    md = torch.from_numpy(m).to(gu.device())
    O2, L2 = gu.run_masked(case, True, m, inputs=inputs, mask_dev=md.expand(B, H, Nq, Nk))
    O3, L3 = gu.run_masked(case, True, m, inputs=inputs,
                           mask_dev=md.expand(B, H, Nq, Nk).contiguous())
    assert np.array_equal(O2, O3) and np.array_equal(L2, L3)


def test_masked_prefill_workload():
    w = ai.WORKLOADS["masked_prefill"]
    case = ai.generate(w)
    sel = gu.sample_rows(w.B, w.H, w.q_len, 32, seed=w.seed + 7)
    O_ref, LSE_ref = gu.oracle_rows(case, w.causal, sel, mask=case["mask"])
    gu.log("masked_prefill: fused")
    O, LSE = gu.run_masked(case, w.causal, case["mask"])
    gu.assert_close(*gu.gather(O, LSE, sel), O_ref, LSE_ref, w.dtype, "masked_prefill", sel)
