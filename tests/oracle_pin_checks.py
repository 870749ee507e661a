"""Pins that tie the fp64 oracle to facts fixed outside it.

Each ``check_*`` takes an oracle library handle and raises AssertionError when
the oracle disagrees with the pages' printed values, a closed form, an
invariance of the definition, or a library-primitive restatement on tiny
inputs.  ``test_oracle_pins.py`` runs them against the real oracle and
``test_oracle_mutants.py`` runs them against deliberately broken copies of it
(each mutant must fail at least one pin).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _run(lib, Q, K, V, scale, causal=False, key_len=None):
    Q = np.asarray(Q, dtype=np.float32)
    K = np.asarray(K, dtype=np.float32)
    V = np.asarray(V, dtype=np.float32)
    return oracle.sdpa(Q, K, V, scale, causal, key_len, lib=lib)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _randn(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


# ------------------------------------------------------------ printed values
def _one_query_scores(x, d=4):
    """q = e0, key j = x_j e0, value j = e_j: output row 0 is softmax(x)."""
    n = len(x)
    d = max(d, n)
    Q = np.zeros((1, 1, n, d), np.float32)
    K = np.zeros((1, 1, n, d), np.float32)
    V = np.zeros((1, 1, n, d), np.float32)
    Q[0, 0, :, 0] = 1.0
    for j, xj in enumerate(x):
        K[0, 0, j, 0] = xj
        V[0, 0, j, j] = 1.0
    return Q, K, V


def check_softmax_worked_example(lib):
    g = _golden("softmax_worked_example.json")
    Q, K, V = _one_query_scores(g["x"])
    O, LSE = _run(lib, Q, K, V, 1.0)
    half = 0.5 * 10.0 ** -g["softmax_decimals"]
    for j, pj in enumerate(g["softmax"]):
        assert abs(O[0, 0, 0, j] - pj) <= half + 1e-12, (j, O[0, 0, 0, j], pj)
    # the normaliser the page prints is exp(LSE) of the row (max is 2 here)
    half_sum = 0.5 * 10.0 ** -g["sum_exp_decimals"]
    assert abs(math.exp(LSE[0, 0, 0]) - g["sum_exp"]) <= half_sum + 1e-12
    # every row has the same scores, so every row agrees
    assert np.allclose(O[0, 0], O[0, 0, 0], atol=0, rtol=0)


def check_softmax_saturation_example(lib):
    g = _golden("softmax_saturation_example.json")
    Q, K, V = _one_query_scores(g["x"])
    O, _ = _run(lib, Q, K, V, 1.0)
    assert O[0, 0, 0, g["winner"]] >= g["winner_prob_at_least"]
    assert O[0, 0, 0].sum() == 1.0 or abs(O[0, 0, 0].sum() - 1.0) < 1e-12


def check_dot_product_example(lib):
    g = _golden("dot_product_example.json")
    d = 8
    Q = np.zeros((1, 1, 1, d), np.float32)
    K = np.zeros((1, 1, 1, d), np.float32)
    Q[0, 0, 0, :3] = g["q"]
    K[0, 0, 0, :3] = g["k"]
    V = _randn(_rng(3), (1, 1, 1, d))
    O, LSE = _run(lib, Q, K, V, 1.0)
    # one visible key: its score is the log-sum-exp, its value is the output
    assert LSE[0, 0, 0] == g["dot"]
    assert np.array_equal(O[0, 0, 0], V[0, 0, 0].astype(np.float64))


def check_sqrt_d_example(lib):
    g = _golden("sqrt_d_example.json")
    d = g["d"]
    Q = np.ones((1, 1, 1, d), np.float32)
    K = np.ones((1, 1, 1, d), np.float32)
    V = np.ones((1, 1, 1, d), np.float32)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    _, LSE = _run(lib, Q, K, V, scale)
    # q.k = d, scaled by 1/sqrt(d), gives sqrt(d) (up to the float32 scale)
    assert abs(LSE[0, 0, 0] - g["sqrt_d"]) <= 0.5 * 10.0 ** -g["sqrt_d_decimals"]
    assert abs(LSE[0, 0, 0] - d * scale) <= 1e-12


# ------------------------------------------------------------ closed forms
def check_hand_case(lib):
    """N=2, d=1, q=1, k=(0,1), v=(1,0), scale 1, worked out by hand."""
    Q = np.array([1.0, 1.0], np.float32).reshape(1, 1, 2, 1)
    K = np.array([0.0, 1.0], np.float32).reshape(1, 1, 2, 1)
    V = np.array([1.0, 0.0], np.float32).reshape(1, 1, 2, 1)
    O, LSE = _run(lib, Q, K, V, 1.0)
    e = math.e
    for i in range(2):
        assert abs(O[0, 0, i, 0] - 1.0 / (1.0 + e)) < 1e-15
        assert abs(LSE[0, 0, i] - math.log(1.0 + e)) < 1e-15
    O, LSE = _run(lib, Q, K, V, 1.0, causal=True)
    assert O[0, 0, 0, 0] == 1.0 and LSE[0, 0, 0] == 0.0
    assert abs(O[0, 0, 1, 0] - 1.0 / (1.0 + e)) < 1e-15


def check_zero_query_gives_mean(lib):
    """Q = 0: every visible key has weight 1/n, so O is the mean of visible V rows."""
    rng = _rng(11)
    B, H, N, d = 2, 2, 37, 8
    Q = np.zeros((B, H, N, d), np.float32)
    K = _randn(rng, (B, H, N, d))
    V = _randn(rng, (B, H, N, d))
    key_len = np.array([23, 37], np.int32)
    for causal in (False, True):
        O, LSE = _run(lib, Q, K, V, 0.7, causal, key_len)
        for b in range(B):
            for h in range(H):
                for i in range(N):
                    n = key_len[b] if not causal else min(key_len[b], i + 1)
                    ref = V[b, h, :n].astype(np.float64).mean(axis=0)
                    assert np.allclose(O[b, h, i], ref, rtol=0, atol=1e-14)
                    assert abs(LSE[b, h, i] - math.log(n)) < 1e-14


def check_identical_keys(lib):
    """All keys equal: uniform weights; LSE = scale q.k + log n."""
    rng = _rng(12)
    N, d = 19, 16
    Q = _randn(rng, (1, 1, N, d))
    k = _randn(rng, (d,))
    K = np.broadcast_to(k, (1, 1, N, d)).copy()
    V = _randn(rng, (1, 1, N, d))
    scale = 0.25
    O, LSE = _run(lib, Q, K, V, scale, causal=True)
    for i in range(N):
        ref = V[0, 0, :i + 1].astype(np.float64).mean(axis=0)
        assert np.allclose(O[0, 0, i], ref, rtol=0, atol=1e-13)
        s = scale * float(np.dot(Q[0, 0, i].astype(np.float64), k.astype(np.float64)))
        assert abs(LSE[0, 0, i] - (s + math.log(i + 1))) < 1e-12


def check_single_dominant_score(lib):
    """Key t scores a, every other key scores 0: O = (e^a V_t + sum_{j!=t} V_j)/(e^a + n - 1)."""
    rng = _rng(13)
    N, d, t = 12, 8, 5
    V = _randn(rng, (1, 1, N, d)).astype(np.float64)
    for a in (0.5, 3.0, 30.0):
        Q = np.zeros((1, 1, N, d), np.float32)
        K = np.zeros((1, 1, N, d), np.float32)
        Q[..., 0] = 1.0
        K[0, 0, t, 0] = a
        O, LSE = _run(lib, Q, K, V.astype(np.float32), 1.0)
        ea = math.exp(a)
        ref = (ea * V[0, 0, t] + V[0, 0].sum(axis=0) - V[0, 0, t]) / (ea + N - 1)
        for i in range(N):
            assert np.allclose(O[0, 0, i], ref, rtol=1e-13, atol=1e-13)
            assert abs(LSE[0, 0, i] - math.log(ea + N - 1)) < 1e-12
    # the limit: a huge score returns that value row
    Q = np.zeros((1, 1, N, d), np.float32)
    K = np.zeros((1, 1, N, d), np.float32)
    Q[..., 0] = 1.0
    K[0, 0, t, 0] = 1000.0
    O, LSE = _run(lib, Q, K, V.astype(np.float32), 1.0)
    assert np.array_equal(O[0, 0, 3], V[0, 0, t])
    assert LSE[0, 0, 3] == 1000.0


def check_causal_row_zero(lib):
    """Causal row 0 sees only key 0: O_0 = V_0, LSE_0 = scale q_0.k_0."""
    rng = _rng(14)
    B, H, N, d = 2, 3, 9, 32
    Q, K, V = (_randn(rng, (B, H, N, d)) for _ in range(3))
    scale = 0.125
    O, LSE = _run(lib, Q, K, V, scale, causal=True)
    for b in range(B):
        for h in range(H):
            assert np.array_equal(O[b, h, 0], V[b, h, 0].astype(np.float64))
            s = scale * float(np.dot(Q[b, h, 0].astype(np.float64), K[b, h, 0].astype(np.float64)))
            assert abs(LSE[b, h, 0] - s) < 1e-13


def check_rows_sum_to_one(lib):
    """V = 1: each output element is the sum of a row of P, which is 1."""
    rng = _rng(15)
    B, H, N, d = 2, 2, 40, 8
    Q = _randn(rng, (B, H, N, d), 2.0)
    K = _randn(rng, (B, H, N, d), 2.0)
    V = np.ones((B, H, N, d), np.float32)
    for causal in (False, True):
        O, _ = _run(lib, Q, K, V, 0.5, causal, np.array([40, 7], np.int32))
        assert np.allclose(O, 1.0, rtol=0, atol=1e-14)


def check_empty_rows(lib):
    """key_len = 0 (or negative): O = 0, LSE = -inf; key_len > N clamps to N."""
    rng = _rng(16)
    B, H, N, d = 3, 1, 5, 4
    Q, K, V = (_randn(rng, (B, H, N, d)) for _ in range(3))
    O, LSE = _run(lib, Q, K, V, 1.0, False, np.array([0, -3, 99], np.int32))
    assert np.all(O[0:2] == 0.0) and np.all(np.isneginf(LSE[0:2]))
    O_full, LSE_full = _run(lib, Q, K, V, 1.0, False, None)
    assert np.array_equal(O[2], O_full[2]) and np.array_equal(LSE[2], LSE_full[2])


# ------------------------------------------------------------ invariances
def check_mask_reduction(lib):
    """key_len = L equals unmasked attention over K[:L], V[:L]; causal row i
    equals unmasked attention over the prefix K[:i+1], V[:i+1]."""
    rng = _rng(17)
    B, H, N, d = 2, 2, 21, 8
    Q, K, V = (_randn(rng, (B, H, N, d)) for _ in range(3))
    key_len = np.array([13, 1], np.int32)
    O, LSE = _run(lib, Q, K, V, 0.3, False, key_len)
    for b in range(B):
        L = key_len[b]
        Ob, LSEb = _masked_prefix(lib, Q[b:b + 1], K[b:b + 1], V[b:b + 1], L, 0.3)
        assert np.allclose(O[b], Ob[0], rtol=1e-14, atol=1e-14)
        assert np.allclose(LSE[b], LSEb[0], rtol=1e-14, atol=1e-14)
    O, LSE = _run(lib, Q, K, V, 0.3, True, None)
    for i in (0, 1, 7, N - 1):
        Oi, LSEi = _masked_prefix(lib, Q, K, V, i + 1, 0.3)
        assert np.allclose(O[:, :, i], Oi[:, :, i], rtol=1e-14, atol=1e-14)
        assert np.allclose(LSE[:, :, i], LSEi[:, :, i], rtol=1e-14, atol=1e-14)


def _masked_prefix(lib, Q, K, V, L, scale):
    """Unmasked attention of every query row against the first L keys only.

    The oracle takes equal query and key lengths, so each query row i is
    repeated L times against K[:L], V[:L] and output row 0 is kept."""
    B, H, N, d = Q.shape
    O = np.zeros((B, H, N, d))
    LSE = np.zeros((B, H, N))
    for i in range(N):
        Qi = np.repeat(Q[:, :, i:i + 1], L, axis=2)
        Oi, LSEi = _run(lib, Qi, K[:, :, :L], V[:, :, :L], scale)
        O[:, :, i] = Oi[:, :, 0]
        LSE[:, :, i] = LSEi[:, :, 0]
    return O, LSE


def check_shift_invariance(lib):
    """K_j += u for every j multiplies every weight's numerator and the
    denominator alike: O unchanged, LSE_i += scale q_i.u."""
    rng = _rng(18)
    B, H, N, d = 1, 2, 24, 8
    Q, K, V = (_randn(rng, (B, H, N, d)) for _ in range(3))
    K = (np.round(K * 256.0) / 256.0).astype(np.float32)  # multiples of 2^-8
    u = np.zeros(d, np.float32)
    u[[0, 3]] = [0.5, -0.25]  # shifts by multiples of 2^-8 stay exact
    K2 = (K + u).astype(np.float32)
    assert np.array_equal(K2 - u, K)  # shift was exact in float32
    for causal in (False, True):
        O1, L1 = _run(lib, Q, K, V, 0.5, causal)
        O2, L2 = _run(lib, Q, K2, V, 0.5, causal)
        shift = 0.5 * (Q.astype(np.float64) @ u.astype(np.float64))
        assert np.allclose(O1, O2, rtol=1e-12, atol=1e-12)
        assert np.allclose(L2, L1 + shift, rtol=0, atol=1e-12)


def check_permutation_invariance(lib):
    """Non-causal, unmasked: permuting (K, V) rows together leaves O
    unchanged; permuting Q rows permutes O rows."""
    rng = _rng(19)
    B, H, N, d = 1, 1, 31, 16
    Q, K, V = (_randn(rng, (B, H, N, d)) for _ in range(3))
    perm = rng.permutation(N)
    O1, L1 = _run(lib, Q, K, V, 0.25)
    O2, L2 = _run(lib, Q, K[:, :, perm], V[:, :, perm], 0.25)
    assert np.allclose(O1, O2, rtol=1e-13, atol=1e-13)
    assert np.allclose(L1, L2, rtol=1e-13, atol=1e-13)
    O3, L3 = _run(lib, Q[:, :, perm], K, V, 0.25)
    assert np.array_equal(O3, O1[:, :, perm]) and np.array_equal(L3, L1[:, :, perm])


def check_weighted_average(lib):
    """O is linear in V and each O_ic lies within [min_j V_jc, max_j V_jc]
    over visible keys (a convex combination of value rows)."""
    rng = _rng(20)
    B, H, N, d = 1, 2, 33, 8
    Q, K = _randn(rng, (B, H, N, d), 1.5), _randn(rng, (B, H, N, d), 1.5)
    V1, V2 = _randn(rng, (B, H, N, d)), _randn(rng, (B, H, N, d))
    # multiples of 2^-8 so that 2 V1 - V2 / 2 is exact in float32
    V1 = (np.round(V1 * 256.0) / 256.0).astype(np.float32)
    V2 = (np.round(V2 * 256.0) / 256.0).astype(np.float32)
    for causal in (False, True):
        O1, _ = _run(lib, Q, K, V1, 0.4, causal)
        O2, _ = _run(lib, Q, K, V2, 0.4, causal)
        O12, _ = _run(lib, Q, K, (2.0 * V1 - 0.5 * V2).astype(np.float32), 0.4, causal)
        assert np.allclose(O12, 2.0 * O1 - 0.5 * O2, rtol=1e-12, atol=1e-12)
        for h in range(H):
            for i in range(N):
                n = i + 1 if causal else N
                lo = V1[0, h, :n].min(axis=0) - 1e-14
                hi = V1[0, h, :n].max(axis=0) + 1e-14
                assert np.all(O1[0, h, i] >= lo) and np.all(O1[0, h, i] <= hi)


# ------------------------------------------------------------ library restatement
def textbook_numpy(Q, K, V, scale, causal=False, key_len=None, add_mask=None):
    """softmax(scale Q K^T + mask) V with numpy matmul/exp/sum on float64 copies.

    Q is [B, H, Nq, d], K and V [B, Hkv, Nk, d]: the key/value heads are
    expanded with np.repeat (consecutive query heads share one).  The mask
    is -inf above the diagonal that ends at the last query and key
    (np.tril with offset Nk - Nq; the plain lower triangle when Nq = Nk) and
    at keys j >= key_len[b], plus ``add_mask`` (any array that broadcasts to
    [B, H, Nq, Nk]) added to the scaled scores."""
    Q, K, V = (np.asarray(x, np.float64) for x in (Q, K, V))
    B, H, Nq, d = Q.shape
    G = H // K.shape[1]
    K = np.repeat(K, G, axis=1)
    V = np.repeat(V, G, axis=1)
    Nk = K.shape[2]
    S = scale * np.matmul(Q, np.swapaxes(K, -1, -2))
    if add_mask is not None:
        S = S + np.asarray(add_mask, np.float64)
    mask = np.zeros((B, 1, Nq, Nk))
    if causal:
        mask = mask + np.where(np.tril(np.ones((Nq, Nk)), k=Nk - Nq) > 0, 0.0, -np.inf)
    if key_len is not None:
        cols = np.arange(Nk)[None, :]
        kl = np.clip(np.asarray(key_len), 0, Nk)[:, None]
        mask = mask + np.where(cols < kl, 0.0, -np.inf)[:, None, None, :]
    S = S + mask
    with np.errstate(invalid="ignore"):
        m = S.max(axis=-1, keepdims=True) if Nk > 0 else np.full((B, H, Nq, 1), -np.inf)
        E = np.exp(S - m)
        l = E.sum(axis=-1, keepdims=True)
        P = E / l
        O = np.matmul(P, V)
        LSE = (m + np.log(l))[..., 0]
    empty = ~np.isfinite(m[..., 0])
    O[empty] = 0.0
    LSE[empty] = -np.inf
    return O, LSE


def check_textbook_numpy(lib):
    rng = _rng(21)
    for (B, H, N, d, causal, kl) in [(1, 1, 5, 3, False, None), (2, 3, 17, 8, True, None),
                                     (3, 2, 16, 32, False, [0, 9, 16]),
                                     (2, 2, 29, 64, True, [5, 29])]:
        Q, K, V = (_randn(rng, (B, H, N, d), 1.7) for _ in range(3))
        key_len = None if kl is None else np.array(kl, np.int32)
        O, LSE = _run(lib, Q, K, V, 0.37, causal, key_len)
        Oref, LSEref = textbook_numpy(Q, K, V, 0.37, causal, key_len)
        assert np.allclose(O, Oref, rtol=1e-12, atol=1e-12)
        fin = np.isfinite(LSEref)
        assert np.array_equal(fin, np.isfinite(LSE))
        assert np.allclose(LSE[fin], LSEref[fin], rtol=1e-12, atol=1e-12)


def check_online_merge_matches(lib):
    """Blockwise online-softmax merges over random splits and merge orders
    equal the two-pass oracle."""
    from oracle import online_merge as om
    rng = _rng(22)
    B, H, N, d = 1, 2, 50, 8
    Q, K, V = (_randn(rng, (B, H, N, d), 2.0) for _ in range(3))
    scale = 0.6
    O, LSE = _run(lib, Q, K, V, scale)
    for h in range(H):
        for i in (0, 13, 49):
            s = scale * (K[0, h].astype(np.float64) @ Q[0, h, i].astype(np.float64))
            for trial in range(6):
                cuts = np.sort(rng.choice(np.arange(1, N), size=rng.integers(1, 8),
                                          replace=False))
                parts = np.split(np.arange(N), cuts)
                summ = [om.block_summary(s[p], V[0, h, p]) for p in parts]
                while len(summ) > 1:  # merge random adjacent pairs (any tree)
                    k = int(rng.integers(0, len(summ) - 1))
                    summ[k:k + 2] = [om.merge(summ[k], summ[k + 1])]
                m, l, o = summ[0]
                assert np.allclose(o, O[0, h, i], rtol=1e-12, atol=1e-12)
                assert abs(om.lse(summ[0]) - LSE[0, h, i]) < 1e-12


# ------------------------------------------------------------ cross-attention and grouped heads
def _run_general(lib, Q, K, V, scale, causal=False, key_len=None, mask=None):
    Q = np.asarray(Q, dtype=np.float32)
    K = np.asarray(K, dtype=np.float32)
    V = np.asarray(V, dtype=np.float32)
    return oracle.attn(Q, K, V, scale, causal, key_len, mask=mask, lib=lib)


def check_grouped_heads_equal_repeated_heads(lib):
    """Hkv < H equals self-attention shapes with each key/value head copied to
    the H / Hkv consecutive query heads that share it (np.repeat)."""
    rng = _rng(31)
    B, H, Hkv, N, d = 2, 6, 2, 23, 16
    Q = _randn(rng, (B, H, N, d), 1.5)
    K = _randn(rng, (B, Hkv, N, d), 1.5)
    V = _randn(rng, (B, Hkv, N, d))
    Kr, Vr = np.repeat(K, H // Hkv, axis=1), np.repeat(V, H // Hkv, axis=1)
    for causal, kl in ((False, None), (True, np.array([23, 11], np.int32))):
        O, LSE = _run_general(lib, Q, K, V, 0.3, causal, kl)
        Or, LSEr = _run(lib, Q, Kr, Vr, 0.3, causal, kl)
        assert np.array_equal(O, Or) and np.array_equal(LSE, LSEr)


def check_cross_textbook_numpy(lib):
    """Different query and key lengths and grouped heads against numpy."""
    rng = _rng(32)
    for (B, H, Hkv, Nq, Nk, d, causal, kl) in [
            (1, 4, 1, 3, 17, 8, True, None), (2, 4, 2, 19, 7, 16, True, None),
            (2, 3, 3, 5, 40, 32, False, [0, 33]), (1, 8, 2, 11, 29, 8, True, [20]),
            (2, 2, 1, 1, 64, 16, True, [64, 9])]:
        Q = _randn(rng, (B, H, Nq, d), 1.7)
        K = _randn(rng, (B, Hkv, Nk, d), 1.7)
        V = _randn(rng, (B, Hkv, Nk, d))
        key_len = None if kl is None else np.array(kl, np.int32)
        O, LSE = _run_general(lib, Q, K, V, 0.37, causal, key_len)
        Oref, LSEref = textbook_numpy(Q, K, V, 0.37, causal, key_len)
        assert np.allclose(O, Oref, rtol=1e-12, atol=1e-12)
        fin = np.isfinite(LSEref)
        assert np.array_equal(fin, np.isfinite(LSE))
        assert np.allclose(LSE[fin], LSEref[fin], rtol=1e-12, atol=1e-12)


def check_causal_queries_are_the_last_rows(lib):
    """Bottom-right alignment: causal attention of the last Nq query rows
    against all Nk keys equals rows Nk-Nq .. Nk-1 of causal self-attention
    over the Nk rows; a single query row sees every key."""
    rng = _rng(33)
    B, H, N, d = 2, 2, 30, 8
    Q, K, V = (_randn(rng, (B, H, N, d)) for _ in range(3))
    O_self, LSE_self = _run(lib, Q, K, V, 0.45, causal=True)
    for nq in (1, 4, 13):
        O, LSE = _run_general(lib, Q[:, :, N - nq:], K, V, 0.45, causal=True)
        assert np.array_equal(O, O_self[:, :, N - nq:])
        assert np.array_equal(LSE, LSE_self[:, :, N - nq:])
    O1, LSE1 = _run_general(lib, Q[:, :, :1], K, V, 0.45, causal=True)
    O2, LSE2 = _run_general(lib, Q[:, :, :1], K, V, 0.45, causal=False)
    assert np.array_equal(O1, O2) and np.array_equal(LSE1, LSE2)


def check_cross_zero_query_prefix_means(lib):
    """Q = 0 with Nq != Nk: query i averages the value rows up to key
    i + Nk - Nq (causal), or all of them; more queries than keys leaves the
    first Nq - Nk rows empty (O = 0, LSE = -inf)."""
    rng = _rng(34)
    for Nq, Nk in ((5, 12), (12, 5)):
        B, H, Hkv, d = 1, 4, 2, 8
        Q = np.zeros((B, H, Nq, d), np.float32)
        K = _randn(rng, (B, Hkv, Nk, d))
        V = _randn(rng, (B, Hkv, Nk, d))
        for causal in (False, True):
            O, LSE = _run_general(lib, Q, K, V, 1.0, causal)
            for h in range(H):
                hk = h // (H // Hkv)
                for i in range(Nq):
                    n = min(Nk, i + Nk - Nq + 1) if causal else Nk
                    if n <= 0:
                        assert np.all(O[0, h, i] == 0.0) and np.isneginf(LSE[0, h, i])
                        continue
                    ref = V[0, hk, :n].astype(np.float64).mean(axis=0)
                    assert np.allclose(O[0, h, i], ref, rtol=0, atol=1e-14)
                    assert abs(LSE[0, h, i] - math.log(n)) < 1e-14


def check_sparse_selection_equals_full_rows(lib):
    """Rows picked by a shuffled, sparse (b, h, i) selection, with repeats,
    equal the same rows of the full result bit for bit and numpy's
    textbook rows, for grouped heads, Nq != Nk, both structural masks and an
    additive mask.  Selected row t is the t-th triple, not the t-th row of
    the tensor: reading the query, the causal position or the mask row from
    t instead of (b, h, i) fails here (every full-result pin selects the
    rows in order, where the two coincide)."""
    rng = _rng(35)
    for (B, H, Hkv, Nq, Nk, d, causal, kl, mshape) in [
            (2, 6, 2, 9, 14, 8, True, [14, 5], None),
            (3, 4, 1, 12, 7, 16, True, [7, 0, 3], None),
            (2, 4, 4, 10, 10, 8, False, [10, 6], (2, 4, 10, 10)),
            (2, 6, 3, 5, 16, 8, True, None, (5, 16))]:
        Q = _randn(rng, (B, H, Nq, d), 1.5)
        K = _randn(rng, (B, Hkv, Nk, d), 1.5)
        V = _randn(rng, (B, Hkv, Nk, d))
        m = None if mshape is None else _randn(rng, mshape, 1.5)
        key_len = None if kl is None else np.array(kl, np.int32)
        O, LSE = _run_general(lib, Q, K, V, 0.41, causal, key_len, mask=m)
        Oref, LSEref = textbook_numpy(Q, K, V, 0.41, causal, key_len, add_mask=m)
        n = B * H * Nq
        flat = rng.choice(n, size=n // 3, replace=False)
        flat = np.concatenate([flat, flat[:3]])  # repeated rows, out of order
        rng.shuffle(flat)
        b, rest = np.divmod(flat, H * Nq)
        h, i = np.divmod(rest, Nq)
        sel = np.stack([b, h, i], axis=1).astype(np.int64)
        Os, LSEs = oracle.attn_rows(Q, K, V, 0.41, causal, key_len, sel, mask=m, lib=lib)
        assert np.array_equal(Os, O[b, h, i])
        assert np.array_equal(LSEs, LSE[b, h, i])
        assert np.allclose(Os, Oref[b, h, i], rtol=1e-12, atol=1e-12)
        fin = np.isfinite(LSEref[b, h, i])
        assert np.array_equal(fin, np.isfinite(LSEs))
        assert np.allclose(LSEs[fin], LSEref[b, h, i][fin], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ additive mask
def check_mask_minus_inf_is_a_structural_mask(lib):
    """An additive mask of -inf above the end-aligned diagonal equals the
    causal flag, -inf at keys j >= L equals key_len = L, and a row whose mask
    is -inf everywhere has no visible key (O = 0, LSE = -inf)."""
    rng = _rng(41)
    for Nq, Nk in ((20, 20), (7, 30), (30, 7)):
        B, H, Hkv, d = 2, 4, 2, 8
        Q = _randn(rng, (B, H, Nq, d), 1.5)
        K = _randn(rng, (B, Hkv, Nk, d), 1.5)
        V = _randn(rng, (B, Hkv, Nk, d))
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        causal_mask = np.where(j <= i + Nk - Nq, 0.0, -np.inf).astype(np.float32)
        O1, L1 = _run_general(lib, Q, K, V, 0.4, causal=True)
        O2, L2 = _run_general(lib, Q, K, V, 0.4, mask=causal_mask)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
        kl = np.array([Nk, max(Nk // 3, 1)], np.int32)
        pad = np.broadcast_to(np.where(np.arange(Nk)[None, :] < kl[:, None], 0.0, -np.inf)
                              [:, None, None, :], (B, 1, Nq, Nk)).astype(np.float32)
        O1, L1 = _run_general(lib, Q, K, V, 0.4, key_len=kl)
        O2, L2 = _run_general(lib, Q, K, V, 0.4, mask=pad)
        assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    m = np.zeros((Nq, Nk), np.float32)
    m[3, :] = -np.inf
    O, L = _run_general(lib, Q, K, V, 0.4, mask=m)
    assert np.all(O[:, :, 3] == 0.0) and np.all(np.isneginf(L[:, :, 3]))
    assert np.all(np.isfinite(L[:, :, :3]))


def check_mask_log_weights_closed_form(lib):
    """Q = 0 and mask = log w: the weights are w_ij / sum_j w_ij, so
    O_i = sum_j w_ij v_j / sum_j w_ij and LSE_i = log sum_j w_ij.  A
    different, non-symmetric w per (b, h) pins the mask's indexing."""
    rng = _rng(42)
    B, H, Hkv, Nq, Nk, d = 2, 3, 3, 5, 9, 4
    Q = np.zeros((B, H, Nq, d), np.float32)
    K = _randn(rng, (B, Hkv, Nk, d))
    V = _randn(rng, (B, Hkv, Nk, d))
    W = rng.uniform(0.05, 3.0, size=(B, H, Nq, Nk))
    mask = np.log(W).astype(np.float32)
    W = np.exp(mask.astype(np.float64))  # the weights the float32 mask encodes
    O, LSE = _run_general(lib, Q, K, V, 0.9, mask=mask)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                w = W[b, h, i]
                ref = (w[:, None] * V[b, h].astype(np.float64)).sum(axis=0) / w.sum()
                assert np.allclose(O[b, h, i], ref, rtol=1e-13, atol=1e-13)
                assert abs(LSE[b, h, i] - math.log(w.sum())) < 1e-13


def check_mask_textbook_numpy(lib):
    """A random finite mask, with and without the structural masks and
    grouped heads, against numpy."""
    rng = _rng(43)
    for (B, H, Hkv, Nq, Nk, d, causal, kl, mshape) in [
            (1, 2, 2, 9, 9, 8, False, None, (9, 9)),
            (2, 4, 2, 6, 13, 16, True, [13, 4], (2, 4, 6, 13)),
            (2, 3, 1, 11, 5, 8, True, None, (1, 3, 11, 5)),
            (3, 2, 2, 8, 8, 32, False, [8, 0, 3], (3, 1, 8, 8))]:
        Q = _randn(rng, (B, H, Nq, d), 1.5)
        K = _randn(rng, (B, Hkv, Nk, d), 1.5)
        V = _randn(rng, (B, Hkv, Nk, d))
        m = _randn(rng, mshape, 2.0)
        key_len = None if kl is None else np.array(kl, np.int32)
        O, LSE = _run_general(lib, Q, K, V, 0.37, causal, key_len, mask=m)
        Oref, LSEref = textbook_numpy(Q, K, V, 0.37, causal, key_len, add_mask=m)
        assert np.allclose(O, Oref, rtol=1e-12, atol=1e-12)
        fin = np.isfinite(LSEref)
        assert np.array_equal(fin, np.isfinite(LSE))
        assert np.allclose(LSE[fin], LSEref[fin], rtol=1e-12, atol=1e-12)


def check_mask_broadcast_equals_copies(lib):
    """A shared [Nq, Nk] mask (strides 0) equals the same mask copied to every
    (b, h), and a per-row constant added to the mask moves LSE by it and
    leaves O unchanged."""
    rng = _rng(44)
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 7, 12, 8
    Q = _randn(rng, (B, H, Nq, d))
    K = _randn(rng, (B, Hkv, Nk, d))
    V = _randn(rng, (B, Hkv, Nk, d))
    m = (np.round(_randn(rng, (Nq, Nk)) * 256.0) / 256.0).astype(np.float32)  # m + c exact
    O1, L1 = _run_general(lib, Q, K, V, 0.5, True, mask=m)
    O2, L2 = _run_general(lib, Q, K, V, 0.5, True,
                          mask=np.broadcast_to(m, (B, H, Nq, Nk)).copy())
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    c = (np.arange(Nq, dtype=np.float32) * 0.25 - 1.0)[:, None]
    mc = (m + c).astype(np.float32)
    assert np.array_equal(mc - c, m)  # the shift was exact in float32
    O3, L3 = _run_general(lib, Q, K, V, 0.5, True, mask=mc)
    assert np.allclose(O3, O1, rtol=1e-12, atol=1e-12)
    assert np.allclose(L3, L1 + c[:, 0], rtol=0, atol=1e-12)


# ------------------------------------------------- arbitrary-precision brute force
def _decimal_attention(Q, K, V, scale, causal, key_len, digits=40):
    """The definition evaluated in decimal arithmetic at ``digits`` digits,
    from the exact values of the fp32 inputs: per row, the visible keys'
    scores, their max, the sum of exponentials, the weighted average of V
    and the log-sum-exp.  Returns (O, LSE) as Python lists of Decimals
    (LSE None for a row with no visible key)."""
    import decimal
    ctx = decimal.Context(prec=digits)
    D = decimal.Decimal
    B, H, N, d = Q.shape
    sc = D(float(np.float32(scale)))
    O, LSE = {}, {}
    for b in range(B):
        L = N if key_len is None else max(0, min(N, int(key_len[b])))
        for h in range(H):
            for i in range(N):
                vis = [j for j in range(L) if not causal or j <= i]
                if not vis:
                    O[b, h, i] = [D(0)] * d
                    LSE[b, h, i] = None
                    continue
                s = {}
                for j in vis:
                    acc = D(0)
                    for c in range(d):
                        acc = ctx.add(acc, ctx.multiply(D(float(Q[b, h, i, c])), D(float(K[b, h, j, c]))))
                    s[j] = ctx.multiply(sc, acc)
                m = max(s.values())
                e = {j: ctx.exp(ctx.subtract(s[j], m)) for j in vis}
                l = sum(e.values(), D(0))
                O[b, h, i] = [ctx.divide(sum((ctx.multiply(e[j], D(float(V[b, h, j, c]))) for j in vis), D(0)), l)
                              for c in range(d)]
                LSE[b, h, i] = ctx.add(m, ctx.ln(l))
    return O, LSE


def check_decimal_brute_force(lib):
    """The fp64 oracle agrees with a 40-digit decimal evaluation of the
    definition to fp64 rounding level, on small random cases with both
    masks: a dropped term, a wrong index or a single-precision step anywhere
    in the oracle shows up far above 1e-12."""
    rng = _rng(4242)
    for causal, key_len in ((False, None), (True, None), (False, [3, 0]), (True, [5, 2])):
        Q = _randn(rng, (2, 2, 5, 4), 1.5)
        K = _randn(rng, (2, 2, 5, 4), 1.5)
        V = _randn(rng, (2, 2, 5, 4))
        scale = 0.5
        O, LSE = _run(lib, Q, K, V, scale, causal, key_len)
        Od, Ld = _decimal_attention(Q, K, V, scale, causal, key_len)
        for (b, h, i), row in Od.items():
            for c, x in enumerate(row):
                assert abs(float(O[b, h, i, c]) - float(x)) <= 1e-12 * (1.0 + abs(float(x))), \
                    (causal, key_len, b, h, i, c, float(O[b, h, i, c]), float(x))
            if Ld[b, h, i] is None:
                assert np.isneginf(LSE[b, h, i])
            else:
                assert abs(float(LSE[b, h, i]) - float(Ld[b, h, i])) <= 1e-12, (causal, key_len, b, h, i)


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
