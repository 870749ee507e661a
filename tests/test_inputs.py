"""Host logic of the seeded input generator (CPU only)."""
import numpy as np
import torch

import attn_inputs as ai


def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(7))
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 3,
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, -3.0e38, 1e-40, -1e-40,
                  np.inf, -np.inf], np.float32),
        # exact ties between two bf16 values: nearest-even decides
        (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = ai.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    back = ai.bits_to_f32(ai.f32_to_bf16_bits(x), ai.BF16)
    assert np.all(np.isnan(back))


def test_decode_is_exact_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = ai.bits_to_f32(bits, ai.F16)
    ref16 = torch.from_numpy(bits.view(np.int16)).view(torch.float16).float().numpy()
    same = (f16 == ref16) | (np.isnan(f16) & np.isnan(ref16))
    assert same.all()
    b16 = ai.bits_to_f32(bits, ai.BF16)
    refb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    same = (b16 == refb) | (np.isnan(b16) & np.isnan(refb))
    assert same.all()
    # round trip: every finite pattern rounds back to itself
    fin = np.isfinite(f16)
    assert np.array_equal(ai.f32_to_f16_bits(f16[fin]), bits[fin])
    fin = np.isfinite(b16)
    assert np.array_equal(ai.f32_to_bf16_bits(b16[fin]), bits[fin])


def test_workloads_are_deterministic_and_shaped():
    w = ai.WORKLOADS["reranker"]
    a = ai.generate(w)
    b = ai.generate(w)
    for k in ("Q", "K", "V", "key_len"):
        assert np.array_equal(a[k], b[k])
    assert a["Q"].shape == (50, 12, 256, 32) and a["Q"].dtype == np.uint16
    assert a["key_len"].shape == (50,)
    assert a["key_len"].min() >= 48 and a["key_len"].max() <= 256
    c = ai.generate(w, seed=w.seed + 1)
    assert not np.array_equal(a["Q"], c["Q"])


def test_workload_table():
    t = ai.WORKLOADS
    assert [t[k].shape for k in ai.WORKLOAD_ORDER] == [
        (1, 1, 64, 32), (50, 12, 256, 32), (1, 32, 4096, 128),
        (8, 16, 2048, 64), (1, 32, 32768, 128)]
    assert [t[k].dtype for k in ai.WORKLOAD_ORDER] == ["f16", "f16", "f16", "bf16", "bf16"]
    assert [t[k].causal for k in ai.WORKLOAD_ORDER] == [False, False, True, False, True]
    assert t["prefill"].scale == np.float32(1 / np.sqrt(128))
    assert t["peaky"].q_sigma == 3.0 and t["peaky"].v_sigma == 1.0


def test_peaky_spread():
    x = ai.generate(ai.Workload("p", 1, 1, 4096, 64, ai.BF16, False, False,
                                q_sigma=3.0, k_sigma=3.0, seed=5))
    q = ai.bits_to_f32(x["Q"], ai.BF16)
    v = ai.bits_to_f32(x["V"], ai.BF16)
    assert abs(q.std() - 3.0) < 0.05 and abs(v.std() - 1.0) < 0.02


def test_row_sample_is_distinct_and_sorted():
    w = ai.Workload("s", 1, 4, 1000, 32, ai.BF16, True, False, seed=9, sample_rows=100)
    x = ai.generate(w)
    r = x["rows"]
    assert r.shape == (4, 100)
    for h in range(4):
        assert len(set(r[h].tolist())) == 100 and np.all(np.diff(r[h]) > 0)
        assert r[h].min() >= 0 and r[h].max() < 1000
    sel = ai.sampled_rows_selection(r)
    assert sel.shape == (400, 3) and np.array_equal(sel[:100, 2], r[0])
