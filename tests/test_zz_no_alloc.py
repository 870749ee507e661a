"""attn_fwd_gqa_splitkv_static (the split-key forward that allocates nothing
and keeps its partials in the library's own scratch) against
attn_fwd_gqa_splitkv with a caller workspace and against the fp64 oracle:
two calls in a row, the second on a smaller problem, then the first again."""
import numpy as np
import pytest
import torch

import attn_inputs as ai
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (B, H, Hkv, Nq, Nk, d, dtype, causal, n_splits, key_len)
CALLS = [
    (4, 16, 4, 1, 3000, 128, ai.BF16, True, 4, "random"),   # decode-like, grouped heads
    (2, 8, 8, 100, 700, 64, ai.F16, False, 3, [700, 5]),     # smaller, self-attention heads
]


def _static(case, causal, n_splits):
    import exact_self_attention_amd as attn
    q, k, v, kl = gu.dev_inputs(case)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    attn.attn_fwd_gqa_splitkv_static(q, k, v, o, lse, n_splits=n_splits, scale=float(case["scale"]),
                                     causal=causal, key_len=kl)
    torch.cuda.synchronize()
    return gu.from_dev(o, case["dtype"]), lse.cpu().numpy()


def _check(B, H, Hkv, Nq, Nk, d, dtype, causal, n_splits, key_len, seed):
    case = ai.random_case_general(B, H, Hkv, Nq, Nk, d, dtype, seed=seed, sigma=1.5, key_len=key_len)
    gu.log(f"static scratch B={B} H={H} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} {dtype} causal={causal} "
           f"splits={n_splits}")
    O_s, L_s = _static(case, causal, n_splits)
    O_w, L_w, _ = gu.run_gqa_split(case, causal, n_splits=n_splits)
    # the same kernels on the same inputs: identical to the workspace form
    assert np.array_equal(O_s, O_w)
    assert np.array_equal(L_s, L_w)
    sel = ai.all_rows_selection(B, H, Nq)
    O_ref, L_ref = gu.oracle_rows(case, causal, sel)
    Og, Lg = gu.gather(O_s, L_s, sel)
    gu.assert_close(Og, Lg, O_ref, L_ref, dtype, "static scratch", sel)


def test_static_scratch_matches_workspace_form_and_oracle():
    for n, call in enumerate(CALLS + CALLS[:1]):
        _check(*call, seed=40_000 + n)


def test_static_scratch_rejects_problems_beyond_its_size():
    import exact_self_attention_amd as attn
    # 4 splits x 1 x 32 x 32768 rows x 129 x 4 bytes = 2.2 GB > 64 MiB
    q = torch.zeros(1, 32, 32768, 128, dtype=torch.float16, device=gu.device())
    o = torch.empty_like(q)
    with pytest.raises(attn.AttnError) as e:
        attn.attn_fwd_gqa_splitkv_static(q, q, q, o, None, n_splits=4, scale=0.1, causal=True)
    assert attn.STATUS[e.value.status] == "ATTN_ERR_WORKSPACE"
