"""The C ABI loads, exports what include/attn.h declares, and rejects bad
arguments before touching a device (CPU only: no kernel is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    so = os.path.join(ROOT, "exact_self_attention_amd", "libattn.so")
    if not os.path.exists(so):
        import __graft_entry__
        __graft_entry__.build()
    import exact_self_attention_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "attn_fwd" in names and "attn_fwd_naive" in names
    raw = ctypes.CDLL(lib.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert sorted(lib.EXPORTS) == names


def test_status_strings_and_version(lib):
    for code in range(7):
        s = lib.attn_status_string(code)
        assert s and s != "unknown status"
    assert lib.attn_status_string(99) == "unknown status"
    assert lib.attn_version() == 100


def test_workspace_bytes(lib):
    assert lib.attn_fwd_naive_workspace_bytes(1, 32, 4096) == 32 * 4096 * 4096 * 4
    assert lib.attn_fwd_naive_workspace_bytes(50, 12, 256) == 50 * 12 * 256 * 256 * 4
    assert lib.attn_fwd_naive_workspace_bytes(0, 5, 7) == 0
    assert lib.attn_fwd_naive_workspace_bytes(-1, 5, 7) == 0
    assert lib.attn_fwd_naive_workspace_bytes(1 << 20, 1 << 20, 1 << 20) == 0  # overflow


def test_kernel_names(lib):
    assert lib.attn_fwd_kernel_name(0, 128, 4096, True, False) == "attn_fwd_d128_f16_causal"
    assert lib.attn_fwd_kernel_name(1, 64, 2048, False, False) == "attn_fwd_d64_bf16_full"
    # a head whose keys fit in LDS goes to the short-sequence kernel
    assert lib.attn_fwd_kernel_name(0, 32, 256, False, True) == "attn_fwd_short_d32_f16_full"
    assert lib.attn_fwd_kernel_name(0, 32, 257, False, True) == "attn_fwd_d32_f16_full"
    assert lib.attn_fwd_kernel_name(1, 64, 256, True, False) == "attn_fwd_short_d64_bf16_causal"
    assert lib.attn_fwd_kernel_name(0, 128, 128, False, False) == "attn_fwd_short_d128_f16_full"
    # one query tile per head (129..256 rows at d = 128) takes the deep-ring instance
    assert lib.attn_fwd_kernel_name(0, 128, 129, False, False) == "attn_fwd_deep_d128_f16_full"
    assert lib.attn_fwd_kernel_name(0, 128, 256, True, False) == "attn_fwd_deep_d128_f16_causal"
    assert lib.attn_fwd_kernel_name(0, 128, 257, True, False) == "attn_fwd_d128_f16_causal"
    with pytest.raises(lib.AttnError):
        lib.attn_fwd_kernel_name(0, 48, 256, False, False)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_kernel_name_is_the_general_decision(lib, d):
    """attn_fwd names the kernel attn_fwd_gqa would launch for H = Hkv and
    Nq = Nk = N: the same short / decode / deep / streaming decision."""
    for N in [0, 1, 2, 17, 32, 33, 48, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 512, 1000, 4096]:
        for dtype in (0, 1):
            for causal in (False, True):
                for H in (1, 32):
                    assert lib.attn_fwd_kernel_name(dtype, d, N, causal, False) == \
                        lib.attn_fwd_gqa_kernel_name(dtype, d, H, H, N, N, causal), (d, N, dtype, causal, H)


# Fake, never-dereferenced device addresses: each call below is rejected by
# the argument checks, which run before any HIP call.
A = 0x10000000
MB = 1 << 20


def call_fwd(lib, dtype=0, Q=A, K=A + 64 * MB, V=A + 128 * MB, O=A + 192 * MB, LSE=None,
             B=1, H=2, N=64, d=64, scale=0.125, causal=0, key_len=None):
    return lib.lib.attn_fwd(dtype, Q, K, V, O, LSE, B, H, N, d, scale, causal, key_len, None)


def call_naive(lib, ws=A + 256 * MB, ws_bytes=64 * 64 * 4, **kw):
    a = dict(dtype=0, Q=A, K=A + 64 * MB, V=A + 128 * MB, O=A + 192 * MB, LSE=None,
             B=1, H=2, N=64, d=64, scale=0.125, causal=0, key_len=None)
    a.update(kw)
    return lib.lib.attn_fwd_naive(a["dtype"], a["Q"], a["K"], a["V"], a["O"], a["LSE"],
                                  a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                                  a["key_len"], ws, ws_bytes, None)


INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 1, 2, 3, 4


@pytest.mark.parametrize("kw,code", [
    (dict(d=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(B=-1), INVALID), (dict(N=-5), INVALID), (dict(N=(1 << 30) + 1), INVALID),
    (dict(B=1 << 20, H=1 << 12), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=-0.5), INVALID),
    (dict(Q=None), INVALID), (dict(O=None), INVALID),
    (dict(Q=A + 8), MISALIGNED), (dict(V=A + 128 * MB + 2), MISALIGNED),
    (dict(LSE=A + 300 * MB + 2), MISALIGNED), (dict(key_len=A + 301 * MB + 1), MISALIGNED),
    (dict(O=A + 16), INVALID),                        # O overlaps Q
    (dict(LSE=A + 192 * MB + 1024), INVALID),          # LSE overlaps O
    (dict(key_len=A + 192 * MB + 64), INVALID),        # key_len overlaps O
])
def test_fwd_rejects_bad_arguments(lib, kw, code):
    assert call_fwd(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0),
                                dict(B=0, Q=None, K=None, V=None, O=None)])
def test_empty_problem_is_a_noop(lib, kw):
    assert call_fwd(lib, **kw) == 0
    assert call_naive(lib, ws=None, ws_bytes=0, **kw) == 0


def test_q_k_v_may_alias_each_other(lib):
    # read-only inputs may share memory; such a call gets past the argument
    # checks, so it is only checked here that the overlap test alone does not
    # reject it: use an unsupported d to stop right after.
    assert call_fwd(lib, K=A, V=A, d=48) == UNSUPPORTED


def test_naive_workspace_checks(lib):
    assert call_naive(lib, ws=None) == WORKSPACE
    assert call_naive(lib, ws_bytes=64 * 64 * 4 - 1) == WORKSPACE
    assert call_naive(lib, ws=A + 256 * MB + 4) == MISALIGNED
    assert call_naive(lib, ws=A + 192 * MB) == INVALID  # workspace overlaps O
    assert call_naive(lib, N=65536 * 16) == INVALID     # score grid limit
    assert call_naive(lib, d=80) == UNSUPPORTED


def test_python_layer_checks_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 32, dtype=torch.float16)
    with pytest.raises(ValueError):  # CPU tensors are refused before the C call
        lib.attn_fwd(q, q, q, q.clone(), scale=0.1)
    with pytest.raises(TypeError):
        lib.attn_fwd(q.float(), q.float(), q.float(), q.float(), scale=0.1)


def call_split(lib, n_splits=2, ws=A + 256 * MB, ws_bytes=None, **kw):
    a = dict(dtype=0, Q=A, K=A + 64 * MB, V=A + 128 * MB, O=A + 192 * MB, LSE=None,
             B=1, H=2, N=64, d=64, scale=0.125, causal=0, key_len=None)
    a.update(kw)
    if ws_bytes is None:
        ws_bytes = lib.attn_fwd_splitkv_workspace_bytes(a["B"], a["H"], a["N"], a["d"], max(n_splits, 1))
    return lib.lib.attn_fwd_splitkv(a["dtype"], a["Q"], a["K"], a["V"], a["O"], a["LSE"],
                                    a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                                    a["key_len"], n_splits, ws, ws_bytes, None)


def test_splitkv_workspace_bytes(lib):
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 4, 4096, 128, 4) == 4 * 1 * 4 * 4096 * 129 * 4
    assert lib.attn_fwd_splitkv_workspace_bytes(2, 3, 100, 32, 1) == 2 * 3 * 100 * 33 * 4
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 64, 64, 0) == 0        # no splits
    assert lib.attn_fwd_splitkv_workspace_bytes(1, 1, 64, 64, 4097) == 0     # too many
    assert lib.attn_fwd_splitkv_workspace_bytes(-1, 1, 64, 64, 2) == 0
    assert lib.attn_fwd_splitkv_workspace_bytes(1 << 20, 1 << 20, 1 << 20, 128, 8) == 0  # overflow


def test_splitkv_argument_checks(lib):
    assert call_split(lib, n_splits=0) == INVALID
    assert call_split(lib, n_splits=5000) == INVALID
    assert call_split(lib, ws=None) == WORKSPACE
    need = lib.attn_fwd_splitkv_workspace_bytes(1, 2, 64, 64, 2)
    assert call_split(lib, ws_bytes=need - 1) == WORKSPACE
    assert call_split(lib, ws=A + 256 * MB + 8) == MISALIGNED
    assert call_split(lib, ws=A + 192 * MB) == INVALID       # workspace overlaps O
    assert call_split(lib, d=48) == UNSUPPORTED
    assert call_split(lib, scale=-1.0) == INVALID
    assert call_split(lib, B=0, ws=None, ws_bytes=0) == 0   # empty problem: no-op


def test_splitkv_default_splits_without_device(lib):
    # no usable device here (or a bad argument): the default is 1 split
    assert lib.attn_fwd_splitkv_default_splits(0, 1, 4, 4096, 128, False) >= 1
    assert lib.attn_fwd_splitkv_default_splits(0, 1, 4, 4096, 48, False) == 1


def call_gqa(lib, **kw):
    a = dict(dtype=0, Q=A, K=A + 64 * MB, V=A + 128 * MB, O=A + 192 * MB, LSE=None,
             B=1, H=8, Hkv=2, Nq=64, Nk=128, d=64, scale=0.125, causal=0, key_len=None)
    a.update(kw)
    return lib.lib.attn_fwd_gqa(a["dtype"], a["Q"], a["K"], a["V"], a["O"], a["LSE"],
                                a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                a["scale"], a["causal"], a["key_len"], None)


DEVICE = 6


@pytest.mark.parametrize("kw,code", [
    (dict(Hkv=3), INVALID), (dict(Hkv=0), INVALID), (dict(Hkv=16), INVALID),
    (dict(Hkv=-1), INVALID), (dict(Nq=-1), INVALID), (dict(Nk=-1), INVALID),
    (dict(Nk=(1 << 30) + 1), INVALID),
    (dict(Hkv=1, Nq=(1 << 27) + 1), INVALID),         # 8 heads x Nq rows per slice > 2^30
    (dict(d=96), UNSUPPORTED),
    (dict(K=None), INVALID),
    (dict(O=A + 64 * MB + 4096), INVALID),             # O overlaps K
    (dict(LSE=A + 128 * MB), INVALID),                 # LSE overlaps V
    (dict(K=A + 64 * MB + 8), MISALIGNED),
])
def test_gqa_rejects_bad_arguments(lib, kw, code):
    assert call_gqa(lib, **kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0, Hkv=0), dict(Nq=0),
                                dict(Nq=0, Q=None, K=None, V=None, O=None)])
def test_gqa_empty_problem_is_a_noop(lib, kw):
    assert call_gqa(lib, **kw) == 0


def test_gqa_accepts_what_it_should(lib):
    # these get past every argument check; without a device the call then
    # stops at the device check (on a GPU host it would launch)
    ok_or_device = (0, DEVICE)
    assert call_gqa(lib, Nk=0, K=None, V=None) in ok_or_device   # no keys: rows get O = 0
    assert call_gqa(lib, Hkv=8) in ok_or_device                  # plain multi-head
    assert call_gqa(lib, Hkv=1) in ok_or_device                  # one key/value head
    assert call_gqa(lib, Nq=1, Nk=100000) in ok_or_device        # one query row


def test_gqa_split_and_default_splits_without_device(lib):
    a = (0, A, A + 64 * MB, A + 128 * MB, A + 192 * MB, None, 1, 8, 3, 64, 128, 64, 0.125, 0, None)
    assert lib.lib.attn_fwd_gqa_splitkv(*a, 2, A + 256 * MB, 1 << 20, None) == INVALID  # Hkv=3
    a = (0, A, A + 64 * MB, A + 128 * MB, A + 192 * MB, None, 1, 8, 2, 64, 128, 64, 0.125, 0, None)
    need = lib.attn_fwd_splitkv_workspace_bytes(1, 8, 64, 64, 2)
    assert lib.lib.attn_fwd_gqa_splitkv(*a, 2, A + 256 * MB, need - 1, None) == WORKSPACE
    assert lib.lib.attn_fwd_gqa_splitkv(*a, 0, A + 256 * MB, need, None) == INVALID
    assert lib.attn_fwd_gqa_splitkv_default_splits(0, 1, 8, 3, 1, 4096, 128, True) == 1
    assert lib.attn_fwd_gqa_splitkv_default_splits(0, 1, 8, 2, 1, 4096, 128, True) >= 1


def call_masked(lib, mask=A + 320 * MB, sb=0, sh=0, **kw):
    a = dict(dtype=0, Q=A, K=A + 64 * MB, V=A + 128 * MB, O=A + 192 * MB, LSE=None,
             B=2, H=8, Hkv=2, Nq=64, Nk=128, d=64, scale=0.125, causal=0, key_len=None)
    a.update(kw)
    return lib.lib.attn_fwd_masked(a["dtype"], a["Q"], a["K"], a["V"], a["O"], a["LSE"],
                                   a["B"], a["H"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                                   a["scale"], a["causal"], a["key_len"], mask, sb, sh, None)


def test_masked_argument_checks(lib):
    assert call_masked(lib, mask=None) == INVALID
    assert call_masked(lib, sb=-1) == INVALID
    assert call_masked(lib, sh=-64) == INVALID
    assert call_masked(lib, mask=A + 320 * MB + 2) == MISALIGNED
    assert call_masked(lib, sh=1 << 27) == INVALID              # one batch's mask >= 2 GiB
    assert call_masked(lib, mask=A + 192 * MB + 64) == INVALID  # mask overlaps O
    assert call_masked(lib, Hkv=3) == INVALID
    assert call_masked(lib, B=0) == 0                            # empty: no-op
    assert call_masked(lib, mask=None, B=0) == INVALID
    # the mask may share memory with the read-only inputs; stops at the device check here
    assert call_masked(lib, mask=A + 64 * MB, sb=64 * 128, sh=0) in (0, DEVICE)
    assert call_masked(lib, sb=8 * 64 * 128, sh=64 * 128) in (0, DEVICE)


def test_gqa_kernel_names(lib):
    f16, bf16 = 0, 1
    assert lib.attn_fwd_gqa_kernel_name(f16, 128, 32, 32, 4096, 4096, True) == "attn_fwd_d128_f16_causal"
    assert lib.attn_fwd_gqa_kernel_name(f16, 32, 12, 12, 256, 256, False) == "attn_fwd_short_d32_f16_full"
    # at most 32 query rows per key/value head: the decode kernel
    assert lib.attn_fwd_gqa_kernel_name(bf16, 128, 32, 8, 1, 32768, True) == "attn_fwd_decode_d128_bf16_causal"
    assert lib.attn_fwd_gqa_kernel_name(bf16, 128, 32, 8, 1, 32768, True, n_splits=4) == \
        "attn_fwd_split_decode_d128_bf16_causal"
    assert lib.attn_fwd_gqa_kernel_name(f16, 64, 32, 8, 8, 1000, False) == "attn_fwd_decode_d64_f16_full"
    # at most one 256-row query tile per key/value head: the deep-ring instances
    assert lib.attn_fwd_gqa_kernel_name(bf16, 128, 32, 8, 16, 32768, True) == "attn_fwd_deep_d128_bf16_causal"
    assert lib.attn_fwd_gqa_kernel_name(bf16, 128, 32, 8, 64, 32768, True, n_splits=4) == \
        "attn_fwd_split_deep_d128_bf16_causal"
    assert lib.attn_fwd_gqa_kernel_name(f16, 64, 32, 8, 65, 4096, False) == "attn_fwd_d64_f16_full"
    assert lib.attn_fwd_gqa_kernel_name(f16, 128, 4, 4, 4096, 4096, True, n_splits=4) == \
        "attn_fwd_split_d128_f16_causal"
    assert lib.attn_fwd_gqa_kernel_name(f16, 128, 32, 32, 4096, 4096, True, masked=True) == \
        "attn_fwd_mask_d128_f16_causal"
    assert lib.attn_fwd_gqa_kernel_name(f16, 128, 32, 8, 1, 4096, True, masked=True, n_splits=2) == \
        "attn_fwd_split_mask_d128_f16_causal"
    with pytest.raises(lib.AttnError):
        lib.attn_fwd_gqa_kernel_name(f16, 128, 32, 3, 1, 4096, True)


def test_static_scratch_entry_checks_before_any_device_call(lib):
    """attn_fwd_gqa_splitkv_static rejects a problem whose partials exceed its
    scratch, and bad arguments, before any HIP call (fake pointers here)."""
    f = lib.lib.attn_fwd_gqa_splitkv_static
    GB = 1 << 30   # tensors of 256 MiB each, spaced so that none overlaps
    args = lambda B=1, H=32, Hkv=32, Nq=32768, Nk=32768, d=128, S=4: (
        0, A, A + GB, A + 2 * GB, A + 3 * GB, None, B, H, Hkv, Nq, Nk, d, 0.1, 1, None, S, None)
    WORKSPACE, INVALID = 4, 1
    assert f(*args()) == WORKSPACE                       # 2.2 GB of partials > 64 MiB
    assert f(*args(S=0)) == INVALID
    assert f(*args(Hkv=5)) == INVALID
    assert f(*args(B=0)) == 0                            # empty: no-op
