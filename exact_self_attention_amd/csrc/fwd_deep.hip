// Streaming kernel instances for slices of at most one 256-row query tile
// (decode-like shapes: few query rows against many keys, bound by device
// memory): Q straight to registers and 5-slot K/V rings (fwd_body.h, DEEP).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_body.h"

#define ATTN_DEEP_INSTANCE(NAME, D, BF16, CAUSAL, SPLIT)                           \
    extern "C" __global__ __launch_bounds__(attn::kThreads)                       \
    void NAME(attn::FwdParams p) { attn::fwd_body<D, BF16, CAUSAL, SPLIT, false, true>(p); }

ATTN_DEEP_INSTANCE(attn_fwd_deep_d32_f16_full, 32, false, false, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d32_f16_causal, 32, false, true, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d32_bf16_full, 32, true, false, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d32_bf16_causal, 32, true, true, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d64_f16_full, 64, false, false, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d64_f16_causal, 64, false, true, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d64_bf16_full, 64, true, false, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d64_bf16_causal, 64, true, true, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d128_f16_full, 128, false, false, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d128_f16_causal, 128, false, true, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d128_bf16_full, 128, true, false, false)
ATTN_DEEP_INSTANCE(attn_fwd_deep_d128_bf16_causal, 128, true, true, false)

ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d32_f16_full, 32, false, false, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d32_f16_causal, 32, false, true, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d32_bf16_full, 32, true, false, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d32_bf16_causal, 32, true, true, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d64_f16_full, 64, false, false, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d64_f16_causal, 64, false, true, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d64_bf16_full, 64, true, false, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d64_bf16_causal, 64, true, true, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d128_f16_full, 128, false, false, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d128_f16_causal, 128, false, true, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d128_bf16_full, 128, true, false, true)
ATTN_DEEP_INSTANCE(attn_fwd_split_deep_d128_bf16_causal, 128, true, true, true)

namespace attn {

namespace {
struct DeepEntry {
    FwdKernelFn fn;
    const char *name;
};
#define ATTN_ENTRY(NAME) {NAME, #NAME}
// index: (((split * 3 + d_index) * 2) + bf16) * 2 + causal,
// d_index: 32 -> 0, 64 -> 1, 128 -> 2
const DeepEntry kDeepTable[24] = {
    ATTN_ENTRY(attn_fwd_deep_d32_f16_full),         ATTN_ENTRY(attn_fwd_deep_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_deep_d32_bf16_full),        ATTN_ENTRY(attn_fwd_deep_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_deep_d64_f16_full),         ATTN_ENTRY(attn_fwd_deep_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_deep_d64_bf16_full),        ATTN_ENTRY(attn_fwd_deep_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_deep_d128_f16_full),        ATTN_ENTRY(attn_fwd_deep_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_deep_d128_bf16_full),       ATTN_ENTRY(attn_fwd_deep_d128_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_deep_d32_f16_full),   ATTN_ENTRY(attn_fwd_split_deep_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_split_deep_d32_bf16_full),  ATTN_ENTRY(attn_fwd_split_deep_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_deep_d64_f16_full),   ATTN_ENTRY(attn_fwd_split_deep_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_split_deep_d64_bf16_full),  ATTN_ENTRY(attn_fwd_split_deep_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_deep_d128_f16_full),  ATTN_ENTRY(attn_fwd_split_deep_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_split_deep_d128_bf16_full), ATTN_ENTRY(attn_fwd_split_deep_d128_bf16_causal),
};
#undef ATTN_ENTRY

const DeepEntry &deep_entry(bool bf16, int d, bool causal, bool split) {
    const int di = d == 32 ? 0 : (d == 64 ? 1 : 2);
    return kDeepTable[(((split ? 3 : 0) + di) * 2 + (bf16 ? 1 : 0)) * 2 + (causal ? 1 : 0)];
}
}  // namespace

FwdKernelFn fwd_deep_kernel(bool bf16, int d, bool causal, bool split) {
    return deep_entry(bf16, d, causal, split).fn;
}

const char *fwd_deep_kernel_name(bool bf16, int d, bool causal, bool split) {
    return deep_entry(bf16, d, causal, split).name;
}

}  // namespace attn
