// Kernel choice for attn_fwd: the short-sequence kernel when a slice's keys
// fit in LDS, the streaming kernel otherwise (and always with a mask).
#include "kernels.h"

namespace attn {

namespace {
bool use_short(int d, int64_t Nk) { return Nk <= fwd_short_max_keys(d); }
}  // namespace

hipError_t launch_fwd(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    return use_short(d, p.Nk) && p.mask == nullptr ? launch_fwd_short(bf16, d, causal, p, s)
                             : launch_fwd_fused(bf16, d, causal, p, s);
}

const char *fwd_kernel_name(bool bf16, int d, bool causal, int64_t Nk) {
    return use_short(d, Nk) ? fwd_short_kernel_name(bf16, d, causal)
                           : fwd_fused_kernel_name(bf16, d, causal);
}

}  // namespace attn
