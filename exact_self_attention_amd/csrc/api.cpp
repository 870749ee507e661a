// C ABI of libattn.so (declared in include/attn.h): argument checks,
// dispatch to a kernel instance, launch on the caller's stream.
//
// Every argument check runs before any HIP runtime call, so a rejected call
// never touches the device.  Nothing here allocates device memory.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxSplits = 4096;
constexpr int kMaxDevices = 64;

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Problem shape: Q and O are [B, H, Nq, d], K and V [B, Hkv, Nk, d].
struct Shape {
    int64_t B, H, Hkv, Nq, Nk, d;
    size_t q_elems() const { return (size_t)B * (size_t)H * (size_t)Nq; }   // rows of Q, O, LSE
    size_t kv_elems() const { return (size_t)B * (size_t)Hkv * (size_t)Nk; }  // rows of K, V
};

// Checks shared by every forward entry point.  *empty is set when there is
// nothing to compute (B*H*Nq == 0).  Nk == 0 is not empty: every row then
// has no visible key (O = 0, LSE = -inf), and K and V may be null.
attn_status_t check_args(attn_dtype_t dtype, const void *Q, const void *K, const void *V,
                         const void *O, const float *LSE, const Shape &sh, float scale,
                         const int32_t *key_len, bool *empty) {
    *empty = false;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (sh.B < 0 || sh.H < 0 || sh.Hkv < 0 || sh.Nq < 0 || sh.Nk < 0) return ATTN_ERR_INVALID_ARG;
    if (sh.d != 32 && sh.d != 64 && sh.d != 128) return ATTN_ERR_UNSUPPORTED;
    if (sh.Nq > kMaxN || sh.Nk > kMaxN) return ATTN_ERR_INVALID_ARG;
    if (sh.H > 0 && (sh.Hkv == 0 || sh.Hkv > sh.H || sh.H % sh.Hkv != 0)) return ATTN_ERR_INVALID_ARG;
    if (sh.B > 0 && sh.H > INT32_MAX / sh.B) return ATTN_ERR_INVALID_ARG;
    // query rows per slice (the heads that share a key/value head)
    if (sh.H > 0 && (sh.H / sh.Hkv) * sh.Nq > kMaxN) return ATTN_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || scale < 0.f) return ATTN_ERR_INVALID_ARG;
    if (sh.B == 0 || sh.H == 0 || sh.Nq == 0) {
        *empty = true;
        return ATTN_OK;
    }
    if (Q == nullptr || O == nullptr) return ATTN_ERR_INVALID_ARG;
    if (sh.Nk > 0 && (K == nullptr || V == nullptr)) return ATTN_ERR_INVALID_ARG;
    if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
        return ATTN_ERR_MISALIGNED;
    if (!aligned(LSE, 4) || !aligned(key_len, 4)) return ATTN_ERR_MISALIGNED;
    const size_t qbytes = sh.q_elems() * (size_t)sh.d * 2;
    const size_t kvbytes = sh.kv_elems() * (size_t)sh.d * 2;
    const size_t lbytes = sh.q_elems() * sizeof(float);
    const size_t kbytes = (size_t)sh.B * sizeof(int32_t);
    if (overlaps(O, qbytes, Q, qbytes) || overlaps(O, qbytes, K, kvbytes) ||
        overlaps(O, qbytes, V, kvbytes))
        return ATTN_ERR_INVALID_ARG;
    if (LSE != nullptr &&
        (overlaps(LSE, lbytes, Q, qbytes) || overlaps(LSE, lbytes, K, kvbytes) ||
         overlaps(LSE, lbytes, V, kvbytes) || overlaps(LSE, lbytes, O, qbytes)))
        return ATTN_ERR_INVALID_ARG;
    if (key_len != nullptr &&
        (overlaps(key_len, kbytes, O, qbytes) || overlaps(key_len, kbytes, LSE, lbytes)))
        return ATTN_ERR_INVALID_ARG;
    return ATTN_OK;
}

// Kernel arguments for a checked, non-empty problem.
attn::FwdParams make_params(const void *Q, const void *K, const void *V, void *O, float *LSE,
                            const Shape &sh, float scale, const int32_t *key_len) {
    attn::FwdParams p;
    p.Q = static_cast<const uint16_t *>(Q);
    p.K = static_cast<const uint16_t *>(K);
    p.V = static_cast<const uint16_t *>(V);
    p.O = static_cast<uint16_t *>(O);
    p.LSE = LSE;
    p.key_len = key_len;
    p.M = (sh.H / sh.Hkv) * sh.Nq;
    p.Nk = sh.Nk;
    p.Nq = (int)sh.Nq;
    p.causal_off = (int)(sh.Nk - sh.Nq);
    p.slices = (int)(sh.B * sh.Hkv);
    p.Hkv = (int)sh.Hkv;
    p.n_qtiles = 0;
    p.kv_splits = 1;
    p.split_tiles = 0;
    p.part_O = nullptr;
    p.part_LSE = nullptr;
    p.mask = nullptr;
    p.mask_sb = 0;
    p.mask_sh = 0;
    p.mask_bytes = 0;
    p.xcd_slices = 0;
    // The kernel needs a positive exp2 scale (masked scores are -inf and must
    // map to exactly 0).  A zero scale becomes 1e-30: every score times it
    // rounds to 0 against the fp32 maximum, so all weights stay exactly 1.
    p.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    if (!(p.scale_log2 >= 1e-30f)) p.scale_log2 = 1e-30f;
    return p;
}

// Checks of an additive mask for a checked, non-empty problem; fills the
// mask fields of p.  Element (b, h, i, j) is at b * sb + h * sh + i * Nk + j;
// one batch's part must stay below 2 GiB (the kernel addresses it with
// 32-bit offsets).
attn_status_t check_mask(const float *mask, int64_t sb, int64_t sh, const Shape &sh_, const void *O,
                         const float *LSE, attn::FwdParams *p) {
    if (mask == nullptr || sb < 0 || sh < 0) return ATTN_ERR_INVALID_ARG;
    if (!aligned(mask, 4)) return ATTN_ERR_MISALIGNED;
    const unsigned __int128 per_batch =
        ((unsigned __int128)(sh_.H - 1) * (unsigned __int128)sh +
         (unsigned __int128)sh_.Nq * (unsigned __int128)sh_.Nk) * 4u;
    if (per_batch > (unsigned __int128)(INT32_MAX - 64)) return ATTN_ERR_INVALID_ARG;
    const unsigned __int128 total = (unsigned __int128)(sh_.B - 1) * (unsigned __int128)sb * 4u + per_batch;
    if (total > (unsigned __int128)SIZE_MAX) return ATTN_ERR_INVALID_ARG;
    const size_t qbytes = sh_.q_elems() * (size_t)sh_.d * 2;
    if (overlaps(mask, (size_t)total, O, qbytes) ||
        overlaps(mask, (size_t)total, LSE, LSE ? sh_.q_elems() * 4 : 0))
        return ATTN_ERR_INVALID_ARG;
    p->mask = mask;
    p->mask_sb = sb;
    p->mask_sh = sh;
    p->mask_bytes = (uint32_t)per_batch;
    return ATTN_OK;
}

// The current device must be a gfx950; checked once per device.
attn_status_t check_device() {
    static std::atomic<int> state[kMaxDevices];  // 0 unknown, 1 ok, 2 bad
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return ATTN_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int s = state[dev].load(std::memory_order_relaxed);
        if (s != 0) return s == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

}  // namespace

extern "C" {

attn_status_t attn_fwd_gqa(attn_dtype_t dtype, const void *Q, const void *K, const void *V,
                           void *O, float *LSE, int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                           int64_t Nk, int64_t d, float scale, int causal,
                           const int32_t *key_len, void *stream) {
    const Shape sh{B, H, Hkv, Nq, Nk, d};
    bool empty = false;
    attn_status_t st = check_args(dtype, Q, K, V, O, LSE, sh, scale, key_len, &empty);
    if (st != ATTN_OK || empty) return st;
    st = check_device();
    if (st != ATTN_OK) return st;
    const attn::FwdParams p = make_params(Q, K, V, O, LSE, sh, scale, key_len);
    const hipError_t e = attn::launch_fwd(dtype == ATTN_BF16, (int)d, causal != 0, p,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_fwd_masked(attn_dtype_t dtype, const void *Q, const void *K, const void *V,
                              void *O, float *LSE, int64_t B, int64_t H, int64_t Hkv, int64_t Nq,
                              int64_t Nk, int64_t d, float scale, int causal,
                              const int32_t *key_len, const float *mask, int64_t mask_stride_b,
                              int64_t mask_stride_h, void *stream) {
    const Shape sh{B, H, Hkv, Nq, Nk, d};
    bool empty = false;
    attn_status_t st = check_args(dtype, Q, K, V, O, LSE, sh, scale, key_len, &empty);
    if (st != ATTN_OK) return st;
    if (mask == nullptr || mask_stride_b < 0 || mask_stride_h < 0) return ATTN_ERR_INVALID_ARG;
    if (empty) return ATTN_OK;
    attn::FwdParams p = make_params(Q, K, V, O, LSE, sh, scale, key_len);
    st = check_mask(mask, mask_stride_b, mask_stride_h, sh, O, LSE, &p);
    if (st != ATTN_OK) return st;
    st = check_device();
    if (st != ATTN_OK) return st;
    const hipError_t e = attn::launch_fwd(dtype == ATTN_BF16, (int)d, causal != 0, p,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_fwd(attn_dtype_t dtype, const void *Q, const void *K, const void *V, void *O,
                       float *LSE, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       int causal, const int32_t *key_len, void *stream) {
    return attn_fwd_gqa(dtype, Q, K, V, O, LSE, B, H, H, N, N, d, scale, causal, key_len, stream);
}

attn_status_t attn_fwd_naive(attn_dtype_t dtype, const void *Q, const void *K, const void *V,
                             void *O, float *LSE, int64_t B, int64_t H, int64_t N, int64_t d,
                             float scale, int causal, const int32_t *key_len, void *workspace,
                             size_t workspace_bytes, void *stream) {
    bool empty = false;
    attn_status_t st =
        check_args(dtype, Q, K, V, O, LSE, Shape{B, H, H, N, N, d}, scale, key_len, &empty);
    if (st != ATTN_OK || empty) return st;
    if ((N + 15) / 16 > 65535) return ATTN_ERR_INVALID_ARG;  // grid limit of the score kernel
    const size_t per_head = attn_fwd_naive_workspace_bytes(1, 1, N);
    if (per_head == 0) return ATTN_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < per_head) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_MISALIGNED;
    const size_t elems = (size_t)B * (size_t)H * (size_t)N;
    if (overlaps(workspace, workspace_bytes, Q, elems * d * 2) ||
        overlaps(workspace, workspace_bytes, K, elems * d * 2) ||
        overlaps(workspace, workspace_bytes, V, elems * d * 2) ||
        overlaps(workspace, workspace_bytes, O, elems * d * 2) ||
        overlaps(workspace, workspace_bytes, LSE, LSE ? elems * 4 : 0) ||
        overlaps(workspace, workspace_bytes, key_len, key_len ? (size_t)B * 4 : 0))
        return ATTN_ERR_INVALID_ARG;
    st = check_device();
    if (st != ATTN_OK) return st;

    const int BH = (int)(B * H);
    size_t group = workspace_bytes / per_head;
    if (group > 65535) group = 65535;  // grid limit of the head dimension
    attn::NaiveParams p;
    p.Q = static_cast<const uint16_t *>(Q);
    p.K = static_cast<const uint16_t *>(K);
    p.V = static_cast<const uint16_t *>(V);
    p.O = static_cast<uint16_t *>(O);
    p.LSE = LSE;
    p.key_len = key_len;
    p.S = static_cast<float *>(workspace);
    p.N = N;
    p.d = (int)d;
    p.H = (int)H;
    p.scale = scale;
    p.causal = causal != 0;
    p.bf16 = dtype == ATTN_BF16;
    for (int bh0 = 0; bh0 < BH; bh0 += (int)group) {
        p.bh0 = bh0;
        p.nbh = (int)((size_t)(BH - bh0) < group ? (size_t)(BH - bh0) : group);
        if (attn::launch_naive(p, static_cast<hipStream_t>(stream)) != hipSuccess)
            return ATTN_ERR_LAUNCH;
    }
    return ATTN_OK;
}

}  // extern "C"

namespace {
// The split-key forward, with an additive mask when `masked`.
attn_status_t splitkv(attn_dtype_t dtype, const void *Q, const void *K, const void *V, void *O,
                      float *LSE, int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                      int64_t d, float scale, int causal, const int32_t *key_len, bool masked,
                      const float *mask, int64_t mask_sb, int64_t mask_sh, int64_t n_splits,
                      void *workspace, size_t workspace_bytes, void *stream) {
    const Shape sh{B, H, Hkv, Nq, Nk, d};
    bool empty = false;
    attn_status_t st = check_args(dtype, Q, K, V, O, LSE, sh, scale, key_len, &empty);
    if (st != ATTN_OK) return st;
    if (n_splits < 1 || n_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
    if (masked && (mask == nullptr || mask_sb < 0 || mask_sh < 0)) return ATTN_ERR_INVALID_ARG;
    if (empty) return ATTN_OK;
    const size_t need = attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits);
    if (need == 0) return ATTN_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_ERR_MISALIGNED;
    const size_t qbytes = sh.q_elems() * (size_t)d * 2;
    const size_t kvbytes = sh.kv_elems() * (size_t)d * 2;
    if (overlaps(workspace, workspace_bytes, Q, qbytes) ||
        overlaps(workspace, workspace_bytes, K, kvbytes) ||
        overlaps(workspace, workspace_bytes, V, kvbytes) ||
        overlaps(workspace, workspace_bytes, O, qbytes) ||
        overlaps(workspace, workspace_bytes, LSE, LSE ? sh.q_elems() * 4 : 0) ||
        overlaps(workspace, workspace_bytes, key_len, key_len ? (size_t)B * 4 : 0))
        return ATTN_ERR_INVALID_ARG;
    attn::FwdParams p = make_params(Q, K, V, O, LSE, sh, scale, key_len);
    if (masked) {
        st = check_mask(mask, mask_sb, mask_sh, sh, O, LSE, &p);
        if (st != ATTN_OK) return st;
        if (overlaps(workspace, workspace_bytes, mask,
                     (size_t)(B - 1) * (size_t)mask_sb * 4 + p.mask_bytes))
            return ATTN_ERR_INVALID_ARG;
    }
    st = check_device();
    if (st != ATTN_OK) return st;

    // whole 64-key tiles per split; trailing splits that would be empty for
    // every row are not launched
    const int64_t tiles = (Nk + 63) / 64;
    const int64_t per = tiles > 0 ? (tiles + n_splits - 1) / n_splits : 1;
    const int64_t used = tiles > 0 ? (tiles + per - 1) / per : 1;
    p.kv_splits = (int)used;
    p.split_tiles = (int)per;
    p.part_O = static_cast<float *>(workspace);
    p.part_LSE = p.part_O + (size_t)used * sh.q_elems() * (size_t)d;
    const hipError_t e = attn::launch_fwd_split(dtype == ATTN_BF16, (int)d, causal != 0, p,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
}  // namespace

// Device-resident scratch of attn_fwd_gqa_splitkv_static, for callers that
// cannot allocate: the split partials live in this file-scope array, one
// copy on every device the library runs on, held until the process ends.
// In host code its name is only a stand-in for the device copy: kernels get
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[ATTN_STATIC_SCRATCH_BYTES];

namespace {
struct ScratchAddr {
    std::once_flag once;
    hipError_t err = hipSuccess;
    void *ptr = nullptr;
};
ScratchAddr g_scratch[kMaxDevices];

// The device address of `scratch` on the current device (looked up once per
// device, with that device current), or nullptr.
void *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    ScratchAddr &s = g_scratch[dev];
    std::call_once(s.once, [&s] {
        void *ptr = nullptr;
        s.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        s.ptr = s.err == hipSuccess ? ptr : nullptr;
    });
    return s.ptr;
}
}  // namespace

extern "C" {

attn_status_t attn_fwd_gqa_splitkv_static(attn_dtype_t dtype, const void *Q, const void *K,
                                          const void *V, void *O, float *LSE, int64_t B,
                                          int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk,
                                          int64_t d, float scale, int causal,
                                          const int32_t *key_len, int64_t n_splits,
                                          void *stream) {
    // the argument checks first (no HIP call for a rejected call), then the
    // size limit, then the device and the scratch address
    const Shape sh{B, H, Hkv, Nq, Nk, d};
    bool empty = false;
    attn_status_t st = check_args(dtype, Q, K, V, O, LSE, sh, scale, key_len, &empty);
    if (st != ATTN_OK) return st;
    if (n_splits < 1 || n_splits > kMaxSplits) return ATTN_ERR_INVALID_ARG;
    if (empty) return ATTN_OK;
    const size_t need = attn_fwd_splitkv_workspace_bytes(B, H, Nq, d, n_splits);
    if (need == 0) return ATTN_ERR_INVALID_ARG;
    if (need > (size_t)ATTN_STATIC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    st = check_device();
    if (st != ATTN_OK) return st;
    void *const ws = scratch_on_current_device();
    if (ws == nullptr) return ATTN_ERR_DEVICE;
    return splitkv(dtype, Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, causal, key_len, false,
                   nullptr, 0, 0, n_splits, ws, (size_t)ATTN_STATIC_SCRATCH_BYTES, stream);
}

attn_status_t attn_fwd_gqa_splitkv(attn_dtype_t dtype, const void *Q, const void *K,
                                   const void *V, void *O, float *LSE, int64_t B, int64_t H,
                                   int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                   int causal, const int32_t *key_len, int64_t n_splits,
                                   void *workspace, size_t workspace_bytes, void *stream) {
    return splitkv(dtype, Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, causal, key_len, false,
                   nullptr, 0, 0, n_splits, workspace, workspace_bytes, stream);
}

attn_status_t attn_fwd_masked_splitkv(attn_dtype_t dtype, const void *Q, const void *K,
                                      const void *V, void *O, float *LSE, int64_t B, int64_t H,
                                      int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                      int causal, const int32_t *key_len, const float *mask,
                                      int64_t mask_stride_b, int64_t mask_stride_h,
                                      int64_t n_splits, void *workspace, size_t workspace_bytes,
                                      void *stream) {
    return splitkv(dtype, Q, K, V, O, LSE, B, H, Hkv, Nq, Nk, d, scale, causal, key_len, true,
                   mask, mask_stride_b, mask_stride_h, n_splits, workspace, workspace_bytes,
                   stream);
}

attn_status_t attn_fwd_splitkv(attn_dtype_t dtype, const void *Q, const void *K, const void *V,
                               void *O, float *LSE, int64_t B, int64_t H, int64_t N, int64_t d,
                               float scale, int causal, const int32_t *key_len, int64_t n_splits,
                               void *workspace, size_t workspace_bytes, void *stream) {
    return attn_fwd_gqa_splitkv(dtype, Q, K, V, O, LSE, B, H, H, N, N, d, scale, causal, key_len,
                                n_splits, workspace, workspace_bytes, stream);
}

size_t attn_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d,
                                        int64_t n_splits) {
    if (B < 0 || H < 0 || N < 0 || N > kMaxN || d < 0 || d > 1024 || n_splits < 1 ||
        n_splits > kMaxSplits)
        return 0;
    const unsigned __int128 total = (unsigned __int128)n_splits * (unsigned __int128)B *
                                    (unsigned __int128)H * (unsigned __int128)N *
                                    (unsigned __int128)(d + 1) * 4u;
    if (total > (unsigned __int128)SIZE_MAX) return 0;
    return (size_t)total;
}

int64_t attn_fwd_gqa_splitkv_default_splits(attn_dtype_t dtype, int64_t B, int64_t H,
                                            int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                                            int causal) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return 1;
    if (d != 32 && d != 64 && d != 128) return 1;
    if (B <= 0 || H <= 0 || Hkv <= 0 || Hkv > H || H % Hkv != 0 || Nq <= 0 || Nk <= 0 ||
        Nq > kMaxN || Nk > kMaxN || H > INT32_MAX / B || (H / Hkv) * Nq > kMaxN)
        return 1;
    if (check_device() != ATTN_OK) return 1;
    attn::FwdParams probe = make_params(nullptr, nullptr, nullptr, nullptr, nullptr,
                                        Shape{B, H, Hkv, Nq, Nk, d}, 1.f, nullptr);
    const bool decode = attn::fwd_uses_decode(probe);
    const int resident =
        decode ? attn::fwd_decode_resident_workgroups(dtype == ATTN_BF16, (int)d, causal != 0)
               : attn::fwd_split_resident_workgroups(dtype == ATTN_BF16, (int)d, causal != 0);
    if (resident <= 0) return 1;
    const int64_t tiles = (Nk + 63) / 64;
    int64_t max_s = tiles / 2 > 1 ? tiles / 2 : 1;
    if (max_s > kMaxSplits) max_s = kMaxSplits;
    if (decode) {
        // one work item per key/value head, each over all the keys
        const int64_t items = B * Hkv;
        if (items >= resident) return 1;
        const int64_t s = (resident + items - 1) / items;
        return s > max_s ? max_s : s;
    }
    // work items: (key/value head, 256-row query tile).  A split covers a
    // fixed run of key tiles, and the grid holds only the splits with work
    // (under the causal mask a query tile sees fewer keys the earlier it
    // is).  The count is the largest whose workgroups all fit in one
    // resident round, so that the longest run is as short as it can be.
    const int64_t rows = attn::fwd_query_rows_per_item();
    const int64_t n_qt = ((H / Hkv) * Nq + rows - 1) / rows;
    if (n_qt * B * Hkv >= resident) return 1;
    auto busy = [&](int64_t s) {
        probe.split_tiles = (int)((tiles + s - 1) / s);
        return attn::fwd_split_workgroups(probe, causal != 0);
    };
    // busy() does not decrease as s grows: take the largest s that fits
    int64_t lo = 1, hi = max_s;
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (busy(mid) <= resident) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

int64_t attn_fwd_splitkv_default_splits(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N,
                                        int64_t d, int causal) {
    return attn_fwd_gqa_splitkv_default_splits(dtype, B, H, H, N, N, d, causal);
}

size_t attn_fwd_naive_workspace_bytes(int64_t B, int64_t H, int64_t N) {
    if (B < 0 || H < 0 || N < 0 || N > kMaxN) return 0;
    const unsigned __int128 total = (unsigned __int128)B * (unsigned __int128)H *
                                    (unsigned __int128)N * (unsigned __int128)N * 4u;
    if (total > (unsigned __int128)SIZE_MAX) return 0;
    return (size_t)total;
}

const char *attn_status_string(attn_status_t status) {
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (size, scale, null pointer or aliasing)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or dtype (d must be 32, 64 or 128)";
    case ATTN_ERR_MISALIGNED: return "misaligned pointer (tensors need 16 bytes, LSE and key_len 4)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than the entry point needs";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_DEVICE: return "no usable gfx950 device is current";
    }
    return "unknown status";
}

attn_status_t attn_fwd_kernel_name(attn_dtype_t dtype, int64_t d, int64_t N, int causal,
                                   int has_key_len, char *buf, size_t buf_len) {
    (void)has_key_len;
    // attn_fwd is attn_fwd_gqa with one key/value head per query head and
    // equal lengths, so the same decision names its kernel (the head count
    // does not enter it)
    return attn_fwd_gqa_kernel_name(dtype, d, 1, 1, N, N, causal, 0, 0, buf, buf_len);
}

attn_status_t attn_fwd_gqa_kernel_name(attn_dtype_t dtype, int64_t d, int64_t H, int64_t Hkv,
                                       int64_t Nq, int64_t Nk, int causal, int masked,
                                       int64_t n_splits, char *buf, size_t buf_len) {
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (d != 32 && d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
    if (H < 1 || Hkv < 1 || Hkv > H || H % Hkv != 0 || Nq < 0 || Nk < 0 || Nq > kMaxN ||
        Nk > kMaxN || (H / Hkv) * Nq > kMaxN || n_splits < 0 || n_splits > kMaxSplits)
        return ATTN_ERR_INVALID_ARG;
    if (buf == nullptr || buf_len == 0) return ATTN_ERR_INVALID_ARG;
    const bool bf16 = dtype == ATTN_BF16;
    const bool split = n_splits > 0;
    attn::FwdParams p = make_params(nullptr, nullptr, nullptr, nullptr, nullptr,
                                    Shape{1, H, Hkv, Nq, Nk, d}, 1.f, nullptr);
    p.mask = masked ? reinterpret_cast<const float *>(&p) : nullptr;  // only its presence matters
    const char *name;
    if (masked)
        name = attn::fwd_masked_kernel_name(bf16, (int)d, causal != 0, split);
    else if (!split && Nk <= attn::fwd_short_max_keys((int)d))
        name = attn::fwd_kernel_name(bf16, (int)d, causal != 0, Nk);
    else if (attn::fwd_uses_decode(p))
        name = attn::fwd_decode_kernel_name(bf16, (int)d, causal != 0, split);
    else if (attn::fwd_uses_deep(p))
        name = attn::fwd_deep_kernel_name(bf16, (int)d, causal != 0, split);
    else if (split)
        name = attn::fwd_split_kernel_name(bf16, (int)d, causal != 0);
    else
        name = attn::fwd_fused_kernel_name(bf16, (int)d, causal != 0);
    std::snprintf(buf, buf_len, "%s", name);
    return ATTN_OK;
}

int attn_version(void) { return 100; }

}  // extern "C"
