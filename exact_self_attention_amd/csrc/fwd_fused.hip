// Instances of the streaming kernel (the body is in fwd_body.h), the merge
// kernel of the split-key forward, and their launches.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "fwd_body.h"

#define ATTN_FWD_INSTANCE(NAME, D, BF16, CAUSAL)                                   \
    extern "C" __global__ __launch_bounds__(attn::kThreads)                       \
    void NAME(attn::FwdParams p) { attn::fwd_body<D, BF16, CAUSAL, false, false>(p); }
#define ATTN_SPLIT_INSTANCE(NAME, D, BF16, CAUSAL)                                 \
    extern "C" __global__ __launch_bounds__(attn::kThreads)                       \
    void NAME(attn::FwdParams p) { attn::fwd_body<D, BF16, CAUSAL, true, false>(p); }

ATTN_FWD_INSTANCE(attn_fwd_d32_f16_full, 32, false, false)
ATTN_FWD_INSTANCE(attn_fwd_d32_f16_causal, 32, false, true)
ATTN_FWD_INSTANCE(attn_fwd_d32_bf16_full, 32, true, false)
ATTN_FWD_INSTANCE(attn_fwd_d32_bf16_causal, 32, true, true)
ATTN_FWD_INSTANCE(attn_fwd_d64_f16_full, 64, false, false)
ATTN_FWD_INSTANCE(attn_fwd_d64_f16_causal, 64, false, true)
ATTN_FWD_INSTANCE(attn_fwd_d64_bf16_full, 64, true, false)
ATTN_FWD_INSTANCE(attn_fwd_d64_bf16_causal, 64, true, true)
ATTN_FWD_INSTANCE(attn_fwd_d128_f16_full, 128, false, false)
ATTN_FWD_INSTANCE(attn_fwd_d128_f16_causal, 128, false, true)
ATTN_FWD_INSTANCE(attn_fwd_d128_bf16_full, 128, true, false)
ATTN_FWD_INSTANCE(attn_fwd_d128_bf16_causal, 128, true, true)

ATTN_SPLIT_INSTANCE(attn_fwd_split_d32_f16_full, 32, false, false)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d32_f16_causal, 32, false, true)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d32_bf16_full, 32, true, false)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d32_bf16_causal, 32, true, true)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d64_f16_full, 64, false, false)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d64_f16_causal, 64, false, true)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d64_bf16_full, 64, true, false)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d64_bf16_causal, 64, true, true)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d128_f16_full, 128, false, false)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d128_f16_causal, 128, false, true)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d128_bf16_full, 128, true, false)
ATTN_SPLIT_INSTANCE(attn_fwd_split_d128_bf16_causal, 128, true, true)

namespace attn {
namespace {

// Merge of the key-range splits of every row, one thread per 4 output
// columns: LSE = m + log sum_s exp(LSE_s - m) with m = max_s LSE_s, and
// O = sum_s exp(LSE_s - m) O_s / sum_s exp(LSE_s - m), which is the
// online-softmax merge of "Self-Attention Kernel & Inference Engine from
// Scratch" ("Online Softmax Formulation") applied to whole blocks.  Rows
// whose splits are all empty get O = 0 and LSE = -inf.
struct MergeParams {
    const float *part_O;
    const float *part_LSE;
    uint16_t *O;
    float *LSE;
    int64_t rows;  // B * H * Nq
    int d;
    int splits;
};

// Up to this many splits, all of a row's partial LSEs are loaded at once,
// then the output chunks of the splits that saw a key of the row: two round
// trips to memory instead of one per split and loop.
constexpr int kMergeRegs = 8;

template <bool BF16>
__device__ __forceinline__ void merge_body(const MergeParams &p) {
    const int chunks = p.d / 4;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = t / chunks;
    const int c = (int)(t - row * chunks);
    if (row >= p.rows) return;
    uint16_t *orow = p.O + row * p.d + 4 * c;
    float m = -INFINITY, wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (p.splits <= kMergeRegs) {
        float l[kMergeRegs];
        f32x4 o[kMergeRegs];
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s)
            l[s] = s < p.splits ? p.part_LSE[(int64_t)s * p.rows + row] : -INFINITY;
        // a split that saw no key of the row (LSE = -inf) wrote no output:
        // its partial is not read (causal rows see fewer splits)
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s)
            o[s] = l[s] != -INFINITY
                       ? *reinterpret_cast<const f32x4 *>(p.part_O + ((int64_t)s * p.rows + row) * p.d + 4 * c)
                       : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kMergeRegs; ++s) m = fmaxf(m, l[s]);
        if (m != -INFINITY) {
#pragma unroll
            for (int s = 0; s < kMergeRegs; ++s) {
                // an empty split (LSE -inf) is left out: its partial output
                // was never written, and 0 times whatever it holds may be NaN
                if (l[s] == -INFINITY) continue;
                const float w = fast_exp2((l[s] - m) * 1.44269504088896341f);
                wsum += w;
                acc += w * o[s];
            }
        }
    } else {
        for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.part_LSE[(int64_t)s * p.rows + row]);
        if (m != -INFINITY) {
            for (int s = 0; s < p.splits; ++s) {
                const float l = p.part_LSE[(int64_t)s * p.rows + row];
                if (l == -INFINITY) continue;  // an empty split (its O_s is 0)
                const float w = fast_exp2((l - m) * 1.44269504088896341f);
                wsum += w;
                acc += w * *reinterpret_cast<const f32x4 *>(p.part_O + ((int64_t)s * p.rows + row) * p.d + 4 * c);
            }
        }
    }
    if (m == -INFINITY) {
        *reinterpret_cast<u32x2 *>(orow) = (u32x2){0u, 0u};
        if (p.LSE != nullptr && c == 0) p.LSE[row] = -INFINITY;
        return;
    }
    const float inv = 1.f / wsum;
    *reinterpret_cast<u32x2 *>(orow) =
        (u32x2){pack2<BF16>(acc[0] * inv, acc[1] * inv), pack2<BF16>(acc[2] * inv, acc[3] * inv)};
    if (p.LSE != nullptr && c == 0) p.LSE[row] = m + __builtin_logf(wsum);
}

}  // namespace
}  // namespace attn

extern "C" __global__ __launch_bounds__(256) void attn_fwd_split_merge_f16(attn::MergeParams p) {
    attn::merge_body<false>(p);
}
extern "C" __global__ __launch_bounds__(256) void attn_fwd_split_merge_bf16(attn::MergeParams p) {
    attn::merge_body<true>(p);
}

namespace attn {

namespace {
struct FwdEntry {
    FwdKernelFn fn;
    const char *name;
};
#define ATTN_ENTRY(NAME) {NAME, #NAME}
// index: ((d_index * 2) + bf16) * 2 + causal, d_index: 32 -> 0, 64 -> 1, 128 -> 2
const FwdEntry kFwdTable[12] = {
    ATTN_ENTRY(attn_fwd_d32_f16_full),   ATTN_ENTRY(attn_fwd_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_d32_bf16_full),  ATTN_ENTRY(attn_fwd_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_d64_f16_full),   ATTN_ENTRY(attn_fwd_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_d64_bf16_full),  ATTN_ENTRY(attn_fwd_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_d128_f16_full),  ATTN_ENTRY(attn_fwd_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_d128_bf16_full), ATTN_ENTRY(attn_fwd_d128_bf16_causal),
};
const FwdEntry kSplitTable[12] = {
    ATTN_ENTRY(attn_fwd_split_d32_f16_full),   ATTN_ENTRY(attn_fwd_split_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_split_d32_bf16_full),  ATTN_ENTRY(attn_fwd_split_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_d64_f16_full),   ATTN_ENTRY(attn_fwd_split_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_split_d64_bf16_full),  ATTN_ENTRY(attn_fwd_split_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_d128_f16_full),  ATTN_ENTRY(attn_fwd_split_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_split_d128_bf16_full), ATTN_ENTRY(attn_fwd_split_d128_bf16_causal),
};

#undef ATTN_ENTRY

int d_index(int d) { return d == 32 ? 0 : (d == 64 ? 1 : 2); }
int table_index(bool bf16, int d, bool causal) {
    return (d_index(d) * 2 + (bf16 ? 1 : 0)) * 2 + (causal ? 1 : 0);
}
const FwdEntry &entry(bool bf16, int d, bool causal) { return kFwdTable[table_index(bf16, d, causal)]; }
}  // namespace

const char *fwd_fused_kernel_name(bool bf16, int d, bool causal) {
    return entry(bf16, d, causal).name;
}

bool fwd_uses_deep(const FwdParams &p) { return p.mask == nullptr && p.M <= kBM; }

// Slice-group size of the XCD-blocked launch order (xcd_blocked_tile) for a
// masked forward, or 0 for the plain order.  Only a mask repeated over the
// heads is reused across slices; a group of A slices then shares it when
// the mask is also repeated over batches or the group lies in one batch.
// Among the group sizes the order allows, take the one with the least
// estimated traffic beyond L2: K and V fetched 8 A / S times, each batch's
// mask (S / A) / B times per batch.
int xcd_slice_group(const FwdParams &p, int d) {
    if (p.mask == nullptr || p.mask_sh != 0) return 0;
    const int S = p.slices;
    const double kv = (double)S * (double)p.Nk * d * 4.0;
    const double mask = (double)p.M * (double)p.Nk * 4.0;
    int best = 0;
    double best_cost = 0.0;
    for (int groups = 1; groups <= 8; groups *= 2) {
        if (S % groups != 0) continue;
        const int A = S / groups;
        const int per_slice_xcds = 8 / groups;
        if (p.n_qtiles % per_slice_xcds != 0) continue;
        if (p.mask_sb != 0 && p.Hkv % A != 0) continue;
        const double cost = kv * per_slice_xcds + mask * groups;
        if (best == 0 || cost < best_cost || (cost == best_cost && A < best)) {
            best = A;
            best_cost = cost;
        }
    }
    return best;
}

hipError_t launch_fwd_fused(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    if (fwd_uses_decode(p)) return launch_fwd_decode(bf16, d, causal, false, p, s);
    p.n_qtiles = (int)((p.M + kBM - 1) / kBM);
    p.xcd_slices = xcd_slice_group(p, d);
    const int64_t blocks = (int64_t)p.n_qtiles * p.slices;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const FwdKernelFn fn = p.mask != nullptr ? fwd_masked_kernel(bf16, d, causal, false)
                           : fwd_uses_deep(p) ? fwd_deep_kernel(bf16, d, causal, false)
                                              : entry(bf16, d, causal).fn;
    hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

int fwd_query_rows_per_item() { return kBM; }

const char *fwd_split_kernel_name(bool bf16, int d, bool causal) {
    return kSplitTable[table_index(bf16, d, causal)].name;
}

int fwd_split_resident_workgroups(bool bf16, int d, bool causal) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices][12];
    const int index = table_index(bf16, d, causal);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = cache[dev][index].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(kSplitTable[index].fn), kThreads, 0) != hipSuccess)
        return 0;
    const int r = cus * (per_cu > 0 ? per_cu : 1);
    if (dev < kMaxDevices) cache[dev][index].store(r, std::memory_order_relaxed);
    return r;
}

int64_t fwd_split_workgroups(const FwdParams &p, bool causal) {
    if (p.split_tiles < 1 || p.M <= 0 || p.slices <= 0) return 0;
    const int64_t n_qt = (p.M + kBM - 1) / kBM;
    const int64_t tiles = (p.Nk + kBN - 1) / kBN;
    int64_t busy = 0;
    for (int64_t t = 0; t < n_qt; ++t) {
        int64_t n_all = tiles;
        if (causal) {
            // the highest position among the tile's rows (split_busy)
            const int64_t r_lo = t * kBM, r_hi = std::min<int64_t>(p.M, r_lo + kBM) - 1;
            const int64_t hi = (r_lo / p.Nq == r_hi / p.Nq ? r_hi % p.Nq : p.Nq - 1) + p.causal_off;
            const int64_t kv_end = std::max<int64_t>(0, std::min<int64_t>(p.Nk, hi + 1));
            n_all = (kv_end + kBN - 1) / kBN;
        }
        busy += std::max<int64_t>(1, (n_all + p.split_tiles - 1) / p.split_tiles);
    }
    return busy * p.slices;
}

hipError_t launch_fwd_split(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    p.n_qtiles = (int)((p.M + kBM - 1) / kBM);
    if (p.kv_splits < 1 || p.split_tiles < 1) return hipErrorInvalidConfiguration;
    // only the (query tile, slice, split) workgroups with work, plus one for
    // a tile that sees no key (split_busy)
    const int64_t blocks = fwd_uses_decode(p) ? (int64_t)p.n_qtiles * p.slices * p.kv_splits
                                              : fwd_split_workgroups(p, causal);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipError_t e;
    if (fwd_uses_decode(p)) {
        e = launch_fwd_decode(bf16, d, causal, true, p, s);
    } else {
        const FwdKernelFn fn = p.mask != nullptr ? fwd_masked_kernel(bf16, d, causal, true)
                               : fwd_uses_deep(p) ? fwd_deep_kernel(bf16, d, causal, true)
                                                  : kSplitTable[table_index(bf16, d, causal)].fn;
        hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    MergeParams m;
    m.part_O = p.part_O;
    m.part_LSE = p.part_LSE;
    m.O = p.O;
    m.LSE = p.LSE;
    m.rows = (int64_t)p.slices * p.M;
    m.d = d;
    m.splits = p.kv_splits;
    const int64_t threads = m.rows * (d / 4);
    const int64_t mblocks = (threads + 255) / 256;
    if (mblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bf16 ? attn_fwd_split_merge_bf16 : attn_fwd_split_merge_f16,
                       dim3((unsigned)mblocks), dim3(256), 0, s, m);
    return hipGetLastError();
}

}  // namespace attn
