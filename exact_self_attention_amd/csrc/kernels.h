// Internal interface between the C ABI (api.cpp) and the gfx950 kernels.
// Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Arguments of one fused forward launch.  All pointers are device pointers;
// 16-bit tensors are passed as raw bit patterns.
//
// Q and O are [B, H, Nq, d], K and V [B, Hkv, Nk, d], and query head h reads
// key/value head h / (H / Hkv).  The H / Hkv query heads that share a
// key/value head are consecutive, so their rows form one contiguous block of
// M = (H / Hkv) * Nq rows of Q, O and LSE: a kernel works on slices
// (b, key/value head), each M query rows against Nk keys.  Row r of a slice
// is query r mod Nq of its head; with a causal mask it sees keys
// j <= r mod Nq + causal_off (causal_off = Nk - Nq: the last query row is
// aligned with the last key).  Self-attention is M = Nq = Nk, slices = B*H.
struct FwdParams {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    float *LSE;                 // [B, H, Nq] or nullptr
    const int32_t *key_len;     // [B] or nullptr: valid keys of sequence b
    int64_t M;                  // query rows per slice
    int64_t Nk;                 // keys per slice
    int Nq;                     // query rows per head
    int causal_off;             // Nk - Nq
    int slices;                 // B * Hkv
    int Hkv;
    int n_qtiles;               // ceil(M / query rows per workgroup)
    float scale_log2;           // scale * log2(e), > 0
    // Key-range split (attn_fwd_splitkv): workgroup slice s covers key tiles
    // [s * split_tiles, (s + 1) * split_tiles) and writes its normalised
    // partial output and LSE, in fp32, to part_O / part_LSE.
    int kv_splits;              // 1: no split
    int split_tiles;            // 64-key tiles per split
    float *part_O;              // [kv_splits][slices][M][d]
    float *part_LSE;            // [kv_splits][slices][M]
    // Additive fp32 mask (attn_fwd_masked) or nullptr: element (b, h, i, j)
    // at b * mask_sb + h * mask_sh + i * Nk + j; mask_bytes covers one
    // batch's part (< 2^31).
    const float *mask;
    int64_t mask_sb, mask_sh;
    uint32_t mask_bytes;
    // > 0: XCD-blocked launch order of a masked forward whose mask all the
    // slices share, with groups of this many slices (xcd_blocked_tile).
    int xcd_slices;
};

typedef void (*FwdKernelFn)(FwdParams);

// Streaming kernel (any Nk): 8 waves, 256 query rows per workgroup, K/V
// tiles through LDS rings, matrix-core and softmax phases ping-ponging
// between two wave groups.  p.n_qtiles is filled in here.
hipError_t launch_fwd_fused(bool bf16, int d, bool causal, FwdParams p, hipStream_t s);
const char *fwd_fused_kernel_name(bool bf16, int d, bool causal);

// Split-key forward: the streaming kernel over p.kv_splits key ranges into
// p.part_O / p.part_LSE, then a merge of the partial results into O and LSE
// (LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s).
hipError_t launch_fwd_split(bool bf16, int d, bool causal, FwdParams p, hipStream_t s);
const char *fwd_split_kernel_name(bool bf16, int d, bool causal);
// Workgroups of the split kernel the current device holds at once (0 on error).
int fwd_split_resident_workgroups(bool bf16, int d, bool causal);
// Workgroups of the streaming kernel's split grid: for each query tile the
// splits of p.split_tiles key tiles that have work, at least one, times
// p.slices (the decode kernel has its own grid).
int64_t fwd_split_workgroups(const FwdParams &p, bool causal);
int fwd_query_rows_per_item();

// Streaming kernel instances with the additive mask (plain or split-key);
// launch_fwd_fused and launch_fwd_split take them when p.mask is set.
FwdKernelFn fwd_masked_kernel(bool bf16, int d, bool causal, bool split);
const char *fwd_masked_kernel_name(bool bf16, int d, bool causal, bool split);

// Streaming kernel instances with 5-slot rings and Q straight to registers
// (fwd_deep.hip) for slices of at most one 256-row query tile without a
// mask; launch_fwd_fused and launch_fwd_split take them then.
FwdKernelFn fwd_deep_kernel(bool bf16, int d, bool causal, bool split);
const char *fwd_deep_kernel_name(bool bf16, int d, bool causal, bool split);
bool fwd_uses_deep(const FwdParams &p);

// Decode kernel (fwd_decode.hip) for slices of at most 32 query rows
// without a mask: 4 waves split the key range and merge at the end;
// launch_fwd_fused and launch_fwd_split take it then.
bool fwd_uses_decode(const FwdParams &p);
hipError_t launch_fwd_decode(bool bf16, int d, bool causal, bool split, FwdParams p, hipStream_t s);
const char *fwd_decode_kernel_name(bool bf16, int d, bool causal, bool split);
int fwd_decode_resident_workgroups(bool bf16, int d, bool causal);

// Short-sequence kernel (Nk <= fwd_short_max_keys(d)): 4 waves, 128 query
// rows per workgroup, the slice's whole K and V resident in LDS.
int64_t fwd_short_max_keys(int d);
hipError_t launch_fwd_short(bool bf16, int d, bool causal, FwdParams p, hipStream_t s);
const char *fwd_short_kernel_name(bool bf16, int d, bool causal);

// Dispatch on (dtype, d, Nk, causal): the kernel attn_fwd launches, and its
// name as profilers report it.
hipError_t launch_fwd(bool bf16, int d, bool causal, FwdParams p, hipStream_t s);
const char *fwd_kernel_name(bool bf16, int d, bool causal, int64_t Nk);

// Arguments of the unfused baseline, for heads [bh0, bh0 + nbh).
struct NaiveParams {
    const uint16_t *Q, *K, *V;
    uint16_t *O;
    float *LSE;
    const int32_t *key_len;
    float *S;                   // nbh * N * N fp32 scores, then probabilities
    int64_t N;
    int d;
    int H;
    int bh0;
    int nbh;
    float scale;
    int causal;
    int bf16;
};

hipError_t launch_naive(const NaiveParams &p, hipStream_t s);

}  // namespace attn
