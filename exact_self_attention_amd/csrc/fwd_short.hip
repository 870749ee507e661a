// Fused exact attention forward for short sequences on gfx950 (CDNA4).
//
// When a slice's keys fit in LDS (Nk <= 256 at d <= 64, Nk <= 128 at
// d = 128) the streaming pipeline of the long-sequence kernel only adds
// latency: every tile is used once and the loop is a few tiles long.  Here a
// workgroup of 4 waves owns 128 query rows of one slice (b, key/value head;
// the rows of the query heads that share it, head after head):
//
//   1. all of the slice's visible K and V rows go to LDS at once (direct
//      buffer loads, rows past the valid key length read as zero and are not
//      fetched), and each wave loads the Q fragments of its query rows
//      straight into VGPRs;
//   2. one barrier;
//   3. each wave runs, for every key tile its 32 rows can see,
//      S^T = K_j Q^T on the matrix cores, the online softmax update of
//      "Self-Attention Kernel & Inference Engine from Scratch" (section
//      "Online Softmax Formulation": running max, running normaliser,
//      rescaled output), and O^T += V_j^T P^T, with no further
//      synchronisation, then writes O = O_acc / l and LSE.
//
// A workgroup needs at most 64 KB of LDS (32 KB at d = 32), so several are
// resident per compute unit and their load latencies overlap each other's
// arithmetic.  Masking follows the long-sequence kernel: causal and key-length
// limits end the tile loop early and per-element masks run only on tiles
// that straddle a limit; a masked score is -inf, whose exp2 is exactly 0.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdna4.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace cdna4;

constexpr int short_max_keys_of(int d) { return d >= 128 ? 128 : 256; }
// 4 waves, one per SIMD and per 32 query rows: a workgroup owns 128 query
// rows of one slice.  (One 8-wave workgroup per head, or one 4-wave
// workgroup making two passes, measured slower: fewer waves in flight.)
constexpr int kSWaves = 4;
constexpr int kSBM = kSWaves * kQRows;
// Waves per SIMD the register allocation must allow: as many workgroups as
// LDS holds per compute unit (4 of 32 KB at d = 32, 2 of 64 KB otherwise).
constexpr int short_waves_per_simd(int d) { return d == 32 ? 4 : 2; }

template <int D, bool BF16, bool CAUSAL>
__device__ __forceinline__ void short_body(const FwdParams &p) {
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = kBN * D;                 // halves per K or V tile
    constexpr int TILE_INSTR = kBN * CPR / 64;    // 1 KB load instructions per tile
    constexpr int NT = short_max_keys_of(D) / kBN;  // key tiles held in LDS
    constexpr int SW = kSWaves;
    constexpr int SHARE = 2 * TILE_INSTR / SW;    // K and V loads per wave per tile
    constexpr int KB = kBN / 32;
    constexpr int DK = D / 16;
    constexpr int DB = D / 32;
    static_assert((2 * TILE_INSTR) % SW == 0, "tile load split");
    static_assert(KB == 2, "the softmax arithmetic assumes 64-key tiles");

    __shared__ __attribute__((aligned(1024))) uint16_t sK[NT][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[NT][TILE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    const int S = p.slices;
    const int sl = blockIdx.x % S;
    int qt = blockIdx.x / S;
    const int M = (int)p.M;                // query rows of the slice
    if (CAUSAL) qt = heavy_first_tile(qt, p.n_qtiles, p.Nq, M, kSBM);
    const int Nk = (int)p.Nk;
    const int b = sl / p.Hkv;
    const size_t q_base = (size_t)sl * (size_t)M * D;
    const size_t kv_base = (size_t)sl * (size_t)Nk * D;
    const uint16_t *__restrict__ Qp = p.Q + q_base;
    const uint16_t *__restrict__ Kp = p.K + kv_base;
    const uint16_t *__restrict__ Vp = p.V + kv_base;

    int Lk = Nk;
    if (p.key_len != nullptr) {
        const int v = p.key_len[b];
        Lk = v < 0 ? 0 : (v > Nk ? Nk : v);
    }
    const int q0 = qt * kSBM;
    const int qw0 = q0 + wave * kQRows;           // this wave's 32 query rows
    const int my_q = qw0 + l32;
    // causal: keys up to the highest position of the workgroup's (or the
    // wave's) rows; tiles past the lowest position of a wave's rows need
    // per-element masking
    const CausalRows cr{p.Nq, p.causal_off};
    int kv_end = Lk;
    int wave_lo = 0, wave_hi = 0;
    if (CAUSAL) {
        int lo, hi;
        cr.range(q0, min(q0 + kSBM, M) - 1, lo, hi);
        kv_end = max(0, min(kv_end, hi + 1));
        if (qw0 < M) cr.range(qw0, min(qw0 + kQRows, M) - 1, wave_lo, wave_hi);
    }
    const int my_pos = CAUSAL ? cr.pos(my_q) : 0;
    const int n = (kv_end + kBN - 1) / kBN;       // key tiles of the workgroup (<= NT)
    int n_w = n;                                  // key tiles this wave computes
    if (CAUSAL) n_w = (max(0, min(kv_end, wave_hi + 1)) + kBN - 1) / kBN;
    if (qw0 >= M) n_w = 0;

    // ---- loads: Q fragments to VGPRs (B operand of S^T: query row my_q,
    // dims 16 kk + 8 g .. +7; rows past M are zero), K and V tiles to LDS
    // (same swizzled layout as the long-sequence kernel: load instruction t
    // of a tile fills LDS bytes [1024 t, 1024 t + 1024), lane i physical
    // chunk 64 t + i).  Of a tile's 2 TILE_INSTR loads (K, then V) wave w
    // issues numbers w, w + SW, ...
    u32x4 qreg[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qreg[kk] = my_q < M ? *reinterpret_cast<const u32x4 *>(Qp + (size_t)my_q * D + (2 * kk + g) * 8)
                            : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (t < n) {
            const int rows = min(kBN, Lk - t * kBN);
            const i32x4 rk = make_rsrc(Kp + (size_t)t * kBN * D, (uint32_t)(rows * D * 2));
            const i32x4 rv = make_rsrc(Vp + (size_t)t * kBN * D, (uint32_t)(rows * D * 2));
            const uint32_t kl = (uint32_t)(uintptr_t)(lds_void *)sK[t];
            const uint32_t vl = (uint32_t)(uintptr_t)(lds_void *)sV[t];
#pragma unroll
            for (int i = 0; i < SHARE; ++i) {
                const int u = wave_u + SW * i;
                const bool is_v = u >= TILE_INSTR;
                const int ti = is_v ? u - TILE_INSTR : u;
                const int P = 64 * ti + lane;
                const int row = P / CPR;
                const int ch = (P % CPR) ^ swz<D>(row);
                const uint32_t voff = (uint32_t)(row * D * 2 + ch * 16);
                if (is_v)
                    dma16(rv, vl + (uint32_t)ti * 1024u, voff);
                else
                    dma16(rk, kl + (uint32_t)ti * 1024u, voff);
            }
        }
    }
    wait_tile_loads<0>();
    barrier();

    // ---- this wave's query rows over the visible key tiles
    const float c = p.scale_log2;
    f32x16 oacc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    f32x16 s[KB];
    u32x4 pf[KB][2];
    float m_run = -INFINITY;  // running max of scale*log2(e)*score (may trail the true one)
    float l_run = 0.f;        // this lane's share of the running normaliser

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (j >= n_w) break;
        const uint16_t *kt = sK[j];
        const uint16_t *vt = sV[j];
        // S^T = K_j Q^T
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
                s[kb] = mfma32<BF16>(frag_k<D>(kt, kb, kk, l32, g), qreg[kk], s[kb]);
        // mask the tiles that straddle the key-length or causal limit
        const int j0 = j * kBN;
        if ((j0 + kBN > Lk) || (CAUSAL && j0 + kBN - 1 > wave_lo)) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= my_pos);
                    s[kb][r] = ok ? s[kb][r] : -INFINITY;
                }
        }
        // online softmax with a lazy running max: it moves only when the
        // tile's max exceeds it by more than kLazy, then to kHeadroom above
        // that max; output and normaliser are rescaled by exp2(m_old - m_new)
        const float m_tile = row_max64(s) * c;  // -inf stays -inf (c > 0)
        const bool grow = m_tile > m_run + kLazy;
        if (__any(grow)) {
            const float m_new = grow ? m_tile + kHeadroom : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        }
        l_run += exps64<BF16>(s, c, m_run == -INFINITY ? 0.f : -m_run, pf);
        // O^T += V_j^T P^T
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                oacc[cb] = mfma32<BF16>(frag_v<D>(vt, cb, kc, lane, g), pf[kc >> 1][kc & 1], oacc[cb]);
    }

    // ---- epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l)
    const Halves lh = both_halves(l_run);
    const float l_tot = lh.lo + lh.hi;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_q < M) {
        uint16_t *orow = p.O + q_base + (size_t)my_q * D;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u32x2 w = {pack2<BF16>(oacc[cb][4 * a] * inv, oacc[cb][4 * a + 1] * inv),
                           pack2<BF16>(oacc[cb][4 * a + 2] * inv, oacc[cb][4 * a + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + cb * 32 + a * 8 + g * 4) = w;
            }
        if (p.LSE != nullptr && g == 0)
            p.LSE[(size_t)sl * M + my_q] =
                l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

}  // namespace
}  // namespace attn

#define ATTN_SHORT_INSTANCE(NAME, D, BF16, CAUSAL)                                 \
    extern "C" __global__ __launch_bounds__(attn::kSWaves * 64)                   \
    __attribute__((amdgpu_waves_per_eu(attn::short_waves_per_simd(D))))           \
    void NAME(attn::FwdParams p) { attn::short_body<D, BF16, CAUSAL>(p); }

ATTN_SHORT_INSTANCE(attn_fwd_short_d32_f16_full, 32, false, false)
ATTN_SHORT_INSTANCE(attn_fwd_short_d32_f16_causal, 32, false, true)
ATTN_SHORT_INSTANCE(attn_fwd_short_d32_bf16_full, 32, true, false)
ATTN_SHORT_INSTANCE(attn_fwd_short_d32_bf16_causal, 32, true, true)
ATTN_SHORT_INSTANCE(attn_fwd_short_d64_f16_full, 64, false, false)
ATTN_SHORT_INSTANCE(attn_fwd_short_d64_f16_causal, 64, false, true)
ATTN_SHORT_INSTANCE(attn_fwd_short_d64_bf16_full, 64, true, false)
ATTN_SHORT_INSTANCE(attn_fwd_short_d64_bf16_causal, 64, true, true)
ATTN_SHORT_INSTANCE(attn_fwd_short_d128_f16_full, 128, false, false)
ATTN_SHORT_INSTANCE(attn_fwd_short_d128_f16_causal, 128, false, true)
ATTN_SHORT_INSTANCE(attn_fwd_short_d128_bf16_full, 128, true, false)
ATTN_SHORT_INSTANCE(attn_fwd_short_d128_bf16_causal, 128, true, true)

namespace attn {

namespace {
typedef void (*ShortKernel)(FwdParams);
struct ShortEntry {
    ShortKernel fn;
    const char *name;
};
#define ATTN_ENTRY(NAME) {NAME, #NAME}
// index: ((d_index * 2) + bf16) * 2 + causal, d_index: 32 -> 0, 64 -> 1, 128 -> 2
const ShortEntry kShortTable[12] = {
    ATTN_ENTRY(attn_fwd_short_d32_f16_full),   ATTN_ENTRY(attn_fwd_short_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_short_d32_bf16_full),  ATTN_ENTRY(attn_fwd_short_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_short_d64_f16_full),   ATTN_ENTRY(attn_fwd_short_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_short_d64_bf16_full),  ATTN_ENTRY(attn_fwd_short_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_short_d128_f16_full),  ATTN_ENTRY(attn_fwd_short_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_short_d128_bf16_full), ATTN_ENTRY(attn_fwd_short_d128_bf16_causal),
};
#undef ATTN_ENTRY

const ShortEntry &short_entry(bool bf16, int d, bool causal) {
    const int di = d == 32 ? 0 : (d == 64 ? 1 : 2);
    return kShortTable[(di * 2 + (bf16 ? 1 : 0)) * 2 + (causal ? 1 : 0)];
}
}  // namespace

int64_t fwd_short_max_keys(int d) { return short_max_keys_of(d); }

const char *fwd_short_kernel_name(bool bf16, int d, bool causal) {
    return short_entry(bf16, d, causal).name;
}

hipError_t launch_fwd_short(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    if (p.Nk > fwd_short_max_keys(d)) return hipErrorInvalidValue;
    p.n_qtiles = (int)((p.M + kSBM - 1) / kSBM);
    const int64_t blocks = (int64_t)p.n_qtiles * p.slices;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(short_entry(bf16, d, causal).fn, dim3((unsigned)blocks),
                       dim3(64 * kSWaves), 0, s, p);
    return hipGetLastError();
}

}  // namespace attn
