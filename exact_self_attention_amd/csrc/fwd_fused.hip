// Fused exact attention forward for gfx950 (CDNA4).
//
// One workgroup = 8 waves = one tile of 256 query rows of one (b, h); each
// wave owns 32 query rows.  Key/value tiles of 64 rows stream through LDS.
// Per key tile j, each wave computes
//
//   S^T = K_j Q^T            32x32x16 MFMA, fp16/bf16 in, fp32 out
//   online softmax update    running max m, running sum l, O rescale
//   O^T += V_j^T P^T         32x32x16 MFMA, P taken from the S^T registers
//
// which is the tiled online-softmax forward of "Self-Attention Kernel &
// Inference Engine from Scratch" (sections "Online Softmax Formulation" and
// "CUDA Kernel Structure"): two score blocks merge through the running max
// and normaliser, the output is rescaled by exp(m_old - m_new), and the
// division by the normaliser is deferred to the end.  The gfx950 design:
//
//  * Two wave groups ping-pong.  Waves 0-3 and 4-7 sit on the four SIMDs in
//    pairs.  Phases are separated by workgroup barriers; in every phase one
//    group issues matrix-core work (P.V of the previous tile and Q.K of the
//    current one) while the other runs the softmax of its current tile on
//    the vector ALU, so each SIMD keeps its matrix core and its VALU busy at
//    the same time.
//  * S^T (keys as MFMA rows, queries as columns) keeps one query's scores in
//    one lane: a row max or sum is in-lane work plus one exchange with the
//    lane 32 away (v_permlane32_swap).
//  * The S^T accumulator layout (lane = query + 32*g, register r = key
//    8*(r/4) + 4*g + r%4) is used as the B operand of the P.V MFMA as it
//    is.  V is stored transposed in LDS with keys permuted inside each group
//    of 16 so that lane group g reads its 8 keys with one 128-bit load.
//  * K is stored row-major with 16-byte chunks XOR-swizzled by row, so the
//    128-bit fragment reads of 8 or 16 consecutive rows hit distinct banks.
//  * Q stays in VGPRs.  Global loads of the tiles two phases ahead are in
//    flight while the current ones are used (register staging, then LDS).
//  * exp2 with scale*log2(e) folded into one FMA; the running max is only
//    raised when a tile's max exceeds it by more than 2^8 (lazy rescale):
//    the result is the same, probabilities stay below 256.
//  * Causal and key-padding masks: the loop stops at the last key tile any
//    row of the workgroup can see, each wave skips tiles wholly after its
//    rows, per-element masking only on tiles that straddle a boundary, and
//    key rows past the valid length are never read.  Causal grids launch
//    the heaviest query tiles first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQRows = 32;               // query rows per wave
constexpr int kBM = kWaves * kQRows;     // query rows per workgroup
constexpr int kBN = 64;                  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLazy = 8.0f;            // log2 of the largest unscaled probability

template <bool BF16>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values (round to nearest even), low half first.
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2 v = {lo, hi};
    if constexpr (BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x in the lane 32 away (lanes l and l^32 swap).
__device__ __forceinline__ float other_half(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // r[0] holds the low half of the wave twice, r[1] the high half twice.
    const uint32_t lo = r[0], hi = r[1];
    return __builtin_bit_cast(float, (__lane_id() < 32) ? hi : lo);
}

// Position of key k (0..kBN-1) inside a transposed V tile row.  Within each
// group of 16 keys the order is 0-3, 8-11, 4-7, 12-15, so that the 8 keys a
// lane group holds in the S^T accumulator (4g..4g+3 and 8+4g..8+4g+3) are
// contiguous.
__device__ __forceinline__ int vt_pos(int k) {
    const int kk = k & 15;
    return (k & ~15) | (kk & 3) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

__device__ __forceinline__ uint32_t half_of(u32x4 v, int e) {
    const uint32_t w = v[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// XOR swizzle of the 16-byte chunk index of K tile row `row` (D halves per
// row): rows that share a 256-byte bank window get distinct chunk offsets.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
    constexpr int RP = 128 / D;  // rows per 256 bytes
    constexpr int CPR = D / 8;   // chunks per row
    return (row / RP) % CPR;
}

template <int D, bool BF16, bool CAUSAL>
__device__ __forceinline__ void fwd_body(const FwdParams &p) {
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int KTILE = kBN * D;                // halves per K tile (no padding)
    constexpr int VSTR = kBN + 8;                 // LDS row stride of a V^T tile
    constexpr int VTILE = D * VSTR;
    constexpr int K_CHUNKS = kBN * CPR;
    constexpr int K_PER_T = (K_CHUNKS + kThreads - 1) / kThreads;
    constexpr int KG_RAW = kBN * D / (8 * kThreads);
    constexpr int KG = KG_RAW >= 1 ? KG_RAW : 1;  // keys per thread in a V tile load
    constexpr int V_ITEMS = (kBN / KG) * CPR;
    constexpr int KB = kBN / 32;                  // 32-key blocks per tile
    constexpr int DK = D / 16;                    // 16-deep k-steps of Q.K
    constexpr int DB = D / 32;                    // 32-wide column blocks of O
    static_assert(KG == 1 || KG == 2 || KG == 4, "V tile load shape");
    static_assert(V_ITEMS <= kThreads, "V tile load shape");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * KTILE + 2 * VTILE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int grp = wave >> 2;       // ping-pong group
    const int simd = wave & 3;
    const int rb = 2 * simd + grp;   // this wave's 32-row block in the tile

    const int BH = p.BH;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // heaviest tiles first
    const int N = (int)p.N;
    const int b = bh / p.H;
    const size_t base = (size_t)bh * (size_t)N * D;
    const uint16_t *__restrict__ Qp = p.Q + base;
    const uint16_t *__restrict__ Kp = p.K + base;
    const uint16_t *__restrict__ Vp = p.V + base;

    int Lk = N;
    if (p.key_len != nullptr) {
        const int v = p.key_len[b];
        Lk = v < 0 ? 0 : (v > N ? N : v);
    }
    const int q0 = qt * kBM;
    int kv_end = Lk;
    if (CAUSAL) kv_end = min(kv_end, q0 + kBM);
    const int n = (kv_end + kBN - 1) / kBN;       // key tiles of the workgroup
    const int qw0 = q0 + rb * kQRows;
    const int my_q = qw0 + l32;
    const bool q_ok = my_q < N;
    int n_w = n;                                  // key tiles this wave computes
    if (CAUSAL) n_w = (min(kv_end, qw0 + kQRows) + kBN - 1) / kBN;
    if (qw0 >= N) n_w = 0;

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    u32x4 qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qf[kk] = q_ok ? *reinterpret_cast<const u32x4 *>(Qp + (size_t)my_q * D + kk * 16 + g * 8)
                      : zero4;

    // ---- tile loads: global -> staging registers -> LDS
    u32x4 stg_k[K_PER_T];
    u32x4 stg_v[KG];
    const int v_ch = tid % CPR;
    const int v_grp = tid / CPR;

    auto gload = [&](int tk, int tv) {
#pragma unroll
        for (int i = 0; i < K_PER_T; ++i) {
            const int ci = tid + i * kThreads;
            const int key = tk * kBN + ci / CPR;
            const bool ok = ci < K_CHUNKS && tk < n && key < Lk;
            stg_k[i] = ok ? *reinterpret_cast<const u32x4 *>(Kp + (size_t)key * D + (ci % CPR) * 8)
                          : zero4;
        }
#pragma unroll
        for (int e = 0; e < KG; ++e) {
            const int key = tv * kBN + v_grp * KG + e;
            const bool ok = tid < V_ITEMS && tv < n && key < Lk;
            stg_v[e] = ok ? *reinterpret_cast<const u32x4 *>(Vp + (size_t)key * D + v_ch * 8)
                          : zero4;
        }
    };

    auto swrite = [&](int tk, int tv) {
        if (tk < n) {
            uint16_t *kt = lds + (tk & 1) * KTILE;
#pragma unroll
            for (int i = 0; i < K_PER_T; ++i) {
                const int ci = tid + i * kThreads;
                if (ci < K_CHUNKS) {
                    const int row = ci / CPR;
                    const int c = (ci % CPR) ^ k_swz<D>(row);
                    *reinterpret_cast<u32x4 *>(kt + row * D + c * 8) = stg_k[i];
                }
            }
        }
        if (tv >= 0 && tv < n && tid < V_ITEMS) {
            uint16_t *vt = lds + 2 * KTILE + (tv & 1) * VTILE;
            const int pos = vt_pos(v_grp * KG);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t *dst = vt + (v_ch * 8 + e) * VSTR + pos;
                if constexpr (KG == 4) {
                    u32x2 w = {half_of(stg_v[0], e) | (half_of(stg_v[1], e) << 16),
                               half_of(stg_v[2], e) | (half_of(stg_v[3], e) << 16)};
                    *reinterpret_cast<u32x2 *>(dst) = w;
                } else if constexpr (KG == 2) {
                    *reinterpret_cast<uint32_t *>(dst) =
                        half_of(stg_v[0], e) | (half_of(stg_v[1], e) << 16);
                } else {
                    *dst = (uint16_t)half_of(stg_v[0], e);
                }
            }
        }
    };

    // ---- per-wave state
    f32x16 oacc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    f32x16 s[KB];
    u32x4 pf[KB][2];
    float m_run = -INFINITY;  // running max of scale*log2(e)*score (possibly stale by < kLazy)
    float l_run = 0.f;        // this lane's share of the running normaliser
    const float c = p.scale_log2;

    auto qk = [&](int j) {
        const uint16_t *kt = lds + (j & 1) * KTILE;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
            const int row = kb * 32 + l32;
            const int swz = k_swz<D>(row);
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(
                    kt + row * D + (((2 * kk + g) ^ swz) * 8));
                s[kb] = mfma32<BF16>(a, qf[kk], s[kb]);
            }
        }
    };

    auto pv = [&](int j) {
        const uint16_t *vt = lds + 2 * KTILE + (j & 1) * VTILE;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int kc = 0; kc < 2 * KB; ++kc) {
                const u32x4 a = *reinterpret_cast<const u32x4 *>(
                    vt + (cb * 32 + l32) * VSTR + kc * 16 + g * 8);
                oacc[cb] = mfma32<BF16>(a, pf[kc >> 1][kc & 1], oacc[cb]);
            }
    };

    auto softmax = [&](int j) {
        const int j0 = j * kBN;
        const bool need_mask = (j0 + kBN > Lk) || (CAUSAL && j0 + kBN - 1 > qw0);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= my_q);
                    s[kb][r] = ok ? s[kb][r] : -INFINITY;
                }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[kb][r], s[kb][r + 1]));
        mx = fmaxf(mx, other_half(mx));
        const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
        const bool grow = m_tile > m_run + kLazy;
        if (__any(grow)) {
            const float m_new = grow ? m_tile : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.f;
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float s0 = s[kb][ch * 8 + 2 * w];
                    const float s1 = s[kb][ch * 8 + 2 * w + 1];
                    float p0 = fast_exp2(__builtin_fmaf(s0, c, -m_use));
                    float p1 = fast_exp2(__builtin_fmaf(s1, c, -m_use));
                    if (need_mask) {
                        p0 = (s0 == -INFINITY) ? 0.f : p0;
                        p1 = (s1 == -INFINITY) ? 0.f : p1;
                    }
                    lsum += p0 + p1;
                    pf[kb][ch][w] = pack2<BF16>(p0, p1);
                }
        l_run += lsum;
    };

    // ---- prologue: K tile 0 in LDS, K tile 1 and V tile 0 in flight
    if (n > 0) {
        gload(0, n);
        swrite(0, -1);
        gload(1, 0);
    }
    __syncthreads();

    // ---- phases: group g issues MFMA work for pair j in phase 2j+g and the
    // softmax of tile j in phase 2j+g+1.  K tile j is read in phases 2j and
    // 2j+1, V tile j in 2j+2 and 2j+3; both rings hold two tiles, refilled
    // in phase 2j+1 (K tile j+1, V tile j).
    const int n_phases = n > 0 ? 2 * n + 2 : 0;
    for (int ph = 0; ph < n_phases; ++ph) {
        const int t = ph - grp;
        if (t >= 0) {
            const int j = t >> 1;
            if ((t & 1) == 0) {
                __builtin_amdgcn_s_setprio(1);
                if (j >= 1 && j - 1 < n_w) pv(j - 1);
                if (j < n_w) qk(j);
                __builtin_amdgcn_s_setprio(0);
            } else if (j < n_w) {
                softmax(j);
            }
        }
        if (ph & 1) {
            const int j = ph >> 1;
            swrite(j + 1, j);
            gload(j + 2, j + 1);
        }
        __syncthreads();
    }

    // ---- epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l)
    const float l_tot = l_run + other_half(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (q_ok) {
        uint16_t *orow = p.O + base + (size_t)my_q * D;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u32x2 w = {pack2<BF16>(oacc[cb][4 * a] * inv, oacc[cb][4 * a + 1] * inv),
                           pack2<BF16>(oacc[cb][4 * a + 2] * inv, oacc[cb][4 * a + 3] * inv)};
                *reinterpret_cast<u32x2 *>(orow + cb * 32 + a * 8 + g * 4) = w;
            }
        if (p.LSE != nullptr && g == 0)
            p.LSE[(size_t)bh * N + my_q] =
                l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

}  // namespace
}  // namespace attn

#define ATTN_FWD_INSTANCE(NAME, D, BF16, CAUSAL)                                   \
    extern "C" __global__ __launch_bounds__(attn::kThreads)                       \
    void NAME(attn::FwdParams p) { attn::fwd_body<D, BF16, CAUSAL>(p); }

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

namespace attn {

namespace {
typedef void (*FwdKernel)(FwdParams);
struct FwdEntry {
    FwdKernel fn;
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
#undef ATTN_ENTRY

int d_index(int d) { return d == 32 ? 0 : (d == 64 ? 1 : 2); }
const FwdEntry &entry(bool bf16, int d, bool causal) {
    return kFwdTable[(d_index(d) * 2 + (bf16 ? 1 : 0)) * 2 + (causal ? 1 : 0)];
}
}  // namespace

int fwd_query_tile(int) { return kBM; }

const char *fwd_kernel_name(bool bf16, int d, bool causal) { return entry(bf16, d, causal).name; }

hipError_t launch_fwd(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    p.n_qtiles = (int)((p.N + kBM - 1) / kBM);
    const int64_t blocks = (int64_t)p.n_qtiles * p.BH;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(entry(bf16, d, causal).fn, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace attn
