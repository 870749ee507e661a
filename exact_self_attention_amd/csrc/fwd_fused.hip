// Fused exact attention forward for gfx950 (CDNA4).
//
// One workgroup = 4 waves = one tile of 128 query rows of one (b, h); each
// wave owns 32 query rows.  Per key tile of 64 rows:
//
//   S^T = K_j Q_i^T          on 32x32x16 MFMA (fp16/bf16 in, fp32 out)
//   online softmax update    running max m, running sum l, rescale of O
//   O^T += V_j^T P^T         on 32x32x16 MFMA, P taken straight from the
//                            S^T accumulators (no LDS round trip)
//
// This is the tiled online-softmax forward of "Self-Attention Kernel &
// Inference Engine from Scratch" (sections "Online Softmax Formulation" and
// "CUDA Kernel Structure"): the running max/normaliser merge of two score
// blocks, the output rescaled by exp(m_old - m_new), and the division by the
// normaliser deferred to the end.  The design here is gfx950-specific:
//
//  * Computing S^T (keys as MFMA rows, queries as columns) puts one query's
//    scores in one lane: a row max / row sum is 16 in-lane values per 32-key
//    block plus one exchange with the lane 32 away.
//  * The S^T accumulator layout (lane = query + 32*g, register r = key
//    8*(r/4) + 4*g + r%4) is consumed as the B operand of the P.V MFMA
//    as-is; V is stored transposed in LDS with keys permuted inside each
//    group of 16 so that lane group g reads its 8 keys with one 128-bit LDS
//    load.  The sum over keys does not care about the order; masks use the
//    true key index.
//  * Q stays in VGPRs for the whole loop.  K and V tiles are double
//    buffered in LDS, and the next tile's global loads (128-bit, coalesced)
//    are in flight while the current tile is computed.
//  * Exponentials use exp2 with scale*log2(e) folded into one FMA.
//  * Causal and key-padding masks: the loop stops at the last key tile any
//    row of the workgroup can see; whole-tile skip per wave on the causal
//    diagonal; per-element masking only on tiles that straddle a boundary.
//    Key rows past the valid length are never read (loaded as zeros).
//  * Causal grids launch the heaviest query tiles first.

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

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kQRows = 32;               // query rows per wave
constexpr int kBM = kWaves * kQRows;     // query rows per workgroup
constexpr int kBN = 64;                  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;

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

template <int D, bool BF16, bool CAUSAL>
__device__ __forceinline__ void fwd_body(const FwdParams &p) {
    constexpr int KSTR = D + 8;          // LDS row stride of a K tile (halves)
    constexpr int VSTR = kBN + 8;        // LDS row stride of a V^T tile
    constexpr int KTILE = kBN * KSTR;
    constexpr int VTILE = D * VSTR;
    constexpr int STAGE = KTILE + VTILE;
    constexpr int CPR = D / 8;           // 16-byte chunks per row
    constexpr int K_RPP = kThreads / CPR;
    constexpr int K_PASSES = kBN / K_RPP;
    constexpr int KG = kBN * D / (8 * kThreads);  // keys per thread, V load
    constexpr int KB = kBN / 32;         // 32-key blocks per tile
    constexpr int DK = D / 16;           // 16-deep k-steps of Q.K
    constexpr int DB = D / 32;           // 32-wide column blocks of O
    static_assert(K_PASSES * K_RPP == kBN, "K tile load shape");
    static_assert(KG == 1 || KG == 2 || KG == 4, "V tile load shape");
    static_assert((kBN / KG) * CPR == kThreads, "V tile load shape");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

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
    const int n_tiles = (kv_end + kBN - 1) / kBN;
    const int qw0 = q0 + wave * kQRows;
    const int my_q = qw0 + l32;
    const bool q_ok = my_q < N;

    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    u32x4 qf[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qf[kk] = q_ok ? *reinterpret_cast<const u32x4 *>(Qp + (size_t)my_q * D + kk * 16 + g * 8)
                      : zero4;

    u32x4 kreg[K_PASSES];
    u32x4 vreg[KG];
    const int ld_ch = tid % CPR;
    const int ld_row = tid / CPR;

    auto gload = [&](int t) {
        const int j0 = t * kBN;
#pragma unroll
        for (int ps = 0; ps < K_PASSES; ++ps) {
            const int key = j0 + ps * K_RPP + ld_row;
            kreg[ps] = key < Lk
                ? *reinterpret_cast<const u32x4 *>(Kp + (size_t)key * D + ld_ch * 8) : zero4;
        }
#pragma unroll
        for (int e = 0; e < KG; ++e) {
            const int key = j0 + ld_row * KG + e;
            vreg[e] = key < Lk
                ? *reinterpret_cast<const u32x4 *>(Vp + (size_t)key * D + ld_ch * 8) : zero4;
        }
    };

    auto swrite = [&](int buf) {
        uint16_t *kt = lds + buf * STAGE;
        uint16_t *vt = kt + KTILE;
#pragma unroll
        for (int ps = 0; ps < K_PASSES; ++ps)
            *reinterpret_cast<u32x4 *>(kt + (ps * K_RPP + ld_row) * KSTR + ld_ch * 8) = kreg[ps];
        const int pos = vt_pos(ld_row * KG);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint16_t *dst = vt + (ld_ch * 8 + e) * VSTR + pos;
            if constexpr (KG == 4) {
                u32x2 w = {half_of(vreg[0], e) | (half_of(vreg[1], e) << 16),
                           half_of(vreg[2], e) | (half_of(vreg[3], e) << 16)};
                *reinterpret_cast<u32x2 *>(dst) = w;
            } else if constexpr (KG == 2) {
                *reinterpret_cast<uint32_t *>(dst) = half_of(vreg[0], e) | (half_of(vreg[1], e) << 16);
            } else {
                *dst = (uint16_t)half_of(vreg[0], e);
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float m_run = -INFINITY;  // running max of scale*log2(e)*score
    float l_run = 0.f;        // this lane's share of the running normaliser
    const float c = p.scale_log2;

    if (n_tiles > 0) {
        gload(0);
        swrite(0);
        __syncthreads();
    }
    for (int t = 0; t < n_tiles; ++t) {
        const int cur = t & 1;
        if (t + 1 < n_tiles) gload(t + 1);
        const int j0 = t * kBN;
        const bool wave_active = !CAUSAL || (j0 <= qw0 + kQRows - 1);
        if (wave_active) {
            const uint16_t *kt = lds + cur * STAGE;
            const uint16_t *vt = kt + KTILE;

            // S^T block kb: lane (query l32, group g), register r holds key
            // j0 + 32*kb + 8*(r/4) + 4*g + r%4.
            f32x16 s[KB];
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
                for (int kk = 0; kk < DK; ++kk) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(
                        kt + (kb * 32 + l32) * KSTR + kk * 16 + g * 8);
                    s[kb] = mfma32<BF16>(a, qf[kk], s[kb]);
                }
            }

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
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * c;
            const float m_new = fmaxf(m_run, m_tile);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run - m_use);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;

            // P = exp2(c*s - m), packed to 16 bits as the P.V B operand.
            u32x4 pf[KB][2];
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

            // O^T block cb += V^T[cb rows][keys] . P^T[keys][queries]
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                    for (int ch = 0; ch < 2; ++ch) {
                        const u32x4 a = *reinterpret_cast<const u32x4 *>(
                            vt + (cb * 32 + l32) * VSTR + (kb * 2 + ch) * 16 + g * 8);
                        oacc[cb] = mfma32<BF16>(a, pf[kb][ch], oacc[cb]);
                    }
        }
        if (t + 1 < n_tiles) swrite(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l).
    const float l_tot = l_run + __shfl_xor(l_run, 32);
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
