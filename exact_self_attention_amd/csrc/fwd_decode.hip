// Fused exact attention forward for slices of at most 32 query rows
// (decode: one or a few new queries per head against a long key/value
// history), gfx950.  Such a slice streams every key once and is bound by
// device memory, but in the streaming kernel a single wave would then carry
// all the matrix-core and softmax work of each tile.  Here the 4 waves of a
// workgroup take the same query rows and split the workgroup's key range
// between them: wave w takes 32-key tiles w, w + 4, ... .  Each wave
//
//   * loads its tiles into its own 2-slot LDS ring with direct-to-LDS buffer
//     loads (the next tile is in flight while the current one is used; no
//     workgroup barrier: only the wave that loads a slot reads it),
//   * runs S^T = K_j Q^T, the online softmax update (running max, running
//     normaliser, rescaled output: "Self-Attention Kernel & Inference Engine
//     from Scratch", section "Online Softmax Formulation") and
//     O^T += V_j^T P^T on its tiles,
//
// and the four partial results are merged once at the end through LDS with
// the same identity applied to whole blocks.  The result is O and LSE, or
// with key splits the normalised fp32 partial and LSE of this workgroup's
// range for the merge kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "cdna4.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kDWaves = 4;            // waves per workgroup, one per SIMD
constexpr int kDBN = 32;              // keys per tile
constexpr int kDMaxRows = kQRows;     // query rows per slice (one wave's worth)

template <int D, bool BF16, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void decode_body(const FwdParams &p) {
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = kDBN * D;                // halves per K or V tile
    constexpr int TILE_INSTR = kDBN * CPR / 64;   // 1 KB load instructions per tile
    constexpr int DK = D / 16;
    constexpr int DB = D / 32;
    static_assert(kDMaxRows * D * 4 <= 2 * TILE * 2, "merge scratch fits a wave's K slots");

    __shared__ __attribute__((aligned(1024))) uint16_t sK[kDWaves][2][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[kDWaves][2][TILE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // workgroup -> (key split, slice); all its waves take the slice's rows
    const int S = p.slices;
    const int sp = SPLIT ? (int)blockIdx.x / S : 0;
    const int sl = (int)blockIdx.x - sp * S;
    const int M = (int)p.M;
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
    const int my_q = l32;
    const bool q_ok = my_q < M;
    const CausalRows cr{p.Nq, p.causal_off};
    int kv_end = Lk;
    int rows_lo = 0;
    if (CAUSAL) {
        int hi;
        cr.range(0, M - 1, rows_lo, hi);
        kv_end = max(0, min(kv_end, hi + 1));
    }
    const int my_pos = CAUSAL ? cr.pos(my_q) : 0;
    // this workgroup's key range (whole 64-key units of the split), in
    // 32-key tiles; wave w takes tiles t_lo + w, t_lo + w + 4, ...
    const int k_lo = SPLIT ? sp * p.split_tiles * 64 : 0;
    const int k_hi = SPLIT ? min(kv_end, k_lo + p.split_tiles * 64) : kv_end;
    const int t_lo = k_lo / kDBN;
    const int t_hi = k_hi > k_lo ? (k_hi + kDBN - 1) / kDBN : t_lo;
    const int n_mine = __builtin_amdgcn_readfirstlane(
        t_hi - t_lo > wave_u ? (t_hi - t_lo - wave_u + kDWaves - 1) / kDWaves : 0);

    // Q fragments (B operand of S^T) straight to registers; rows past M are 0
    u32x4 qreg[DK];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
        qreg[kk] = q_ok ? *reinterpret_cast<const u32x4 *>(Qp + (size_t)my_q * D + (2 * kk + g) * 8)
                        : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) asm volatile("" ::"v"(qreg[kk]));  // waited for before any tile load

    // tile loads of this wave's i-th tile into its slot i & 1; load
    // instruction t fills LDS bytes [1024 t, 1024 t + 1024) of the tile, lane
    // i physical chunk 64 t + i (the swizzled layout of the other kernels)
    auto issue_tile = [&](int i) {
        const int tt = t_lo + wave_u + kDWaves * i;
        const int rows = min(kDBN, Lk - tt * kDBN);
        const i32x4 rk = make_rsrc(Kp + (size_t)tt * kDBN * D, (uint32_t)(rows * D * 2));
        const i32x4 rv = make_rsrc(Vp + (size_t)tt * kDBN * D, (uint32_t)(rows * D * 2));
        const uint32_t kl = (uint32_t)(uintptr_t)(lds_void *)sK[wave_u][i & 1];
        const uint32_t vl = (uint32_t)(uintptr_t)(lds_void *)sV[wave_u][i & 1];
#pragma unroll
        for (int t = 0; t < TILE_INSTR; ++t) {
            const int P = 64 * t + lane;
            const int row = P / CPR;
            const int c = (P % CPR) ^ swz<D>(row);
            const uint32_t voff = (uint32_t)(row * D * 2 + c * 16);
            dma16(rk, kl + (uint32_t)t * 1024u, voff);
            dma16(rv, vl + (uint32_t)t * 1024u, voff);
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float m_run = -INFINITY;  // running max of scale*log2(e)*score (may trail the true one)
    float l_run = 0.f;        // this lane's share of the running normaliser
    const float c = p.scale_log2;

    if (n_mine > 0) issue_tile(0);
    for (int i = 0; i < n_mine; ++i) {
        if (i + 1 < n_mine) {
            issue_tile(i + 1);
            wait_tile_loads<2 * TILE_INSTR>();  // tile i has landed, tile i + 1 may be in flight
        } else {
            wait_tile_loads<0>();
        }
        const uint16_t *kt = sK[wave_u][i & 1];
        const uint16_t *vt = sV[wave_u][i & 1];
        const int j0 = (t_lo + wave_u + kDWaves * i) * kDBN;
        // S^T = K_j Q^T
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) s = mfma32<BF16>(frag_k<D>(kt, 0, kk, l32, g), qreg[kk], s);
        // masks on tiles that straddle the key length or a causal limit
        if ((j0 + kDBN > Lk) || (CAUSAL && j0 + kDBN - 1 > rows_lo)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j0 + (r >> 2) * 8 + g * 4 + (r & 3);
                const bool ok = key < Lk && (!CAUSAL || key <= my_pos);
                s[r] = ok ? s[r] : -INFINITY;
            }
        }
        // online softmax with a lazy running max (moves only when the
        // tile's max exceeds it by more than kLazy, then to kHeadroom above)
        const float m_tile = row_max32(s) * c;  // -inf stays -inf (c > 0)
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
        u32x4 pf[2];
        l_run += exps32<BF16>(s, c, m_run == -INFINITY ? 0.f : -m_run, pf);
        // O^T += V_j^T P^T
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int kc = 0; kc < 2; ++kc)
                oacc[cb] = mfma32<BF16>(frag_v<D>(vt, cb, kc, lane, g), pf[kc], oacc[cb]);
    }
    wait_tile_loads<0>();

    // ---- merge of the four waves' partial results.  Each wave writes its
    // unnormalised output (fp32 [32 rows][D]) over its own K slots and its
    // running max and normaliser per row into its V slots.  The 16-byte
    // chunks of a row are XOR-swizzled by the row: a row is 512 B at d = 128,
    // a multiple of the LDS bank width, so unswizzled the 32 rows one
    // instruction touches would all fall on the same banks.
    auto part_at = [&](const uint16_t *slot, int col) -> float * {
        return const_cast<float *>(reinterpret_cast<const float *>(slot)) + l32 * D +
               (((col >> 2) ^ (l32 & (D / 4 - 1))) << 2);
    };
    const Halves lh = both_halves(l_run);
    const float l_mine = lh.lo + lh.hi;
    barrier();  // every wave is done reading its tiles
    float *ml_part = reinterpret_cast<float *>(&sV[wave_u][0][0]);
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *reinterpret_cast<f32x4 *>(part_at(&sK[wave_u][0][0], cb * 32 + a * 8 + g * 4)) =
                (f32x4){oacc[cb][4 * a], oacc[cb][4 * a + 1], oacc[cb][4 * a + 2], oacc[cb][4 * a + 3]};
    if (g == 0) {
        ml_part[l32] = m_run;
        ml_part[32 + l32] = l_mine;
    }
    barrier();
    if (wave_u != 0) return;

    float m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDWaves; ++w)
        m_all = fmaxf(m_all, reinterpret_cast<const float *>(&sV[w][0][0])[l32]);
    float wgt[kDWaves];
    float l_tot = 0.f;
#pragma unroll
    for (int w = 0; w < kDWaves; ++w) {
        const float *ml = reinterpret_cast<const float *>(&sV[w][0][0]);
        const float mw = ml[l32];
        wgt[w] = mw == -INFINITY ? 0.f : fast_exp2(mw - m_all);
        l_tot += wgt[w] * ml[32 + l32];
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_all + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    if (!q_ok) return;
    if (SPLIT) {
        const size_t row = ((size_t)sp * S + sl) * (size_t)M + my_q;
        if (l_tot > 0.f) {
            float *orow = p.part_O + row * D;
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int col = cb * 32 + a * 8 + g * 4;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int w = 0; w < kDWaves; ++w)
                        acc += wgt[w] * *reinterpret_cast<const f32x4 *>(part_at(&sK[w][0][0], col));
                    *reinterpret_cast<f32x4 *>(orow + col) = acc * inv;
                }
        }
        if (g == 0) p.part_LSE[row] = lse;
    } else {
        uint16_t *orow = p.O + q_base + (size_t)my_q * D;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int col = cb * 32 + a * 8 + g * 4;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < kDWaves; ++w)
                    acc += wgt[w] * *reinterpret_cast<const f32x4 *>(part_at(&sK[w][0][0], col));
                acc *= inv;
                *reinterpret_cast<u32x2 *>(orow + col) =
                    (u32x2){pack2<BF16>(acc[0], acc[1]), pack2<BF16>(acc[2], acc[3])};
            }
        if (p.LSE != nullptr && g == 0) p.LSE[(size_t)sl * M + my_q] = lse;
    }
}

}  // namespace
}  // namespace attn

#define ATTN_DECODE_INSTANCE(NAME, D, BF16, CAUSAL, SPLIT)                         \
    extern "C" __global__ __launch_bounds__(attn::kDWaves * 64)                   \
    void NAME(attn::FwdParams p) { attn::decode_body<D, BF16, CAUSAL, SPLIT>(p); }

ATTN_DECODE_INSTANCE(attn_fwd_decode_d32_f16_full, 32, false, false, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d32_f16_causal, 32, false, true, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d32_bf16_full, 32, true, false, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d32_bf16_causal, 32, true, true, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d64_f16_full, 64, false, false, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d64_f16_causal, 64, false, true, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d64_bf16_full, 64, true, false, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d64_bf16_causal, 64, true, true, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d128_f16_full, 128, false, false, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d128_f16_causal, 128, false, true, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d128_bf16_full, 128, true, false, false)
ATTN_DECODE_INSTANCE(attn_fwd_decode_d128_bf16_causal, 128, true, true, false)

ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d32_f16_full, 32, false, false, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d32_f16_causal, 32, false, true, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d32_bf16_full, 32, true, false, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d32_bf16_causal, 32, true, true, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d64_f16_full, 64, false, false, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d64_f16_causal, 64, false, true, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d64_bf16_full, 64, true, false, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d64_bf16_causal, 64, true, true, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d128_f16_full, 128, false, false, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d128_f16_causal, 128, false, true, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d128_bf16_full, 128, true, false, true)
ATTN_DECODE_INSTANCE(attn_fwd_split_decode_d128_bf16_causal, 128, true, true, true)

namespace attn {

namespace {
struct DecodeEntry {
    FwdKernelFn fn;
    const char *name;
};
#define ATTN_ENTRY(NAME) {NAME, #NAME}
// index: (((split * 3 + d_index) * 2) + bf16) * 2 + causal,
// d_index: 32 -> 0, 64 -> 1, 128 -> 2
const DecodeEntry kDecodeTable[24] = {
    ATTN_ENTRY(attn_fwd_decode_d32_f16_full),         ATTN_ENTRY(attn_fwd_decode_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_decode_d32_bf16_full),        ATTN_ENTRY(attn_fwd_decode_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_decode_d64_f16_full),         ATTN_ENTRY(attn_fwd_decode_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_decode_d64_bf16_full),        ATTN_ENTRY(attn_fwd_decode_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_decode_d128_f16_full),        ATTN_ENTRY(attn_fwd_decode_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_decode_d128_bf16_full),       ATTN_ENTRY(attn_fwd_decode_d128_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_decode_d32_f16_full),   ATTN_ENTRY(attn_fwd_split_decode_d32_f16_causal),
    ATTN_ENTRY(attn_fwd_split_decode_d32_bf16_full),  ATTN_ENTRY(attn_fwd_split_decode_d32_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_decode_d64_f16_full),   ATTN_ENTRY(attn_fwd_split_decode_d64_f16_causal),
    ATTN_ENTRY(attn_fwd_split_decode_d64_bf16_full),  ATTN_ENTRY(attn_fwd_split_decode_d64_bf16_causal),
    ATTN_ENTRY(attn_fwd_split_decode_d128_f16_full),  ATTN_ENTRY(attn_fwd_split_decode_d128_f16_causal),
    ATTN_ENTRY(attn_fwd_split_decode_d128_bf16_full), ATTN_ENTRY(attn_fwd_split_decode_d128_bf16_causal),
};
#undef ATTN_ENTRY

int decode_index(bool bf16, int d, bool causal, bool split) {
    const int di = d == 32 ? 0 : (d == 64 ? 1 : 2);
    return (((split ? 3 : 0) + di) * 2 + (bf16 ? 1 : 0)) * 2 + (causal ? 1 : 0);
}
}  // namespace

bool fwd_uses_decode(const FwdParams &p) { return p.mask == nullptr && p.M <= kDMaxRows; }

const char *fwd_decode_kernel_name(bool bf16, int d, bool causal, bool split) {
    return kDecodeTable[decode_index(bf16, d, causal, split)].name;
}

hipError_t launch_fwd_decode(bool bf16, int d, bool causal, bool split, FwdParams p, hipStream_t s) {
    p.n_qtiles = 1;
    const int64_t blocks = (int64_t)p.slices * (split ? p.kv_splits : 1);
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL || p.M > kDMaxRows) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kDecodeTable[decode_index(bf16, d, causal, split)].fn, dim3((unsigned)blocks),
                       dim3(kDWaves * 64), 0, s, p);
    return hipGetLastError();
}

int fwd_decode_resident_workgroups(bool bf16, int d, bool causal) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices][12];
    const int index = decode_index(bf16, d, causal, true);
    const int slot = index - 12;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int v = cache[dev][slot].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(kDecodeTable[index].fn), kDWaves * 64, 0) != hipSuccess)
        return 0;
    const int r = cus * (per_cu > 0 ? per_cu : 1);
    if (dev < kMaxDevices) cache[dev][slot].store(r, std::memory_order_relaxed);
    return r;
}

}  // namespace attn
