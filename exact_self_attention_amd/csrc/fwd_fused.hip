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
//  * K and V tiles go from device memory straight into LDS (buffer loads
//    with the LDS bit: no staging registers; rows past the valid key length
//    fall outside the buffer range and read as zero, so they are never read
//    from memory).  Both rings hold two tiles in separate LDS arrays; a tile
//    is fetched two phases before its first use.
//  * Both tiles are row-major with their 16-byte chunks XOR-swizzled by row
//    so that the 128-bit K fragment reads and the transposing V reads
//    (ds_read_b64_tr_b16) are free of bank conflicts.
//  * S^T (keys as MFMA rows, queries as columns) keeps one query's scores in
//    one lane: a row max or sum is in-lane work plus one exchange with the
//    lane 32 away (v_permlane32_swap).  The S^T accumulator layout (lane =
//    query + 32*g, register r = key 8*(r/4) + 4*g + r%4) is the B operand of
//    the P.V MFMA as it is; the transposing reads deliver V^T in the same key
//    order.
//  * Q is staged in LDS once per workgroup.  exp2 with scale*log2(e) folded
//    into one FMA.  Lazy running max: it moves only when a tile's max
//    exceeds it by more than 2^8, and then a little above that max, so the
//    output and normaliser are rarely rescaled; the result is the same and
//    probabilities stay inside the fp16 range.  At d = 128 the exponentials
//    are first taken against the running max as it stands, and the row max
//    is only computed when a lane's tile sum exceeds 2^15 (rare).
//  * Causal and key-padding masks: the loop stops at the last key tile any
//    row of the workgroup can see, each wave skips tiles wholly after its
//    rows, and per-element masking runs only on tiles that straddle a
//    boundary.  Causal grids launch the heaviest query tiles first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQRows = 32;               // query rows per wave
constexpr int kBM = kWaves * kQRows;     // query rows per workgroup
constexpr int kBN = 64;                  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;
// Lazy running max.  The running max only moves when a tile's max exceeds
// it by more than kLazy (log2 units), and then to kHeadroom above that
// tile's max, so that it rarely has to move again.  Probabilities stay below
// 2^kLazy, and after a move the largest is 2^-kHeadroom.
constexpr float kLazy = 8.0f;
constexpr float kHeadroom = 8.0f;
// At d = 128 the exponentials of a tile are taken against the running max as
// it stands, before any row max is known; they are redone after a move only
// when a lane's sum of the tile's probabilities exceeds kExpFirstBound
// (below the fp16 maximum, so no probability can overflow).
constexpr float kExpFirstBound = 32768.0f;
// Buffer resource word 3 for raw (untyped) 32-bit loads on gfx9-class parts.
constexpr int kBufferWord3 = 0x00020000;

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

// The values of x in lanes l % 32 and l % 32 + 32, for every lane l:
// v_permlane32_swap of x with itself leaves the low half of the wave in
// both halves of the first result and the high half in the second.
struct Halves {
    float lo, hi;
};
__device__ __forceinline__ Halves both_halves(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}

// XOR swizzle of the 16-byte chunk index within row `row` of a tile with D
// halves per row.  It makes (a) the 128-bit fragment reads of 16
// consecutive rows at one logical chunk and (b) the transposing 8-byte reads
// of 4 consecutive rows x 4 consecutive chunks land in distinct bank groups.
template <int D>
__device__ __forceinline__ int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    else return (row >> 2) & 3;
}

// Workgroup barrier without the memory-model waits of __syncthreads: the
// code orders its LDS traffic itself (fragment reads are consumed before the
// barrier; tile loads are waited for explicitly).
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Scheduling pattern: N times (one MFMA, then R LDS reads).
template <int N, int R>
__device__ __forceinline__ void sched_mfma_reads() {
    if constexpr (N > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS read
        sched_mfma_reads<N - 1, R>();
    }
}

__device__ __forceinline__ void wait_tile_loads() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (gfx9 layout) over nbytes bytes at base, stride 0.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t nbytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)nbytes);
    r[3] = kBufferWord3;
    return r;
}

// One wave-wide tile load: lane i copies the 16 bytes at byte offset voff of
// the buffer into LDS at lds_addr + 16 i; bytes past the buffer range read
// as zero.  Written as inline assembly so that the compiler does not add
// waits for these loads before unrelated LDS reads: the kernel waits for
// them itself (wait_tile_loads) before the barrier that publishes a tile.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}

template <int D, bool BF16, bool CAUSAL>
__device__ __forceinline__ void fwd_body(const FwdParams &p) {
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = kBN * D;                 // halves per K or V tile
    constexpr int TILE_INSTR = kBN * CPR / 64;    // 1 KB load instructions per tile
    constexpr int KB = kBN / 32;                  // 32-key blocks per tile
    constexpr int DK = D / 16;                    // 16-deep k-steps of Q.K
    constexpr int DB = D / 32;                    // 32-wide column blocks of O

    __shared__ __attribute__((aligned(1024))) uint16_t sQ[kBM * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sK0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sK1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV1[TILE];

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

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // The query tile goes to LDS once (same swizzled row-major layout as the
    // K tiles; rows past N read as zero); each wave re-reads its Q fragments
    // there instead of holding them in 8 x DK VGPRs.
    {
        constexpr int QI = kBM * CPR / 64;        // 1 KB load instructions
        static_assert(QI % kWaves == 0, "query tile load split");
        const int rows = min(kBM, N - q0);
        const i32x4 rq = make_rsrc(Qp + (size_t)q0 * D, (uint32_t)(rows * D * 2));
        const uint32_t lds = (uint32_t)(uintptr_t)(lds_void *)sQ;
#pragma unroll
        for (int i = 0; i < QI / kWaves; ++i) {
            const int t = wave + kWaves * i;
            const int P = 64 * t + lane;
            const int row = P / CPR;
            const int c = (P % CPR) ^ swz<D>(row);
            dma16(rq, lds + (uint32_t)(wave_u + kWaves * i) * 1024u, (uint32_t)(row * D * 2 + c * 16));
        }
    }

    // ---- tile loads, device memory -> LDS.  Load instruction t of a tile
    // fills LDS bytes [1024 t, 1024 t + 1024); lane i writes 16 bytes at
    // 1024 t + 16 i, i.e. physical chunk P = 64 t + i = row * CPR + chunk'.
    // The lane therefore fetches logical chunk chunk' ^ swz(row).
    // The waves of group A issue the loads of a tile pair at the end of
    // their MFMA work in even phases (a load burst in front of the MFMAs
    // stalls them); instruction t = w + LW i comes from wave w < LW.
    constexpr int LW = 4 < TILE_INSTR ? 4 : TILE_INSTR;
    constexpr int DMA_HALF = TILE_INSTR / LW;     // loads per loader wave per tile
    constexpr int DMA_PER_PHASE = 2 * DMA_HALF;   // K tile + V tile
    static_assert(TILE_INSTR % LW == 0, "tile load split");
    const int loader = wave_u;
    const bool is_loader = loader < LW;
    uint32_t voff[DMA_HALF];
#pragma unroll
    for (int i = 0; i < DMA_HALF; ++i) {
        const int t = (is_loader ? loader : 0) + LW * i;
        const int P = 64 * t + lane;
        const int row = P / CPR;
        const int c = (P % CPR) ^ swz<D>(row);
        voff[i] = (uint32_t)(row * D * 2 + c * 16);
    }
    auto tile_rsrc = [&](const uint16_t *src, int j) -> i32x4 {
        const int j0 = j * kBN;
        const int rows = min(kBN, Lk - j0);
        return make_rsrc(src + (size_t)j0 * D, (uint32_t)(rows * D * 2));
    };
    // Load k (0 <= k < DMA_PER_PHASE) of this loader wave: K tile, then V.
    auto issue_load = [&](int k, bool ld_k, bool ld_v, const i32x4 &rk, const i32x4 &rv,
                          uint16_t *k_dst, uint16_t *v_dst) {
        const int i = k % DMA_HALF;
        const uint32_t t = (uint32_t)(loader + LW * i);
        if (k < DMA_HALF) {
            if (ld_k) dma16(rk, (uint32_t)(uintptr_t)(lds_void *)k_dst + t * 1024u, voff[i]);
        } else {
            if (ld_v) dma16(rv, (uint32_t)(uintptr_t)(lds_void *)v_dst + t * 1024u, voff[i]);
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
    float m_run = -INFINITY;  // running max of scale*log2(e)*score (may trail the true one)
    float l_run = 0.f;        // this lane's share of the running normaliser
    const float c = p.scale_log2;

    // K fragment (A operand of S^T) for 32-key block kb, k-step kk: key row
    // kb*32 + l32, dims 16 kk + 8 g .. +7, one 128-bit read.
    auto frag_k = [&](const uint16_t *kt, int kb, int kk) -> u32x4 {
        const int row = kb * 32 + l32;
        return *reinterpret_cast<const u32x4 *>(kt + row * D + (((2 * kk + g) ^ swz<D>(row)) * 8));
    };
    // Q fragment (B operand of S^T) for k-step kk: query row rb*32 + l32 of
    // the tile, dims 16 kk + 8 g .. +7.
    auto frag_q = [&](int kk) -> u32x4 {
        const int row = rb * 32 + l32;
        return *reinterpret_cast<const u32x4 *>(sQ + row * D + (((2 * kk + g) ^ swz<D>(row)) * 8));
    };
    // V^T fragment (A operand of P.V) for column block cb, 16-key chunk kc:
    // two transposing reads at rows 16 kc + 8 h + 4 g + (lane%16)/4, logical
    // chunk 4 cb + 2 ((lane/16)%2) + (lane%4)/2, 8-byte half lane%2; they
    // return V[16kc + 8h + 4g + t][32 cb + l32] for t = 0..3, the key order
    // of the P registers.
    auto frag_v = [&](const uint16_t *vt, int cb, int kc) -> u32x4 {
        i16x4 part[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 16 * kc + 8 * h + 4 * g + (lane & 15) / 4;
            const int chunk = (4 * cb + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) ^ swz<D>(row);
            part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4 *)(vt + row * D + chunk * 8 + (lane & 1) * 4));
        }
        const u32x2 lo = __builtin_bit_cast(u32x2, part[0]);
        const u32x2 hi = __builtin_bit_cast(u32x2, part[1]);
        return (u32x4){lo[0], lo[1], hi[0], hi[1]};
    };

    // MFMA work of one phase as a list of steps of up to 4 MFMAs: first the
    // P.V steps (one per 32-column block of O, over the 4 key chunks), then
    // the Q.K steps (per 32-key block, 4 k-steps each).  Fragments of step
    // s+1 are read from LDS before the MFMAs of step s are issued, so LDS
    // latency hides behind matrix-core work.
    // A Q.K step covers two k-steps kk for both 32-key blocks: 4 MFMAs,
    // 2 Q fragment reads shared by the two blocks, 4 K fragment reads.
    constexpr int QK_STEPS = DK / 2;
    constexpr int QK_PER = 4;                          // MFMAs per Q.K step
    constexpr int QK_READS = 6;
    constexpr int PV_STEPS = DB;
    auto load_step = [&](int st, const uint16_t *kt, const uint16_t *vt, bool do_pv, u32x4 *f) {
        if (st < PV_STEPS) {
            if (do_pv) {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) f[kc] = frag_v(vt, st, kc);
            }
        } else {
            const int k0 = 2 * (st - PV_STEPS);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                f[3 * i] = frag_q(k0 + i);
                f[3 * i + 1] = frag_k(kt, 0, k0 + i);
                f[3 * i + 2] = frag_k(kt, 1, k0 + i);
            }
        }
    };
    auto mfma_step = [&](int st, bool do_pv, const u32x4 *f) {
        if (st < PV_STEPS) {
            if (do_pv) {
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
                    oacc[st] = mfma32<BF16>(f[kc], pf[kc >> 1][kc & 1], oacc[st]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                s[0] = mfma32<BF16>(f[3 * i + 1], f[3 * i], s[0]);
                s[1] = mfma32<BF16>(f[3 * i + 2], f[3 * i], s[1]);
            }
        }
    };
    constexpr int NST = PV_STEPS + QK_STEPS;
    // One branch-free block (P.V part on or off at compile time); the
    // scheduling hints issue the reads of step s+1 between the MFMAs of
    // step s rather than in one batch after them.
    auto mfma_phase = [&](const uint16_t *kt, const uint16_t *vt, auto pv_tag) {
        constexpr bool DO_PV = decltype(pv_tag)::value;
        constexpr int FIRST = DO_PV ? 0 : PV_STEPS;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        u32x4 f[2][6];
        load_step(FIRST, kt, vt, DO_PV, f[FIRST & 1]);
#pragma unroll
        for (int st = FIRST; st < NST; ++st) {
            if (st + 1 < NST) load_step(st + 1, kt, vt, DO_PV, f[(st + 1) & 1]);
            mfma_step(st, DO_PV, f[st & 1]);
        }
        if constexpr (DO_PV) {
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
            sched_mfma_reads<4 * (PV_STEPS - 1), 2>();
            sched_mfma_reads<2, 2>();
            sched_mfma_reads<2, 1>();
        } else {
            __builtin_amdgcn_sched_group_barrier(0x100, QK_READS, 0);
        }
#pragma unroll
        for (int rep_ = 0; rep_ < QK_STEPS - 1; ++rep_) {
            sched_mfma_reads<2, 2>();
            sched_mfma_reads<2, 1>();
        }
        sched_mfma_reads<QK_PER, 0>();
    };

    auto max3 = [](float a, float b, float c3) -> float {
        float d;
        asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c3));
        return d;
    };
    // Online softmax of tile j.  Masked scores become -inf; since c > 0 their
    // exp2 is exactly 0.  The row max and the row sum are trees (short
    // dependency chains); the normaliser sums the fp32 probabilities.
    // Row max (over both lane halves) of the 32 scores a lane holds.
    auto row_max = [&]() -> float {
        static_assert(KB == 2, "the reductions below assume 32 scores per lane");
        float t1[11];
#pragma unroll
        for (int i = 0; i < 10; ++i)
            t1[i] = max3(s[(3 * i) / 16][(3 * i) % 16], s[(3 * i + 1) / 16][(3 * i + 1) % 16],
                         s[(3 * i + 2) / 16][(3 * i + 2) % 16]);
        t1[10] = fmaxf(s[1][14], s[1][15]);
        const float t2a = max3(t1[0], t1[1], t1[2]), t2b = max3(t1[3], t1[4], t1[5]);
        const float t2c = max3(t1[6], t1[7], t1[8]), t2d = fmaxf(t1[9], t1[10]);
        const float mx = max3(max3(t2a, t2b, t2c), t2d, t2d);
        const Halves mh = both_halves(mx);
        return fmaxf(mh.lo, mh.hi);
    };
    // P = exp2(c s + neg_m) packed to 16 bits into pf; returns this lane's
    // sum of the fp32 values (a tree, for short dependency chains).
    auto exps = [&](float neg_m) -> float {
        float pr[32];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const int i = kb * 16 + ch * 8 + 2 * w;
                    pr[i] = fast_exp2(__builtin_fmaf(s[kb][ch * 8 + 2 * w], c, neg_m));
                    pr[i + 1] = fast_exp2(__builtin_fmaf(s[kb][ch * 8 + 2 * w + 1], c, neg_m));
                    pf[kb][ch][w] = pack2<BF16>(pr[i], pr[i + 1]);
                }
#pragma unroll
        for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w; ++i) pr[i] += pr[i + w];
        return pr[0];
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
        float lsum = 0.f;
        bool max_first = true;
        if (D >= 128 && j > 0) {
            // exponentials first; a sum above the bound (or a row with no
            // running max yet) sends the whole wave to the max-first path
            lsum = exps(m_run == -INFINITY ? 0.f : -m_run);
            max_first = __any(!(lsum <= kExpFirstBound) || m_run == -INFINITY);
        }
        if (max_first) {
            const float m_tile = row_max() * c;  // -inf stays -inf (c > 0)
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
            lsum = exps(m_run == -INFINITY ? 0.f : -m_run);
        }
        l_run += lsum;
    };

    // One phase.  Group A (grp 0) issues the MFMA work of pair j in phase 2j
    // and the softmax of tile j in phase 2j+1; group B runs one phase later.
    // K tile j is read in phases 2j and 2j+1, V tile j in 2j+2 and 2j+3.
    // Tile loads for K j+1 and V j start at phase 2j and are waited for at
    // the end of phase 2j+1.  Slot arrays are passed in statically so the
    // compiler can tell the in-flight loads from the tiles being read.
    auto phase = [&](int ph, const uint16_t *k_cur, const uint16_t *v_prev,
                     uint16_t *k_next, uint16_t *v_cur) {
        const int j = ph >> 1;
        const int t = ph - grp;
        if (t >= 0) {
            const int jj = t >> 1;
            if ((t & 1) == 0) {
                const bool do_pv = jj >= 1 && jj - 1 < n_w;
                const bool do_qk = jj < n_w;
                __builtin_amdgcn_s_setprio(1);
                if (do_qk && do_pv) {
                    mfma_phase(k_cur, v_prev, std::true_type{});
                } else if (do_qk) {
                    mfma_phase(k_cur, v_prev, std::false_type{});
                } else if (do_pv) {
                    u32x4 f[6];
#pragma unroll
                    for (int st = 0; st < PV_STEPS; ++st) {
                        load_step(st, k_cur, v_prev, true, f);
                        mfma_step(st, true, f);
                    }
                }
                __builtin_amdgcn_s_setprio(0);
            } else if (jj < n_w) {
                softmax(jj);
            }
        }
        // tile loads of this phase: K tile j+1 and V tile j, by group A at the
        // end of even phases
        if ((ph & 1) == 0 && is_loader) {
            const bool ld_k = j + 1 < n;
            const bool ld_v = j < n;
            const i32x4 rk = tile_rsrc(Kp, ld_k ? j + 1 : 0);
            const i32x4 rv = tile_rsrc(Vp, ld_v ? j : 0);
#pragma unroll
            for (int k = 0; k < DMA_PER_PHASE; ++k) issue_load(k, ld_k, ld_v, rk, rv, k_next, v_cur);
        }
        if (ph & 1) wait_tile_loads();
        barrier();
    };

    // prologue: K tile 0
    if (n > 0) {
        const i32x4 rk = tile_rsrc(Kp, 0);
        if (is_loader) {
#pragma unroll
            for (int k = 0; k < DMA_HALF; ++k) issue_load(k, true, false, rk, rk, sK0, sV0);
        }
        wait_tile_loads();
    }
    barrier();

    // Phases 4i .. 4i+3 handle tiles j = 2i (slots 0) and j = 2i+1 (slots 1).
    // For group B the "current" tile of an odd phase 2j+1 is tile j as well,
    // so the slot arguments depend only on the phase.
    const int n_phases = n > 0 ? 2 * n + 2 : 0;
    for (int ph = 0; ph < n_phases; ph += 4) {
        phase(ph + 0, sK0, sV1, sK1, sV0);
        if (ph + 1 < n_phases) phase(ph + 1, sK0, sV1, sK1, sV0);
        if (ph + 2 < n_phases) phase(ph + 2, sK1, sV0, sK0, sV1);
        if (ph + 3 < n_phases) phase(ph + 3, sK1, sV0, sK0, sV1);
    }

    // ---- epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l)
    const Halves lh = both_halves(l_run);
    const float l_tot = lh.lo + lh.hi;
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
