#pragma once
// Fused exact attention forward for gfx950 (CDNA4): the streaming kernel's
// body, instantiated by fwd_fused.hip (plain and split-key) and
// fwd_masked.hip (with an additive mask).
//
// One workgroup = 8 waves = one tile of 256 query rows of one slice (b,
// key/value head: the rows of the query heads that share it, head after
// head); each wave owns 32 query rows.  Key/value tiles of 64 rows stream
// through LDS.
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
//    pairs.  In every phase one group issues matrix-core work (P.V of the
//    previous tile and Q.K of the current one) while the other runs the
//    softmax of its current tile on the vector ALU, so each SIMD keeps its
//    matrix core and its VALU busy at the same time.  A workgroup barrier
//    ends every second phase (once per key tile; at d = 128 without a mask,
//    once per two key tiles).
//  * K and V tiles go from device memory straight into LDS (buffer loads
//    with the LDS bit: no staging registers; rows past the valid key length
//    fall outside the buffer range and read as zero, so they are never read
//    from memory).  K and V each cycle through a ring of 3 LDS slots, one
//    array per slot, and a tile is fetched two tiles (four phases) before
//    its first use; 5 slots and four tiles ahead in the deep instances, 5
//    slots and three tiles ahead at d = 128 without a mask.
//  * Both tiles are row-major with their 16-byte chunks XOR-swizzled by row
//    so that the 128-bit K fragment reads and the transposing V reads
//    (ds_read_b64_tr_b16) are free of bank conflicts.
//  * S^T (keys as MFMA rows, queries as columns) keeps one query's scores in
//    one lane: a row max or sum is in-lane work plus one exchange with the
//    lane 32 away (v_permlane32_swap).  The S^T accumulator layout (lane =
//    query + 32*g, register r = key 8*(r/4) + 4*g + r%4) is the B operand of
//    the P.V MFMA as it is; the transposing reads deliver V^T in the same key
//    order.
//  * Q is staged in LDS once per workgroup and moved into each wave's VGPRs
//    (at d = 128 without a mask it is staged in ring slots still free in the
//    prologue; the masked d = 128 instances re-read it from LDS; the deep
//    instances load it straight into VGPRs).  exp2 with scale*log2(e) folded
//    into one FMA.  Lazy running max: it moves only when a tile's max
//    exceeds it by more than 2^8, and then a little above that max, so the
//    output and normaliser are rarely rescaled; the result is the same and
//    probabilities stay inside the fp16 range.  At d = 128 the exponentials
//    are first taken against the running max as it stands, and the row max
//    is only computed when a lane's tile sum exceeds 2^15 (rare).
//  * Causal and key-padding masks: the loop stops at the last key tile any
//    row of the workgroup can see, each wave skips tiles wholly after its
//    rows, and per-element masking runs only on tiles that straddle a
//    boundary.  Causal grids launch the heaviest query tiles first; a masked
//    launch whose mask all slices share groups its work by XCD
//    (xcd_blocked_tile) so that the mask rows are reused in each L2.
//  * The output leaves through LDS (each wave's 32 rows, in the tiles'
//    swizzled layout) as 16-byte stores of whole rows.  The deep instances,
//    which have no query staging area, store 8-byte pieces directly; the
//    split-key instances write fp32 partials.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "cdna4.h"
#include "kernels.h"

namespace attn {
namespace {

using namespace cdna4;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * kQRows;     // query rows per workgroup
// K and V tiles each cycle through kRing LDS slots; a tile is fetched
// kRing - 1 tiles ahead of its first use, so a load has 2 (kRing - 1) - 1
// phases to arrive.
constexpr int kRing = 3;
constexpr int kAhead = kRing - 1;
// Fragment reads run this many MFMA steps (of 4 MFMAs) ahead of their use.
constexpr int kFragAhead = 1;
// Tile loads are issued by all eight waves when d >= this, else by the four
// waves of group A, in both cases right after a wave's matrix-core work (with
// an additive mask: at the start of the softmax phase, before the mask
// loads).  Issuing a 1 KB load can hold a wave up while the vector memory
// unit works through the loads ahead of it; right after its matrix-core
// phase the wave would otherwise wait for its last products anyway.
constexpr int kSpreadLoadsMinD = 128;
// At d = 128 the exponentials of a tile are taken against the running max as
// it stands, before any row max is known; they are redone after a move only
// when a lane's sum of the tile's probabilities exceeds kExpFirstBound
// (below the fp16 maximum, so no probability can overflow).
constexpr float kExpFirstBound = 32768.0f;

// Scheduling pattern: N MFMAs, each followed by its share of R LDS reads
// (the earlier MFMAs take the remainder).
template <int N, int R>
__device__ __forceinline__ void sched_mfma_reads() {
    if constexpr (N > 0) {
        constexpr int here = (R + N - 1) / N;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if constexpr (here > 0) __builtin_amdgcn_sched_group_barrier(0x100, here, 0);  // DS read
        sched_mfma_reads<N - 1, R - here>();
    }
}

// LDS reads of MFMA step st of a phase with PVS P.V steps out of NST: 8
// transposing reads for a P.V step, QKR fragment reads for a Q.K step (4 K
// fragments, plus 2 Q fragments when Q is read from LDS).
template <int NST, int PVS, int QKR>
constexpr int step_reads(int st) {
    return st >= NST ? 0 : (st < PVS ? 8 : QKR);
}
template <int A, int B, int NST, int PVS, int QKR>
constexpr int step_reads_upto() {
    int n = 0;
    for (int st = A; st < B; ++st) n += step_reads<NST, PVS, QKR>(st);
    return n;
}
// Steps ST .. NST-1: each step's 4 MFMAs with the reads of step
// ST + kFragAhead spread between them.
template <int ST, int NST, int PVS, int QKR>
__device__ __forceinline__ void sched_steps() {
    if constexpr (ST < NST) {
        sched_mfma_reads<4, step_reads<NST, PVS, QKR>(ST + kFragAhead)>();
        sched_steps<ST + 1, NST, PVS, QKR>();
    }
}

// MASK: an fp32 additive mask is added to the scaled scores.  Its values for
// a tile are loaded into VGPRs (a lane's 32 values are 8 16-byte pieces of
// its query's row) in the softmax phase before the tile's own, right after
// that phase's tile loads, so the loads it must wait for are never newer
// than the mask.  With a mask every wave issues tile loads at the start of
// its softmax phase, and at d = 128 Q fragments are read from LDS instead of
// being held in VGPRs (the mask values take those registers).
// LDS for the query tile, allocated only by the instances that stage it.
template <int HALVES>
struct QStage {
    __device__ static uint16_t *get() {
        __shared__ __attribute__((aligned(1024))) uint16_t buf[HALVES];
        return buf;
    }
};
template <>
struct QStage<0> {
    __device__ static uint16_t *get() { return nullptr; }
};

// DEEP: for slices of at most one query tile (decode-like shapes, which
// stream K/V and are bound by device memory), Q goes from device memory
// straight to registers instead of through LDS, and the freed LDS deepens
// the K/V rings to 5 slots, so 4 tiles of loads are in flight instead of 2.
// Splits of query tile qt that have work when the keys are split into runs
// of p.split_tiles tiles: those that start before the end of the keys its
// rows see (all Nk keys, or under the causal mask up to the highest position
// among its rows), and at least one, so that every tile has a workgroup.
// fwd_split_workgroups computes the same counts on the host.
template <bool CAUSAL>
__device__ __forceinline__ int split_busy(const FwdParams &p, int qt) {
    int kv_end = (int)p.Nk;
    if (CAUSAL) {
        const int q0 = qt * kBM;
        int lo, hi;
        CausalRows{p.Nq, p.causal_off}.range(q0, min(q0 + kBM, (int)p.M) - 1, lo, hi);
        kv_end = max(0, min(kv_end, hi + 1));
    }
    const int n_all = (kv_end + kBN - 1) / kBN;
    return max(1, (n_all + p.split_tiles - 1) / p.split_tiles);
}

template <int D, bool BF16, bool CAUSAL, bool SPLIT, bool MASK, bool DEEP = false>
__device__ __forceinline__ void fwd_body(const FwdParams &p) {
    static_assert(!(DEEP && MASK), "the deep-ring instances have no mask");
    // PAIRED (d = 128 without a mask): a workgroup barrier every second key
    // tile instead of every tile (after key tile 0, so that the prologue
    // waits only for it, then after odd key tiles), with 5-slot rings and
    // tiles fetched three ahead (a batch then overwrites the
    // slots of tiles two and three back, which a barrier always separates
    // from it).  The query tile is staged in ring slots that the prologue
    // leaves free (K 3-4 and V 2-3) and is moved to VGPRs before the first
    // batch overwrites them.  Loop cycles per key tile fall by 1.4-2.8%; at
    // d = 64 the same measured 1.6% slower on peaky.
    constexpr bool PAIRED = !MASK && !DEEP && D == 128;
    constexpr bool Q_IN_RING = PAIRED;
    constexpr int RING = DEEP || PAIRED ? 5 : kRing;
    constexpr int AHEAD = PAIRED ? 3 : RING - 1;
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = kBN * D;                 // halves per K or V tile
    constexpr int TILE_INSTR = kBN * CPR / 64;    // 1 KB load instructions per tile
    constexpr int KB = kBN / 32;                  // 32-key blocks per tile
    constexpr int DK = D / 16;                    // 16-deep k-steps of Q.K
    constexpr int DB = D / 32;                    // 32-wide column blocks of O

    __shared__ __attribute__((aligned(1024))) uint16_t sK[RING][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[RING][TILE];
    uint16_t *const sQ = QStage<DEEP || Q_IN_RING ? 0 : kBM * D>::get();
    // the two 128-row halves of the staged query tile
    static_assert(!Q_IN_RING || 2 * TILE == (kBM / 2) * D, "a query half fills two ring slots");
    auto q_half = [&](int h) -> uint16_t * {
        if constexpr (Q_IN_RING)
            return h == 0 ? &sK[3][0] : &sV[2][0];
        else
            return h == 0 ? sQ : sQ + (kBM / 2) * D;
    };

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int grp = wave >> 2;       // ping-pong group
    const int simd = wave & 3;
    const int rb = 2 * simd + grp;   // this wave's 32-row block in the tile

    const int S = p.slices;
    const int M = (int)p.M;                // query rows of the slice
    // workgroup -> (query tile, slice, key split)
    int sl, qt, sp = 0;
    int sp_busy = 1;                       // splits of this tile with work
    if constexpr (SPLIT) {
        // The grid lists the query tiles in launch order, each with its
        // splits that have work (split_busy) for every slice, the splits of
        // one slice adjacent.  Under the causal mask the counts differ, and
        // the tile is found from their running total, 64 tiles per step.
        const int i = (int)blockIdx.x;
        int k_sel, pre;
        if constexpr (!CAUSAL) {
            sp_busy = p.kv_splits;
            k_sel = i / (S * sp_busy);
            pre = k_sel * sp_busy;
        } else {
            k_sel = -1;
            pre = 0;
            int base = 0;
            for (int k0 = 0; k0 < p.n_qtiles; k0 += 64) {
                const int k = k0 + lane;
                const int bk = k < p.n_qtiles
                                   ? split_busy<CAUSAL>(p, heavy_first_tile(k, p.n_qtiles, p.Nq, M, kBM))
                                   : 0;
                int incl = bk;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int t = __shfl_up(incl, off, 64);
                    if (lane >= off) incl += t;
                }
                const unsigned long long hit = __ballot(k < p.n_qtiles && (base + incl) * S > i);
                if (hit != 0ull) {
                    // (one value per wave: kept in scalar registers)
                    const int L = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
                    sp_busy = __builtin_amdgcn_readfirstlane(__shfl(bk, L, 64));
                    pre = base + __builtin_amdgcn_readfirstlane(__shfl(incl, L, 64)) - sp_busy;
                    k_sel = k0 + L;
                    break;
                }
                base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
            }
            if (k_sel < 0) return;  // not in the grid's list (the same for every wave)
        }
        const int r = i - pre * S;
        sl = r / sp_busy;
        sp = r - sl * sp_busy;
        qt = CAUSAL ? heavy_first_tile(k_sel, p.n_qtiles, p.Nq, M, kBM) : k_sel;
    } else {
        const int wg = (int)blockIdx.x;
        sl = wg % S;
        qt = wg / S;
        if (MASK && p.xcd_slices > 0)
            xcd_blocked_tile(wg, p.n_qtiles, S, p.xcd_slices, CAUSAL, p.Nq, M, kBM, qt, sl);
        else if (CAUSAL)
            qt = heavy_first_tile(qt, p.n_qtiles, p.Nq, M, kBM);
    }
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
    const int q0 = qt * kBM;
    const int qw0 = q0 + rb * kQRows;
    const int my_q = qw0 + l32;
    const bool q_ok = my_q < M;
    // causal: the workgroup needs keys up to the highest position of its
    // rows, a wave up to the highest of its own; tiles past the lowest
    // position of a wave's rows need per-element masking
    const CausalRows cr{p.Nq, p.causal_off};
    int kv_end = Lk;
    int wave_lo = 0, wave_hi = 0;
    if (CAUSAL) {
        int lo, hi;
        cr.range(q0, min(q0 + kBM, M) - 1, lo, hi);
        kv_end = max(0, min(kv_end, hi + 1));
        if (qw0 < M) cr.range(qw0, min(qw0 + kQRows, M) - 1, wave_lo, wave_hi);
    }
    const int my_pos = CAUSAL ? cr.pos(my_q) : 0;
    // key tiles j_begin .. j_begin + n - 1 (all visible tiles unless split)
    const int n_all = (kv_end + kBN - 1) / kBN;
    const int j_begin = SPLIT ? sp * p.split_tiles : 0;
    const int n = SPLIT ? max(0, min(n_all - j_begin, p.split_tiles)) : n_all;
    int n_w = n;                                  // key tiles this wave computes
    if (CAUSAL) n_w = max(0, min(n, (max(0, min(kv_end, wave_hi + 1)) + kBN - 1) / kBN - j_begin));
    if (qw0 >= M) n_w = 0;
    n_w = __builtin_amdgcn_readfirstlane(n_w);  // one value per wave
    if (SPLIT && n == 0) {
        // no row of the tile sees a key of this split: its partial rows get
        // only LSE = -inf, which the merge reads as "no output", and so do
        // those of the splits after the tile's last busy one, which have no
        // workgroup (n is the same for the whole workgroup, so every wave
        // leaves here)
        const int r = q0 + tid;
        if (tid < kBM && r < M)
            for (int s2 = sp; s2 < (sp == sp_busy - 1 ? p.kv_splits : sp + 1); ++s2)
                p.part_LSE[((size_t)s2 * S + sl) * (size_t)M + r] = -INFINITY;
        return;
    }


    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // The query tile goes to LDS once (same swizzled row-major layout as the
    // K tiles; rows past N read as zero); each wave re-reads its Q fragments
    // there instead of holding them in 8 x DK VGPRs.
    if constexpr (!DEEP) {
        constexpr int QI = kBM * CPR / 64;        // 1 KB load instructions
        static_assert(QI % kWaves == 0, "query tile load split");
        const int rows = min(kBM, M - q0);
        const i32x4 rq = make_rsrc(Qp + (size_t)q0 * D, (uint32_t)(rows * D * 2));
#pragma unroll
        for (int i = 0; i < QI / kWaves; ++i) {
            const int t = wave + kWaves * i;
            const int P = 64 * t + lane;
            const int row = P / CPR;
            const int c = (P % CPR) ^ swz<D>(row);
            // instruction T fills bytes [1024 T, 1024 T + 1024) of the tile:
            // half T / (QI / 2), the swizzle of a row unchanged by the split
            const int T = wave_u + kWaves * i;
            const uint32_t lds = (uint32_t)(uintptr_t)(lds_void *)q_half(T / (QI / 2));
            dma16(rq, lds + (uint32_t)(T % (QI / 2)) * 1024u, (uint32_t)(row * D * 2 + c * 16));
        }
    }

    // ---- tile loads, device memory -> LDS.  Load instruction t of a tile
    // fills LDS bytes [1024 t, 1024 t + 1024); lane i writes 16 bytes at
    // 1024 t + 16 i, i.e. physical chunk P = 64 t + i = row * CPR + chunk'.
    // The lane therefore fetches logical chunk chunk' ^ swz(row).
    // Batch jb is K tile jb + AHEAD and V tile jb + AHEAD - 1 (2 TILE_INSTR
    // instructions); each of the NLD loader waves issues SHARE of them,
    // instruction t = wave + NLD i (K for t < TILE_INSTR, then V).  Issuing a
    // 1 KB load can stall the issuing wave while the vector memory front end
    // is busy, so the loads go where a wave has slack (see kSpreadLoads).
    constexpr bool kSpreadLoads = D >= kSpreadLoadsMinD || MASK;
    constexpr int BATCH = 2 * TILE_INSTR;
    constexpr int NLD = kSpreadLoads ? kWaves : kWaves / 2;
    constexpr int SHARE = BATCH / NLD;             // loads per loader per batch
    static_assert(BATCH % NLD == 0, "tile load split");
    const bool is_loader = wave_u < NLD;
    uint32_t voff[SHARE];
    uint32_t lds_off[SHARE];
    bool ld_is_v[SHARE];
#pragma unroll
    for (int i = 0; i < SHARE; ++i) {
        const int t = (is_loader ? wave_u : 0) + NLD * i;
        const int tt = t % TILE_INSTR;
        ld_is_v[i] = t >= TILE_INSTR;
        lds_off[i] = (uint32_t)tt * 1024u;
        const int P = 64 * tt + lane;
        const int row = P / CPR;
        const int c = (P % CPR) ^ swz<D>(row);
        voff[i] = (uint32_t)(row * D * 2 + c * 16);
    }
    // Buffer over key tile j, clipped at the last valid key; a tile at or
    // past the workgroup's last one gets an empty range, so its loads write
    // zeros to LDS without touching memory (and every batch has the same
    // number of instructions, which the waits below count on).
    auto tile_rsrc = [&](const uint16_t *src, int j) -> i32x4 {
        const int j0 = (j + j_begin) * kBN;
        const int rows = j < n ? min(kBN, Lk - j0) : 0;
        return make_rsrc(src + (size_t)(j < n ? j0 : 0) * D, (uint32_t)(rows * D * 2));
    };
    auto issue_batch = [&](int jb, const uint16_t *k_dst, const uint16_t *v_dst) {
        const i32x4 rk = tile_rsrc(Kp, jb + AHEAD);
        const i32x4 rv = tile_rsrc(Vp, jb + AHEAD - 1);
        const uint32_t kl = (uint32_t)(uintptr_t)(lds_void *)k_dst;
        const uint32_t vl = (uint32_t)(uintptr_t)(lds_void *)v_dst;
#pragma unroll
        for (int i = 0; i < SHARE; ++i) {
            if (ld_is_v[i])
                dma16(rv, vl + lds_off[i], voff[i]);
            else
                dma16(rk, kl + lds_off[i], voff[i]);
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
    // with a mask the scores become scale*s + mask (one FMA each) before the
    // softmax, which then takes them with the factor log2(e)
    const float c_sm = MASK ? kLog2e : c;
    const float c_mask = c * kLn2;  // the scale itself

    // Additive mask: this lane's query row of it.  Row r of the slice is
    // query r mod Nq of head kvh * (M / Nq) + r / Nq; the buffer spans this
    // batch's mask, and the key offset of a tile goes in the scalar offset.
    const float *mask_b = MASK ? p.mask + (size_t)b * (size_t)p.mask_sb : nullptr;
    int mask_voff = 0;
    if constexpr (MASK) {
        const int r = q_ok ? my_q : 0;
        const int64_t head = (int64_t)(sl % p.Hkv) * (M / p.Nq) + r / p.Nq;
        mask_voff = (int)((head * p.mask_sh + (int64_t)(r % p.Nq) * Nk + 4 * g) * 4);
    }
    f32x4 mreg[MASK ? KB : 1][4];
    // The mask values of key tile j (tile j of the wave's range, read as
    // zero-length past the wave's last tile so that every wave issues the
    // same loads), lane-ordered like the S^T registers: piece q of block kb
    // holds keys kb*32 + 8q + 4g .. +3.
    auto issue_mask = [&](int j_any) {
        // j is the same in every lane (the resource must be scalar)
        const int j = __builtin_amdgcn_readfirstlane(j_any);
        const bool live = j < n_w;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)mask_b, (short)0, live ? (int)p.mask_bytes : 0, kBufferWord3);
        const int soff = live ? (j + j_begin) * kBN * 4 : 0;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                mreg[kb][q] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, mask_voff + (kb * 32 + 8 * q) * 4,
                                                                 soff, 0));
    };
    // scores of the tile in s -> log2(e) * (scale * score + mask)
    auto apply_mask = [&]() {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kb][r] = __builtin_fmaf(s[kb][r], c_mask, mreg[kb][r >> 2][r & 3]);
        // keep these before the tile loads that follow (the compiler's wait
        // for the mask must not cover them)
        asm volatile("" : "+v"(s[0]), "+v"(s[1]));
    };

    auto frag_k = [&](const uint16_t *kt, int kb, int kk) -> u32x4 {
        return cdna4::frag_k<D>(kt, kb, kk, l32, g);
    };
    // Q fragment (B operand of S^T) for k-step kk: query row rb*32 + l32 of
    // the tile, dims 16 kk + 8 g .. +7 (same layout as a K fragment).
    auto frag_q = [&](int kk) -> u32x4 { return cdna4::frag_k<D>(q_half(rb >> 2), rb & 3, kk, l32, g); };
    auto frag_v = [&](const uint16_t *vt, int cb, int kc) -> u32x4 {
        return cdna4::frag_v<D>(vt, cb, kc, lane, g);
    };

    // MFMA work of one phase as a list of steps of 4 MFMAs each: first the
    // P.V steps (one per 32-column block of O, over the 4 key chunks: 8
    // transposing reads), then the Q.K steps (two k-steps for both 32-key
    // blocks: 4 K fragment reads; the Q fragments sit in VGPRs).  The
    // fragments of step s + kFragAhead are read while the MFMAs of step s
    // issue, from a ring of kFragAhead + 1 fragment sets, so each read has
    // kFragAhead steps of matrix-core work to arrive in.
    constexpr int QK_STEPS = DK / 2;
    constexpr int PV_STEPS = DB;
    constexpr int NST = PV_STEPS + QK_STEPS;
    constexpr bool kQInRegs = !(MASK && D >= 128);
    constexpr int QKR = kQInRegs ? 4 : 6;
    u32x4 qreg[kQInRegs ? DK : 1];
    auto load_step = [&](int st, const uint16_t *kt, const uint16_t *vt, u32x4 *f) {
        if (st < PV_STEPS) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) f[kc] = frag_v(vt, st, kc);
        } else {
            const int k0 = 2 * (st - PV_STEPS);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                f[2 * i] = frag_k(kt, 0, k0 + i);
                f[2 * i + 1] = frag_k(kt, 1, k0 + i);
                if constexpr (!kQInRegs) f[4 + i] = frag_q(k0 + i);
            }
        }
    };
    auto mfma_step = [&](int st, const u32x4 *f) {
        if (st < PV_STEPS) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                oacc[st] = mfma32<BF16>(f[kc], pf[kc >> 1][kc & 1], oacc[st]);
        } else {
            const int k0 = 2 * (st - PV_STEPS);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const u32x4 qf = kQInRegs ? qreg[k0 + i] : f[4 + i];
                s[0] = mfma32<BF16>(f[2 * i], qf, s[0]);
                s[1] = mfma32<BF16>(f[2 * i + 1], qf, s[1]);
            }
        }
    };
    // One branch-free block (P.V and Q.K parts on or off at compile time);
    // the scheduling hints place the reads of step s + kFragAhead between
    // the MFMAs of step s.
    auto mfma_phase = [&](const uint16_t *kt, const uint16_t *vt, auto pv_tag, auto qk_tag) {
        constexpr bool DO_PV = decltype(pv_tag)::value;
        constexpr bool DO_QK = decltype(qk_tag)::value;
        constexpr int FIRST = DO_PV ? 0 : PV_STEPS;
        constexpr int LAST = DO_QK ? NST : PV_STEPS;
        constexpr int NF = kFragAhead + 1;
        if constexpr (DO_QK) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        }
        u32x4 f[NF][kQInRegs ? 4 : 6];
#pragma unroll
        for (int st = FIRST; st < FIRST + kFragAhead; ++st)
            if (st < LAST) load_step(st, kt, vt, f[st % NF]);
#pragma unroll
        for (int st = FIRST; st < LAST; ++st) {
            if (st + kFragAhead < LAST) load_step(st + kFragAhead, kt, vt, f[(st + kFragAhead) % NF]);
            mfma_step(st, f[st % NF]);
        }
        __builtin_amdgcn_sched_group_barrier(
            0x100, step_reads_upto<FIRST, FIRST + kFragAhead, LAST, PV_STEPS, QKR>(), 0);
        sched_steps<FIRST, LAST, PV_STEPS, QKR>();
    };

    // Online softmax of tile j.  Masked scores become -inf; since c > 0 their
    // exp2 is exactly 0.  The row max and the row sum are trees (short
    // dependency chains); the normaliser sums the fp32 probabilities.
    static_assert(KB == 2, "the softmax arithmetic assumes 64-key tiles");
    auto row_max = [&]() -> float { return row_max64(s); };
    // (at d = 64 the vector ALU bounds the loop, and fp16 sums take the
    // packed probabilities two at a time with v_dot2: exps_blocks)
    auto exps = [&](float neg_m) -> float {
        if constexpr (D == 64)
            return exps_blocks<BF16, 2>(s, c_sm, neg_m, pf);
        else
            return exps64<BF16>(s, c_sm, neg_m, pf);
    };
    auto softmax = [&](int j) {
        const int j0 = (j + j_begin) * kBN;
        const bool need_mask = (j0 + kBN > Lk) || (CAUSAL && j0 + kBN - 1 > wave_lo);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + kb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
                    const bool ok = key < Lk && (!CAUSAL || key <= my_pos);
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
            const float m_tile = row_max() * c_sm;  // -inf stays -inf (c_sm > 0)
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
    // Batch j (K tile j+AHEAD, V tile j+AHEAD-1, both first read in phase
    // 2(j+AHEAD)) is issued in phase 2j by group A after its matrix-core
    // work and, with kSpreadLoads, in phase 2j+1 by group B after its own
    // (with a mask: by group B in phase 2j and group A in phase 2j+1, at the
    // start of their softmax of tile j).  It is waited for
    // at the end of phase 2(j+AHEAD)-1, when each loader's share of the
    // AHEAD-1 later batches may still be in flight.  Its slots were last
    // read in phase 2j-1.  Slot arrays are passed in statically so the
    // compiler can tell the in-flight loads from the tiles being read.
    auto phase = [&](int ph, const uint16_t *k_cur, const uint16_t *v_prev,
                     const uint16_t *k_next, const uint16_t *v_next) {
        const int j = ph >> 1;
        const int t = ph - grp;
        // A wave's softmax phases are those with t odd (t = -1: group B's
        // first phase, which only loads).  With a mask: apply tile t/2's
        // mask, issue the tile loads, then load tile t/2 + 1's mask.
        if (MASK && (t & 1) && t >= 1 && (t >> 1) < n_w) apply_mask();
        constexpr bool kLoadsAfterMfma = !MASK;
        if (kSpreadLoads && !kLoadsAfterMfma && (ph & 1) != grp) issue_batch(ph >> 1, k_next, v_next);
        if (MASK && (t & 1)) issue_mask((t >> 1) + 1);
        if (t >= 0) {
            const int jj = t >> 1;
            if ((t & 1) == 0) {
                const bool do_pv = jj >= 1 && jj - 1 < n_w;
                const bool do_qk = jj < n_w;
                __builtin_amdgcn_s_setprio(1);
                if (do_qk && do_pv) {
                    mfma_phase(k_cur, v_prev, std::true_type{}, std::true_type{});
                } else if (do_qk) {
                    mfma_phase(k_cur, v_prev, std::false_type{}, std::true_type{});
                } else if (do_pv) {
                    mfma_phase(k_cur, v_prev, std::true_type{}, std::false_type{});
                }
                __builtin_amdgcn_s_setprio(0);
                if (kSpreadLoads && kLoadsAfterMfma) issue_batch(ph >> 1, k_next, v_next);
            } else if (jj < n_w) {
                softmax(jj);
            }
        }
        if (!kSpreadLoads && (ph & 1) == 0 && is_loader) issue_batch(ph >> 1, k_next, v_next);
        // Tiles are published and ring slots released only at the end of
        // odd phases (the newest batch, and with a mask the 8 mask loads
        // issued after it, may stay in flight), so that is the only place a
        // workgroup barrier is needed.  Between two of them each wave runs
        // its matrix-core phase and its softmax phase back to back: the two
        // waves of a SIMD start them in opposite order, so they still
        // overlap, and the waves are not forced into step twice per tile.
        if constexpr (PAIRED) {
            // after key tile 0 (its batch and the next may still be in
            // flight), then after every odd key tile (only the newest batch)
            if (ph == 1) {
                wait_tile_loads<(AHEAD - 1) * SHARE>();
                barrier();
            } else if ((ph & 3) == 3) {
                wait_tile_loads<(AHEAD - 2) * SHARE>();
                barrier();
            }
        } else if (ph & 1) {
            wait_tile_loads<(AHEAD - 1) * SHARE + (MASK ? 8 : 0)>();
            barrier();
        }
    };

    if constexpr (DEEP) {
        // this wave's Q fragments straight from device memory (rows past M
        // are zero), waited for here, before any tile load is issued (the
        // compiler's wait for them then covers no tile load)
#pragma unroll
        for (int kk = 0; kk < DK; ++kk)
            qreg[kk] = my_q < M ? *reinterpret_cast<const u32x4 *>(Qp + (size_t)my_q * D + (2 * kk + g) * 8)
                                : (u32x4){0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) asm volatile("" ::"v"(qreg[kk]));
    }

    // prologue: K tile 0, then the batches of the virtual phases -2(AHEAD-1)
    // .. -2 (K tiles 1 .. AHEAD-1 and V tiles 0 .. AHEAD-2); only K tile 0
    // (and the Q tile) must have arrived before the first phase.
    const int n_phases = n > 0 ? 2 * n + 2 : 0;
    if (n > 0 && is_loader) {
        const i32x4 rk = tile_rsrc(Kp, 0);
        const uint32_t kl = (uint32_t)(uintptr_t)(lds_void *)sK[0];
#pragma unroll
        for (int i = 0; i < SHARE; ++i)
            if (!ld_is_v[i]) dma16(rk, kl + lds_off[i], voff[i]);
#pragma unroll
        for (int jb = 1 - AHEAD; jb < 0; ++jb)
            issue_batch(jb, sK[(jb + AHEAD) % RING], sV[(jb + AHEAD - 1) % RING]);
        wait_tile_loads<(AHEAD - 1) * SHARE>();
    } else {
        wait_tile_loads<0>();
    }
    barrier();
    // group A's first softmax phase comes before any phase of its own that
    // loads a mask (group B loads tile 0's in its first phase)
    if (MASK && grp == 0) issue_mask(0);

    if constexpr (kQInRegs && !DEEP) {
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) qreg[kk] = frag_q(kk);
    }
    if constexpr (Q_IN_RING) {
        // every wave holds its Q fragments before the first batch of the
        // loop overwrites their slots
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) asm volatile("" ::"v"(qreg[kk]));
        barrier();
    }

    // Phases 2 RING i + 2u and + 1 handle tile j = RING i + u, whose K tile
    // sits in slot u; slots therefore depend only on the unrolled position.
    for (int ph = 0; ph < n_phases; ph += 2 * RING) {
#pragma unroll
        for (int u = 0; u < 2 * RING; ++u) {
            const int t = u >> 1;
            if (ph + u < n_phases)
                phase(ph + u, sK[t], sV[(t + RING - 1) % RING], sK[(t + AHEAD) % RING],
                      sV[(t + AHEAD - 1) % RING]);
        }
    }
    // loads of tiles past the last one (empty ranges) may still be in flight
    wait_tile_loads<0>();

    // ---- epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l)
    const Halves lh = both_halves(l_run);
    const float l_tot = lh.lo + lh.hi;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (SPLIT) {
        // this split's normalised partial output and its LSE, in fp32; a row
        // with no visible key in the split gets only LSE = -inf (the merge
        // then ignores its output)
        if (q_ok) {
            const size_t row = ((size_t)sp * S + sl) * (size_t)M + my_q;
            float *orow = p.part_O + row * D;
            if (l_tot > 0.f)
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 w = {oacc[cb][4 * a] * inv, oacc[cb][4 * a + 1] * inv,
                               oacc[cb][4 * a + 2] * inv, oacc[cb][4 * a + 3] * inv};
                    *reinterpret_cast<f32x4 *>(orow + cb * 32 + a * 8 + g * 4) = w;
                }
            if (g == 0) {
                p.part_LSE[row] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
                // the splits after the tile's last busy one have no workgroup
                if (sp == sp_busy - 1)
                    for (int s2 = sp + 1; s2 < p.kv_splits; ++s2)
                        p.part_LSE[((size_t)s2 * S + sl) * (size_t)M + my_q] = -INFINITY;
            }
        }
    } else if constexpr (!DEEP) {
        // The wave's 32 output rows go through its own 32 rows of the query
        // staging area (it is their only reader and has read them for the
        // last time), in the swizzled layout of the K/V tiles, and leave as
        // 16-byte stores of whole rows: one instruction writes 4 rows.
        // (in ring slots at d = 128: every wave must be past its last tile)
        if constexpr (Q_IN_RING) barrier();
        char *stage = reinterpret_cast<char *>(q_half(rb >> 2)) + (size_t)(rb & 3) * kQRows * D * 2;
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                u32x2 w = {pack2<BF16>(oacc[cb][4 * a] * inv, oacc[cb][4 * a + 1] * inv),
                           pack2<BF16>(oacc[cb][4 * a + 2] * inv, oacc[cb][4 * a + 3] * inv)};
                const int chunk = (cb * 4 + a) ^ swz<D>(l32);
                *reinterpret_cast<u32x2 *>(stage + l32 * D * 2 + chunk * 16 + g * 8) = w;
            }
#pragma unroll
        for (int it = 0; it < kQRows * CPR / 64; ++it) {
            const int c = it * 64 + lane;
            const int row = c / CPR, ch = c % CPR;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stage + row * D * 2 + (ch ^ swz<D>(row)) * 16);
            if (qw0 + row < M)
                *reinterpret_cast<u32x4 *>(p.O + q_base + (size_t)(qw0 + row) * D + ch * 8) = v;
        }
        if (q_ok && p.LSE != nullptr && g == 0)
            p.LSE[(size_t)sl * M + my_q] =
                l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
    } else if (q_ok) {
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

