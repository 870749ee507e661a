// Fused exact attention forward for gfx950 (CDNA4).
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
// Tile loads are issued by all waves at the start of their softmax phases
// when d >= this (the matrix-core phase is then the longer one), else by the
// four waves of group A right after their matrix-core work in even phases
// (the softmax phase is then the longer one).
constexpr int kSpreadLoadsMinD = 128;
// At d = 128 the exponentials of a tile are taken against the running max as
// it stands, before any row max is known; they are redone after a move only
// when a lane's sum of the tile's probabilities exceeds kExpFirstBound
// (below the fp16 maximum, so no probability can overflow).
constexpr float kExpFirstBound = 32768.0f;

// Scheduling pattern: N times (one MFMA, then R LDS reads).
template <int N, int R>
__device__ __forceinline__ void sched_mfma_reads() {
    if constexpr (N > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);  // DS read
        sched_mfma_reads<N - 1, R>();
    }
}

// LDS reads of MFMA step st of a phase with PVS P.V steps out of NST: 8
// transposing reads for a P.V step, 4 K fragment reads for a Q.K step.
template <int NST, int PVS>
constexpr int step_reads(int st) {
    return st >= NST ? 0 : (st < PVS ? 8 : 4);
}
template <int A, int B, int NST, int PVS>
constexpr int step_reads_upto() {
    int n = 0;
    for (int st = A; st < B; ++st) n += step_reads<NST, PVS>(st);
    return n;
}
// Steps ST .. NST-1: each step's 4 MFMAs with the reads of step
// ST + kFragAhead spread evenly between them.
template <int ST, int NST, int PVS>
__device__ __forceinline__ void sched_steps() {
    if constexpr (ST < NST) {
        sched_mfma_reads<4, step_reads<NST, PVS>(ST + kFragAhead) / 4>();
        sched_steps<ST + 1, NST, PVS>();
    }
}

template <int D, bool BF16, bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void fwd_body(const FwdParams &p) {
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = kBN * D;                 // halves per K or V tile
    constexpr int TILE_INSTR = kBN * CPR / 64;    // 1 KB load instructions per tile
    constexpr int KB = kBN / 32;                  // 32-key blocks per tile
    constexpr int DK = D / 16;                    // 16-deep k-steps of Q.K
    constexpr int DB = D / 32;                    // 32-wide column blocks of O

    __shared__ __attribute__((aligned(1024))) uint16_t sQ[kBM * D];
    __shared__ __attribute__((aligned(1024))) uint16_t sK[kRing][TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t sV[kRing][TILE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int grp = wave >> 2;       // ping-pong group
    const int simd = wave & 3;
    const int rb = 2 * simd + grp;   // this wave's 32-row block in the tile

    const int S = p.slices;
    // workgroup -> (key split, query tile, slice)
    const int per_split = p.n_qtiles * S;
    const int sp = SPLIT ? (int)blockIdx.x / per_split : 0;
    const int wg = (int)blockIdx.x - sp * per_split;
    const int sl = wg % S;
    int qt = wg / S;
    const int M = (int)p.M;                // query rows of the slice
    if (CAUSAL) qt = heavy_first_tile(qt, p.n_qtiles, p.Nq, M, kBM);
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

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    // The query tile goes to LDS once (same swizzled row-major layout as the
    // K tiles; rows past N read as zero); each wave re-reads its Q fragments
    // there instead of holding them in 8 x DK VGPRs.
    {
        constexpr int QI = kBM * CPR / 64;        // 1 KB load instructions
        static_assert(QI % kWaves == 0, "query tile load split");
        const int rows = min(kBM, M - q0);
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
    // Batch jb is K tile jb + kAhead and V tile jb + kAhead - 1 (2 TILE_INSTR
    // instructions); each of the NLD loader waves issues SHARE of them,
    // instruction t = wave + NLD i (K for t < TILE_INSTR, then V).  Issuing a
    // 1 KB load can stall the issuing wave while the vector memory front end
    // is busy, so the loads go where a wave has slack (see kSpreadLoads).
    constexpr bool kSpreadLoads = D >= kSpreadLoadsMinD;
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
        const i32x4 rk = tile_rsrc(Kp, jb + kAhead);
        const i32x4 rv = tile_rsrc(Vp, jb + kAhead - 1);
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

    auto frag_k = [&](const uint16_t *kt, int kb, int kk) -> u32x4 {
        return cdna4::frag_k<D>(kt, kb, kk, l32, g);
    };
    // Q fragment (B operand of S^T) for k-step kk: query row rb*32 + l32 of
    // the tile, dims 16 kk + 8 g .. +7 (same layout as a K fragment).
    auto frag_q = [&](int kk) -> u32x4 { return cdna4::frag_k<D>(sQ, rb, kk, l32, g); };
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
    u32x4 qreg[DK];
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
                s[0] = mfma32<BF16>(f[2 * i], qreg[k0 + i], s[0]);
                s[1] = mfma32<BF16>(f[2 * i + 1], qreg[k0 + i], s[1]);
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
        u32x4 f[NF][4];
#pragma unroll
        for (int st = FIRST; st < FIRST + kFragAhead; ++st)
            if (st < LAST) load_step(st, kt, vt, f[st % NF]);
#pragma unroll
        for (int st = FIRST; st < LAST; ++st) {
            if (st + kFragAhead < LAST) load_step(st + kFragAhead, kt, vt, f[(st + kFragAhead) % NF]);
            mfma_step(st, f[st % NF]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, step_reads_upto<FIRST, FIRST + kFragAhead, LAST, PV_STEPS>(), 0);
        sched_steps<FIRST, LAST, PV_STEPS>();
    };

    // Online softmax of tile j.  Masked scores become -inf; since c > 0 their
    // exp2 is exactly 0.  The row max and the row sum are trees (short
    // dependency chains); the normaliser sums the fp32 probabilities.
    static_assert(KB == 2, "the softmax arithmetic assumes 64-key tiles");
    auto row_max = [&]() -> float { return row_max64(s); };
    auto exps = [&](float neg_m) -> float { return exps64<BF16>(s, c, neg_m, pf); };
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
    // Batch j (K tile j+kAhead, V tile j+kAhead-1, both first read in phase
    // 2(j+kAhead)) is issued in phase 2j (group A, after its matrix-core
    // work) or, with kSpreadLoads, by group B in phase 2j and group A in
    // phase 2j+1 (at the start of their softmax of tile j).  It is waited for
    // at the end of phase 2(j+kAhead)-1, when each loader's share of the
    // kAhead-1 later batches may still be in flight.  Its slots were last
    // read in phase 2j-1.  Slot arrays are passed in statically so the
    // compiler can tell the in-flight loads from the tiles being read.
    auto phase = [&](int ph, const uint16_t *k_cur, const uint16_t *v_prev,
                     const uint16_t *k_next, const uint16_t *v_next) {
        if (kSpreadLoads && (ph & 1) != grp) issue_batch(ph >> 1, k_next, v_next);
        const int j = ph >> 1;
        const int t = ph - grp;
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
            } else if (jj < n_w) {
                softmax(jj);
            }
        }
        if (!kSpreadLoads && (ph & 1) == 0 && is_loader) issue_batch(ph >> 1, k_next, v_next);
        if (ph & 1) wait_tile_loads<(kAhead - 1) * SHARE>();
        barrier();
    };

    // prologue: K tile 0, then the batches of the virtual phases -2(kAhead-1)
    // .. -2 (K tiles 1 .. kAhead-1 and V tiles 0 .. kAhead-2); only K tile 0
    // (and the Q tile) must have arrived before the first phase.
    const int n_phases = n > 0 ? 2 * n + 2 : 0;
    if (n > 0 && is_loader) {
        const i32x4 rk = tile_rsrc(Kp, 0);
        const uint32_t kl = (uint32_t)(uintptr_t)(lds_void *)sK[0];
#pragma unroll
        for (int i = 0; i < SHARE; ++i)
            if (!ld_is_v[i]) dma16(rk, kl + lds_off[i], voff[i]);
#pragma unroll
        for (int jb = 1 - kAhead; jb < 0; ++jb)
            issue_batch(jb, sK[(jb + kAhead) % kRing], sV[(jb + kAhead - 1) % kRing]);
        wait_tile_loads<(kAhead - 1) * SHARE>();
    } else {
        wait_tile_loads<0>();
    }
    barrier();

#pragma unroll
    for (int kk = 0; kk < DK; ++kk) qreg[kk] = frag_q(kk);

    // Phases 2 kRing i + 2u and + 1 handle tile j = kRing i + u, whose K tile
    // sits in slot u; slots therefore depend only on the unrolled position.
    for (int ph = 0; ph < n_phases; ph += 2 * kRing) {
#pragma unroll
        for (int u = 0; u < 2 * kRing; ++u) {
            const int t = u >> 1;
            if (ph + u < n_phases)
                phase(ph + u, sK[t], sV[(t + kRing - 1) % kRing], sK[(t + kAhead) % kRing],
                      sV[(t + kAhead - 1) % kRing]);
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
            if (g == 0)
                p.part_LSE[row] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
        }
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

#define ATTN_FWD_INSTANCE(NAME, D, BF16, CAUSAL)                                   \
    extern "C" __global__ __launch_bounds__(attn::kThreads)                       \
    void NAME(attn::FwdParams p) { attn::fwd_body<D, BF16, CAUSAL, false>(p); }
#define ATTN_SPLIT_INSTANCE(NAME, D, BF16, CAUSAL)                                 \
    extern "C" __global__ __launch_bounds__(attn::kThreads)                       \
    void NAME(attn::FwdParams p) { attn::fwd_body<D, BF16, CAUSAL, true>(p); }

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

template <bool BF16>
__device__ __forceinline__ void merge_body(const MergeParams &p) {
    const int chunks = p.d / 4;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t row = t / chunks;
    const int c = (int)(t - row * chunks);
    if (row >= p.rows) return;
    float m = -INFINITY;
    for (int s = 0; s < p.splits; ++s) m = fmaxf(m, p.part_LSE[(int64_t)s * p.rows + row]);
    uint16_t *orow = p.O + row * p.d + 4 * c;
    if (m == -INFINITY) {
        *reinterpret_cast<u32x2 *>(orow) = (u32x2){0u, 0u};
        if (p.LSE != nullptr && c == 0) p.LSE[row] = -INFINITY;
        return;
    }
    float wsum = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.splits; ++s) {
        const float l = p.part_LSE[(int64_t)s * p.rows + row];
        if (l == -INFINITY) continue;  // an empty split (its O_s is 0)
        const float w = fast_exp2((l - m) * 1.44269504088896341f);
        wsum += w;
        acc += w * *reinterpret_cast<const f32x4 *>(p.part_O + ((int64_t)s * p.rows + row) * p.d + 4 * c);
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

hipError_t launch_fwd_fused(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    p.n_qtiles = (int)((p.M + kBM - 1) / kBM);
    const int64_t blocks = (int64_t)p.n_qtiles * p.slices;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(entry(bf16, d, causal).fn, dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
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

hipError_t launch_fwd_split(bool bf16, int d, bool causal, FwdParams p, hipStream_t s) {
    p.n_qtiles = (int)((p.M + kBM - 1) / kBM);
    const int64_t blocks = (int64_t)p.n_qtiles * p.slices * p.kv_splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL || p.kv_splits < 1 || p.split_tiles < 1)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(kSplitTable[table_index(bf16, d, causal)].fn, dim3((unsigned)blocks),
                       dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
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
