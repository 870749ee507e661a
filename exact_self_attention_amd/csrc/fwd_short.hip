// Fused exact attention forward for short sequences on gfx950 (CDNA4).
//
// For short key ranges (Nk <= 256 at d <= 64, Nk <= 128 at d = 128) the
// streaming kernel's deep pipeline and wave specialisation only add latency:
// a slice has at most four 64-key tiles.  Here a workgroup of 4 waves owns
// 128 query rows of one slice (b, key/value head; the rows of the query
// heads that share it, head after head):
//
//   1. each wave loads the Q fragments of its query rows straight into
//      VGPRs, and the workgroup loads the first key tiles (K and V) into an
//      LDS ring (as many slots as short_ring_of(d)) with direct buffer loads
//      (rows past the valid key length read as zero and are not fetched);
//   2. for every key tile its 32 rows can see, each wave runs
//      S^T = K_j Q^T on the matrix cores, the online softmax update of
//      "Self-Attention Kernel & Inference Engine from Scratch" (section
//      "Online Softmax Formulation": running max, running normaliser,
//      rescaled output), and O^T += V_j^T P^T.  Only Q and tile 0 are
//      waited for before the first tile; a barrier before each later tile
//      publishes it, so the work on the first tiles overlaps the arrival of
//      the rest.  When a slice has more tiles than slots, that barrier also
//      frees the slot of the previous tile, and the tile RING - 1 ahead is
//      loaded into it;
//   3. O = O_acc / l goes through LDS to coalesced stores, with LSE.
//
// The softmax arithmetic (exponentials, row max, row sum) bounds this kernel
// at d = 32, so it is trimmed: after the first tile the exponentials come
// first and the row max only when they could overflow, fp16 row sums add
// the packed probabilities two at a time (exps_blocks), a last tile whose
// second 32 keys no row of the wave sees is computed as one 32-key block,
// and the per-element mask compares a constant per register with one
// per-lane limit.
//
// A workgroup needs 32 KB of LDS at d = 32, 48 KB at d = 64 and 64 KB at
// d = 128, and 4, 3 or 2 workgroups are resident per compute unit.  (Five
// of 32 KB do not fit on gfx950, although the occupancy query reports 5; at
// 31 KB five do.)  Masking follows the long-sequence kernel: causal and
// key-length limits end the tile loop early and per-element masks run only
// on tiles that straddle a limit; a masked score is -inf, whose exp2 is
// exactly 0.

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
// LDS slots for K and V tiles: all four tiles at d = 32 (32 KB), a ring of
// three at d = 64 (48 KB instead of 64: 3 workgroups per compute unit
// instead of 2, measured 18% faster at 256 keys), both tiles at d = 128
// (64 KB).  At d = 32 a ring of 2 or 3 (5 workgroups per compute unit)
// measured no faster: the softmax arithmetic, not the latency, bounds it.
constexpr int short_ring_of(int d) { return d == 64 ? 3 : short_max_keys_of(d) / kBN; }
// Waves per SIMD the register allocation must allow: as many workgroups as
// LDS holds per compute unit.
constexpr int short_waves_per_simd(int d) { return d == 32 ? 4 : (d == 64 ? 3 : 2); }
// After the first tile the exponentials are taken against the running max
// before any row max is known; they are redone after a max update only when
// a lane's sum of the tile's probabilities exceeds this bound (below the
// fp16 maximum, so no probability can overflow) or the lane has no running
// max yet.
constexpr float kShortExpFirstBound = 32768.0f;

// LDS slot I of the K (IS_V false) or V ring: one array per slot, so that the
// compiler, which sees the tile loads, can tell a slot still being filled
// from one being read.
template <int D, int I, bool IS_V>
struct ShortSlot {
    __device__ static uint16_t *get() {
        __shared__ __attribute__((aligned(1024))) uint16_t buf[kBN * D];
        return buf;
    }
};

template <int D, bool BF16, bool CAUSAL>
__device__ __forceinline__ void short_body(const FwdParams &p) {
    constexpr int CPR = D / 8;                    // 16-byte chunks per row
    constexpr int TILE = kBN * D;                 // halves per K or V tile
    constexpr int TILE_INSTR = kBN * CPR / 64;    // 1 KB load instructions per tile
    constexpr int NT = short_max_keys_of(D) / kBN;  // key tiles of a slice at most
    constexpr int RING = short_ring_of(D);        // LDS slots per K and V
    static_assert(RING >= 2 && RING <= NT, "ring depth");
    constexpr int SW = kSWaves;
    constexpr int SHARE = 2 * TILE_INSTR / SW;    // K and V loads per wave per tile
    constexpr int KB = kBN / 32;
    constexpr int DK = D / 16;
    constexpr int DB = D / 32;
    static_assert((2 * TILE_INSTR) % SW == 0, "tile load split");
    static_assert(KB == 2, "the softmax arithmetic assumes 64-key tiles");

    static_assert(RING <= 4, "ring slots");
    uint16_t *const sK[4] = {ShortSlot<D, 0, false>::get(), ShortSlot<D, 1, false>::get(),
                             RING > 2 ? ShortSlot<D, 2, false>::get() : nullptr,
                             RING > 3 ? ShortSlot<D, 3, false>::get() : nullptr};
    uint16_t *const sV[4] = {ShortSlot<D, 0, true>::get(), ShortSlot<D, 1, true>::get(),
                             RING > 2 ? ShortSlot<D, 2, true>::get() : nullptr,
                             RING > 3 ? ShortSlot<D, 3, true>::get() : nullptr};

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
    static_assert(TILE_INSTR % SW == 0, "a load's tile (K or V) is the same in every wave");
    // Every wave issues the same loads whatever the key length: a tile at or
    // past the last visible one gets an empty range (its loads write zeros
    // and read no memory), so the number of loads in flight at each point is
    // known at compile time, to the explicit waits and to the compiler's.
    auto issue_tile = [&](int t) {
        const int rows = t < n ? min(kBN, Lk - t * kBN) : 0;
        const size_t off = t < n ? (size_t)t * kBN * D : 0;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Kp + off), (short)0, rows * D * 2, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(Vp + off), (short)0, rows * D * 2, kBufferWord3);
#pragma unroll
        for (int i = 0; i < SHARE; ++i) {
            const int u = wave_u + SW * i;
            const bool is_v = SW * i >= TILE_INSTR;
            const int ti = is_v ? u - TILE_INSTR : u;
            const int P = 64 * ti + lane;
            const int row = P / CPR;
            const int ch = (P % CPR) ^ swz<D>(row);
            const uint32_t voff = (uint32_t)(row * D * 2 + ch * 16);
            uint16_t *slot = is_v ? sV[t % RING] : sK[t % RING];
            dma16_tracked(is_v ? rv : rk, (lds_void *)(slot + ti * 512), voff);
        }
    };
    // Q first, then the first RING tiles.  Only tile 0 (and Q) must have
    // arrived before the first tile's work; each later tile is waited for
    // when its turn comes, so the work on the first tiles overlaps the
    // arrival of the rest.
#pragma unroll
    for (int t = 0; t < RING; ++t) issue_tile(t);
    wait_tile_loads<(RING - 1) * SHARE>();
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) asm volatile("" ::"v"(qreg[kk]));
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
    // keys that some row of this wave sees, and that this lane's row sees
    const int wave_lim = CAUSAL ? min(kv_end, wave_hi + 1) : kv_end;
    const int row_lim = CAUSAL ? min(Lk, my_pos + 1) : Lk;

#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (j >= n) break;
        if (j > 0) {
            // Tile j is in once the loads issued after its own are all that
            // may still be in flight: those of tiles j + 1 .. j + RING - 2
            // (below NT).  With fewer slots than tiles, tile j + RING - 1
            // then goes to the slot of tile j - 1, which every wave is past
            // after this barrier.
            wait_tile_loads_upto<SHARE>((min(j + RING - 2, NT - 1) - j) * SHARE);
            barrier();
            if constexpr (NT > RING) {
                if (j + RING - 1 < NT) issue_tile(j + RING - 1);
            }
        }
        if (j >= n_w) continue;
        const uint16_t *kt = sK[j % RING];
        const uint16_t *vt = sV[j % RING];
        const int j0 = j * kBN;
        if (wave_lim - j0 <= 32) {
            // a last tile whose second half no row of the wave sees: one
            // 32-key block
            f32x16 s1;
#pragma unroll
            for (int r = 0; r < 16; ++r) s1[r] = 0.f;
#pragma unroll
            for (int kk = 0; kk < DK; ++kk) s1 = mfma32<BF16>(frag_k<D>(kt, 0, kk, l32, g), qreg[kk], s1);
            if (j0 + 32 > wave_lim || (CAUSAL && j0 + 31 > wave_lo)) {
                const int lim = row_lim - j0 - 4 * g;
#pragma unroll
                for (int r = 0; r < 16; ++r) s1[r] = (r >> 2) * 8 + (r & 3) < lim ? s1[r] : -INFINITY;
            }
            f32x16 sb[1] = {s1};
            u32x4 pf1[1][2];
            float lsum = 0.f;
            bool max_first = true;
            if (j > 0) {
                lsum = exps_blocks<BF16, 1>(sb, c, m_run == -INFINITY ? 0.f : -m_run, pf1);
                max_first = __any(!(lsum <= kShortExpFirstBound) || m_run == -INFINITY);
            }
            if (max_first) {
                const float m_tile = row_max32(s1) * c;
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
                lsum = exps_blocks<BF16, 1>(sb, c, m_run == -INFINITY ? 0.f : -m_run, pf1);
            }
            l_run += lsum;
#pragma unroll
            for (int cb = 0; cb < DB; ++cb)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
                    oacc[cb] = mfma32<BF16>(frag_v<D>(vt, cb, kc, lane, g), pf1[0][kc], oacc[cb]);
            continue;
        }
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
        // mask the tiles that straddle the key-length or causal limit:
        // register r of block kb holds key j0 + 32 kb + 8 (r / 4) + 4 g + r % 4
        if ((j0 + kBN > Lk) || (CAUSAL && j0 + kBN - 1 > wave_lo)) {
            const int lim = row_lim - j0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[kb][r] = kb * 32 + (r >> 2) * 8 + (r & 3) < lim ? s[kb][r] : -INFINITY;
        }
        // online softmax with a lazy running max: it moves only when the
        // tile's max exceeds it by more than kLazy, then to kHeadroom above
        // that max; output and normaliser are rescaled by exp2(m_old - m_new).
        // After the first tile, exponentials first (kShortExpFirstBound).
        float lsum = 0.f;
        bool max_first = true;
        if (j > 0) {
            lsum = exps_blocks<BF16, 2>(s, c, m_run == -INFINITY ? 0.f : -m_run, pf);
            max_first = __any(!(lsum <= kShortExpFirstBound) || m_run == -INFINITY);
        }
        if (max_first) {
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
            lsum = exps_blocks<BF16, 2>(s, c, m_run == -INFINITY ? 0.f : -m_run, pf);
        }
        l_run += lsum;
        // O^T += V_j^T P^T
#pragma unroll
        for (int cb = 0; cb < DB; ++cb)
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
                oacc[cb] = mfma32<BF16>(frag_v<D>(vt, cb, kc, lane, g), pf[kc >> 1][kc & 1], oacc[cb]);
    }

    // ---- epilogue: O = O_acc / l, LSE = ln(2) * (m + log2 l).  O is staged
    // in LDS (the K tiles' space, free once every wave is past its last
    // tile), so that each store instruction writes whole 16-byte chunks of
    // consecutive rows.  From the accumulator layout each lane would write
    // 8-byte pieces, spread over 32 rows per instruction: with loads and
    // arithmetic taken out, those stores alone took 3.9 us at 600 x 256
    // rows of d = 32, the staged ones 2.7 us.
    const Halves lh = both_halves(l_run);
    const float l_tot = lh.lo + lh.hi;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    static_assert(2 * TILE >= kSBM * D, "the output tile fits in the first two K slots");
    // loads of tiles the loop did not reach (empty ranges, zeros) may still
    // be writing their slots
    wait_tile_loads<0>();
    barrier();
    // This wave's 32 rows, row-major with the tiles' XOR swizzle of 16-byte
    // chunks (the 32 rows a write instruction touches spread over the banks).
    uint16_t *so = sK[wave >> 1] + (wave & 1) * kQRows * D;
    const int wsw = swz<D>(l32);
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            u32x2 w = {pack2<BF16>(oacc[cb][4 * a] * inv, oacc[cb][4 * a + 1] * inv),
                       pack2<BF16>(oacc[cb][4 * a + 2] * inv, oacc[cb][4 * a + 3] * inv)};
            *reinterpret_cast<u32x2 *>(so + l32 * D + (((cb * 4 + a) ^ wsw) * 8) + g * 4) = w;
        }
    // each wave reads back only what it wrote: LDS keeps a wave's order
    uint16_t *ob = p.O + q_base + (size_t)qw0 * D;
#pragma unroll
    for (int k = 0; k < kQRows * CPR / 64; ++k) {
        const int L = lane + 64 * k;
        const int row = L / CPR, ch = L % CPR;
        const u32x4 v = *reinterpret_cast<const u32x4 *>(so + row * D + ((ch ^ swz<D>(row)) * 8));
        if (qw0 + row < M) *reinterpret_cast<u32x4 *>(ob + L * 8) = v;
    }
    if (my_q < M && p.LSE != nullptr && g == 0)
        p.LSE[(size_t)sl * M + my_q] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
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
