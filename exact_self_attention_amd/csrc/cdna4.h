// gfx950 (CDNA4) device building blocks shared by the attention kernels:
// vector types, the 32x32x16 matrix-core product, 16-bit packing, exp2, the
// cross-half lane exchange, the LDS tile swizzle and fragment reads, the
// softmax arithmetic on a wave's scores, the raw workgroup barrier, buffer
// resources, direct-to-LDS 16-byte loads (inline and compiler-tracked) with
// their counted waits, the causal row positions of a slice, and the launch
// orders (heaviest query tiles first; XCD-blocked for a shared mask).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace cdna4 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kQRows = 32;               // query rows per wave
constexpr int kBN = 64;                  // keys per tile
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
// Lazy running max.  The running max only moves when a tile's max exceeds
// it by more than kLazy (log2 units), and then to kHeadroom above that
// tile's max, so that it rarely has to move again.  Probabilities stay below
// 2^kLazy, and after a move the largest is 2^-kHeadroom.
constexpr float kLazy = 8.0f;
constexpr float kHeadroom = 8.0f;
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

// Waits until at most KEEP of this wave's vector-memory loads are still in
// flight (loads complete in issue order).
template <int KEEP>
__device__ __forceinline__ void wait_tile_loads() {
    static_assert(KEEP >= 0 && KEEP < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KEEP) : "memory");
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

// The same load through the compiler's builtin.  The compiler then counts it
// in the waits it inserts itself (before a use of registers loaded earlier,
// before LDS reads of the array it writes) and tells LDS arrays apart, so
// loads into other arrays do not hold up reads of this one.
__device__ __forceinline__ void dma16_tracked(__amdgpu_buffer_rsrc_t rsrc, lds_void *lds,
                                              uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds, 16, (int)voff, 0, 0, 0);
}

// Waits until at most k of this wave's vector-memory loads are in flight,
// for k a multiple of STEP up to 3 STEP (rounded up to one).
template <int STEP>
__device__ __forceinline__ void wait_tile_loads_upto(int k) {
    if (k >= 3 * STEP) wait_tile_loads<3 * STEP>();
    else if (k >= 2 * STEP) wait_tile_loads<2 * STEP>();
    else if (k >= STEP) wait_tile_loads<STEP>();
    else wait_tile_loads<0>();
}

// v_max3_f32: the largest of three floats in one instruction.
__device__ __forceinline__ float max3(float a, float b, float c) {
    float d;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

// Fragment reads from a K or V tile of kBN rows x D halves, row-major with
// swizzled 16-byte chunks (swz), for a wave whose lane is l32 + 32 g.
//
// K fragment (A operand of S^T = K Q^T) for 32-key block kb, k-step kk: key
// row kb*32 + l32, dims 16 kk + 8 g .. +7, one 128-bit read.
template <int D>
__device__ __forceinline__ u32x4 frag_k(const uint16_t *kt, int kb, int kk, int l32, int g) {
    const int row = kb * 32 + l32;
    return *reinterpret_cast<const u32x4 *>(kt + row * D + (((2 * kk + g) ^ swz<D>(row)) * 8));
}
// V^T fragment (A operand of O^T += V^T P^T) for column block cb, 16-key
// chunk kc: two transposing reads at rows 16 kc + 8 h + 4 g + (lane%16)/4,
// logical chunk 4 cb + 2 ((lane/16)%2) + (lane%4)/2, 8-byte half lane%2;
// they return V[16kc + 8h + 4g + t][32 cb + l32] for t = 0..3, the key
// order of the P registers taken from the S^T accumulators.
template <int D>
__device__ __forceinline__ u32x4 frag_v(const uint16_t *vt, int cb, int kc, int lane, int g) {
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
}

// Softmax arithmetic on the scores of one 64-key tile as a wave holds them
// in two S^T accumulators: lane l32 + 32 g has query l32's scores of keys
// 8 (r/4) + 4 g + r%4 (block 0) and 32 + the same (block 1), r = 0..15.
//
// Row max (over both lane halves) of the 32 scores a lane holds: a tree of
// v_max3 (short dependency chains) and one cross-half exchange.
__device__ __forceinline__ float row_max64(const f32x16 (&s)[2]) {
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
}
// P = exp2(c s + neg_m), packed to 16 bits into pf (the B operand layout of
// the P.V product); returns this lane's sum of the fp32 values (a tree).
template <bool BF16>
__device__ __forceinline__ float exps64(const f32x16 (&s)[2], float c, float neg_m,
                                        u32x4 (&pf)[2][2]) {
    float pr[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
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
}

// Row max of a 32-key block (S^T layout: one query column per lane pair).
__device__ __forceinline__ float row_max32(const f32x16 &s) {
    float t[6];
#pragma unroll
    for (int i = 0; i < 5; ++i) t[i] = max3(s[3 * i], s[3 * i + 1], s[3 * i + 2]);
    t[5] = s[15];
    const float mx = max3(max3(t[0], t[1], t[2]), t[3], max3(t[4], t[5], t[5]));
    const Halves mh = both_halves(mx);
    return fmaxf(mh.lo, mh.hi);
}
// P = exp2(c s + neg_m) for a 32-key block, packed into pf[ch] (16-key
// chunks, the B operand of the P.V product); returns the lane's fp32 sum.
template <bool BF16>
__device__ __forceinline__ float exps32(const f32x16 &s, float c, float neg_m, u32x4 (&pf)[2]) {
    float pr[16];
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int i = ch * 8 + 2 * w;
            pr[i] = fast_exp2(__builtin_fmaf(s[i], c, neg_m));
            pr[i + 1] = fast_exp2(__builtin_fmaf(s[i + 1], c, neg_m));
            pf[ch][w] = pack2<BF16>(pr[i], pr[i + 1]);
        }
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) pr[i] += pr[i + w];
    return pr[0];
}

typedef __fp16 f16x2s __attribute__((ext_vector_type(2)));
// P = exp2(c s + neg_m) for NB 32-key blocks, packed into pf; returns the
// lane's sum.  With fp16 probabilities the sum is taken over the packed
// values, two per v_dot2_f32_f16 against (1, 1) in fp32 (16 + 3 instead of
// 31 additions per 64 keys): it is then the sum of exactly the rounded
// values the P.V product weights V with, within 2^-11 relative of the sum
// of the unrounded ones.  With bf16 (2^-8) the fp32 values are summed.
template <bool BF16, int NB>
__device__ __forceinline__ float exps_blocks(const f32x16 (&s)[NB], float c, float neg_m,
                                             u32x4 (&pf)[NB][2]) {
    float pr[16 * NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const int i = kb * 16 + ch * 8 + 2 * w;
                pr[i] = fast_exp2(__builtin_fmaf(s[kb][ch * 8 + 2 * w], c, neg_m));
                pr[i + 1] = fast_exp2(__builtin_fmaf(s[kb][ch * 8 + 2 * w + 1], c, neg_m));
                pf[kb][ch][w] = pack2<BF16>(pr[i], pr[i + 1]);
            }
    if constexpr (BF16) {
#pragma unroll
        for (int w = 8 * NB; w >= 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < w; ++i) pr[i] += pr[i + w];
        return pr[0];
    } else {
        const f16x2s one = {(__fp16)1.0f, (__fp16)1.0f};
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // (a vector element as the operand of __builtin_bit_cast
                    // compiles to element 0: copy it out first)
                    const uint32_t word = pf[kb][ch][w];
                    acc[w] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2s, word), one, acc[w], false);
                }
        return (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
}

// Causal positions of a slice's query rows.  The rows of the query heads
// that share a key/value head follow each other, nq rows per head, so row r
// is query r mod nq of its head and sees keys j <= r mod nq + off.
struct CausalRows {
    int nq;   // query rows per head
    int off;  // keys minus query rows per head
    __device__ __forceinline__ int pos(int r) const { return r % nq + off; }
    // Lowest and highest position among rows r_lo .. r_hi (r_lo <= r_hi).
    // Rows on both sides of a head boundary include a first row (position
    // off) and a last one (position nq - 1 + off).
    __device__ __forceinline__ void range(int r_lo, int r_hi, int &lo, int &hi) const {
        const int h_lo = r_lo / nq, h_hi = r_hi / nq;
        if (h_lo == h_hi) {
            lo = r_lo - h_lo * nq + off;
            hi = r_hi - h_hi * nq + off;
        } else {
            lo = off;
            hi = nq - 1 + off;
        }
    }
};

// Launch order of a slice's query tiles (rows_per_tile rows each) under a
// causal mask, most visible keys first, so that the last workgroups to start
// are the cheapest.  A tile's work grows with its rows' positions.  When each
// head's nq rows split into whole tiles, tile t of every one of the m / nq
// heads has the same work: launch index i then goes over t downwards and,
// for each t, over the heads.  Otherwise the tiles go from last to first.
__device__ __forceinline__ int heavy_first_tile(int i, int n_tiles, int nq, int m,
                                                int rows_per_tile) {
    const int heads = m / nq;
    if (heads > 1 && nq % rows_per_tile == 0) {
        const int per_head = nq / rows_per_tile;
        return (i % heads) * per_head + (per_head - 1 - i / heads);
    }
    return n_tiles - 1 - i;
}

// Launch order of a forward whose additive mask all S slices share.  The
// n_qt * S workgroups are dealt round-robin to the 8 XCDs, each with its own
// L2; here XCD x works on a block of A slices and n_qt * S / (8 A) query
// tiles, so that a query tile's mask rows are read by A slices on one XCD
// (fetched S / A times in all, instead of up to 8 times per tile) while a
// slice's K and V are fetched by 8 A / S XCDs.  The query tiles go to the
// XCDs in a snake over their ranks (heaviest first under a causal mask), so
// every XCD gets the same work, and each XCD runs its tiles heaviest first.
// Needs S % A == 0, 8 % (S / A) == 0 and n_qt % (8 A / S) == 0.
__device__ __forceinline__ void xcd_blocked_tile(int b, int n_qt, int S, int A, bool causal, int nq,
                                                 int m, int rows_per_tile, int &qt, int &sl) {
    constexpr int kXcds = 8;
    const int x = b % kXcds, local = b / kXcds;
    const int slice_groups = S / A;
    const int tile_groups = kXcds / slice_groups;
    const int sg = x % slice_groups, tg = x / slice_groups;
    const int i = local / A;  // this XCD's i-th query tile, heaviest first
    sl = sg * A + local % A;
    const int rank = i * tile_groups + ((i & 1) ? tile_groups - 1 - tg : tg);
    qt = causal ? heavy_first_tile(rank, n_qt, nq, m, rows_per_tile) : rank;
}

}  // namespace cdna4
}  // namespace attn
