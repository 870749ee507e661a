// Unfused baseline: three launches that materialise the scores and the
// probabilities in device memory, as in "Tensor Parallelism with CUDA -
// Standard Attention" (sections "Why This Ordering?" and "The Naive HBM
// Algorithm") and "Naive Attention Kernel" (sections 1 and 3):
//
//   qk       one thread per score: S_ij = scale * q_i . k_j      (writes S)
//   softmax  one workgroup per row: max, exponential sum, then normalise in
//            place (S becomes P); also writes LSE
//   pv       one thread per output element: O_ic = sum_j P_ij v_jc
//
// Arithmetic is fp32 from the widened fp16/bf16 inputs.  Only visible scores
// are computed and read: a row's visible keys are the prefix j < n_vis(i),
// n_vis(i) = min(L_b, i + 1) under causal masking, else L_b.  No tiling, no
// matrix cores, no fusion across the three steps: this is the reference point
// the fused kernel is measured against.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace attn {
namespace {

constexpr int kSoftmaxThreads = 256;

__device__ __forceinline__ float widen(uint16_t bits, bool bf16) {
    if (bf16) return __uint_as_float((uint32_t)bits << 16);
    return (float)__builtin_bit_cast(_Float16, bits);
}

__device__ __forceinline__ uint16_t narrow(float x, bool bf16) {
    if (bf16) return __builtin_bit_cast(uint16_t, (__bf16)x);
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

__device__ __forceinline__ int visible_keys(const NaiveParams &p, int b, int64_t i) {
    int64_t L = p.N;
    if (p.key_len != nullptr) {
        const int64_t v = p.key_len[b];
        L = v < 0 ? 0 : (v > p.N ? p.N : v);
    }
    if (p.causal && i + 1 < L) L = i + 1;
    return (int)L;
}

__global__ __launch_bounds__(256) void attn_naive_qk(NaiveParams p) {
    const int64_t j = (int64_t)blockIdx.x * 16 + threadIdx.x;
    const int64_t i = (int64_t)blockIdx.y * 16 + threadIdx.y;
    const int z = blockIdx.z;
    const int bh = p.bh0 + z;
    if (i >= p.N || j >= p.N) return;
    if (j >= visible_keys(p, bh / p.H, i)) return;
    const size_t base = (size_t)bh * p.N * p.d;
    const uint16_t *q = p.Q + base + (size_t)i * p.d;
    const uint16_t *k = p.K + base + (size_t)j * p.d;
    const bool bf16 = p.bf16 != 0;
    float acc = 0.f;
    for (int c = 0; c < p.d; ++c) acc = __builtin_fmaf(widen(q[c], bf16), widen(k[c], bf16), acc);
    p.S[((size_t)z * p.N + i) * p.N + j] = p.scale * acc;
}

__device__ float block_reduce(float v, bool is_max, float *red) {
    for (int off = 32; off > 0; off >>= 1) {
        const float o = __shfl_xor(v, off);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kSoftmaxThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

__global__ __launch_bounds__(kSoftmaxThreads) void attn_naive_softmax(NaiveParams p) {
    __shared__ float red[kSoftmaxThreads / 64];
    const int64_t i = blockIdx.x;
    const int z = blockIdx.y;
    const int bh = p.bh0 + z;
    const int n = visible_keys(p, bh / p.H, i);
    float *row = p.S + ((size_t)z * p.N + i) * p.N;

    float m = -INFINITY;
    for (int j = threadIdx.x; j < n; j += kSoftmaxThreads) m = fmaxf(m, row[j]);
    m = block_reduce(m, true, red);
    float l = 0.f;
    for (int j = threadIdx.x; j < n; j += kSoftmaxThreads) l += expf(row[j] - m);
    l = block_reduce(l, false, red);
    const float inv = 1.f / l;
    for (int j = threadIdx.x; j < n; j += kSoftmaxThreads) row[j] = expf(row[j] - m) * inv;
    if (threadIdx.x == 0 && p.LSE != nullptr)
        p.LSE[(size_t)bh * p.N + i] = n > 0 ? m + logf(l) : -INFINITY;
}

__global__ __launch_bounds__(256) void attn_naive_pv(NaiveParams p) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int z = blockIdx.y;
    const int bh = p.bh0 + z;
    if (idx >= p.N * p.d) return;
    const int64_t i = idx / p.d;
    const int c = (int)(idx % p.d);
    const int n = visible_keys(p, bh / p.H, i);
    const float *prow = p.S + ((size_t)z * p.N + i) * p.N;
    const uint16_t *v = p.V + (size_t)bh * p.N * p.d + c;
    const bool bf16 = p.bf16 != 0;
    float acc = 0.f;
    for (int j = 0; j < n; ++j) acc = __builtin_fmaf(prow[j], widen(v[(size_t)j * p.d], bf16), acc);
    p.O[(size_t)bh * p.N * p.d + idx] = narrow(acc, bf16);
}

}  // namespace

hipError_t launch_naive(const NaiveParams &p, hipStream_t s) {
    const unsigned tiles = (unsigned)((p.N + 15) / 16);
    hipLaunchKernelGGL(attn_naive_qk, dim3(tiles, tiles, p.nbh), dim3(16, 16), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_naive_softmax, dim3((unsigned)p.N, p.nbh), dim3(kSoftmaxThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned pv_blocks = (unsigned)((p.N * p.d + 255) / 256);
    hipLaunchKernelGGL(attn_naive_pv, dim3(pv_blocks, p.nbh), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace attn
