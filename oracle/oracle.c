/*
 * TEST INFRASTRUCTURE -- not part of the product path.
 *
 * Plain, slow, fp64 CPU oracle for exact scaled-dot-product attention.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header or constant with the HIP
 * library.
 *
 * What it computes, for every selected (batch b, head h, query row i):
 *
 *   S_ij = scale * (q_i . k_j)            for every visible key j
 *   P_ij = exp(S_ij - max_j S_ij) / sum_j exp(S_ij - max_j S_ij)
 *   O_i  = sum_j P_ij v_j
 *   LSE_i = max_j S_ij + log(sum_j exp(S_ij - max_j S_ij))
 *
 * This is the textbook definition O = softmax(Q K^T / sqrt(d)) V of
 * "Tensor Parallelism with CUDA - Standard Attention" (sections "Step 1:
 * QK^T", "What is a Dot Product?", "Step 2: Softmax" -- the max-subtracted,
 * numerically stable form -- and "Step 3: PV"), with the scale passed in as
 * an argument, and the masked five-step form of "Naive Attention Kernel"
 * (section 1, "Standard Attention: Step by Step") where the mask is
 * structural: a masked key gets probability exactly zero.
 *
 * Shapes: Q and O are [B, H, Nq, d]; K and V are [B, Hkv, Nk, d] with H a
 * multiple of Hkv.  Self-attention is Hkv = H and Nq = Nk.  Different
 * query and key lengths (cross-attention) and fewer key/value heads than
 * query heads (grouped-query attention) are the extensions the
 * "cuda-reranker" page lists as future work; it does not define them, so
 * this oracle fixes the usual reading: query head h reads key/value head
 * floor(h / (H / Hkv)), i.e. consecutive query heads share one.
 *
 * Visible keys (the readings this oracle fixes where the pages are silent):
 *   - key j is visible iff j < L_b, where L_b = clamp(key_len[b], 0, Nk) when
 *     a key-length array is given (a key-side padding mask, "cuda-reranker"),
 *     else L_b = Nk;
 *   - with causal masking additionally j <= i + (Nk - Nq): the query rows
 *     are aligned with the last Nq keys (bottom-right), which is j <= i
 *     (top-left) when Nq = Nk;
 *   - a row with no visible key has O_i = 0 and LSE_i = -inf.
 *
 * Additive mask (optional): S_ij = scale * (q_i . k_j) + mask_ij, the five
 * steps of "Naive Attention Kernel" (section 1: scores, scale, add the mask,
 * softmax, product with V), with a float mask element per (query, key).  The
 * mask of (b, h) starts at element b * mask_sb + h * mask_sh and is row-major
 * [Nq, Nk]; a stride of 0 shares one mask (the pages' [S, S]) across batch or
 * heads.  An element of -inf removes its key like a structural mask; a row
 * whose visible scores are all -inf is a row with no visible key.
 *
 * The score row is materialised in full (one row at a time), followed by two
 * passes (max, then exponential sum), then the weighted sum of value rows.
 * Inputs are float32 arrays holding the exact widening of the fp16/bf16 bits
 * under test; all arithmetic is double precision with the C library's exp and
 * log.  Built without fast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Q: [B, H, Nq, d]; K, V: [B, Hkv, Nk, d]; all row-major float32.
 * key_len: [B] or NULL.  mask: float32 additive mask or NULL, element
 * (b, h, i, j) at b * mask_sb + h * mask_sh + i * Nk + j.
 * sel: n_sel triples (b, h, i) as int64, h a query head, i a query row.
 * O: [n_sel, d] double; LSE: [n_sel] double.
 * Returns 0, or -1 on a bad argument or a failed allocation.
 */
int oracle_attn_rows(const float *Q, const float *K, const float *V,
                     int64_t B, int64_t H, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d,
                     double scale, int causal, const int32_t *key_len,
                     const float *mask, int64_t mask_sb, int64_t mask_sh,
                     const int64_t *sel, int64_t n_sel,
                     double *O, double *LSE)
{
    if (B < 0 || H < 0 || Hkv <= 0 || H % Hkv != 0 || Nq < 0 || Nk < 0 || d <= 0 ||
        n_sel < 0 || mask_sb < 0 || mask_sh < 0)
        return -1;
    for (int64_t t = 0; t < n_sel; ++t) {
        int64_t b = sel[3 * t], h = sel[3 * t + 1], i = sel[3 * t + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= Nq) return -1;
    }
    const int64_t group = H / Hkv;   /* query heads per key/value head */
    int failed = 0;

#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double *p = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (s == NULL || p == NULL) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < n_sel; ++t) {
            if (s == NULL || p == NULL) continue;
            int64_t b = sel[3 * t], h = sel[3 * t + 1], i = sel[3 * t + 2];
            int64_t hk = h / group;  /* the key/value head query head h reads */
            const float *q  = Q + ((b * H + h) * Nq + i) * d;
            const float *kb = K + (b * Hkv + hk) * Nk * d;
            const float *vb = V + (b * Hkv + hk) * Nk * d;
            double *o = O + t * d;

            /* visible keys are j < n_vis */
            int64_t L = Nk;
            if (key_len != NULL) {
                L = key_len[b];
                if (L < 0) L = 0;
                if (L > Nk) L = Nk;
            }
            int64_t n_vis = L;
            /* causal: query row i sits at key position i + Nk - Nq */
            int64_t pos = i + (Nk - Nq);
            if (causal && pos + 1 < n_vis) n_vis = pos + 1 > 0 ? pos + 1 : 0;

            if (n_vis == 0) {
                for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
                LSE[t] = -INFINITY;
                continue;
            }

            /* scores S_ij = scale * q_i . k_j (+ mask_ij) */
            const float *mrow = mask == NULL ? NULL : mask + b * mask_sb + h * mask_sh + i * Nk;
            for (int64_t j = 0; j < n_vis; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += (double)q[c] * (double)kb[j * d + c];
                s[j] = scale * dot;
                if (mrow != NULL) s[j] += (double)mrow[j];
            }
            /* pass 1: row maximum */
            double m = s[0];
            for (int64_t j = 1; j < n_vis; ++j)
                if (s[j] > m) m = s[j];
            if (m == -INFINITY) {  /* every visible key masked out by -inf */
                for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
                LSE[t] = -INFINITY;
                continue;
            }
            /* pass 2: normaliser, then probabilities */
            double l = 0.0;
            for (int64_t j = 0; j < n_vis; ++j) {
                p[j] = exp(s[j] - m);
                l += p[j];
            }
            for (int64_t j = 0; j < n_vis; ++j) p[j] /= l;
            /* O_i = sum_j P_ij v_j */
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            for (int64_t j = 0; j < n_vis; ++j)
                for (int64_t c = 0; c < d; ++c)
                    o[c] += p[j] * (double)vb[j * d + c];
            LSE[t] = m + log(l);
        }
        free(s);
        free(p);
    }
    return failed ? -1 : 0;
}
