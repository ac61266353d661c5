/*
 * CPU oracle for the MoE token dispatch / combine path.
 *
 * TEST INFRASTRUCTURE ONLY. Plain, slow C that states what the path
 * computes. Only the tests, the smoke check and the benchmark's CPU baseline
 * use it; the HIP library never links, includes or calls it, and the two
 * share no source. Build: gcc -O2 -std=c11 -fPIC -shared (no fast-math, SSE
 * arithmetic, default round-to-nearest-even mode), single-threaded. The same
 * source is also built with -fopenmp: the only pragmas spread independent
 * per-token, per-row or per-block iterations over threads; counting, offsets and the
 * stable placement stay serial, and no arithmetic changes.
 *
 * Sources (Perplexity engineering posts):
 *  [EPMC] "Efficient and portable mixture-of-experts communication",
 *         sections Introduction, Dispatch, Combine.
 *  [EFA]  "Enabling trillion-parameter models on AWS EFA",
 *         sections Send and receive buffers, Dispatch and Combine,
 *         Evaluation (dispatch/combine latency).
 *  [DSV3] DeepSeek-V3 report excerpts quoted on the third and fourth pages
 *         (fine-grained 1x128 activation quantisation; gating kept in its
 *         original precision; combine components kept in BF16).
 *
 * Readings where the pages are silent (each is repeated where it is used):
 *  - selection is on the raw fp32 logits, descending, ties to the lower
 *    expert index, IEEE comparison (so -0 == +0);
 *  - weights are the router softmax restricted to the selected experts and
 *    renormalised to sum to one, computed in fp64 and rounded once to fp32;
 *  - within an expert segment rows are in token order (a stable layout);
 *  - segments are padded to a multiple of row_align rows; pad rows carry a
 *    zero payload, zero scales and row_src = -1;
 *  - destination groups are contiguous expert ranges of E/G experts;
 *  - FP8 is OCP E4M3 (bias 7, max 448, no infinities); the scale of a
 *    1x128 block is s = amax / 448 (fp32 division); each element is the fp32
 *    quotient x / s rounded to nearest-even E4M3 and saturated to +-448;
 *    an all-zero block has s = 0 and all codes 0x00;
 *  - a slot whose expert id lies outside [0, E) is dropped: it is not
 *    counted, gets dst_row = -1 and contributes nothing to combine;
 *  - combine accumulates in fp64 in slot order and rounds once to bf16.
 *
 * Parity status: every function below is pinned by the CPU tests (brute
 * force, library routines, closed forms, invariants). The composition of
 * the whole chain has no printed values on the pages to pin against.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops below use: 1 unless built with OpenMP. */
int oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- bf16 */

static float bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round a finite double to the nearest bfloat16, ties to even, in one step
 * (no intermediate rounding to float). bf16 keeps 8 significant bits and the
 * float exponent range; below 2^-126 the spacing is the subnormal 2^-133. */
uint16_t oracle_bf16_from_double(double d) {
    uint16_t sign = signbit(d) ? 0x8000u : 0u;
    double a = fabs(d);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);                 /* a = m * 2^ex, m in [0.5, 1) */
    int q = ex - 8;                /* spacing of 8-bit significands: 2^(ex-8) */
    if (q < -133) q = -133;        /* subnormal bf16 spacing */
    double n = nearbyint(ldexp(a, -q));   /* exact scaling, then RNE */
    double v = ldexp(n, q);
    if (v >= 0x1p128) return (uint16_t)(sign | 0x7F80u);   /* overflow: inf */
    float f = (float)v;            /* exact: v has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* ---------------------------------------------------------------- e4m3 */

/* OCP E4M3 (FN variant) value of a code; 0x7F / 0xFF are NaN. */
float oracle_e4m3_value(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);            /* subnormal: m/8 * 2^-6 */
    else v = ldexp(8.0 + m, e - 7 - 3);              /* (1 + m/8) * 2^(e-7) */
    return (float)(s ? -v : v);
}

/* Round a finite float to nearest-even E4M3, saturating to +-448 (0x7E).
 * Spacing: 2^-9 below 2^-6 (subnormals), else 2^(e-3) for a in [2^e, 2^(e+1)).
 * The rounded significand n (0..16) is added to the exponent field so a
 * carry from n == 16 moves to the next binade by itself. */
uint8_t oracle_e4m3_encode(float v) {
    uint8_t sign = signbit(v) ? 0x80u : 0u;
    double a = fabs((double)v);
    if (isnan(v)) return (uint8_t)(sign | 0x7Fu);
    if (a > 448.0) return (uint8_t)(sign | 0x7Eu);    /* saturate to +-448 */
    if (a < 0x1p-6) {
        int n = (int)nearbyint(ldexp(a, 9));          /* 0..8; 8 = 2^-6 = 0x08 */
        return (uint8_t)(sign | n);
    }
    int ex;
    frexp(a, &ex);
    int e = ex - 1;                                   /* a in [2^e, 2^(e+1)) */
    int n = (int)nearbyint(ldexp(a, 3 - e));          /* 8..16 */
    int code = ((e + 7) << 3) + (n - 8);             /* <= 0x7E since a <= 448 */
    return (uint8_t)(sign | code);
}

/* Quantise one 1x128 block: s = amax/448 (fp32), q = E4M3(fp32(x/s)). */
void oracle_quantize_block(const uint16_t* x, uint8_t* q, float* s_out) {
    float amax = 0.0f;
    for (int i = 0; i < 128; i++) {
        float a = fabsf(bf16_value(x[i]));
        if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    *s_out = s;
    for (int i = 0; i < 128; i++) {
        if (amax == 0.0f) { q[i] = 0; continue; }
        float y = bf16_value(x[i]) / s;               /* correctly rounded fp32 */
        q[i] = oracle_e4m3_encode(y);
    }
}

/* ---------------------------------------------------------------- routing */

/* Router gate: softmax over the E logits of each token, the top-k experts by
 * score, and weights renormalised over the selected experts ([EPMC]
 * Introduction; gating in original precision per [DSV3]). Softmax is strictly
 * increasing in the logit, so ranking by logit is ranking by probability;
 * ranking on the fp32 logits avoids ties that rounding of probabilities would
 * create. Slot j holds the j-th best expert. */
void oracle_route_topk(const float* logits, int64_t T, int E, int k,
                       int32_t* topk_idx, float* topk_w) {
#pragma omp parallel
    {
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    unsigned char* taken = (unsigned char*)malloc((size_t)E);
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const float* l = logits + t * (int64_t)E;
        /* softmax over all experts, in fp64 */
        double lmax = l[0];
        for (int e = 1; e < E; e++) if (l[e] > lmax) lmax = l[e];
        double z = 0.0;
        for (int e = 0; e < E; e++) { p[e] = exp((double)l[e] - lmax); z += p[e]; }
        for (int e = 0; e < E; e++) p[e] /= z;
        /* top-k: repeatedly take the best remaining expert */
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* ties keep lower e */
            }
            taken[best] = 1;
            topk_idx[t * k + j] = best;
        }
        /* renormalise the selected probabilities */
        double sel = 0.0;
        for (int j = 0; j < k; j++) sel += p[topk_idx[t * k + j]];
        for (int j = 0; j < k; j++)
            topk_w[t * k + j] = (float)(p[topk_idx[t * k + j]] / sel);
    }
    free(p);
    free(taken);
    }
}

/* ---------------------------------------------------------------- dispatch */

/* Count tokens per expert, turn the (padded) counts into segment offsets by a
 * running sum, then place every (token, slot) pair into its expert's
 * contiguous segment ([EFA] Dispatch and Combine: per-expert counts, their
 * cumulative sum gives the offsets used to pack tokens into contiguous
 * per-expert send buffers; [EPMC] Dispatch: payload, scales and the token's
 * index are packed together, source and token index kept per row).
 *
 * Layout produced:
 *   expert_counts[e]   tokens routed to e (unpadded)
 *   expert_offsets[e]  first row of e's segment; expert_offsets[E] = rows used
 *   group_offsets[g]   = expert_offsets[g * E / G]  (group g = send buffer g)
 *   row_src[r]         t * k + j of the pair stored in row r, -1 for pad rows
 *   dst_row[t * k + j] row holding that pair, -1 if the slot is dropped
 *   out[r]             x[t] (bf16 copy) or its E4M3 codes, scales[r][b] per
 *                      128-channel block
 * Rows at and beyond expert_offsets[E] are not written.
 * Returns the number of rows used. */
int64_t oracle_dispatch(const uint16_t* x, const int32_t* topk_idx,
                        int64_t T, int H, int E, int k, int groups,
                        int row_align, int fp8,
                        void* out, float* scales,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* group_offsets, int32_t* row_src,
                        int32_t* dst_row) {
    const int64_t TK = T * (int64_t)k;
    /* counts */
    for (int e = 0; e < E; e++) expert_counts[e] = 0;
    for (int64_t i = 0; i < TK; i++) {
        int e = topk_idx[i];
        if (e >= 0 && e < E) expert_counts[e]++;
    }
    /* padded counts -> offsets (exclusive running sum) */
    expert_offsets[0] = 0;
    for (int e = 0; e < E; e++) {
        int64_t c = expert_counts[e];
        int64_t padded = (c + row_align - 1) / row_align * row_align;
        expert_offsets[e + 1] = (int32_t)(expert_offsets[e] + padded);
    }
    if (group_offsets) {
        int per = E / groups;
        for (int g = 0; g <= groups; g++) group_offsets[g] = expert_offsets[g * per];
    }
    /* stable placement: experts in order, tokens in order within an expert */
    for (int64_t i = 0; i < TK; i++) dst_row[i] = -1;
    for (int e = 0; e < E; e++) {
        int64_t r = expert_offsets[e];
        for (int64_t t = 0; t < T; t++)
            for (int j = 0; j < k; j++)
                if (topk_idx[t * k + j] == e) {
                    dst_row[t * k + j] = (int32_t)r;
                    row_src[r] = (int32_t)(t * k + j);
                    r++;
                }
        for (; r < expert_offsets[e + 1]; r++) row_src[r] = -1;   /* pad rows */
    }
    /* payload */
    const int nb = H / 128;
#pragma omp parallel
    {
    uint8_t* qrow = fp8 ? (uint8_t*)malloc((size_t)H) : NULL;
    float* srow = fp8 ? (float*)malloc(sizeof(float) * (size_t)(nb > 0 ? nb : 1)) : NULL;
#pragma omp for schedule(static)
    for (int64_t t = 0; t < T; t++) {
        const uint16_t* xr = x + t * (int64_t)H;
        if (fp8)
            for (int b = 0; b < nb; b++)
                oracle_quantize_block(xr + 128 * b, qrow + 128 * b, srow + b);
        for (int j = 0; j < k; j++) {
            int64_t r = dst_row[t * k + j];
            if (r < 0) continue;
            if (fp8) {
                memcpy((uint8_t*)out + r * H, qrow, (size_t)H);
                memcpy(scales + r * nb, srow, sizeof(float) * (size_t)nb);
            } else {
                memcpy((uint16_t*)out + r * H, xr, sizeof(uint16_t) * (size_t)H);
            }
        }
    }
    free(qrow);
    free(srow);
    }
    /* pad rows: zero payload and zero scales */
    for (int e = 0; e < E; e++)
        for (int64_t r = expert_offsets[e] + expert_counts[e]; r < expert_offsets[e + 1]; r++) {
            if (fp8) {
                memset((uint8_t*)out + r * H, 0, (size_t)H);
                for (int b = 0; b < nb; b++) scales[r * nb + b] = 0.0f;
            } else {
                memset((uint16_t*)out + r * H, 0, sizeof(uint16_t) * (size_t)H);
            }
        }
    return expert_offsets[E];
}

/* ---------------------------------------------------------------- experts */

/* Stand-in experts used around the path (not part of it): row r of expert e
 * becomes bf16(fp32(v) * c_e) with c_e = fp32((e+1)/E), or c_e = 1 when
 * identity is set; v is the bf16 row or, for FP8 rows, code value * scale in
 * fp32. Pad rows become zero. Rows at and beyond num_rows are not written. */
void oracle_expert_scale(const void* disp, const float* scales,
                         const int32_t* row_src, const int32_t* topk_idx,
                         int64_t num_rows, int H, int E, int fp8, int identity,
                         uint16_t* expert_out) {
    const int nb = H / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < num_rows; r++) {
        uint16_t* o = expert_out + r * H;
        if (row_src[r] < 0) { memset(o, 0, sizeof(uint16_t) * (size_t)H); continue; }
        int e = topk_idx[row_src[r]];
        float c = identity ? 1.0f : (float)(e + 1) / (float)E;
        for (int h = 0; h < H; h++) {
            float v;
            if (fp8) v = oracle_e4m3_value(((const uint8_t*)disp)[r * H + h]) * scales[r * nb + h / 128];
            else v = bf16_value(((const uint16_t*)disp)[r * H + h]);
            float prod = v * c;
            o[h] = oracle_bf16_from_double((double)prod);
        }
    }
}

/* ---------------------------------------------------------------- combine */

/* Weighted sum of each token's expert outputs with the router weights
 * ([EPMC] Introduction: the final activation is the weighted average of the
 * selected experts' outputs; Combine: the receiver reads each expert's row
 * through the routing table and applies its weight; [EFA] Evaluation: the
 * accumulation happens only on the receiving side). Accumulated in fp64 in
 * slot order, rounded once to bf16. Dropped slots (dst_row < 0) add nothing. */
void oracle_combine(const uint16_t* expert_out, const int32_t* dst_row,
                    const float* topk_w, int64_t T, int H, int k, uint16_t* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; t++)
        for (int h = 0; h < H; h++) {
            double acc = 0.0;
            for (int j = 0; j < k; j++) {
                int64_t r = dst_row[t * k + j];
                if (r < 0) continue;
                acc += (double)topk_w[t * k + j] * (double)bf16_value(expert_out[r * H + h]);
            }
            y[t * H + h] = oracle_bf16_from_double(acc);
        }
}

/* ---------------------------------------------------------------- helpers */

/* Many 1x128 blocks (the sweeps of the FP8 tests): block b of x [n, 128]
 * quantised as oracle_quantize_block into q [n, 128] and s[b]. */
void oracle_quantize_blocks(const uint16_t* x, int64_t n, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < n; b++) oracle_quantize_block(x + 128 * b, q + 128 * b, s + b);
}

/* Elementwise encoders used by the tests that sweep the E4M3 rounding. */
void oracle_e4m3_encode_array(const float* v, uint8_t* out, int64_t n) {
    for (int64_t i = 0; i < n; i++) out[i] = oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_encode_bits(uint32_t start, int64_t count, uint8_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        uint32_t u = start + (uint32_t)i;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = oracle_e4m3_encode(f);
    }
}

/* ---------------------------------------------------------------- sender-side */

/* Combine with partial sums on the sending side ([EFA] Evaluation: the
 * sender accumulates to cut the bytes transferred, at a possible cost in
 * accuracy; here a destination group stands for the sending rank). For token
 * t the distinct groups g = topk_idx[t,j] / (E/G) of its live slots are taken
 * in ascending order; partial row p of t is
 *   P[t,p] = bf16( sum over slots j of group g_p, in slot order, of w[t,j] * eo[dst_row[t,j]] )
 * (fp64 accumulation, one rounding: the row travels as bf16), and
 *   y[t] = bf16( sum over p of P[t,p] )  (fp64, one rounding).
 * partial has room for k rows per token ([T, k, H]); count[t] = rows used. */
void oracle_combine_sender(const uint16_t* expert_out, const int32_t* dst_row,
                           const float* topk_w, const int32_t* topk_idx,
                           int64_t T, int H, int E, int k, int groups,
                           uint16_t* partial, int32_t* count, uint16_t* y) {
    const int per = E / groups;
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    double* tot = (double*)malloc(sizeof(double) * (size_t)H);
    for (int64_t t = 0; t < T; t++) {
        for (int h = 0; h < H; h++) tot[h] = 0.0;
        int n = 0, prev = -1;
        for (;;) {
            int g = -1;                                   /* next larger group */
            for (int j = 0; j < k; j++) {
                int e = topk_idx[t * k + j];
                if (dst_row[t * k + j] < 0 || e < 0 || e >= E) continue;
                int gj = e / per;
                if (gj > prev && (g < 0 || gj < g)) g = gj;
            }
            if (g < 0) break;
            for (int h = 0; h < H; h++) acc[h] = 0.0;
            for (int j = 0; j < k; j++) {
                int e = topk_idx[t * k + j];
                int64_t r = dst_row[t * k + j];
                if (r < 0 || e < 0 || e >= E || e / per != g) continue;
                for (int h = 0; h < H; h++)
                    acc[h] += (double)topk_w[t * k + j] * (double)bf16_value(expert_out[r * H + h]);
            }
            uint16_t* prow = partial + (t * k + n) * (int64_t)H;
            for (int h = 0; h < H; h++) {
                prow[h] = oracle_bf16_from_double(acc[h]);
                tot[h] += (double)bf16_value(prow[h]);
            }
            n++;
            prev = g;
        }
        count[t] = n;
        for (int h = 0; h < H; h++) y[t * H + h] = oracle_bf16_from_double(tot[h]);
    }
    free(acc);
    free(tot);
}

/* ---------------------------------------------------------------- routing variants */

/* Shared experts treated as routed ones (DeepSeek-V3 excerpt on the third
 * page: each token selects 8 routed experts plus the shared expert, which is
 * always chosen). Slots 0..k-1 are the routed top-k of oracle_route_topk;
 * slots k..k+n_shared-1 hold experts E..E+n_shared-1 with weight shared_w.
 * Row stride of the outputs is k + n_shared. */
void oracle_route_topk_shared(const float* logits, int64_t T, int E, int k, int n_shared,
                              float shared_w, int32_t* topk_idx, float* topk_w) {
    const int ks = k + n_shared;
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    float* w = (float*)malloc(sizeof(float) * (size_t)k);
    for (int64_t t = 0; t < T; t++) {
        oracle_route_topk(logits + t * (int64_t)E, 1, E, k, idx, w);
        for (int j = 0; j < k; j++) {
            topk_idx[t * ks + j] = idx[j];
            topk_w[t * ks + j] = w[j];
        }
        for (int s = 0; s < n_shared; s++) {
            topk_idx[t * ks + k + s] = E + s;
            topk_w[t * ks + k + s] = shared_w;
        }
    }
    free(idx);
    free(w);
}

/* Redundant replicas (DeepSeek-V3 excerpts: experts with heavy load get extra
 * copies hosted as separate experts). Logical expert e owns the physical
 * experts replica_base[e] .. replica_base[e+1]-1; token t goes to copy
 * t mod (number of copies). Ids outside [0, E) pass through unchanged. */
void oracle_route_replicas(int32_t* topk_idx, int64_t T, int k, int E,
                           const int32_t* replica_base) {
    for (int64_t t = 0; t < T; t++)
        for (int j = 0; j < k; j++) {
            int e = topk_idx[t * k + j];
            if (e < 0 || e >= E) continue;
            int n = replica_base[e + 1] - replica_base[e];
            topk_idx[t * k + j] = replica_base[e] + (int)(t % n);
        }
}

/* ---------------------------------------------------------------- grouped GEMM consumer */

/* Weight quantisation ([DSV3] fine-grained quantisation: weights are grouped
 * and scaled per 128x128 block, i.e. per 128 output channels per 128 input
 * channels). w is fp32 [N, K] row-major (K contiguous), N and K multiples of
 * 128. For block (nb, kb): s = amax / 448 (fp32 division, the same reading as
 * the 1x128 activation blocks), every element is E4M3(w / s); an all-zero
 * block has s = 0 and codes 0x00. Scales are [N/128, K/128] row-major. */
void oracle_quantize_weights(const float* w, int64_t N, int64_t K, uint8_t* q, float* s) {
    const int64_t KB = K / 128;
    for (int64_t nb = 0; nb < N / 128; nb++)
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f;
            for (int64_t n = nb * 128; n < nb * 128 + 128; n++)
                for (int64_t k = kb * 128; k < kb * 128 + 128; k++)
                    amax = fmaxf(amax, fabsf(w[n * K + k]));
            const float sc = amax / 448.0f;
            s[nb * KB + kb] = sc;
            for (int64_t n = nb * 128; n < nb * 128 + 128; n++)
                for (int64_t k = kb * 128; k < kb * 128 + 128; k++)
                    q[n * K + k] = amax == 0.0f ? 0 : oracle_e4m3_encode(w[n * K + k] / sc);
        }
}

/* One output of the grouped GEMM. Row r belongs to expert e. Following the
 * [DSV3] description of FP8 GEMM with fine-grained scales: the product is
 * summed over each 128-element interval of the inner dimension, that partial
 * is multiplied by the row's activation scale for the interval and the weight
 * block's scale, and the result is added to the accumulator. Here every step
 * is in fp64: products of two E4M3 values are exact, the sums round once per
 * addition. mag is the same sum over absolute values (the size against which
 * rounding of the sum is measured). */
static void gemm_entry(const uint8_t* a, const float* a_scales, const uint8_t* w,
                       const float* w_scales, int N, int K, int e, int64_t r, int n,
                       double* val, double* mag) {
    const int KB = K / 128;
    const uint8_t* ar = a + r * (int64_t)K;
    const uint8_t* wn = w + ((int64_t)e * N + n) * (int64_t)K;
    const float* wsc = w_scales + ((int64_t)e * (N / 128) + n / 128) * KB;
    double acc = 0.0, accabs = 0.0;
    for (int b = 0; b < KB; b++) {
        double part = 0.0, partabs = 0.0;
        for (int k = b * 128; k < b * 128 + 128; k++) {
            const double p = (double)oracle_e4m3_value(ar[k]) * (double)oracle_e4m3_value(wn[k]);
            part += p;
            partabs += fabs(p);
        }
        const double f = (double)a_scales[r * KB + b] * (double)wsc[b];
        acc += f * part;
        accabs += fabs(f) * partabs;
    }
    *val = acc;
    *mag = accabs;
}

/* Expert of a row: the e with off[e] <= r < off[e+1]; -1 past off[E]. */
static int row_expert(const int32_t* off, int E, int64_t r) {
    for (int e = 0; e < E; e++)
        if (r >= off[e] && r < off[e + 1]) return e;
    return -1;
}

/* Grouped GEMM over the segments moe dispatch lays out (expert e owns rows
 * [off[e], off[e+1]) of a, pad rows included):
 *   y[r, n] = bf16( sum_b a_s[r,b] w_s[e, n/128, b] sum_{k in b} a[r,k] w[e,n,k] )
 * a: E4M3 [rows, K], a_scales fp32 [rows, K/128], w: E4M3 [E, N, K] (K
 * contiguous), w_scales fp32 [E, N/128, K/128]. y64 and mag (may be NULL)
 * receive the fp64 sum and its absolute-value sum. Rows at or past off[E] are
 * not written. */
void oracle_grouped_gemm_fp8(const uint8_t* a, const float* a_scales, const int32_t* off, int E,
                             const uint8_t* w, const float* w_scales, int N, int K,
                             uint16_t* y, double* y64, double* mag) {
    for (int64_t r = 0; r < off[E]; r++) {
        const int e = row_expert(off, E, r);
        if (e < 0) continue; /* off[0] > 0: rows before the first segment */
        for (int n = 0; n < N; n++) {
            double v, m;
            gemm_entry(a, a_scales, w, w_scales, N, K, e, r, n, &v, &m);
            y[r * N + n] = oracle_bf16_from_double(v);
            if (y64) y64[r * N + n] = v;
            if (mag) mag[r * N + n] = m;
        }
    }
}

/* The same outputs at count chosen (row, column) positions; rows must lie
 * below off[E]. Outputs are [count]. */
void oracle_grouped_gemm_fp8_at(const uint8_t* a, const float* a_scales, const int32_t* off, int E,
                                const uint8_t* w, const float* w_scales, int N, int K,
                                const int64_t* rows, const int32_t* cols, int64_t count,
                                uint16_t* y, double* y64, double* mag) {
    for (int64_t i = 0; i < count; i++) {
        const int e = row_expert(off, E, rows[i]);
        double v = 0.0, m = 0.0;
        if (e >= 0)
            gemm_entry(a, a_scales, w, w_scales, N, K, e, rows[i], cols[i], &v, &m);
        y[i] = oracle_bf16_from_double(v);
        if (y64) y64[i] = v;
        if (mag) mag[i] = m;
    }
}
