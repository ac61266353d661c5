// Top-k of a logit row by sorting networks on packed candidates.
//
// "Efficient and portable mixture-of-experts communication", Introduction:
// the router's scores are a probability distribution over the experts and the
// top-K experts are kept; softmax is strictly increasing, so the ranking is
// the ranking of the logits.
//
// Each candidate (logit l, expert e) is packed into one double whose order is
// the ranking order: exponent fixed at 1 (so every value lies in [2, 4), no
// sign, no subnormal, no NaN) and a 52-bit mantissa
//   order_key(l) (32 bits) | 0 (10 bits) | 1023 - e (10 bits),
// where order_key is the uint32 whose unsigned order is the numeric order of
// the fp32 logit with -0 taken as +0. A larger logit gives a larger double;
// equal logits give the larger double to the lower expert. All candidates of
// a row are distinct, so plain v_max_f64 / v_min_f64 compare-exchanges sort
// them exactly, ties included, and the expert travels inside the key.
// 2.0 (key 0) lies below every real candidate (finite logits have keys of at
// least 0x00800000) and pads lists and rows.
//
// A token is owned by S adjacent lanes (S a power of two, at most 16, inside
// one DPP row). Lane g holds the 16-byte chunks g, g+S, g+2S, ... of the row.
// It sorts its candidates in groups of K with a bitonic network and keeps the
// best K in a sorted list (merge of two sorted lists: elementwise maximum of
// one list and the other reversed, which is bitonic, then a bitonic half
// cleaner). The S lanes' lists are then merged by a butterfly over DPP lane
// permutes, after which every lane of the group holds the token's top K.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr double kCandNone = 2.0;
// 16-byte chunks of the logit row a lane can hold (48 candidates).
constexpr int kRouteChunks = 12;

__device__ __forceinline__ double cand_pack(float v, int e) {
    const uint32_t key = order_key(v);
    // {0x400, key} >> 12 keeps 0x40000000 | key >> 12: exponent field 0x400
    const uint32_t hi = __builtin_amdgcn_alignbit(0x400u, key, 12);
    const uint32_t lo = (key << 20) | (uint32_t)(1023 - e);
    return __hiloint2double((int)hi, (int)lo);
}

__device__ __forceinline__ uint32_t cand_key(double d) {
    return ((uint32_t)__double2hiint(d) << 12) | ((uint32_t)__double2loint(d) >> 20);
}

__device__ __forceinline__ int cand_expert(double d) {
    return 1023 - (int)((uint32_t)__double2loint(d) & 1023u);
}

// Maximum and minimum of two packed candidates. The packed values are never
// NaN (their exponent field is fixed), so the plain VALU instructions are
// used directly: fmax / fmin would add a NaN-quieting pass over every operand
// that the compiler cannot prove canonical (all of them, since they are built
// from integer operations).
__device__ __forceinline__ double dmax(double a, double b) {
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ double dmin(double a, double b) {
    double r;
    asm("v_min_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// a <- larger, b <- smaller
__device__ __forceinline__ void cmpx(double& a, double& b) {
    const double hi = dmax(a, b);
    const double lo = dmin(a, b);
    a = hi;
    b = lo;
}

// Bitonic sort of K values, descending.
template <int K>
__device__ __forceinline__ void sort_desc(double (&v)[K]) {
#pragma unroll
    for (int blk = 2; blk <= K; blk <<= 1)
#pragma unroll
        for (int j = blk >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < K; i++) {
                const int l = i ^ j;
                if (l > i) {
                    if ((i & blk) == 0) cmpx(v[i], v[l]);
                    else cmpx(v[l], v[i]);
                }
            }
}

// a <- the K largest of a and b, descending; a and b sorted descending.
template <int K>
__device__ __forceinline__ void merge_top(double (&a)[K], const double (&b)[K]) {
#pragma unroll
    for (int i = 0; i < K; i++) a[i] = dmax(a[i], b[K - 1 - i]);
#pragma unroll
    for (int j = K >> 1; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < K; i++) {
            const int l = i ^ j;
            if (l > i) cmpx(a[i], a[l]);
        }
}

// The value of lane (lane ^ D) inside an aligned group of 2D lanes (D < 16),
// through a DPP permute: xor 1, xor 2, then mirrors within 8 and within 16
// lanes (after the earlier rounds every lane of a half holds the same list,
// so any partner in the other half serves).
template <int D>
__device__ __forceinline__ double dpp_partner(double v) {
    constexpr int ctrl = D == 1 ? 0xB1 : D == 2 ? 0x4E : D == 4 ? 0x141 : 0x140;
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), ctrl, 0xF, 0xF, false);
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), ctrl, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

template <int D, int K>
__device__ __forceinline__ void merge_with_partner(double (&list)[K]) {
    double other[K];
#pragma unroll
    for (int q = 0; q < K; q++) other[q] = dpp_partner<D>(list[q]);
    merge_top<K>(list, other);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Top K candidates of the token owned by this lane's group of S lanes (lane
// g of the group). row: the token's logits (16-byte aligned, E % 4 == 0);
// live == false gives a list of padding. Every lane of the group must run
// this together (the butterfly reads the other lanes' registers).
template <int S, int K>
__device__ __forceinline__ void route_token(const float* __restrict__ row, bool live, int E, int g,
                                            double (&list)[K]) {
    static_assert(S >= 1 && S <= 16 && (S & (S - 1)) == 0, "S: power of two up to 16");
    static_assert(K == 2 || K == 4 || K == 8, "K: 2, 4 or 8");
    constexpr int M = 4 * kRouteChunks;   // candidates per lane
    // every chunk load is issued before any arithmetic; chunk i of lane g
    // holds experts 4(g + S i) .. 4(g + S i) + 3
    f32x4 ch[kRouteChunks];
    const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
#pragma unroll
    for (int i = 0; i < kRouteChunks; i++) {
        ch[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const int c = g + S * i;
        if (live && 4 * c < E) ch[i] = __builtin_nontemporal_load(row4 + c);
    }
#pragma unroll
    for (int q = 0; q < K; q++) list[q] = kCandNone;
#pragma unroll
    for (int m0 = 0; m0 < M; m0 += K) {
        // group-uniform: past the row's end no lane holds candidates
        if (4 * S * (m0 / 4) >= E) continue;
        double grp[K];
#pragma unroll
        for (int q = 0; q < K; q++) {
            const int m = m0 + q;
            const int e = 4 * (g + S * (m / 4)) + (m % 4);
            grp[q] = (live && e < E) ? cand_pack(ch[m / 4][m % 4], e) : kCandNone;
        }
        sort_desc<K>(grp);
        if (m0 == 0) {
#pragma unroll
            for (int q = 0; q < K; q++) list[q] = grp[q];
        } else {
            merge_top<K>(list, grp);
        }
    }
    if (S > 1) merge_with_partner<1, K>(list);
    if (S > 2) merge_with_partner<2, K>(list);
    if (S > 4) merge_with_partner<4, K>(list);
    if (S > 8) merge_with_partner<8, K>(list);
}

// Weights of the first k entries of a top-K list: exp(l_j - l_0) over their
// sum (fp32, slot order, true division, so k == 1 gives exactly 1). Lane g
// of the group writes slots j with j % S == g: topk_idx / topk_w at
// [t * ks + j]; slots k .. k + n_shared - 1 hold the always-chosen experts
// E .. E + n_shared - 1 with weight shared_w. s_ids, when given, receives the
// routed experts at [tl * k + j].
template <int S, int K>
__device__ __forceinline__ void write_route(const double (&list)[K], int g, int64_t t, int tl,
                                            int E, int k, int ks, int n_shared, float shared_w,
                                            int32_t* __restrict__ topk_idx,
                                            float* __restrict__ topk_w, int32_t* s_ids) {
    const float m = key_value(cand_key(list[0]));
    float ex[K];
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < K; j++) {
        ex[j] = 0.0f;
        if (j < k) {
            ex[j] = expf(key_value(cand_key(list[j])) - m);
            sum += ex[j];
        }
    }
#pragma unroll
    for (int j = 0; j < K; j++) {
        if (j < k && (j % S) == g) {
            const int e = cand_expert(list[j]);
            topk_idx[t * ks + j] = e;
            topk_w[t * ks + j] = ex[j] / sum;
            if (s_ids) s_ids[tl * k + j] = e;
        }
    }
    for (int sh = g; sh < n_shared; sh += S) {
        topk_idx[t * ks + k + sh] = E + sh;
        topk_w[t * ks + k + sh] = shared_w;
    }
}

// Lanes per token for T rows of E logits: each lane holds at most
// kRouteChunks chunks of 4; beyond that, more lanes per token (shorter
// per-lane work, one more merge round each doubling) while the grid has
// fewer than about 2048 waves, so that small batches still spread over the
// chip.
inline int route_lanes(int64_t T, int E) {
    int S = 1;
    while (S < 16 && 4 * kRouteChunks * S < E) S <<= 1;
    while (S < 16 && 4 * S < E && T * S < 2048 * 64) S <<= 1;
    return S;
}

// The sorting-network path applies to k <= 8, E % 4 == 0 (16-byte chunks),
// rows short enough for 16 lanes, and a 16-byte aligned logit array.
inline bool route_sort_applies(const float* logits, int E, int k) {
    return k <= 8 && E % 4 == 0 && E <= 16 * 4 * kRouteChunks &&
           (reinterpret_cast<uintptr_t>(logits) & 15u) == 0;
}

inline int route_list_len(int k) { return k <= 2 ? 2 : k <= 4 ? 4 : 8; }

}  // namespace moe
