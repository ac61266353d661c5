// K1: router gate. Per token: top-k experts by logit and their softmax
// weights renormalised over the chosen k.
//
// Two kernels. k_route_sort (k <= 8, E <= 768, E % 4 == 0, 16-byte aligned
// rows) sorts packed candidates with compare-exchange networks (topk_sort.h).
// k_route_topk below handles every other shape (k up to 1024, any E) in k
// rounds of a wave-wide maximum.
//
// "Efficient and portable mixture-of-experts communication", Introduction:
// the router is a small linear layer giving a probability distribution over
// experts; the top-K experts are used and the output is their weighted
// average. Softmax is strictly increasing, so ranking by logit is ranking by
// probability, and p_j / sum_chosen p_i = exp(l_j - m) / sum_chosen exp(l_i - m)
// for any m: the full-E denominator cancels and is never formed.
//
// Layout: a group of S lanes (S = next power of two >= E, at most 64) owns one
// token; lane g of the group holds experts g, g+S, g+2S, ... (NV per lane), so
// the logit row is read with coalesced loads. Each of the k rounds:
//   1. every lane takes the best of its remaining candidates (strict >, so
//      equal logits keep the lower expert),
//   2. the group maximum of the lanes' order keys (uint32 whose order is the
//      numeric order, -0 taken as +0) comes from a butterfly over DPP row
//      permutes and the gfx950 permlane16/permlane32 swaps (registers only),
//   3. a ballot of the lanes holding that maximum names the winner; if several
//      lanes tie, a second butterfly takes the smallest expert index,
//   4. the winning lane retires that candidate.
// Round r's winner is kept by lane r (by lane r % 64 in register r / 64 when
// k > 64), which then writes slot r of the output.
#include "moe_device.h"
#include "launch.h"
#include "topk_sort.h"

namespace moe {

namespace {

constexpr int kDppRowMirror = 0x140;   // lane i <-> 15-i within each row of 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Butterfly over aligned groups of S lanes; OP(a, b) must be commutative and
// associative. Every lane of a group ends with the group's result.
template <int S, typename F>
__device__ __forceinline__ uint32_t group_reduce(uint32_t v, F op) {
    if (S > 1) v = op(v, dpp_u32<kDppQuadXor1>(v));
    if (S > 2) v = op(v, dpp_u32<kDppQuadXor2>(v));
    if (S > 4) v = op(v, dpp_u32<kDppRowHalfMirror>(v));
    if (S > 8) v = op(v, dpp_u32<kDppRowMirror>(v));
    if (S > 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = op(p[0], p[1]);
    }
    if (S > 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = op(p[0], p[1]);
    }
    return v;
}

struct UMax {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
struct UMin {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; }
};
struct FAdd {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }
};

}  // namespace

constexpr int kRouteThreads = 256;

template <int S, int NV>
__global__ __launch_bounds__(kRouteThreads) void k_route_topk(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int ks, int n_shared,
                                                    float shared_w, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
    constexpr uint32_t kNone = 0xFFFFFFFFu;
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane & (S - 1);
    const int base = lane & ~(S - 1);          // first lane of this group
    constexpr int kTokensPerWave = kWave / S;
    const int64_t wave = (int64_t)blockIdx.x * (kRouteThreads / kWave) +
                         __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform
    const int64_t t = wave * kTokensPerWave + lane / S;
    const bool live = t < T;

    // candidates as order keys (unsigned order == numeric order, -0 == +0);
    // 0 marks an empty slot, real keys are never 0
    uint32_t c[NV];
    if constexpr (S == kWave) {
        // one token per wave: the row goes through a wave-uniform range
        // descriptor, so all NV loads issue back to back (lanes past the row,
        // or a token past T, read 0)
        const auto rs = range_rsrc(logits + (live ? t : 0) * (int64_t)E, live ? 4 * E : 0);
        uint32_t bits[NV];   // raw fp32 bit patterns
#pragma unroll
        for (int i = 0; i < NV; i++)
            bits[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * (g + S * i), 0, 0);
#pragma unroll
        for (int i = 0; i < NV; i++)
            c[i] = (live && g + S * i < E) ? order_key(__uint_as_float(bits[i])) : 0u;
    } else {
        // several tokens per wave, one candidate per lane
        static_assert(NV == 1, "groups narrower than a wave hold one candidate per lane");
        c[0] = (live && g < E) ? order_key(logits[t * (int64_t)E + g]) : 0u;
    }

    if constexpr (S == kWave) {
        // One token per wave. Round r's winner (key and expert, wave-uniform)
        // is written into lane r of sel_key / sel_e when r < 64; rounds past
        // 64 (only when k > 64) go to the per-slot registers below.
        uint32_t sel_key = 0u;
        int sel_e = 0;
        uint32_t hi_key[NV];
        int hi_e[NV];
#pragma unroll
        for (int i = 0; i < NV; i++) {
            hi_key[i] = 0u;
            hi_e[i] = 0;
        }
        uint32_t first = 0u;
        for (int r = 0; r < k; r++) {
            uint32_t best = c[0];
#pragma unroll
            for (int i = 1; i < NV; i++) best = best > c[i] ? best : c[i];
            const uint32_t m = group_reduce<S>(best, UMax());
            const uint64_t mask = __ballot(best == m);
            // the holding lane's first slot with the maximum (lowest expert)
            int slot = NV - 1;
#pragma unroll
            for (int i = NV - 2; i >= 0; i--) slot = c[i] == m ? i : slot;
            int we;
            if (__popcll(mask) == 1) {
                const int wl = (int)__builtin_ctzll(mask);
                we = wl + S * __builtin_amdgcn_readlane(slot, wl);
            } else {
                // several lanes hold the maximum: the smallest expert index wins
                we = (int)group_reduce<S>(best == m ? (uint32_t)(g + S * slot) : kNone, UMin());
            }
            const int clear = (lane == (we & (S - 1))) ? (int)((uint32_t)we / S) : NV;
#pragma unroll
            for (int i = 0; i < NV; i++) c[i] = (i == clear) ? 0u : c[i];
            if (r == 0) first = m;
            if (r < kWave) {
                sel_key = lane == r ? m : sel_key;
                sel_e = lane == r ? we : sel_e;
            } else if (lane == (r & (kWave - 1))) {
#pragma unroll
                for (int i = 1; i < NV; i++)
                    if (i == r / kWave) {
                        hi_key[i] = m;
                        hi_e[i] = we;
                    }
            }
        }
        // weights: exp(l_j - l_max) / sum over the chosen, fp32, true division
        const float lmax = key_value(first);
        const float ex0 = lane < k ? expf(key_value(sel_key) - lmax) : 0.0f;
        float part = ex0;
        float exh[NV];
#pragma unroll
        for (int i = 1; i < NV; i++) {
            exh[i] = (lane + kWave * i < k) ? expf(key_value(hi_key[i]) - lmax) : 0.0f;
            part += exh[i];
        }
        const float sum = __uint_as_float(group_reduce<S>(__float_as_uint(part), FAdd()));
        if (live) {
            if (lane < k) {
                topk_idx[t * ks + lane] = sel_e;
                topk_w[t * ks + lane] = ex0 / sum;
            }
#pragma unroll
            for (int i = 1; i < NV; i++) {
                const int r = lane + kWave * i;
                if (r < k) {
                    topk_idx[t * ks + r] = hi_e[i];
                    topk_w[t * ks + r] = exh[i] / sum;
                }
            }
            for (int sh = lane; sh < n_shared; sh += kWave) {
                topk_idx[t * ks + k + sh] = E + sh;
                topk_w[t * ks + k + sh] = shared_w;
            }
        }
    } else {
        // Groups narrower than a wave: one candidate per lane, so the lowest
        // holding lane of a group is its lowest expert.
        uint32_t sel_key = 0u;
        int sel_e = 0;
        uint32_t first = 0u;
        for (int r = 0; r < k; r++) {
            const uint32_t m = group_reduce<S>(c[0], UMax());
            const uint64_t mask = __ballot(c[0] == m && c[0] != 0u);
            const uint64_t gmask = (mask >> base) & ((1ull << S) - 1ull);
            const int we = gmask ? (int)__builtin_ctzll(gmask) : 0;
            if (g == we) c[0] = 0u;
            if (r == 0) first = m;
            if (g == r) {
                sel_key = m;
                sel_e = we;
            }
        }
        const float ex = g < k ? expf(key_value(sel_key) - key_value(first)) : 0.0f;
        const float sum = __uint_as_float(group_reduce<S>(__float_as_uint(ex), FAdd()));
        if (live && g < k) {
            topk_idx[t * ks + g] = sel_e;
            topk_w[t * ks + g] = ex / sum;
        }
        if (live)
            for (int sh = g; sh < n_shared; sh += S) {
                topk_idx[t * ks + k + sh] = E + sh;
                topk_w[t * ks + k + sh] = shared_w;
            }
    }
}

// Sorting-network path: S lanes per token, 256 / S tokens per block.
template <int S, int K>
__global__ __launch_bounds__(kRouteThreads) void k_route_sort(
    const float* __restrict__ logits, int64_t T, int E, int k, int ks, int n_shared,
    float shared_w, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int tl = threadIdx.x / S;
    const int g = threadIdx.x & (S - 1);
    const int64_t t = (int64_t)blockIdx.x * (kRouteThreads / S) + tl;
    const bool live = t < T;
    double list[K];
    route_token<S, K>(logits + (live ? t : 0) * (int64_t)E, live, E, g, list);
    if (live)
        write_route<S, K>(list, g, t, tl, E, k, ks, n_shared, shared_w, topk_idx, topk_w,
                          nullptr);
}

struct RouteArgs {
    const float* logits;
    int64_t T;
    int E, k, ks, n_shared;
    float shared_w;
    int32_t* topk_idx;
    float* topk_w;
};

template <int S, int NV>
static void launch_s(const RouteArgs& a, hipStream_t stream, int64_t blocks) {
    k_route_topk<S, NV><<<dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream>>>(
        a.logits, a.T, a.E, a.k, a.ks, a.n_shared, a.shared_w, a.topk_idx, a.topk_w);
}

template <int S, int K>
static void launch_sort(const RouteArgs& a, hipStream_t stream, int64_t blocks) {
    k_route_sort<S, K><<<dim3((unsigned)blocks), dim3(kRouteThreads), 0, stream>>>(
        a.logits, a.T, a.E, a.k, a.ks, a.n_shared, a.shared_w, a.topk_idx, a.topk_w);
}

template <int K>
static void launch_sort_k(int S, const RouteArgs& a, hipStream_t stream, int64_t blocks) {
    switch (S) {
        case 1: launch_sort<1, K>(a, stream, blocks); break;
        case 2: launch_sort<2, K>(a, stream, blocks); break;
        case 4: launch_sort<4, K>(a, stream, blocks); break;
        case 8: launch_sort<8, K>(a, stream, blocks); break;
        default: launch_sort<16, K>(a, stream, blocks); break;
    }
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int n_shared,
                             float shared_w, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream, LaunchInfo* info, bool run) {
    if (route_sort_applies(logits, E, k)) {
        const int S = route_lanes(T, E);
        const int64_t tokens_per_block = kRouteThreads / S;
        const int64_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
        if (info) *info = LaunchInfo{blocks, kRouteThreads, 0, S};
        if (!run || blocks == 0) return hipSuccess;
        const RouteArgs a{logits, T, E, k, k + n_shared, n_shared, shared_w, topk_idx, topk_w};
        switch (route_list_len(k)) {
            case 2: launch_sort_k<2>(S, a, stream, blocks); break;
            case 4: launch_sort_k<4>(S, a, stream, blocks); break;
            default: launch_sort_k<8>(S, a, stream, blocks); break;
        }
        return hipGetLastError();
    }
    int S = 1;
    while (S < E && S < kWave) S <<= 1;
    const int nv = (E + S - 1) / S;
    const int threads = kRouteThreads;
    const int64_t tokens_per_block = (threads / kWave) * (kWave / S);
    const int64_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
    if (info) *info = LaunchInfo{blocks, threads, 0, S};
    if (!run || blocks == 0) return hipSuccess;
    const RouteArgs a{logits, T, E, k, k + n_shared, n_shared, shared_w, topk_idx, topk_w};
    switch (S) {
        case 1: launch_s<1, 1>(a, stream, blocks); break;
        case 2: launch_s<2, 1>(a, stream, blocks); break;
        case 4: launch_s<4, 1>(a, stream, blocks); break;
        case 8: launch_s<8, 1>(a, stream, blocks); break;
        case 16: launch_s<16, 1>(a, stream, blocks); break;
        case 32: launch_s<32, 1>(a, stream, blocks); break;
        default:
            if (nv <= 1) launch_s<64, 1>(a, stream, blocks);
            else if (nv <= 2) launch_s<64, 2>(a, stream, blocks);
            else if (nv <= 4) launch_s<64, 4>(a, stream, blocks);
            else if (nv <= 8) launch_s<64, 8>(a, stream, blocks);
            else launch_s<64, 16>(a, stream, blocks);
    }
    return hipGetLastError();
}

// Redundant replicas: logical expert e owns physical experts
// replica_base[e] .. replica_base[e+1]-1 and token t uses copy t mod count.
__global__ __launch_bounds__(256) void k_route_replicas(int32_t* __restrict__ topk_idx, int64_t T,
                                                        int k, int E,
                                                        const int32_t* __restrict__ replica_base) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= T * k) return;
    const int e = topk_idx[i];
    if ((unsigned)e >= (unsigned)E) return;
    const int b = replica_base[e];
    const int n = replica_base[e + 1] - b;
    if (n <= 0) return;
    topk_idx[i] = b + (int)((i / k) % n);
}

hipError_t launch_route_replicas(int32_t* topk_idx, int64_t T, int k, int E,
                                 const int32_t* replica_base, hipStream_t stream) {
    const int64_t n = T * k;
    const int64_t blocks = (n + 255) / 256;
    if (blocks == 0) return hipSuccess;
    k_route_replicas<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(topk_idx, T, k, E,
                                                                      replica_base);
    return hipGetLastError();
}

}  // namespace moe
