// K1: router gate. Per token: top-k experts by logit and their softmax
// weights renormalised over the chosen k.
//
// "Efficient and portable mixture-of-experts communication", Introduction:
// the router is a small linear layer giving a probability distribution over
// experts; the top-K experts are used and the output is their weighted
// average. Softmax is strictly increasing, so ranking by logit is ranking by
// probability, and p_j / sum_chosen p_i = exp(l_j - m) / sum_chosen exp(l_i - m)
// for any m: the full-E denominator cancels and is never formed.
//
// Layout: a group of S lanes (S = next power of two >= E, at most 64) owns one
// token; lane g of the group holds experts g, g+S, g+2S, ... (NV per lane),
// so the logit row is read with coalesced loads. Each of the k rounds takes
// the group maximum of a packed (order key, ~expert) word with xor shuffles,
// and the lane owning the winner clears it. Round r's winner is kept by lane
// r % S in register slot r / S, which then writes slot r of the output.
#include "moe_device.h"
#include "launch.h"

namespace moe {

template <int NV>
__global__ __launch_bounds__(256) void k_route_topk(const float* __restrict__ logits,
                                                    int64_t T, int E, int k, int S,
                                                    int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane & (S - 1);
    const int tokens_per_wave = kWave / S;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    const int64_t t = wave * tokens_per_wave + lane / S;
    const bool live = t < T;

    uint64_t cand[NV];
    const float* row = logits + (live ? t : 0) * (int64_t)E;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int e = g + S * i;
        cand[i] = (live && e < E) ? topk_pack(row[e], e) : 0ull;
    }

    uint64_t sel[NV];
#pragma unroll
    for (int i = 0; i < NV; i++) sel[i] = 0ull;
    uint64_t first = 0ull;

    for (int r = 0; r < k; r++) {
        uint64_t best = cand[0];
#pragma unroll
        for (int i = 1; i < NV; i++) best = cand[i] > best ? cand[i] : best;
        for (int m = S >> 1; m > 0; m >>= 1) {
            const uint64_t o = shfl_xor_u64(best, m);
            best = o > best ? o : best;
        }
        if (r == 0) first = best;
        const int we = topk_expert(best);
        if ((we & (S - 1)) == g) {
            const int slot = we / S;
#pragma unroll
            for (int i = 0; i < NV; i++)
                if (i == slot) cand[i] = 0ull;
        }
        if ((r & (S - 1)) == g) {
            const int slot = r / S;
#pragma unroll
            for (int i = 0; i < NV; i++)
                if (i == slot) sel[i] = best;
        }
    }

    // weights: exp(l_j - l_max) / sum over the chosen, fp32, true division
    const float m = topk_value(first);
    float ex[NV];
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; i++) {
        const int r = g + S * i;
        ex[i] = (r < k) ? expf(topk_value(sel[i]) - m) : 0.0f;
        part += ex[i];
    }
    for (int msk = S >> 1; msk > 0; msk >>= 1) part += shfl_xor_f32(part, msk);

    if (live) {
#pragma unroll
        for (int i = 0; i < NV; i++) {
            const int r = g + S * i;
            if (r < k) {
                topk_idx[t * k + r] = topk_expert(sel[i]);
                topk_w[t * k + r] = ex[i] / part;
            }
        }
    }
}

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k,
                             int32_t* topk_idx, float* topk_w, hipStream_t stream,
                             LaunchInfo* info) {
    int S = 1;
    while (S < E && S < kWave) S <<= 1;
    const int nv = (E + S - 1) / S;
    const int threads = 256;
    const int64_t tokens_per_block = (threads / kWave) * (kWave / S);
    const int64_t blocks = (T + tokens_per_block - 1) / tokens_per_block;
    if (info) {
        info->grid = blocks;
        info->block = threads;
        info->lds = 0;
        info->param = S;
    }
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(threads);
    if (nv <= 1)
        k_route_topk<1><<<grid, block, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w);
    else if (nv <= 2)
        k_route_topk<2><<<grid, block, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w);
    else if (nv <= 4)
        k_route_topk<4><<<grid, block, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w);
    else if (nv <= 8)
        k_route_topk<8><<<grid, block, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w);
    else
        k_route_topk<16><<<grid, block, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w);
    return hipGetLastError();
}

}  // namespace moe
