// Combine with sender-side partial sums, as a sending and a receiving half.
#include "moe_device.h"
#include "launch.h"

namespace moe {

namespace {
constexpr int kCombineThreads = 128;
constexpr int kCombineWaves = kCombineThreads / kWave;
constexpr int kSlotBatch = 8;
}  // namespace

// Combine split into a sending and a receiving half with partial sums on the
// sending side ("Enabling trillion-parameter models on AWS EFA", Evaluation:
// DeepEP accumulates on the sender to cut the bytes transferred, which may
// cost accuracy; the Perplexity kernels accumulate on the receiver only). A
// destination group stands for the rank that hosts a range of experts.
//
// send: one wave per (token, chunk). For each distinct group of the token's
// live slots, in ascending group order, the weighted sum of that group's rows
// (fp32, slot order) is rounded to bf16 (the wire format) and written as the
// token's next partial row: partial[t, p] at (t*k + p) * H. count[t] = rows.
// recv: y[t] = bf16(sum over p < count[t] of partial[t, p]) in fp32.

__device__ __forceinline__ void fma8(float* acc, float w, const uint4& v) {
    float f[8];
    unpack8(v, f);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = fmaf(w, f[i], acc[i]);
}

__device__ __forceinline__ uint4 pack8(const float* acc) {
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    return o;
}

__global__ __launch_bounds__(kCombineThreads) void k_combine_send(
    const uint16_t* __restrict__ expert_out, const int32_t* __restrict__ dst_row,
    const float* __restrict__ topk_w, const int32_t* __restrict__ topk_idx, int64_t T, int H,
    int E, int k, int per_group, uint16_t* __restrict__ partial, int32_t* __restrict__ count) {
    const int C = H / 8;
    const int CW = (C + kWave - 1) / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kCombineWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = gw / CW;
    if (t >= T) return;
    const int chunk = (int)(gw - t * CW);
    const int u = chunk * kWave + lane;
    const int row_bytes = 2 * H;
    const unsigned char* eo = reinterpret_cast<const unsigned char*>(expert_out);
    unsigned char* pb = reinterpret_cast<unsigned char*>(partial);
    const int32_t* rows = dst_row + t * k;
    const float* ws = topk_w + t * k;
    const int32_t* ids = topk_idx + t * k;

    // group of every live slot (-1 for dropped slots)
    auto group_of = [&](int j) -> int {
        const int e = ids[j];
        return (rows[j] >= 0 && (unsigned)e < (unsigned)E) ? e / per_group : -1;
    };
    int pos = 0;
    if (k <= kSlotBatch) {
        // all rows in registers, then one pass per distinct group
        int r[kSlotBatch], g[kSlotBatch];
        float wj[kSlotBatch];
        uint4 v[kSlotBatch];
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; jj++) {
            r[jj] = jj < k ? rows[jj] : -1;
            wj[jj] = jj < k ? ws[jj] : 0.0f;
            g[jj] = jj < k ? group_of(jj) : -1;
            v[jj] = load16_nt(range_rsrc(eo + (g[jj] >= 0 ? (int64_t)r[jj] * row_bytes : 0),
                                         g[jj] >= 0 ? row_bytes : 0),
                              16 * u);
        }
        int prev = -1;
        for (;;) {
            int gs = 0x7FFFFFFF;
#pragma unroll
            for (int jj = 0; jj < kSlotBatch; jj++)
                if (g[jj] > prev && g[jj] < gs) gs = g[jj];
            if (gs == 0x7FFFFFFF) break;
            float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int jj = 0; jj < kSlotBatch; jj++)
                if (g[jj] == gs) fma8(acc, wj[jj], v[jj]);
            if (u < C) store16_nt(pb + (t * k + pos) * (int64_t)row_bytes + 16 * (int64_t)u, pack8(acc));
            pos++;
            prev = gs;
        }
    } else {
        // many slots: one pass over the slots per distinct group
        int prev = -1;
        for (;;) {
            int gs = 0x7FFFFFFF;
            for (int j = 0; j < k; j++) {
                const int gj = group_of(j);
                if (gj > prev && gj < gs) gs = gj;
            }
            if (gs == 0x7FFFFFFF) break;
            float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
            for (int j = 0; j < k; j++) {
                if (group_of(j) != gs) continue;
                fma8(acc, ws[j],
                     load16_nt(range_rsrc(eo + (int64_t)rows[j] * row_bytes, row_bytes), 16 * u));
            }
            if (u < C) store16_nt(pb + (t * k + pos) * (int64_t)row_bytes + 16 * (int64_t)u, pack8(acc));
            pos++;
            prev = gs;
        }
    }
    if (chunk == 0 && lane == 0) count[t] = pos;
}

__global__ __launch_bounds__(kCombineThreads) void k_combine_recv(
    const uint16_t* __restrict__ partial, const int32_t* __restrict__ count, int64_t T, int H,
    int k, uint16_t* __restrict__ y) {
    const int C = H / 8;
    const int CW = (C + kWave - 1) / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kCombineWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = gw / CW;
    if (t >= T) return;
    const int u = (int)(gw - t * CW) * kWave + lane;
    const int row_bytes = 2 * H;
    int n = count[t];
    n = n < 0 ? 0 : (n > k ? k : n);
    // the token's used partial rows as one range: reads past them give zeros
    const auto rs = range_rsrc(reinterpret_cast<const unsigned char*>(partial) +
                                   t * k * (int64_t)row_bytes,
                               n * row_bytes);
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < n; p0 += kSlotBatch) {
        uint4 v[kSlotBatch];
#pragma unroll
        for (int pp = 0; pp < kSlotBatch; pp++)
            v[pp] = load16_nt(rs, (p0 + pp < n) ? (p0 + pp) * row_bytes + 16 * u : n * row_bytes);
#pragma unroll
        for (int pp = 0; pp < kSlotBatch; pp++)
            if (p0 + pp < n) {
                float f[8];
                unpack8(v[pp], f);
#pragma unroll
                for (int i = 0; i < 8; i++) acc[i] += f[i];
            }
    }
    if (u < C)
        store16_nt(reinterpret_cast<unsigned char*>(y) + t * (int64_t)row_bytes + 16 * (int64_t)u,
                   pack8(acc));
}

hipError_t launch_combine_send(const void* expert_out, const int32_t* dst_row,
                               const float* topk_w, const int32_t* topk_idx, int64_t T, int H,
                               int E, int k, int groups, void* partial, int32_t* count,
                               hipStream_t stream, LaunchInfo* info, bool run) {
    const int CW = (H / 8 + kWave - 1) / kWave;
    const int64_t blocks = (T * CW + kCombineWaves - 1) / kCombineWaves;
    if (info) *info = LaunchInfo{blocks, kCombineThreads, 0, CW};
    if (!run || blocks == 0) return hipSuccess;
    k_combine_send<<<dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream>>>(
        static_cast<const uint16_t*>(expert_out), dst_row, topk_w, topk_idx, T, H, E, k,
        E / groups, static_cast<uint16_t*>(partial), count);
    return hipGetLastError();
}

hipError_t launch_combine_recv(const void* partial, const int32_t* count, int64_t T, int H,
                               int k, void* y, hipStream_t stream, LaunchInfo* info,
                               bool run) {
    const int CW = (H / 8 + kWave - 1) / kWave;
    const int64_t blocks = (T * CW + kCombineWaves - 1) / kCombineWaves;
    if (info) *info = LaunchInfo{blocks, kCombineThreads, 0, CW};
    if (!run || blocks == 0) return hipSuccess;
    k_combine_recv<<<dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream>>>(
        static_cast<const uint16_t*>(partial), count, T, H, k, static_cast<uint16_t*>(y));
    return hipGetLastError();
}

}  // namespace moe
