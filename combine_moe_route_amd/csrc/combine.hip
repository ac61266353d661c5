// K5: combine. y[t] = bf16( sum_j w[t,j] * expert_out[dst_row[t,j]] ), fp32
// accumulation in slot order, one rounding to bf16.
//
// "Efficient and portable mixture-of-experts communication", Combine: the
// receiving kernel reads each expert's row through the routing table and
// weights it by the router's weight, writing into caller-owned tensors.
// "Enabling trillion-parameter models on AWS EFA", Evaluation: accumulation
// happens only on the receiving side (no sender-side partial sums).
//
// Layout: one wave per (token, 64 x 16-byte chunk of the row). The token's
// k row indices and weights are wave-uniform and come in through scalar
// loads; each lane then issues up to 8 independent 16-byte row loads before
// any arithmetic, so a wave keeps 8 KB of gathers in flight. Loads and the
// output store carry the non-temporal hint: every byte is touched once, and
// on MI355X streaming accesses sustain clearly more HBM bandwidth than
// cached ones for this 8-to-1 gather.
//
// Also the stand-in experts used by tests and the benchmark around the path.
#include "moe_device.h"
#include "launch.h"

namespace moe {

// Two waves per block: at both prefill shapes 128-thread blocks ran the
// combine 2-3 % faster than 64-, 256- or 512-thread blocks (same-box traces).
constexpr int kCombineThreads = 128;
constexpr int kCombineWaves = kCombineThreads / kWave;
constexpr int kSlotBatch = 8;

__global__ __launch_bounds__(kCombineThreads) void k_combine(const uint16_t* __restrict__ expert_out,
                                                             const int32_t* __restrict__ dst_row,
                                                             const float* __restrict__ topk_w,
                                                             int64_t T, int H, int k,
                                                             uint16_t* __restrict__ y) {
    const int C = H / 8;                        // 16-byte units per row
    const int CW = (C + kWave - 1) / kWave;     // waves per token
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gw = (int64_t)blockIdx.x * kCombineWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = gw / CW;
    if (t >= T) return;
    const int u = (int)(gw - t * CW) * kWave + lane;
    const int row_bytes = 2 * H;
    const unsigned char* eo = reinterpret_cast<const unsigned char*>(expert_out);
    const int32_t* rows = dst_row + t * k;
    const float* ws = topk_w + t * k;

    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.0f;

    for (int j0 = 0; j0 < k; j0 += kSlotBatch) {
        // routing table (scalar loads), then all row gathers, then the
        // arithmetic in slot order. Each gather goes through a buffer
        // descriptor spanning exactly the expert row: a dropped slot gets an
        // empty descriptor and lanes past the row end read past num_records,
        // so both read zeros without a branch.
        int r[kSlotBatch];
        float wj[kSlotBatch];
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; jj++) {
            const bool in = (j0 + kSlotBatch <= k) || (j0 + jj < k);
            r[jj] = in ? rows[j0 + jj] : -1;
            wj[jj] = in ? ws[j0 + jj] : 0.0f;
        }
        uint4 v[kSlotBatch];
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; jj++) {
            const bool live = r[jj] >= 0;
            if (!live) wj[jj] = 0.0f;
            v[jj] = load16_nt(range_rsrc(eo + (live ? (int64_t)r[jj] * row_bytes : 0),
                                         live ? row_bytes : 0),
                              16 * u);
        }
#pragma unroll
        for (int jj = 0; jj < kSlotBatch; jj++) {
            float f[8];
            unpack8(v[jj], f);
#pragma unroll
            for (int i = 0; i < 8; i++) acc[i] = fmaf(wj[jj], f[i], acc[i]);
        }
    }
    if (u < C) {
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        store16_nt(reinterpret_cast<unsigned char*>(y) + t * (int64_t)row_bytes + 16 * (int64_t)u, o);
    }
}

hipError_t launch_combine(const void* expert_out, const int32_t* dst_row, const float* topk_w,
                          int64_t T, int H, int k, void* y, hipStream_t stream,
                          LaunchInfo* info, bool run) {
    const int C = H / 8;
    const int CW = (C + kWave - 1) / kWave;
    const int64_t waves = T * CW;
    const int64_t blocks = (waves + kCombineWaves - 1) / kCombineWaves;
    if (info) *info = LaunchInfo{blocks, kCombineThreads, 0, CW};
    if (!run || blocks == 0) return hipSuccess;
    k_combine<<<dim3((unsigned)blocks), dim3(kCombineThreads), 0, stream>>>(
        static_cast<const uint16_t*>(expert_out), dst_row, topk_w, T, H, k,
        static_cast<uint16_t*>(y));
    return hipGetLastError();
}

// ---------------------------------------------------------------- harness experts

constexpr int kExpertThreads = 256;

// One block per row (grid-stride). Row r of expert e: bf16(v * c_e).
__global__ __launch_bounds__(kExpertThreads) void k_expert_scale(
    const unsigned char* __restrict__ disp, const float* __restrict__ disp_scales,
    const int32_t* __restrict__ row_src, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ expert_offsets, int64_t max_rows, int H, int E, int fp8,
    int identity, uint16_t* __restrict__ expert_out) {
    const int64_t used = expert_offsets[E];
    const int C = H / 8;
    const int nb = H / 128;
    for (int64_t r = blockIdx.x; r < used && r < max_rows; r += gridDim.x) {
        const int src = row_src[r];
        float c = 0.0f;
        if (src >= 0) {
            const int e = topk_idx[src];
            c = identity ? 1.0f : (float)(e + 1) / (float)E;
        }
        uint4* o = reinterpret_cast<uint4*>(expert_out + r * (int64_t)H);
        for (int u = threadIdx.x; u < C; u += kExpertThreads) {
            if (src < 0) {
                o[u] = make_uint4(0u, 0u, 0u, 0u);
                continue;
            }
            float f[8];
            if (fp8) {
                const uint2 q = *reinterpret_cast<const uint2*>(disp + r * (int64_t)H + 8 * (int64_t)u);
                const float s = disp_scales[r * nb + (8 * u) / 128];
#pragma unroll
                for (int i = 0; i < 4; i++) f[i] = e4m3_to_f32(q.x, i) * s;
#pragma unroll
                for (int i = 0; i < 4; i++) f[4 + i] = e4m3_to_f32(q.y, i) * s;
            } else {
                const uint4 v = *reinterpret_cast<const uint4*>(disp + r * 2 * (int64_t)H + 16 * (int64_t)u);
                unpack8(v, f);
            }
            uint4 out;
            out.x = pack_bf16x2(f[0] * c, f[1] * c);
            out.y = pack_bf16x2(f[2] * c, f[3] * c);
            out.z = pack_bf16x2(f[4] * c, f[5] * c);
            out.w = pack_bf16x2(f[6] * c, f[7] * c);
            o[u] = out;
        }
    }
}

hipError_t launch_expert_scale(const void* disp, const float* disp_scales,
                               const int32_t* row_src, const int32_t* topk_idx,
                               const int32_t* expert_offsets, int64_t max_rows, int H,
                               int E, bool fp8, bool identity, void* expert_out,
                               hipStream_t stream) {
    if (max_rows <= 0) return hipSuccess;
    const int64_t blocks = max_rows < 65536 ? max_rows : 65536;
    k_expert_scale<<<dim3((unsigned)blocks), dim3(kExpertThreads), 0, stream>>>(
        static_cast<const unsigned char*>(disp), disp_scales, row_src, topk_idx, expert_offsets,
        max_rows, H, E, fp8 ? 1 : 0, identity ? 1 : 0, static_cast<uint16_t*>(expert_out));
    return hipGetLastError();
}

}  // namespace moe
