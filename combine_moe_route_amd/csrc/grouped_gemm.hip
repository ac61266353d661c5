// Grouped GEMM over the padded FP8 segments written by the dispatch.
//
// Expert e owns rows [off[e], off[e+1]) of the dispatched activations a
// (E4M3, 1x128 block scales). Every row of that segment is multiplied by the
// expert's weight matrix w[e] (E4M3 [N, K], one fp32 scale per 128x128 block):
//
//   y[r, n] = bf16( sum_b a_s[r, b] w_s[e, n/128, b] sum_{k in block b} a[r, k] w[e, n, k] )
//
// This is the fine-grained FP8 GEMM of the DeepSeek-V3 report (section on
// quantisation and accumulation precision): the matrix cores sum one
// 128-element interval of the inner dimension, and that partial is scaled by
// both block scales and added into fp32 accumulators held in vector
// registers. On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers exactly one
// interval for a 16x16 output tile, so each MFMA result is promoted at once.
//
// Work split: segments are cut into 128-row tiles (a small kernel lists them
// from the device-side offsets, so the host never reads them); a workgroup
// computes a 128 x 256 output tile with 8 waves of 64 x 64. Both operands of
// each 128-wide k-block are staged through LDS (XOR-swizzled 16-byte chunks,
// double-buffered, one barrier per k-block).
#include "launch.h"
#include "moe_device.h"

namespace moe {
namespace {

constexpr int kBM = 128;             // rows per tile
constexpr int kBN = 256;             // output columns per tile
constexpr int kBK = 128;             // inner-dimension block (one scale interval)
constexpr int kGemmThreads = 512;    // 8 waves: 2 along rows x 4 along columns
constexpr int kTileListThreads = 1024;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tile list: tile t covers rows [row0, min(row0 + kBM, seg_end)) of expert e.
// Packed as int4 {row0, seg_end, e, 0}. Segment bounds are clamped to the
// row capacity, so no tile reaches past the buffers whatever the offsets
// hold. count[0] = number of tiles (at most max_tiles, which the host derives
// from the capacity).
__global__ __launch_bounds__(kTileListThreads) void k_gemm_tiles(
    const int32_t* __restrict__ off, int E, int max_rows, int max_tiles,
    int4* __restrict__ tiles, int32_t* __restrict__ count) {
    __shared__ int s_scan[kTileListThreads];
    const int e = threadIdx.x;
    int r0 = 0, r1 = 0, nt = 0;
    if (e < E) {
        r0 = min(max(off[e], 0), max_rows);
        r1 = min(max(off[e + 1], 0), max_rows);
        nt = r1 > r0 ? (r1 - r0 + kBM - 1) / kBM : 0;
    }
    s_scan[e] = nt;
    __syncthreads();
    for (int d = 1; d < kTileListThreads; d <<= 1) {
        const int v = e >= d ? s_scan[e - d] : 0;
        __syncthreads();
        s_scan[e] += v;
        __syncthreads();
    }
    const int base = s_scan[e] - nt;
    for (int i = 0; i < nt && base + i < max_tiles; i++)
        tiles[base + i] = make_int4(r0 + i * kBM, r1, e, 0);
    if (e == kTileListThreads - 1) count[0] = min(s_scan[e], max_tiles);
}

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kBK + ((chunk ^ (row & 7)) << 4);
}

__device__ __forceinline__ i32x8 frag(const uint8_t* s, int row, int half) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(s + swz(row, 2 * half));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(s + swz(row, 2 * half + 1));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm_fp8(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scales,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    uint16_t* __restrict__ y, int N, int K) {
    const int n_tiles_n = N / kBN;
    const int tile = blockIdx.x / n_tiles_n;
    const int nt = blockIdx.x - tile * n_tiles_n;
    if (tile >= tile_count[0]) return;
    const int4 td = tiles[tile];
    const int row0 = td.x, e = td.z;
    const int rows = min(kBM, td.y - row0);
    const int KB = K / kBK;
    const int n0 = nt * kBN;

    __shared__ __attribute__((aligned(16))) uint8_t sA[2][kBM * kBK];
    __shared__ __attribute__((aligned(16))) uint8_t sW[2][kBN * kBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 2, wn = wave & 3;

    // Rows past the tile's end read as zero through the descriptor bound.
    const __amdgpu_buffer_rsrc_t ra = range_rsrc(a + (int64_t)row0 * K, rows * K);
    const __amdgpu_buffer_rsrc_t rw = range_rsrc(w + ((int64_t)e * N + n0) * K, kBN * K);
    const __amdgpu_buffer_rsrc_t rsa = range_rsrc(a_scales + (int64_t)row0 * KB, rows * KB * 4);
    const float* wsc = w_scales + ((int64_t)e * (N / 128) + (n0 + wn * 64) / 128) * KB;

    // Global -> register staging: A 2 x 16 B, W 4 x 16 B per thread.
    int a_off[2], a_lds[2], w_off[4], w_lds[4];
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int idx = tid + i * kGemmThreads, r = idx >> 3, c = idx & 7;
        a_off[i] = r * K + c * 16;
        a_lds[i] = swz(r, c);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int idx = tid + i * kGemmThreads, r = idx >> 3, c = idx & 7;
        w_off[i] = r * K + c * 16;
        w_lds[i] = swz(r, c);
    }
    // Activation-scale rows this lane needs: one per 16-row fragment.
    int sa_off[4];
#pragma unroll
    for (int i = 0; i < 4; i++) sa_off[i] = (wm * 64 + i * 16 + (lane & 15)) * KB * 4;

    // Two register stages: k-block b+2 is fetched while b is computed and
    // b+1 (fetched one k-block earlier) is written to the other LDS buffer.
    u32x4 ga[2][2], gw[2][4];
    float sa[2][4], sw[2];
    auto fetch = [&](int st, int b) {
#pragma unroll
        for (int i = 0; i < 2; i++)
            ga[st][i] = __builtin_amdgcn_raw_buffer_load_b128(ra, a_off[i] + b * kBK, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++)
            gw[st][i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_off[i] + b * kBK, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++)
            sa[st][i] = __uint_as_float(
                __builtin_amdgcn_raw_buffer_load_b32(rsa, sa_off[i] + b * 4, 0, 0));
        sw[st] = wsc[b];
    };
    auto stash = [&](int st, int buf) {
#pragma unroll
        for (int i = 0; i < 2; i++) *reinterpret_cast<u32x4*>(&sA[buf][a_lds[i]]) = ga[st][i];
#pragma unroll
        for (int i = 0; i < 4; i++) *reinterpret_cast<u32x4*>(&sW[buf][w_lds[i]]) = gw[st][i];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int half = lane >> 4;
    auto compute = [&](int buf, const float* fs) {
        i32x8 xf[4], wf[4];
#pragma unroll
        for (int i = 0; i < 4; i++) xf[i] = frag(sA[buf], wm * 64 + i * 16 + (lane & 15), half);
#pragma unroll
        for (int j = 0; j < 4; j++) wf[j] = frag(sW[buf], wn * 64 + j * 16 + (lane & 15), half);
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    wf[j], xf[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; r++) acc[i][j][r] = fmaf(p[r], fs[i], acc[i][j][r]);
            }
    };

    fetch(0, 0);
    if (KB > 1) fetch(1, 1);
    stash(0, 0);
    __syncthreads();

    // Stage st of the registers holds k-block b while b is computed from LDS
    // buffer b & 1; the loop body is written out for b even and b odd so
    // that every register index is a constant.
    for (int b = 0; b < KB; b += 2) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; i++) f[i] = sa[0][i] * sw[0];
        if (b + 2 < KB) fetch(0, b + 2);
        compute(0, f);
        if (b + 1 < KB) stash(1, 1);
        __syncthreads();
        if (b + 1 >= KB) break;

#pragma unroll
        for (int i = 0; i < 4; i++) f[i] = sa[1][i] * sw[1];
        if (b + 3 < KB) fetch(1, b + 3);
        compute(1, f);
        if (b + 2 < KB) stash(0, 0);
        __syncthreads();
    }

    // Lane holds, for fragment pair (i, j), row 16i + lane%16 and the four
    // consecutive columns 16j + 4*(lane/16) .. +3.
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = wm * 64 + i * 16 + (lane & 15);
        if (r >= rows) continue;
        uint16_t* yr = y + (int64_t)(row0 + r) * N + n0 + wn * 64 + 4 * half;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint2 v = make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                                       pack_bf16x2(acc[i][j][2], acc[i][j][3]));
            *reinterpret_cast<uint2*>(yr + j * 16) = v;
        }
    }
}

}  // namespace

int64_t gemm_max_tiles(int64_t max_rows, int E) { return (max_rows + kBM - 1) / kBM + E; }

size_t gemm_workspace_bytes(int64_t max_rows, int E) {
    return 256 + (size_t)gemm_max_tiles(max_rows, E) * sizeof(int4);
}

hipError_t launch_grouped_gemm_fp8(const void* a, const float* a_scales,
                                   const int32_t* expert_offsets, const void* w,
                                   const float* w_scales, int E, int N, int K, int64_t max_rows,
                                   void* y, void* workspace, hipStream_t stream,
                                   LaunchInfo info[2]) {
    const int64_t max_tiles = gemm_max_tiles(max_rows, E);
    int32_t* count = static_cast<int32_t*>(workspace);
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256);
    hipLaunchKernelGGL(k_gemm_tiles, dim3(1), dim3(kTileListThreads), 0, stream, expert_offsets,
                       E, (int)max_rows, (int)max_tiles, tiles, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t grid = max_tiles * (N / kBN);
    hipLaunchKernelGGL(k_grouped_gemm_fp8, dim3((unsigned)grid), dim3(kGemmThreads), 0, stream,
                       static_cast<const uint8_t*>(a), a_scales, static_cast<const uint8_t*>(w),
                       w_scales, tiles, count, static_cast<uint16_t*>(y), N, K);
    if (info) {
        info[0] = LaunchInfo{1, kTileListThreads, 0, 0};
        info[1] = LaunchInfo{grid, kGemmThreads, 2 * (kBM + kBN) * kBK, kBN};
    }
    return hipGetLastError();
}

}  // namespace moe
