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
// interval for a 16x16 output tile, so each MFMA result is promoted right
// away (the last row group of a k-block at the start of the next one).
//
// Work split: segments are cut into row tiles (a small kernel lists them
// from the device-side offsets, so the host never reads them); a workgroup
// computes one tile of 256 output columns with 8 waves. Tiles are 256 rows
// when the capacity holds prefill-sized segments and 128 rows otherwise (the
// shapes are described at Shape below). Each 128-wide k-block of both
// operands and of the activation scales goes from memory straight into LDS
// with buffer_load ... lds (no staging registers), into a ring of stages, and
// the loads of a later k-block are issued at the top of the current one,
// right after the barrier that frees their stage. One barrier
// per k-block; the wait before it counts this wave's outstanding DMA
// explicitly, because the fence of __syncthreads would drain the prefetch as
// well.
#include "launch.h"
#include "moe_device.h"

#include <type_traits>

namespace moe {
namespace {

constexpr int kBMin = 128;           // rows per tile of the smaller shape (sizes the tile list)
constexpr int kBN = 256;             // output columns per tile
constexpr int kBK = 128;             // inner-dimension block (one scale interval)
constexpr int kGemmThreads = 512;    // 8 waves: 2 along rows x 4 along columns
constexpr int kTileListThreads = 1024;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tile list: tile t covers rows [row0, min(row0 + bm, seg_end)) of expert e.
// Packed as int4 {row0, seg_end, e, 0}. Segment bounds are clamped to the
// row capacity, so no tile reaches past the buffers whatever the offsets
// hold. count[0] = number of tiles (at most max_tiles, which the host derives
// from the capacity).
__global__ __launch_bounds__(kTileListThreads) void k_gemm_tiles(
    const int32_t* __restrict__ off, int E, int max_rows, int max_tiles, int bm,
    int4* __restrict__ tiles, int32_t* __restrict__ count) {
    __shared__ int s_scan[kTileListThreads];
    const int e = threadIdx.x;
    int r0 = 0, r1 = 0, nt = 0;
    if (e < E) {
        r0 = min(max(off[e], 0), max_rows);
        r1 = min(max(off[e + 1], 0), max_rows);
        nt = r1 > r0 ? (r1 - r0 + bm - 1) / bm : 0;
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
        tiles[base + i] = make_int4(r0 + i * bm, r1, e, 0);
    if (e == kTileListThreads - 1) count[0] = min(s_scan[e], max_tiles);
}

// LDS layout of a staged k-block: row-major 128-byte rows of 16-byte chunks,
// chunk c of row r stored at chunk c ^ key(r), key(r) = (r & 7) ^ ((r >> 3) & 1).
// A fragment read has lanes on consecutive rows at the same logical chunk.
// Any 8 consecutive rows from a multiple of 8 get 8 distinct physical chunks,
// so 8 lanes cover 128 bytes of distinct banks; and within 16 rows from a
// multiple of 16 the even rows, like the odd ones, also get 8 distinct chunks,
// so 16 lanes cover 256 bytes of distinct banks when a row's two halves of
// the bank space alternate. (A swizzle on (r >> 1) alone left rows r and r + 1
// on the same chunk; the counters showed about one bank-conflict cycle per LDS
// access.)
__device__ __forceinline__ int chunk_key(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kBK + ((chunk ^ chunk_key(row)) << 4);
}

[[maybe_unused]] __device__ __forceinline__ i32x8 frag(const uint8_t* s, int row, int half) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(s + swz(row, 2 * half));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(s + swz(row, 2 * half + 1));
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Wait until at most n vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima, i.e. not waited for).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// Workgroup barrier without the release/acquire fences of __syncthreads
// (those would wait for every load in flight, including the LDS DMA of the
// k-blocks being prefetched). The memory clobber keeps the compiler from
// moving LDS accesses across it; completion of the DMA a wave needs is
// waited for explicitly before it.
[[maybe_unused]] __device__ __forceinline__ void lds_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

// Tile shapes. Both use 8 waves and 256 output columns; the row count picks
// the rest:
//   128 rows: 2 x 4 waves of 64 x 64, three LDS stages (48 KB each), two
//             k-blocks in flight while one is computed;
//   256 rows: 4 x 2 waves of 64 x 128, two LDS stages (64 KB each). Each
//             k-block is twice the work, which covers the load of the next
//             one, and every loaded byte feeds twice the MFMAs. W fragments
//             are read in two halves of 64 columns to stay within 256 VGPRs.
template <int BM>
struct Shape {
    static constexpr int kWavesM = BM / 64;              // 2 or 4
    static constexpr int kWavesN = 8 / kWavesM;          // 4 or 2
    static constexpr int kWaveCols = kBN / kWavesN;      // 64 or 128
    static constexpr int kHalves = kWaveCols / 64;       // W fragment halves: 1 or 2
    static constexpr int kStages = BM == 128 ? 3 : 2;
    static constexpr int kAChunks = BM / 64;             // 1 KB A chunks per wave and stage
    static constexpr int kOps = kAChunks + 4 + 1;        // DMA loads per wave and stage
};

template <int BM>
__device__ __forceinline__ void gemm_body(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scales,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    uint16_t* __restrict__ y, int N, int K) {
    using SH = Shape<BM>;
    constexpr int kStages = SH::kStages;
    const int n_tiles_n = N / kBN;
    const int tile = blockIdx.x / n_tiles_n;
    const int nt = blockIdx.x - tile * n_tiles_n;
    if (tile >= tile_count[0]) return;
    const int4 td = tiles[tile];
    const int row0 = td.x, e = td.z;
    const int rows = min(BM, td.y - row0);
    const int KB = K / kBK;
    const int n0 = nt * kBN;

    // One array per stage, so that the compiler can tell a DMA into one stage
    // from reads of another (the third stage is used by 128-row tiles only).
    __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * kBK], sA1[BM * kBK], sA2[BM * kBK];
    __shared__ __attribute__((aligned(1024))) uint8_t sW0[kBN * kBK], sW1[kBN * kBK], sW2[kBN * kBK];
    // Activation scales of the k-block for each wave's 64 rows.
    __shared__ __attribute__((aligned(256))) float sS0[8 * 64], sS1[8 * 64], sS2[8 * 64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / SH::kWavesN, wn = wave % SH::kWavesN;

    // Rows past the tile's end read as zero through the descriptor bound.
    const __amdgpu_buffer_rsrc_t ra = range_rsrc(a + (int64_t)row0 * K, rows * K);
    const __amdgpu_buffer_rsrc_t rw = range_rsrc(w + ((int64_t)e * N + n0) * K, kBN * K);
    const __amdgpu_buffer_rsrc_t rsa = range_rsrc(a_scales + (int64_t)row0 * KB, rows * KB * 4);
    const float* wsc =
        w_scales + ((int64_t)e * (N / 128) + (n0 + wn * SH::kWaveCols) / 128) * KB;

    // LDS DMA: each wave instruction fills 1 KB of a stage (64 lanes x 16 B,
    // lane order). LDS 16-byte slot p of a stage is (row p/8, physical chunk
    // p%8); the lane loads the logical chunk that the swizzle puts there.
    int a_goff[SH::kAChunks], w_goff[4];
#pragma unroll
    for (int i = 0; i < SH::kAChunks; i++) {
        const int p = (wave * SH::kAChunks + i) * 64 + lane, r = p >> 3;
        a_goff[i] = r * K + (((p & 7) ^ chunk_key(r)) << 4);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int p = (wave * 4 + i) * 64 + lane, r = p >> 3;
        w_goff[i] = r * K + (((p & 7) ^ chunk_key(r)) << 4);
    }
    // Scale DMA: lane l fetches the scale of the wave's row l (rows past the
    // tile's end read 0 through the descriptor bound).
    const int s_goff = (wm * 64 + lane) * KB * 4;

    float sw[kStages];
    auto stageA = [&](auto st) -> uint8_t* {
        if constexpr (decltype(st)::value == 0) return sA0;
        else if constexpr (decltype(st)::value == 1) return sA1;
        else return sA2;
    };
    auto stageW = [&](auto st) -> uint8_t* {
        if constexpr (decltype(st)::value == 0) return sW0;
        else if constexpr (decltype(st)::value == 1) return sW1;
        else return sW2;
    };
    auto stageS = [&](auto st) -> float* {
        if constexpr (decltype(st)::value == 0) return sS0;
        else if constexpr (decltype(st)::value == 1) return sS1;
        else return sS2;
    };
    // Piece q (0..3) of a stage's DMA: W chunk q, a share of the A chunks
    // (all of them over the four pieces) and, with q = 3, the scales.
    auto issue_part = [&](auto st, int b, int q) {
        constexpr int S = decltype(st)::value;
        uint8_t* A = stageA(st);
        uint8_t* W = stageW(st);
        for (int i = q * SH::kAChunks / 4; i < (q + 1) * SH::kAChunks / 4; i++)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void*)(A + (wave * SH::kAChunks + i) * 1024),
                16, a_goff[i] + b * kBK, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void*)(W + (wave * 4 + q) * 1024), 16,
            w_goff[q] + b * kBK, 0, 0, 0);
        if (q == 3) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsa, (__attribute__((address_space(3))) void*)(stageS(st) + wave * 64), 4,
                s_goff + b * 4, 0, 0, 0);
            sw[S] = wsc[b];
        }
    };
    auto issue = [&](auto st, int b) {
#pragma unroll
        for (int q = 0; q < 4; q++) issue_part(st, b, q);
    };

    f32x4 acc[4][4 * SH::kHalves];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4 * SH::kHalves; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int half = lane >> 4;
    // The last row group's MFMA results of a k-block, promoted at the start of
    // the next one (zeros before the first: adding +0 products to the +0 start
    // of the accumulators changes nothing).
    f32x4 pend[4];
#pragma unroll
    for (int j = 0; j < 4; j++) pend[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float pend_f = 0.0f;
    // One k-block from stage st; the DMA into stage nst (k-block nb) is
    // issued first.
    auto compute = [&](auto st, auto nst, int nb) {
        constexpr int S = decltype(st)::value;
        const uint8_t* A = stageA(st);
        const uint8_t* W = stageW(st);
        const float* Ssc = stageS(st) + wave * 64;
#pragma unroll
        for (int q = 0; q < 4; q++) issue_part(nst, nb, q);
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; i++) f[i] = Ssc[i * 16 + (lane & 15)] * sw[S];
        i32x8 xf[4];
#pragma unroll
        for (int i = 0; i < 4; i++) xf[i] = frag(A, wm * 64 + i * 16 + (lane & 15), half);
        // the previous k-block's last promotion, while the fragments load
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                acc[3][(SH::kHalves - 1) * 4 + j][r] =
                    fmaf(pend[j][r], pend_f, acc[3][(SH::kHalves - 1) * 4 + j][r]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hh = 0; hh < SH::kHalves; hh++) {
            i32x8 wf[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
                wf[j] = frag(W, wn * SH::kWaveCols + hh * 64 + j * 16 + (lane & 15), half);
            // Row group i: four MFMAs; their results are promoted while the
            // next group's MFMAs run (two groups of partials live at a time).
            f32x4 prev[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                f32x4 cur[4];
#pragma unroll
                for (int j = 0; j < 4; j++)
                    cur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf[j], xf[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                // keep the promotion of the previous group after this group's
                // MFMAs: hoisted above them, it would wait for the previous
                // group's results instead of running beside this group
                __builtin_amdgcn_sched_barrier(0);
                if (i > 0) {
#pragma unroll
                    for (int j = 0; j < 4; j++)
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            acc[i - 1][hh * 4 + j][r] =
                                fmaf(prev[j][r], f[i - 1], acc[i - 1][hh * 4 + j][r]);
                }
#pragma unroll
                for (int j = 0; j < 4; j++) prev[j] = cur[j];
                __builtin_amdgcn_sched_barrier(0);
            }
            if (hh + 1 < SH::kHalves) {
#pragma unroll
                for (int j = 0; j < 4; j++)
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[3][hh * 4 + j][r] = fmaf(prev[j][r], f[3], acc[3][hh * 4 + j][r]);
            } else {
                // promoted at the start of the next k-block (or after the loop)
#pragma unroll
                for (int j = 0; j < 4; j++) pend[j] = prev[j];
                pend_f = f[3];
            }
        }
    };

    // One k-block: the DMA of its stage (this wave's part) is complete once
    // at most the loads of the k-blocks after it are in flight (kStages - 2 of
    // them); the barrier then makes every wave's part visible and guarantees
    // that all waves are done with the stage the new prefetch overwrites
    // (read in the previous step). The prefetch is always issued, clamped to
    // the last k-block, so the loop has one shape; clamped copies land in a
    // stage that is never read.
    constexpr int kAhead = kStages - 1;
    auto step = [&](auto st, int b) {
        constexpr int S = decltype(st)::value;
        wait_vmcnt<SH::kOps * (kAhead - 1)>();
        lds_barrier();
        compute(st, std::integral_constant<int, (S + kAhead) % kStages>{}, min(b + kAhead, KB - 1));
    };

    issue(std::integral_constant<int, 0>{}, 0);
    if constexpr (kAhead > 1) issue(std::integral_constant<int, 1>{}, min(1, KB - 1));
    int b = 0;
    for (; b + kStages <= KB; b += kStages) {
        step(std::integral_constant<int, 0>{}, b);
        step(std::integral_constant<int, 1>{}, b + 1);
        if constexpr (kStages > 2) step(std::integral_constant<int, 2>{}, b + 2);
    }
    if (b < KB) step(std::integral_constant<int, 0>{}, b);
    if constexpr (kStages > 2)
        if (b + 1 < KB) step(std::integral_constant<int, 1>{}, b + 1);
    // No LDS DMA may still be writing when the workgroup's LDS is released.
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int r = 0; r < 4; r++)
            acc[3][(SH::kHalves - 1) * 4 + j][r] =
                fmaf(pend[j][r], pend_f, acc[3][(SH::kHalves - 1) * 4 + j][r]);

    // Lane holds, for fragment pair (i, j), row 16i + lane%16 and the four
    // consecutive columns 16j + 4*(lane/16) .. +3.
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = wm * 64 + i * 16 + (lane & 15);
        if (r >= rows) continue;
        uint16_t* yr = y + (int64_t)(row0 + r) * N + n0 + wn * SH::kWaveCols + 4 * half;
#pragma unroll
        for (int j = 0; j < 4 * SH::kHalves; j++) {
            const uint2 v = make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]),
                                       pack_bf16x2(acc[i][j][2], acc[i][j][3]));
            *reinterpret_cast<uint2*>(yr + j * 16) = v;
        }
    }
}

// One kernel per tile shape (the body is shared).
__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm_fp8_m128(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scales,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    uint16_t* __restrict__ y, int N, int K) {
    gemm_body<128>(a, a_scales, w, w_scales, tiles, tile_count, y, N, K);
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_grouped_gemm_fp8_m256(
    const uint8_t* __restrict__ a, const float* __restrict__ a_scales,
    const uint8_t* __restrict__ w, const float* __restrict__ w_scales,
    const int4* __restrict__ tiles, const int32_t* __restrict__ tile_count,
    uint16_t* __restrict__ y, int N, int K) {
    gemm_body<256>(a, a_scales, w, w_scales, tiles, tile_count, y, N, K);
}

}  // namespace

int64_t gemm_max_tiles(int64_t max_rows, int E) { return (max_rows + kBMin - 1) / kBMin + E; }

size_t gemm_workspace_bytes(int64_t max_rows, int E) {
    return 256 + (size_t)gemm_max_tiles(max_rows, E) * sizeof(int4);
}

hipError_t launch_grouped_gemm_fp8(const void* a, const float* a_scales,
                                   const int32_t* expert_offsets, const void* w,
                                   const float* w_scales, int E, int N, int K, int64_t max_rows,
                                   void* y, void* workspace, hipStream_t stream,
                                   LaunchInfo info[2], bool run) {
    // 256-row tiles when the capacity allows segments of prefill size (an
    // expert's last tile is then a small part of its work), else 128.
    const int bm = max_rows >= 512 * (int64_t)E ? 256 : 128;
    const int64_t max_tiles = gemm_max_tiles(max_rows, E);   // bounds either height
    const int64_t grid = max_tiles * (N / kBN);
    if (info) {
        info[0] = LaunchInfo{1, kTileListThreads, 0, 0};
        info[1] = LaunchInfo{grid, kGemmThreads,
                             (size_t)(bm == 256 ? 2 : 3) * (bm + kBN) * kBK, bm};
    }
    if (!run) return hipSuccess;
    int32_t* count = static_cast<int32_t*>(workspace);
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(workspace) + 256);
    hipLaunchKernelGGL(k_gemm_tiles, dim3(1), dim3(kTileListThreads), 0, stream, expert_offsets,
                       E, (int)max_rows, (int)max_tiles, bm, tiles, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const auto* a8 = static_cast<const uint8_t*>(a);
    const auto* w8 = static_cast<const uint8_t*>(w);
    auto* y16 = static_cast<uint16_t*>(y);
    if (bm == 256)
        k_grouped_gemm_fp8_m256<<<dim3((unsigned)grid), dim3(kGemmThreads), 0, stream>>>(
            a8, a_scales, w8, w_scales, tiles, count, y16, N, K);
    else
        k_grouped_gemm_fp8_m128<<<dim3((unsigned)grid), dim3(kGemmThreads), 0, stream>>>(
            a8, a_scales, w8, w_scales, tiles, count, y16, N, K);
    return hipGetLastError();
}

}  // namespace moe
