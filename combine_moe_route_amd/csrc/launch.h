// Internal launchers shared by the C ABI (api.hip) and the kernel files.
// Arguments are assumed validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Largest expert count the kernels accept (MOE_MAX_EXPERTS of the C ABI).
constexpr int kMaxExperts = 1024;

struct LaunchInfo {
    int64_t grid = 0;
    int block = 0;
    size_t lds = 0;
    int64_t param = 0;           // kernel-specific: lanes per token, tokens per block, ...
    const char* name = nullptr;  // for the launch log
};

// A launch packet counts work-items in 32 bits (grid_size_x) and blocks in
// 31: a kernel fits when blocks * threads < 2^32 and blocks < 2^31.
inline bool launch_fits(const LaunchInfo& i) {
    return i.grid >= 0 && i.grid < ((int64_t)1 << 31) &&
           i.grid * (int64_t)i.block < ((int64_t)1 << 32);
}

// Every launcher below fills `info` (one entry per kernel it enqueues, in
// order) before launching anything; with run == false it only fills `info`,
// so callers can check the geometry of a whole call before the first launch.

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int n_shared,
                             float shared_w, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream, LaunchInfo* info, bool run = true);

hipError_t launch_route_replicas(int32_t* topk_idx, int64_t T, int k, int E,
                                 const int32_t* replica_base, hipStream_t stream);

struct DispatchArgs {
    const void* x;
    const int32_t* topk_idx;     // routing table; written here first when logits != nullptr
    const float* logits;         // [T, E]: route inside the dispatch (moe_route_dispatch), or nullptr
    float* topk_w;               // [T, k] router weights out, with logits
    int64_t T;
    int H, E, k, groups, row_align;
    bool fp8;
    void* out;
    float* out_scales;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* group_offsets;
    int32_t* row_src;
    int32_t* dst_row;
    uint8_t* tile_counts;   // workspace [tiles, E]
    int32_t* tile_base;     // workspace [tiles, E]
    uint8_t* tile_rank;     // workspace [T, k]
    int64_t max_rows;       // rows in out / out_scales / row_src
};

// Tokens per count tile (16, 32 or 64, growing with T; at most 64, so tile
// counts and in-tile ranks fit a byte) and the tile count.
int dispatch_tile_tokens(int64_t T);
int64_t dispatch_tiles(int64_t T);

// Workspace layout (each part 256-byte aligned): byte tile counts
// [tiles, E] at counts_off, tile prefixes int32 [tiles, E] at base_off, byte
// in-tile ranks [T, k] at rank_off; total bytes. Nothing is kept between
// calls.
struct DispatchWorkspace {
    int tile_tokens;
    int64_t tiles;
    size_t counts_off, base_off, rank_off, total;
};
DispatchWorkspace dispatch_workspace(int64_t T, int E, int k);

// Up to four kernels: [route (only when routing falls back to its own
// kernel)], count (with routing inside when it applies), [scan (small
// batches scan inside the scatter)], scatter. *n gets the number of kernels.
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream, LaunchInfo info[4], int* n,
                           bool run = true);

hipError_t launch_combine(const void* expert_out, const int32_t* dst_row, const float* topk_w,
                          int64_t T, int H, int k, void* y, hipStream_t stream,
                          LaunchInfo* info, bool run = true);

hipError_t launch_combine_send(const void* expert_out, const int32_t* dst_row,
                               const float* topk_w, const int32_t* topk_idx, int64_t T, int H,
                               int E, int k, int groups, void* partial, int32_t* count,
                               hipStream_t stream, LaunchInfo* info, bool run = true);

hipError_t launch_combine_recv(const void* partial, const int32_t* count, int64_t T, int H,
                               int k, void* y, hipStream_t stream, LaunchInfo* info,
                               bool run = true);

hipError_t launch_expert_scale(const void* disp, const float* disp_scales,
                               const int32_t* row_src, const int32_t* topk_idx,
                               const int32_t* expert_offsets, int64_t max_rows, int H,
                               int E, bool fp8, bool identity, void* expert_out,
                               hipStream_t stream);

// Grouped GEMM: tile-list workspace size and launcher (tile list + GEMM).
size_t gemm_workspace_bytes(int64_t max_rows, int E);
int64_t gemm_max_tiles(int64_t max_rows, int E);
hipError_t launch_grouped_gemm_fp8(const void* a, const float* a_scales,
                                   const int32_t* expert_offsets, const void* w,
                                   const float* w_scales, int E, int N, int K, int64_t max_rows,
                                   void* y, void* workspace, hipStream_t stream,
                                   LaunchInfo info[2], bool run = true);

}  // namespace moe
