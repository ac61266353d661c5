// Internal launchers shared by the C ABI (api.hip) and the kernel files.
// Arguments are assumed validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Tokens per tile of the dispatch histogram (one thread per token).
constexpr int kTileTokens = 256;

struct LaunchInfo {
    int64_t grid = 0;
    int block = 0;
    size_t lds = 0;
    int64_t param = 0;   // kernel-specific: lanes per token, tokens per block, ...
};

hipError_t launch_route_topk(const float* logits, int64_t T, int E, int k, int n_shared,
                             float shared_w, int32_t* topk_idx, float* topk_w,
                             hipStream_t stream, LaunchInfo* info);

hipError_t launch_route_replicas(int32_t* topk_idx, int64_t T, int k, int E,
                                 const int32_t* replica_base, hipStream_t stream);

struct DispatchArgs {
    const void* x;
    const int32_t* topk_idx;
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
    int32_t* tile_counts;   // workspace [tiles, E]
    int32_t* tile_rank;     // workspace [T, k]
    int64_t max_rows;       // rows in out / out_scales / row_src
};

int64_t dispatch_tiles(int64_t T);

// Workspace layout: tile counts [tiles, E], then (256-byte aligned) in-tile
// ranks [T, k]. Returns the byte offset of the ranks; *total gets the size.
size_t dispatch_workspace_layout(int64_t T, int E, int k, size_t* total);

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream, LaunchInfo info[3]);

hipError_t launch_combine(const void* expert_out, const int32_t* dst_row, const float* topk_w,
                          int64_t T, int H, int k, void* y, hipStream_t stream,
                          LaunchInfo* info);

hipError_t launch_combine_send(const void* expert_out, const int32_t* dst_row,
                               const float* topk_w, const int32_t* topk_idx, int64_t T, int H,
                               int E, int k, int groups, void* partial, int32_t* count,
                               hipStream_t stream, LaunchInfo* info);

hipError_t launch_combine_recv(const void* partial, const int32_t* count, int64_t T, int H,
                               int k, void* y, hipStream_t stream, LaunchInfo* info);

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
                                   LaunchInfo info[2]);

}  // namespace moe
