// C ABI of libmoeroute: host-side argument checks, then kernel launches on the
// caller's stream. No allocation, no global mutable state, no device->host
// copies. Every check runs before the first HIP call, so invalid arguments
// return an error without touching the GPU.
#include <stdio.h>
#include <stdlib.h>

#include <mutex>

#include "../../include/moe_route.h"
#include "launch.h"

namespace {

constexpr int64_t kInt32Max = 2147483647;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool log_enabled() {
    static const int on = [] {
        const char* v = getenv("MOE_ROUTE_LOG");
        return (v && v[0] == '1') ? 1 : 0;
    }();
    return on != 0;
}

void log_launch(const char* what, const moe::LaunchInfo& i) {
    fprintf(stderr, "[moe_route] %s grid=%lld block=%d lds=%zu param=%lld\n", what,
            (long long)i.grid, i.block, i.lds, (long long)i.param);
}

int64_t max_rows_of(int64_t T, int E, int k, int row_align) {
    if (T < 0 || k < 1 || E < k || E > MOE_MAX_EXPERTS || row_align < 1 || row_align > 1024)
        return -1;
    const int64_t tk = T * (int64_t)k;   // T < 2^62 is implied by the check below
    if (T > kInt32Max) return -1;
    const int64_t rows = tk + (int64_t)E * (row_align - 1);
    return rows > kInt32Max ? -1 : rows;
}

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// True when every kernel of a planned call fits a launch packet.
bool all_fit(const moe::LaunchInfo* info, int n) {
    for (int i = 0; i < n; i++)
        if (!moe::launch_fits(info[i])) return false;
    return true;
}

}  // namespace

extern "C" {

int moe_route_topk(const float* logits, int64_t T, int E, int k, int32_t* topk_idx,
                   float* topk_w, void* stream) {
    if (T < 0 || k < 1 || E < k || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (T * (int64_t)k > kInt32Max || T * (int64_t)E > ((int64_t)1 << 40)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_idx || !topk_w) return MOE_ENULL;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_EALIGN;
    moe::LaunchInfo info;
    (void)moe::launch_route_topk(logits, T, E, k, 0, 0.0f, topk_idx, topk_w, nullptr, &info, false);
    if (!all_fit(&info, 1)) return MOE_EINVAL;
    const hipError_t e = moe::launch_route_topk(logits, T, E, k, 0, 0.0f, topk_idx, topk_w,
                                                static_cast<hipStream_t>(stream), &info);
    if (log_enabled()) log_launch("route_topk", info);
    return status_of(e);
}

int moe_route_topk_shared(const float* logits, int64_t T, int E, int k, int n_shared,
                          float shared_w, int32_t* topk_idx, float* topk_w, void* stream) {
    if (T < 0 || k < 1 || E < k || n_shared < 0 || E + n_shared > MOE_MAX_EXPERTS)
        return MOE_EINVAL;
    if (T * (int64_t)(k + n_shared) > kInt32Max || T * (int64_t)E > ((int64_t)1 << 40))
        return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_idx || !topk_w) return MOE_ENULL;
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4)) return MOE_EALIGN;
    moe::LaunchInfo info;
    (void)moe::launch_route_topk(logits, T, E, k, n_shared, shared_w, topk_idx, topk_w, nullptr, &info,
                           false);
    if (!all_fit(&info, 1)) return MOE_EINVAL;
    const hipError_t e = moe::launch_route_topk(logits, T, E, k, n_shared, shared_w, topk_idx,
                                                topk_w, static_cast<hipStream_t>(stream), &info);
    if (log_enabled()) log_launch("route_topk_shared", info);
    return status_of(e);
}

int moe_route_replicas(int32_t* topk_idx, int64_t T, int k, int E, const int32_t* replica_base,
                       void* stream) {
    if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (T * (int64_t)k > kInt32Max) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !replica_base) return MOE_ENULL;
    if (!aligned(topk_idx, 4) || !aligned(replica_base, 4)) return MOE_EALIGN;
    return status_of(moe::launch_route_replicas(topk_idx, T, k, E, replica_base,
                                                static_cast<hipStream_t>(stream)));
}

int64_t moe_dispatch_max_rows(int64_t T, int E, int k, int row_align) {
    return max_rows_of(T, E, k, row_align);
}

size_t moe_dispatch_workspace_bytes(int64_t T, int E, int k, int groups) {
    if (max_rows_of(T, E, k, 1) < 0 || groups < 1 || E % groups != 0) return 0;
    return moe::dispatch_workspace(T, E, k).total;
}

}  // extern "C"

namespace {

// Checks and launches of a dispatch call. Sizes and options are checked
// first (MOE_EINVAL, including the launch geometry), then pointers
// (MOE_ENULL), alignment (MOE_EALIGN) and the workspace size (MOE_ENOSPC);
// nothing is launched unless every check passes. With library_ws the
// workspace is the library's own scratch (only its size is checked); with
// run == false the checks run and nothing is launched.
int dispatch_impl(const float* logits, float* topk_w, const void* x, const int32_t* topk_idx,
                  int64_t T, int H, int E, int k, int groups, int row_align, int out_dtype,
                  void* out, float* out_scales, int32_t* expert_counts, int32_t* expert_offsets,
                  int32_t* group_offsets, int32_t* row_src, int32_t* dst_row, void* workspace,
                  size_t workspace_bytes, hipStream_t stream, bool library_ws = false,
                  bool run = true) {
    const bool route = logits != nullptr || topk_w != nullptr;   // moe_route_dispatch
    // sizes and options
    const int64_t max_rows = max_rows_of(T, E, k, row_align);
    if (max_rows < 0) return MOE_EINVAL;
    if (route && T * (int64_t)E > ((int64_t)1 << 40)) return MOE_EINVAL;
    if (groups < 1 || groups > E || E % groups != 0) return MOE_EINVAL;
    if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_FP8_E4M3) return MOE_EINVAL;
    const bool fp8 = out_dtype == MOE_OUT_FP8_E4M3;
    if (H < 1 || H > 65536 || H % (fp8 ? 128 : 8) != 0) return MOE_EINVAL;
    moe::DispatchArgs a;
    a.x = x;
    a.topk_idx = topk_idx;
    a.logits = logits;
    a.topk_w = topk_w;
    a.T = T;
    a.H = H;
    a.E = E;
    a.k = k;
    a.groups = groups;
    a.row_align = row_align;
    a.fp8 = fp8;
    a.out = out;
    a.out_scales = out_scales;
    a.expert_counts = expert_counts;
    a.expert_offsets = expert_offsets;
    a.group_offsets = group_offsets;
    a.row_src = row_src;
    a.dst_row = dst_row;
    const moe::DispatchWorkspace ws = moe::dispatch_workspace(T, E, k);
    unsigned char* wsb = static_cast<unsigned char*>(workspace);
    a.tile_counts = wsb + ws.counts_off;
    a.tile_base = reinterpret_cast<int32_t*>(wsb + ws.base_off);
    a.tile_rank = wsb + ws.rank_off;
    a.max_rows = max_rows;
    moe::LaunchInfo info[4];
    int nk = 0;
    // geometry (route_sort_applies looks only at the logits address)
    (void)moe::launch_dispatch(a, nullptr, info, &nk, false);
    if (!all_fit(info, nk)) return MOE_EINVAL;
    // required pointers
    if (!expert_counts || !expert_offsets) return MOE_ENULL;
    if (T > 0 && (!x || !topk_idx || !dst_row)) return MOE_ENULL;
    if (route && T > 0 && (!logits || !topk_w)) return MOE_ENULL;
    if (max_rows > 0 && (!out || !row_src)) return MOE_ENULL;
    if (fp8 && max_rows > 0 && !out_scales) return MOE_ENULL;
    // alignment
    if (!aligned(x, 16) || !aligned(out, 16)) return MOE_EALIGN;
    if (!aligned(topk_idx, 4) || !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) ||
        !aligned(group_offsets, 4) || !aligned(row_src, 4) || !aligned(dst_row, 4) ||
        !aligned(workspace, 16) || (fp8 && !aligned(out_scales, 4)))
        return MOE_EALIGN;
    if (route && (!aligned(logits, 4) || !aligned(topk_w, 4))) return MOE_EALIGN;
    // workspace
    if (workspace_bytes < ws.total) return MOE_ENOSPC;
    if (!library_ws && ws.total > 0 && !workspace) return MOE_ENULL;
    if (!run) return MOE_OK;

    const hipError_t e = moe::launch_dispatch(a, stream, info, &nk);
    if (log_enabled())
        for (int i = 0; i < nk; i++) log_launch(info[i].name ? info[i].name : "dispatch", info[i]);
    return status_of(e);
}

}  // namespace

extern "C" {

int moe_dispatch(const void* x, const int32_t* topk_idx, int64_t T, int H, int E, int k,
                 int groups, int row_align, int out_dtype, void* out, float* out_scales,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* group_offsets,
                 int32_t* row_src, int32_t* dst_row, void* workspace, size_t workspace_bytes,
                 void* stream) {
    return dispatch_impl(nullptr, nullptr, x, topk_idx, T, H, E, k, groups, row_align, out_dtype,
                         out, out_scales, expert_counts, expert_offsets, group_offsets, row_src,
                         dst_row, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

int moe_route_dispatch(const float* logits, const void* x, int64_t T, int H, int E, int k,
                       int groups, int row_align, int out_dtype, int32_t* topk_idx,
                       float* topk_w, void* out, float* out_scales, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* group_offsets, int32_t* row_src,
                       int32_t* dst_row, void* workspace, size_t workspace_bytes, void* stream) {
    // at least one of logits / topk_w must be non-null to select routing (a
    // null one is then reported by the pointer checks); an empty batch needs
    // neither and still writes zero counts and offsets
    if (!logits && !topk_w && T > 0) return MOE_ENULL;
    return dispatch_impl(logits, topk_w, x, topk_idx, T, H, E, k, groups, row_align, out_dtype,
                         out, out_scales, expert_counts, expert_offsets, group_offsets, row_src,
                         dst_row, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---------------------------------------------------------------- no-alloc dispatch
//
// Scratch of moe_dispatch_no_alloc: one array per GPU, resident for the life
// of the process. In host code `scratch` names a host-side stand-in, not the
// device array, so its address is looked up once per device with
// hipGetSymbolAddress and only that pointer is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MOE_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device), or nullptr on a HIP error.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int moe_dispatch_no_alloc(const void* x, const int32_t* topk_idx, int64_t T, int H, int E, int k,
                          int groups, int row_align, int out_dtype, void* out, float* out_scales,
                          int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* group_offsets, int32_t* row_src, int32_t* dst_row,
                          void* stream) {
    // every check first, with no HIP call (a request needing more scratch
    // than the array holds fails here with MOE_ENOSPC)
    const int st = dispatch_impl(nullptr, nullptr, x, topk_idx, T, H, E, k, groups, row_align,
                                 out_dtype, out, out_scales, expert_counts, expert_offsets,
                                 group_offsets, row_src, dst_row, nullptr,
                                 MOE_NO_ALLOC_SCRATCH_BYTES, nullptr, /*library_ws=*/true,
                                 /*run=*/false);
    if (st != MOE_OK) return st;
    void* ws = device_scratch();
    if (!ws) return MOE_EHIP;
    return dispatch_impl(nullptr, nullptr, x, topk_idx, T, H, E, k, groups, row_align, out_dtype,
                         out, out_scales, expert_counts, expert_offsets, group_offsets, row_src,
                         dst_row, ws, MOE_NO_ALLOC_SCRATCH_BYTES,
                         static_cast<hipStream_t>(stream), /*library_ws=*/true);
}

int moe_combine(const void* expert_out, const int32_t* dst_row, const float* topk_w, int64_t T,
                int H, int k, void* y, void* stream) {
    if (T < 0 || k < 1 || k > MOE_MAX_EXPERTS || H < 1 || H > 65536 || H % 8 != 0)
        return MOE_EINVAL;
    if (T > kInt32Max || T * (int64_t)k > kInt32Max) return MOE_EINVAL;
    moe::LaunchInfo info;
    (void)moe::launch_combine(expert_out, dst_row, topk_w, T, H, k, y, nullptr, &info, false);
    if (!all_fit(&info, 1)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!expert_out || !dst_row || !topk_w || !y) return MOE_ENULL;
    if (!aligned(expert_out, 16) || !aligned(y, 16)) return MOE_EALIGN;
    if (!aligned(dst_row, 4) || !aligned(topk_w, 4)) return MOE_EALIGN;
    const hipError_t e = moe::launch_combine(expert_out, dst_row, topk_w, T, H, k, y,
                                             static_cast<hipStream_t>(stream), &info);
    if (log_enabled()) log_launch("combine", info);
    return status_of(e);
}

int moe_combine_send(const void* expert_out, const int32_t* dst_row, const float* topk_w,
                     const int32_t* topk_idx, int64_t T, int H, int E, int k, int groups,
                     void* partial, int32_t* partial_count, void* stream) {
    if (T < 0 || k < 1 || E < k || E > MOE_MAX_EXPERTS || H < 1 || H > 65536 || H % 8 != 0)
        return MOE_EINVAL;
    if (groups < 1 || groups > E || E % groups != 0) return MOE_EINVAL;
    if (T > kInt32Max || T * (int64_t)k > kInt32Max) return MOE_EINVAL;
    moe::LaunchInfo info;
    (void)moe::launch_combine_send(expert_out, dst_row, topk_w, topk_idx, T, H, E, k, groups, partial,
                             partial_count, nullptr, &info, false);
    if (!all_fit(&info, 1)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!expert_out || !dst_row || !topk_w || !topk_idx || !partial || !partial_count)
        return MOE_ENULL;
    if (!aligned(expert_out, 16) || !aligned(partial, 16)) return MOE_EALIGN;
    if (!aligned(dst_row, 4) || !aligned(topk_w, 4) || !aligned(topk_idx, 4) ||
        !aligned(partial_count, 4))
        return MOE_EALIGN;
    const hipError_t e = moe::launch_combine_send(expert_out, dst_row, topk_w, topk_idx, T, H, E,
                                                  k, groups, partial, partial_count,
                                                  static_cast<hipStream_t>(stream), &info);
    if (log_enabled()) log_launch("combine_send", info);
    return status_of(e);
}

int moe_combine_recv(const void* partial, const int32_t* partial_count, int64_t T, int H, int k,
                     void* y, void* stream) {
    if (T < 0 || k < 1 || k > MOE_MAX_EXPERTS || H < 1 || H > 65536 || H % 8 != 0)
        return MOE_EINVAL;
    if (T > kInt32Max || T * (int64_t)k > kInt32Max) return MOE_EINVAL;
    moe::LaunchInfo info;
    (void)moe::launch_combine_recv(partial, partial_count, T, H, k, y, nullptr, &info, false);
    if (!all_fit(&info, 1)) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!partial || !partial_count || !y) return MOE_ENULL;
    if (!aligned(partial, 16) || !aligned(y, 16)) return MOE_EALIGN;
    if (!aligned(partial_count, 4)) return MOE_EALIGN;
    const hipError_t e = moe::launch_combine_recv(partial, partial_count, T, H, k, y,
                                                  static_cast<hipStream_t>(stream), &info);
    if (log_enabled()) log_launch("combine_recv", info);
    return status_of(e);
}

int moe_harness_expert_scale(const void* disp, const float* disp_scales, const int32_t* row_src,
                             const int32_t* topk_idx, const int32_t* expert_offsets,
                             int64_t max_rows, int H, int E, int out_dtype, int identity,
                             void* expert_out, void* stream) {
    if (max_rows < 0 || max_rows > kInt32Max || E < 1 || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
    if (out_dtype != MOE_OUT_BF16 && out_dtype != MOE_OUT_FP8_E4M3) return MOE_EINVAL;
    const bool fp8 = out_dtype == MOE_OUT_FP8_E4M3;
    if (H < 1 || H > 65536 || H % (fp8 ? 128 : 8) != 0) return MOE_EINVAL;
    if (!expert_offsets) return MOE_ENULL;
    if (max_rows == 0) return MOE_OK;
    if (!disp || !row_src || !topk_idx || !expert_out || (fp8 && !disp_scales)) return MOE_ENULL;
    if (!aligned(disp, 16) || !aligned(expert_out, 16)) return MOE_EALIGN;
    return status_of(moe::launch_expert_scale(disp, disp_scales, row_src, topk_idx, expert_offsets,
                                              max_rows, H, E, fp8, identity != 0, expert_out,
                                              static_cast<hipStream_t>(stream)));
}

size_t moe_grouped_gemm_workspace_bytes(int64_t max_rows, int E) {
    if (max_rows < 0 || max_rows > kInt32Max || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    return moe::gemm_workspace_bytes(max_rows, E);
}

int moe_grouped_gemm_fp8(const void* a, const float* a_scales, const int32_t* expert_offsets,
                         const void* w, const float* w_scales, int E, int N, int K,
                         int64_t max_rows, void* y, void* workspace, size_t workspace_bytes,
                         void* stream) {
    if (E < 1 || E > MOE_MAX_EXPERTS || max_rows < 0 || max_rows > kInt32Max) return MOE_EINVAL;
    if (N < 256 || N > (1 << 20) || N % 256 != 0) return MOE_EINVAL;
    if (K < 128 || K > (1 << 20) || K % 128 != 0) return MOE_EINVAL;
    {
        moe::LaunchInfo plan[2];
        (void)moe::launch_grouped_gemm_fp8(nullptr, nullptr, nullptr, nullptr, nullptr, E, N, K,
                                     max_rows, nullptr, nullptr, nullptr, plan, false);
        if (!all_fit(plan, 2)) return MOE_EINVAL;
    }
    if (max_rows == 0) return MOE_OK;
    if (!a || !a_scales || !expert_offsets || !w || !w_scales || !y || !workspace)
        return MOE_ENULL;
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(a_scales, 4) || !aligned(w_scales, 4) ||
        !aligned(expert_offsets, 4) || !aligned(y, 8) || !aligned(workspace, 16))
        return MOE_EALIGN;
    if (workspace_bytes < moe::gemm_workspace_bytes(max_rows, E)) return MOE_ENOSPC;
    moe::LaunchInfo info[2];
    const hipError_t e = moe::launch_grouped_gemm_fp8(a, a_scales, expert_offsets, w, w_scales, E,
                                                      N, K, max_rows, y, workspace,
                                                      static_cast<hipStream_t>(stream), info);
    if (log_enabled()) {
        log_launch("gemm_tiles", info[0]);
        log_launch("grouped_gemm_fp8", info[1]);
    }
    return status_of(e);
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument (size, count or option out of range)";
        case MOE_ENOSPC: return "workspace smaller than moe_dispatch_workspace_bytes";
        case MOE_EALIGN: return "pointer not aligned (16 bytes for payloads, 4 for the rest)";
        case MOE_EHIP: return "HIP kernel launch failed";
        case MOE_ENULL: return "required pointer is NULL";
        default: return "unknown status";
    }
}

}  // extern "C"
