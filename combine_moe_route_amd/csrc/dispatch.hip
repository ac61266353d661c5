// Dispatch: per-expert counts, segment offsets, and the stable scatter of
// token rows into per-expert contiguous buffers (optionally FP8 with 1x128
// scales).
//
// "Enabling trillion-parameter models on AWS EFA", Dispatch and Combine:
// token counts per expert come first (accumulated with atomics in shared
// memory), their cumulative sum gives the offsets at which tokens are packed
// into contiguous per-expert send buffers. "Efficient and portable
// mixture-of-experts communication", Dispatch: activations, block scales and
// the token index are packed together; the receiver there fills its buffers
// in a non-deterministic order, which this layout replaces with token order
// inside every expert segment.
//
// Three kernels on the caller's stream:
//   K2 k_tile_hist  one block per tile of 256 tokens. Each wave ORs its
//                   lanes' bits into a per-wave 64-bit mask per expert in LDS
//                   (atomic OR, so skewed experts do not serialise on a
//                   counter). A token's rank within the tile for expert e is
//                   the popcount of the lower lanes' bits plus the counts of
//                   the earlier waves. Writes the tile's counts [tile, E] and
//                   each slot's in-tile rank [T, k] (both in the workspace).
//   K3 k_scan       one block. Per expert, an exclusive scan over tiles turns
//                   tile counts into each tile's first row inside the segment
//                   (this is what makes the order stable); totals are padded
//                   to row_align and scanned over experts into offsets; group
//                   offsets are read off the expert offsets.
//   K4 k_scatter    one wave per (token, row chunk): rows = segment offset +
//                   tile base + in-tile rank; reads each x row once with
//                   16-byte streaming loads and stores it to its k rows (FP8:
//                   one quantisation per token, k stores); the chunk-0 wave
//                   publishes dst_row / row_src. Leading blocks zero pad rows.
#include "moe_device.h"
#include "launch.h"

namespace moe {

constexpr int kHistWaves = kTileTokens / kWave;   // 4

int64_t dispatch_tiles(int64_t T) { return (T + kTileTokens - 1) / kTileTokens; }

size_t dispatch_workspace_layout(int64_t T, int E, int k, size_t* total) {
    const size_t counts = (size_t)dispatch_tiles(T) * (size_t)E * sizeof(int32_t);
    const size_t rank_off = (counts + 255) / 256 * 256;
    *total = rank_off + (size_t)T * (size_t)k * sizeof(int32_t);
    return rank_off;
}

// ---------------------------------------------------------------- K2

__global__ __launch_bounds__(kTileTokens) void k_tile_hist(const int32_t* __restrict__ topk_idx,
                                                           int64_t T, int E, int k,
                                                           int32_t* __restrict__ tile_counts,
                                                           int32_t* __restrict__ tile_rank) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* mask = reinterpret_cast<uint64_t*>(smem);               // [waves][E]
    int32_t* before = reinterpret_cast<int32_t*>(mask + kHistWaves * E);  // [waves][E]

    const int tid = threadIdx.x;
    const int w = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kTileTokens + tid;
    const bool live = t < T;

    for (int i = tid; i < kHistWaves * E; i += kTileTokens) mask[i] = 0ull;
    __syncthreads();

    const uint64_t bit = 1ull << lane;
    if (live) {
        for (int j = 0; j < k; j++) {
            const int e = topk_idx[t * k + j];
            if ((unsigned)e < (unsigned)E) atomicOr(&mask[w * E + e], bit);
        }
    }
    __syncthreads();

    for (int e = tid; e < E; e += kTileTokens) {
        int run = 0;
#pragma unroll
        for (int v = 0; v < kHistWaves; v++) {
            before[v * E + e] = run;
            run += __popcll(mask[v * E + e]);
        }
        tile_counts[(int64_t)blockIdx.x * E + e] = run;
    }
    __syncthreads();

    if (live) {
        const uint64_t lower = bit - 1ull;
        for (int j = 0; j < k; j++) {
            const int e = topk_idx[t * k + j];
            int r = -1;
            if ((unsigned)e < (unsigned)E) r = before[w * E + e] + __popcll(mask[w * E + e] & lower);
            tile_rank[t * k + j] = r;
        }
    }
}

// ---------------------------------------------------------------- K3

constexpr int kScanThreads = 1024;

__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __builtin_amdgcn_ds_bpermute(((lane - d) & (kWave - 1)) << 2, v);
        if (lane >= d) v += o;
    }
    return v;
}

__global__ __launch_bounds__(kScanThreads) void k_scan(int32_t* __restrict__ tile_counts,
                                                       int64_t tiles, int E, int row_align,
                                                       int groups,
                                                       int32_t* __restrict__ expert_counts,
                                                       int32_t* __restrict__ expert_offsets,
                                                       int32_t* __restrict__ group_offsets) {
    __shared__ int32_t s_off[1025];
    __shared__ int32_t s_wave[kScanThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int e = tid;

    // per expert: exclusive scan over tiles (in place), total count
    int cnt = 0;
    if (e < E) {
        int64_t b = 0;
        for (; b + 4 <= tiles; b += 4) {
            const int c0 = tile_counts[(b + 0) * E + e];
            const int c1 = tile_counts[(b + 1) * E + e];
            const int c2 = tile_counts[(b + 2) * E + e];
            const int c3 = tile_counts[(b + 3) * E + e];
            tile_counts[(b + 0) * E + e] = cnt;
            tile_counts[(b + 1) * E + e] = cnt + c0;
            tile_counts[(b + 2) * E + e] = cnt + c0 + c1;
            tile_counts[(b + 3) * E + e] = cnt + c0 + c1 + c2;
            cnt += c0 + c1 + c2 + c3;
        }
        for (; b < tiles; b++) {
            const int c = tile_counts[b * E + e];
            tile_counts[b * E + e] = cnt;
            cnt += c;
        }
    }
    const int padded = (e < E) ? (cnt + row_align - 1) / row_align * row_align : 0;

    // block-wide exclusive scan of the padded counts over experts
    const int incl = wave_inclusive_sum(padded);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int v = lane < kScanThreads / kWave ? s_wave[lane] : 0;
        const int vi = wave_inclusive_sum(v);
        if (lane < kScanThreads / kWave) s_wave[lane] = vi - v;   // exclusive over waves
    }
    __syncthreads();
    const int excl = s_wave[wave] + incl - padded;
    if (e < E) {
        expert_counts[e] = cnt;
        expert_offsets[e] = excl;
        s_off[e] = excl;
        if (e == E - 1) {
            expert_offsets[E] = excl + padded;
            s_off[E] = excl + padded;
        }
    }
    __syncthreads();
    if (group_offsets != nullptr)
        for (int g = tid; g <= groups; g += kScanThreads) group_offsets[g] = s_off[g * (E / groups)];
    const int64_t n = tiles * E;
    for (int64_t i = tid; i < n; i += kScanThreads) tile_counts[i] += s_off[i % E];
}

// ---------------------------------------------------------------- K4

constexpr int kScatterThreads = 256;

// Zero the pad rows of one expert's segment, or the part of them this
// block owns (pad rows of expert e: [offsets[e] + counts[e], offsets[e+1])).
__device__ void zero_pad_rows(int pb, int pad_blocks_per_expert, int pad_rows_per_block, int H,
                              bool fp8, const int32_t* __restrict__ expert_counts,
                              const int32_t* __restrict__ expert_offsets,
                              unsigned char* __restrict__ out, float* __restrict__ scales,
                              int32_t* __restrict__ row_src) {
    const int e = pb / pad_blocks_per_expert;
    const int part = pb - e * pad_blocks_per_expert;
    const int first = expert_offsets[e] + expert_counts[e];
    const int npad = expert_offsets[e + 1] - first;
    const int lo = part * pad_rows_per_block;
    const int hi = min(npad, lo + pad_rows_per_block);
    if (lo >= hi) return;
    const int rows = hi - lo;
    const int64_t row_bytes = fp8 ? (int64_t)H : 2 * (int64_t)H;
    const int units = (int)(row_bytes / 16);
    const int64_t r0 = (int64_t)first + lo;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int u = threadIdx.x; u < rows * units; u += kScatterThreads) {
        const int rr = u / units;
        const int c = u - rr * units;
        *reinterpret_cast<uint4*>(out + (r0 + rr) * row_bytes + 16 * (int64_t)c) = z;
    }
    if (fp8) {
        const int nb = H / 128;
        for (int i = threadIdx.x; i < rows * nb; i += kScatterThreads) scales[r0 * nb + i] = 0.0f;
    }
    for (int i = threadIdx.x; i < rows; i += kScatterThreads) row_src[r0 + i] = -1;
}

constexpr int kScatterWaves = kScatterThreads / kWave;

// One wave per (token, chunk of 64 lane units). A lane unit is 8 bf16 (16
// bytes) for bf16 rows, or 16 bf16 in / 16 E4M3 codes out for FP8 rows, where
// each aligned group of 8 lanes holds one 1x128 block. The token index is
// wave-uniform, so its expert ids, in-tile ranks and tile bases come in
// through scalar loads; the x row is read once through a range descriptor
// (lanes past the row read zeros) and stored to each of the token's rows.
template <bool FP8>
__global__ __launch_bounds__(kScatterThreads) void k_scatter(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ expert_counts, const int32_t* __restrict__ expert_offsets,
    int64_t T, int H, int E, int k, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    float* __restrict__ scales, int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row) {
    if ((int)blockIdx.x < pad_blocks) {
        zero_pad_rows(blockIdx.x, pad_blocks_per_expert, pad_rows_per_block, H, FP8,
                      expert_counts, expert_offsets, out, scales, row_src);
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int U = FP8 ? H / 16 : H / 8;            // lane units per row
    const int CW = (U + kWave - 1) / kWave;        // waves per token
    const int64_t gw = (int64_t)(blockIdx.x - pad_blocks) * kScatterWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = gw / CW;
    if (t >= T) return;
    const int chunk = (int)(gw - t * CW);
    const int u = chunk * kWave + lane;
    const bool active = u < U;

    // the token's activations: issued first so the row bookkeeping below
    // overlaps the load latency
    const auto xr = range_rsrc(x + t * (int64_t)H, 2 * H);
    uint4 a, b;
    if (FP8) {
        a = load16_nt(xr, 32 * u);
        b = load16_nt(xr, 32 * u + 16);
    } else {
        a = load16_nt(xr, 16 * u);
    }

    uint4 q = make_uint4(0u, 0u, 0u, 0u);
    float s = 0.0f;
    if (FP8) {
        float f[16];
        unpack8(a, f);
        unpack8(b, f + 8);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(f[i]));
        amax = group8_max(amax);
        s = amax / 448.0f;
        if (amax != 0.0f) {
            q.x = f32x4_to_e4m3(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
            q.y = f32x4_to_e4m3(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
            q.z = f32x4_to_e4m3(f[8] / s, f[9] / s, f[10] / s, f[11] / s);
            q.w = f32x4_to_e4m3(f[12] / s, f[13] / s, f[14] / s, f[15] / s);
        }
    }
    const int nb = H / 128;
    const bool scale_lane = FP8 && (u & 7) == 0;

    const int64_t p0 = t * k;
    const int32_t* tb = tile_base + (t / kTileTokens) * E;
    for (int j0 = 0; j0 < k; j0 += 8) {
        // destination rows of slots j0 .. j0+7: segment offset + tile's
        // first row in the segment (tile_base) + in-tile rank
        int r[8];
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
            r[jj] = -1;
            if (j0 + jj < k) {
                const int e = topk_idx[p0 + j0 + jj];
                if ((unsigned)e < (unsigned)E) {
                    const int rr = tb[e] + tile_rank[p0 + j0 + jj];
                    r[jj] = (rr < 0 || rr >= max_rows) ? -1 : rr;   // never write outside
                }
            }
        }
        if (chunk == 0) {
            int mine = -1;
#pragma unroll
            for (int jj = 0; jj < 8; jj++) mine = (lane == jj) ? r[jj] : mine;
            if (lane < 8 && j0 + lane < k) {
                dst_row[p0 + j0 + lane] = mine;
                if (mine >= 0) row_src[mine] = (int32_t)(p0 + j0 + lane);
            }
        }
        if (active) {
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
                if (r[jj] < 0) continue;
                if (FP8) {
                    *reinterpret_cast<uint4*>(out + (int64_t)r[jj] * H + 16 * (int64_t)u) = q;
                    if (scale_lane) scales[(int64_t)r[jj] * nb + (u >> 3)] = s;
                } else {
                    *reinterpret_cast<uint4*>(out + (int64_t)r[jj] * 2 * H + 16 * (int64_t)u) = a;
                }
            }
        }
    }
}

// ---------------------------------------------------------------- launch

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream, LaunchInfo info[3]) {
    const int64_t tiles = dispatch_tiles(a.T);
    hipError_t err;

    // K2
    const size_t hist_lds = (size_t)kHistWaves * a.E * (sizeof(uint64_t) + sizeof(int32_t));
    if (info) info[0] = LaunchInfo{tiles, kTileTokens, hist_lds, 0};
    if (tiles > 0) {
        k_tile_hist<<<dim3((unsigned)tiles), dim3(kTileTokens), hist_lds, stream>>>(
            a.topk_idx, a.T, a.E, a.k, a.tile_counts, a.tile_rank);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }

    // K3
    if (info) info[1] = LaunchInfo{1, kScanThreads, 0, 0};
    k_scan<<<1, kScanThreads, 0, stream>>>(a.tile_counts, tiles, a.E, a.row_align, a.groups,
                                            a.expert_counts, a.expert_offsets, a.group_offsets);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    // K4: leading blocks zero pad rows, then one wave per (token, chunk)
    const int units = a.fp8 ? a.H / 16 : a.H / 8;
    const int64_t waves_per_token = (units + kWave - 1) / kWave;
    const int64_t token_blocks = (a.T * waves_per_token + kScatterWaves - 1) / kScatterWaves;
    int pad_per_expert = 0, pad_rows_per_block = 0;
    if (a.row_align > 1 && a.T > 0) {
        pad_per_expert = a.row_align - 1 < 4 ? a.row_align - 1 : 4;
        pad_rows_per_block = (a.row_align - 1 + pad_per_expert - 1) / pad_per_expert;
    }
    const int64_t pad_blocks = (int64_t)a.E * pad_per_expert;
    const int64_t blocks = pad_blocks + token_blocks;
    if (info) info[2] = LaunchInfo{blocks, kScatterThreads, 0, waves_per_token};
    if (blocks == 0) return hipSuccess;
    unsigned char* out = static_cast<unsigned char*>(a.out);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (a.fp8)
        k_scatter<true><<<dim3((unsigned)blocks), dim3(kScatterThreads), 0, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_counts, a.expert_counts, a.expert_offsets, a.T,
            a.H, a.E, a.k, a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block, out,
            a.out_scales, a.row_src, a.dst_row);
    else
        k_scatter<false><<<dim3((unsigned)blocks), dim3(kScatterThreads), 0, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_counts, a.expert_counts, a.expert_offsets, a.T,
            a.H, a.E, a.k, a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block, out,
            a.out_scales, a.row_src, a.dst_row);
    return hipGetLastError();
}

}  // namespace moe
