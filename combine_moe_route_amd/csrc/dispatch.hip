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
//                   offsets are read off the expert offsets. Several threads
//                   share an expert, each scanning a contiguous tile range.
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

    // expert ids are loaded in batches of 8 before any LDS atomic, so the
    // loads are in flight together; the first batch stays in registers for
    // the ranking pass
    const uint64_t bit = 1ull << lane;
    int e0[8];
#pragma unroll
    for (int jj = 0; jj < 8; jj++) e0[jj] = (live && jj < k) ? topk_idx[t * k + jj] : -1;
#pragma unroll
    for (int jj = 0; jj < 8; jj++)
        if ((unsigned)e0[jj] < (unsigned)E) atomicOr(&mask[w * E + e0[jj]], bit);
    if (live) {
        for (int j0 = 8; j0 < k; j0 += 8) {
            int e[8];
#pragma unroll
            for (int jj = 0; jj < 8; jj++) e[jj] = (j0 + jj < k) ? topk_idx[t * k + j0 + jj] : -1;
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                if ((unsigned)e[jj] < (unsigned)E) atomicOr(&mask[w * E + e[jj]], bit);
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
        for (int j0 = 0; j0 < k; j0 += 8) {
            int e[8];
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                e[jj] = j0 == 0 ? e0[jj] : ((j0 + jj < k) ? topk_idx[t * k + j0 + jj] : -1);
#pragma unroll
            for (int jj = 0; jj < 8; jj++) {
                if (j0 + jj >= k) break;
                int r = -1;
                if ((unsigned)e[jj] < (unsigned)E)
                    r = before[w * E + e[jj]] + __popcll(mask[w * E + e[jj]] & lower);
                tile_rank[t * k + j0 + jj] = r;
            }
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

// Threads are laid out as tid = p * Ep + e (Ep = E rounded up to a power of
// two): P = 1024 / Ep threads share expert e, thread p owning a contiguous
// range of tiles. Pass 1 sums each range with independent loads in batches of
// 8; an LDS exchange gives each range its start inside the expert's segment;
// the p == 0 threads scan the padded totals over experts; pass 2 rewrites the
// tile counts as tile bases (segment offset + rows of earlier tiles).
__global__ __launch_bounds__(kScanThreads) void k_scan(int32_t* __restrict__ tile_counts,
                                                       int64_t tiles, int E, int row_align,
                                                       int groups,
                                                       int32_t* __restrict__ expert_counts,
                                                       int32_t* __restrict__ expert_offsets,
                                                       int32_t* __restrict__ group_offsets) {
    __shared__ int32_t s_part[kScanThreads];
    __shared__ int32_t s_off[1025];
    __shared__ int32_t s_wave[kScanThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    int Ep = 1;
    while (Ep < E) Ep <<= 1;
    const int P = kScanThreads / Ep;
    const int e = tid & (Ep - 1);
    const int p = tid / Ep;
    const bool real = e < E;
    const int64_t per = (tiles + P - 1) / P;
    const int64_t b0 = min(tiles, (int64_t)p * per);
    const int64_t b1 = min(tiles, b0 + per);

    // pass 1: rows of this expert in tiles [b0, b1); the first 8 counts stay
    // in registers for pass 2
    int part = 0;
    int c0[8];
#pragma unroll
    for (int i = 0; i < 8; i++) c0[i] = (real && b0 + i < b1) ? tile_counts[(b0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < 8; i++) part += c0[i];
    if (real) {
        for (int64_t b = b0 + 8; b < b1; b += 8) {
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; i++) c[i] = (b + i < b1) ? tile_counts[(b + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; i++) part += c[i];
        }
    }
    s_part[tid] = part;
    __syncthreads();
    int before = 0, cnt = 0;
    for (int q = 0; q < P; q++) {
        const int v = s_part[q * Ep + e];
        before += q < p ? v : 0;
        cnt += v;
    }
    const int padded = (p == 0 && real) ? (cnt + row_align - 1) / row_align * row_align : 0;

    // exclusive scan of the padded totals over experts (the p == 0 threads
    // are tid 0 .. Ep-1, in expert order; all others add zero)
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
    if (p == 0 && real) {
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

    // pass 2: tile bases
    if (real) {
        int run = s_off[e] + before;
        for (int64_t b = b0; b < b1; b += 8) {
            int c[8];
#pragma unroll
            for (int i = 0; i < 8; i++)
                c[i] = b == b0 ? c0[i] : ((b + i < b1) ? tile_counts[(b + i) * E + e] : 0);
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (b + i < b1) {
                    tile_counts[(b + i) * E + e] = run;
                    run += c[i];
                }
        }
    }
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
    for (int u = threadIdx.x; u < rows * units; u += blockDim.x) {
        const int rr = u / units;
        const int c = u - rr * units;
        *reinterpret_cast<uint4*>(out + (r0 + rr) * row_bytes + 16 * (int64_t)c) = z;
    }
    if (fp8) {
        const int nb = H / 128;
        for (int i = threadIdx.x; i < rows * nb; i += blockDim.x) scales[r0 * nb + i] = 0.0f;
    }
    for (int i = threadIdx.x; i < rows; i += blockDim.x) row_src[r0 + i] = -1;
}

constexpr int kScatterWaves = kScatterThreads / kWave;

// Destination rows of slots j0 .. j0+7 of token t: segment offset + tile's
// first row in the segment (tile_base) + in-tile rank; -1 for dropped slots.
__device__ __forceinline__ void slot_rows(const int32_t* __restrict__ topk_idx,
                                          const int32_t* __restrict__ tile_rank,
                                          const int32_t* __restrict__ tb, int64_t p0, int j0,
                                          int k, int E, int64_t max_rows, int r[8]) {
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
}

// The wave that owns slots j0 .. j0+7 publishes dst_row and row_src for them.
__device__ __forceinline__ void publish_rows(int lane, int64_t p0, int j0, int k, const int r[8],
                                             int32_t* __restrict__ dst_row,
                                             int32_t* __restrict__ row_src) {
    int mine = -1;
#pragma unroll
    for (int jj = 0; jj < 8; jj++) mine = (lane == jj) ? r[jj] : mine;
    if (lane < 8 && j0 + lane < k) {
        dst_row[p0 + j0 + lane] = mine;
        if (mine >= 0) row_src[mine] = (int32_t)(p0 + j0 + lane);
    }
}

// bf16 rows. One wave per (token, chunk of 64 lane units of 8 bf16 = 16
// bytes). The token index is wave-uniform, so its expert ids, in-tile ranks
// and tile bases come in through scalar loads; the x row is read once through
// a range descriptor (lanes past the row read zeros) and stored to each of the
// token's rows.
__global__ __launch_bounds__(kScatterThreads) void k_scatter_bf16(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ expert_counts, const int32_t* __restrict__ expert_offsets,
    int64_t T, int H, int E, int k, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row) {
    if ((int)blockIdx.x < pad_blocks) {
        zero_pad_rows(blockIdx.x, pad_blocks_per_expert, pad_rows_per_block, H, false,
                      expert_counts, expert_offsets, out, nullptr, row_src);
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int U = H / 8;                           // 16-byte units per row
    const int CW = (U + kWave - 1) / kWave;        // waves per token
    const int64_t gw = (int64_t)(blockIdx.x - pad_blocks) * kScatterWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = gw / CW;
    if (t >= T) return;
    const int chunk = (int)(gw - t * CW);
    const int u = chunk * kWave + lane;

    const uint4 a = load16_nt(range_rsrc(x + t * (int64_t)H, 2 * H), 16 * u);
    const int64_t p0 = t * k;
    const int32_t* tb = tile_base + (t / kTileTokens) * E;
    for (int j0 = 0; j0 < k; j0 += 8) {
        int r[8];
        slot_rows(topk_idx, tile_rank, tb, p0, j0, k, E, max_rows, r);
        if (chunk == 0) publish_rows(lane, p0, j0, k, r, dst_row, row_src);
        if (u < U) {
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                if (r[jj] >= 0)
                    *reinterpret_cast<uint4*>(out + (int64_t)r[jj] * 2 * H + 16 * (int64_t)u) = a;
        }
    }
}

// FP8 rows. One block per token, W waves; wave w handles row chunks w, w+W,
// ... of 64 lane units, a unit being 16 bf16 in (32 bytes) and 16 E4M3 codes
// out (16 bytes), so each aligned group of 8 lanes holds one 1x128 block and
// reduces its amax over DPP. The token is quantised once; its codes are stored
// to each destination row, and its 1x128 scales are staged in LDS and written
// to each row's scale segment with one contiguous store (instead of many small
// pieces from different waves, which cost HBM read-modify-write cycles).
__global__ __launch_bounds__(1024) void k_scatter_fp8(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_base,
    const int32_t* __restrict__ expert_counts, const int32_t* __restrict__ expert_offsets,
    int64_t T, int H, int E, int k, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    float* __restrict__ scales, int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row) {
    extern __shared__ float s_scale[];             // [H / 128]
    if ((int)blockIdx.x < pad_blocks) {
        zero_pad_rows(blockIdx.x, pad_blocks_per_expert, pad_rows_per_block, H, true,
                      expert_counts, expert_offsets, out, scales, row_src);
        return;
    }
    const int64_t t = blockIdx.x - pad_blocks;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int W = blockDim.x / kWave;
    const int U = H / 16;                          // lane units per row
    const int CW = (U + kWave - 1) / kWave;
    const int nb = H / 128;
    const auto xr = range_rsrc(x + t * (int64_t)H, 2 * H);
    const int64_t p0 = t * k;
    const int32_t* tb = tile_base + (t / kTileTokens) * E;

    for (int chunk = w; chunk < CW; chunk += W) {
        const int u = chunk * kWave + lane;
        const uint4 a = load16_nt(xr, 32 * u);
        const uint4 b = load16_nt(xr, 32 * u + 16);
        float f[16];
        unpack8(a, f);
        unpack8(b, f + 8);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) amax = fmaxf(amax, fabsf(f[i]));
        amax = group8_max(amax);
        const float s = amax / 448.0f;
        uint4 q = make_uint4(0u, 0u, 0u, 0u);
        if (amax != 0.0f) {
            q.x = f32x4_to_e4m3(f[0] / s, f[1] / s, f[2] / s, f[3] / s);
            q.y = f32x4_to_e4m3(f[4] / s, f[5] / s, f[6] / s, f[7] / s);
            q.z = f32x4_to_e4m3(f[8] / s, f[9] / s, f[10] / s, f[11] / s);
            q.w = f32x4_to_e4m3(f[12] / s, f[13] / s, f[14] / s, f[15] / s);
        }
        if (u < U && (u & 7) == 0) s_scale[u >> 3] = s;
        for (int j0 = 0; j0 < k; j0 += 8) {
            int r[8];
            slot_rows(topk_idx, tile_rank, tb, p0, j0, k, E, max_rows, r);
            if (chunk == 0) publish_rows(lane, p0, j0, k, r, dst_row, row_src);
            if (u < U) {
#pragma unroll
                for (int jj = 0; jj < 8; jj++)
                    if (r[jj] >= 0)
                        *reinterpret_cast<uint4*>(out + (int64_t)r[jj] * H + 16 * (int64_t)u) = q;
            }
        }
    }
    __syncthreads();
    // scale segments: wave w writes the segments of slots w, w+W, ...
    for (int j = w; j < k; j += W) {
        const int e = topk_idx[p0 + j];
        if ((unsigned)e >= (unsigned)E) continue;
        const int rr = tb[e] + tile_rank[p0 + j];
        if (rr < 0 || rr >= max_rows) continue;
        for (int i = lane; i < nb; i += kWave) scales[(int64_t)rr * nb + i] = s_scale[i];
    }
}

// ---------------------------------------------------------------- launch

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream, LaunchInfo info[3],
                           bool run) {
    const int64_t tiles = dispatch_tiles(a.T);
    hipError_t err;

    // geometry of the three kernels first
    const size_t hist_lds = (size_t)kHistWaves * a.E * (sizeof(uint64_t) + sizeof(int32_t));
    int pad_per_expert = 0, pad_rows_per_block = 0;
    if (a.row_align > 1 && a.T > 0) {
        pad_per_expert = a.row_align - 1 < 4 ? a.row_align - 1 : 4;
        pad_rows_per_block = (a.row_align - 1 + pad_per_expert - 1) / pad_per_expert;
    }
    const int64_t pad_blocks = (int64_t)a.E * pad_per_expert;
    int fp8_waves = (a.H / 16 + kWave - 1) / kWave;
    if (fp8_waves > 16) fp8_waves = 16;
    const int fp8_threads = fp8_waves * kWave > kScatterThreads ? fp8_waves * kWave : kScatterThreads;
    const int64_t bf16_waves_per_token = (a.H / 8 + kWave - 1) / kWave;
    const int64_t scatter_blocks =
        a.fp8 ? pad_blocks + a.T
              : pad_blocks + (a.T * bf16_waves_per_token + kScatterWaves - 1) / kScatterWaves;
    if (info) {
        info[0] = LaunchInfo{tiles, kTileTokens, hist_lds, 0};
        info[1] = LaunchInfo{1, kScanThreads, 0, 0};
        info[2] = a.fp8 ? LaunchInfo{scatter_blocks, fp8_threads,
                                     (size_t)(a.H / 128) * sizeof(float), fp8_waves}
                        : LaunchInfo{scatter_blocks, kScatterThreads, 0, bf16_waves_per_token};
    }
    if (!run) return hipSuccess;

    // K2
    if (tiles > 0) {
        k_tile_hist<<<dim3((unsigned)tiles), dim3(kTileTokens), hist_lds, stream>>>(
            a.topk_idx, a.T, a.E, a.k, a.tile_counts, a.tile_rank);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }

    // K3
    k_scan<<<1, kScanThreads, 0, stream>>>(a.tile_counts, tiles, a.E, a.row_align, a.groups,
                                            a.expert_counts, a.expert_offsets, a.group_offsets);
    if ((err = hipGetLastError()) != hipSuccess) return err;

    // K4: leading blocks zero pad rows, then the token work
    unsigned char* out = static_cast<unsigned char*>(a.out);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (a.fp8) {
        // one block per token, one wave per 64-unit chunk (at most 16 waves)
        const size_t lds = (size_t)(a.H / 128) * sizeof(float);
        if (scatter_blocks == 0) return hipSuccess;
        k_scatter_fp8<<<dim3((unsigned)scatter_blocks), dim3(fp8_threads), lds, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_counts, a.expert_counts, a.expert_offsets, a.T,
            a.H, a.E, a.k, a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block, out,
            a.out_scales, a.row_src, a.dst_row);
    } else {
        if (scatter_blocks == 0) return hipSuccess;
        k_scatter_bf16<<<dim3((unsigned)scatter_blocks), dim3(kScatterThreads), 0, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_counts, a.expert_counts, a.expert_offsets, a.T,
            a.H, a.E, a.k, a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block, out,
            a.row_src, a.dst_row);
    }
    return hipGetLastError();
}

}  // namespace moe
