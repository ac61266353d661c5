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
// Two launches on the caller's stream:
//   count   one block per tile of TT tokens (TT = 16, 32 or 64 by T). The
//           block ORs one bit per (token, slot) into a 64-bit mask per expert
//           in LDS (atomic OR: a skewed expert costs no serialised counter),
//           writes the tile's counts [tile, E] and, per slot, the token's rank
//           within the tile for its expert (popcount of the lower tokens'
//           bits). In moe_route_dispatch the same block first routes its
//           tokens (top-k by sorting networks, topk_sort.h). Then it takes a
//           ticket; the block that takes the last ticket (atomicInc wraps the
//           counter back to zero for the next call) scans: per expert, an
//           exclusive sum over tiles turns tile counts into each tile's first
//           row inside the segment (this makes the order stable); totals are
//           padded to row_align and summed over experts into offsets; group
//           offsets are read off the expert offsets.
//   scatter one wave per (token, row chunk): rows = tile base + in-tile rank;
//           reads each x row once with 16-byte streaming loads and stores it
//           to its k rows (FP8: one quantisation per token, k stores); the
//           chunk-0 wave publishes dst_row / row_src. Leading blocks zero the
//           pad rows.
#include "moe_device.h"
#include "launch.h"
#include "topk_sort.h"

namespace moe {

int dispatch_tile_tokens(int64_t T) { return T <= 1024 ? 16 : T <= 4096 ? 32 : 64; }

int64_t dispatch_tiles(int64_t T) {
    const int TT = dispatch_tile_tokens(T);
    return (T + TT - 1) / TT;
}

DispatchWorkspace dispatch_workspace(int64_t T, int E, int k) {
    DispatchWorkspace w;
    w.tile_tokens = dispatch_tile_tokens(T);
    w.tiles = dispatch_tiles(T);
    w.counts_off = 256;   // [0, 256): the ticket counter (word 0)
    const size_t counts = (size_t)w.tiles * (size_t)E * sizeof(int32_t);
    w.rank_off = (w.counts_off + counts + 255) / 256 * 256;
    w.total = w.rank_off + (size_t)T * (size_t)k * sizeof(int32_t);
    return w;
}

static int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// ---------------------------------------------------------------- count

// Tile histogram and in-tile ranks. ids(p) is the expert of pair p = tl * k + j
// of the tile (token tl, slot j), npairs = tokens in the tile * k. Writes the
// tile's counts tile_counts[tile * E + e] and rank[p] (the tile's slice of the
// [T, k] rank array; -1 for a slot whose expert is outside [0, E)).
template <typename Ids>
__device__ __forceinline__ void count_tile(Ids ids, int npairs, int k, int E, int64_t tile,
                                           uint64_t* s_mask, int32_t* __restrict__ tile_counts,
                                           int32_t* __restrict__ rank) {
    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    for (int i = tid; i < E; i += NT) s_mask[i] = 0ull;
    __syncthreads();
    for (int p = tid; p < npairs; p += NT) {
        const int e = ids(p);
        if ((unsigned)e < (unsigned)E) atomicOr(&s_mask[e], 1ull << (p / k));
    }
    __syncthreads();
    for (int i = tid; i < E; i += NT) tile_counts[tile * E + i] = __popcll(s_mask[i]);
    for (int p = tid; p < npairs; p += NT) {
        const int e = ids(p);
        int r = -1;
        if ((unsigned)e < (unsigned)E) r = __popcll(s_mask[e] & ((1ull << (p / k)) - 1ull));
        rank[p] = r;
    }
}

__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __builtin_amdgcn_ds_bpermute(((lane - d) & (kWave - 1)) << 2, v);
        if (lane >= d) v += o;
    }
    return v;
}

// True in every thread of the block that finishes last. Each block's global
// writes are released (device-scope fence) before it takes its ticket; the
// last block acquires before it reads what the others wrote. atomicInc wraps
// the counter to zero on the last ticket, ready for the next launch.
__device__ __forceinline__ bool last_block(uint32_t* ticket) {
    __shared__ int s_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicInc(ticket, gridDim.x - 1) == gridDim.x - 1;
    __syncthreads();
    const bool last = s_last != 0;
    if (last) __threadfence();
    return last;
}

constexpr int kScanBatch = 16;

// Scan over tiles by one block of NT >= Ep threads (Ep = E rounded up to a
// power of two), laid out as tid = p * Ep + e: P = NT / Ep threads share
// expert e, thread p owning a contiguous range of tiles. Pass 1 sums each
// range with batches of independent loads; an LDS exchange gives each range
// its start inside the expert's segment; the p == 0 threads (tid 0 .. Ep-1,
// in expert order) scan the padded totals over experts; pass 2 rewrites the
// tile counts as tile bases (segment offset + rows of earlier tiles).
__device__ void scan_tiles(int32_t* __restrict__ tile_counts, int64_t tiles, int E, int row_align,
                           int groups, int32_t* __restrict__ expert_counts,
                           int32_t* __restrict__ expert_offsets,
                           int32_t* __restrict__ group_offsets) {
    __shared__ int32_t s_part[1024];
    __shared__ int32_t s_off[kMaxExperts + 1];
    __shared__ int32_t s_wave[1024 / kWave];

    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    int Ep = 1;
    while (Ep < E) Ep <<= 1;
    const int P = NT / Ep;
    const int e = tid & (Ep - 1);
    const int p = tid / Ep;
    const bool real = e < E;
    const int64_t per = (tiles + P - 1) / P;
    const int64_t b0 = min(tiles, (int64_t)p * per);
    const int64_t b1 = min(tiles, b0 + per);

    int part = 0;
    if (real) {
        for (int64_t b = b0; b < b1; b += kScanBatch) {
            int c[kScanBatch];
#pragma unroll
            for (int i = 0; i < kScanBatch; i++)
                c[i] = (b + i < b1) ? tile_counts[(b + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kScanBatch; i++) part += c[i];
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

    // exclusive scan of the padded totals over experts (only the p == 0
    // threads contribute; they come first, in expert order)
    const int incl = wave_inclusive_sum(padded);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int v = lane < NT / kWave ? s_wave[lane] : 0;
        const int vi = wave_inclusive_sum(v);
        if (lane < NT / kWave) s_wave[lane] = vi - v;
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
        for (int gi = tid; gi <= groups; gi += NT) group_offsets[gi] = s_off[gi * (E / groups)];

    if (real) {
        int run = s_off[e] + before;
        for (int64_t b = b0; b < b1; b += kScanBatch) {
            int c[kScanBatch];
#pragma unroll
            for (int i = 0; i < kScanBatch; i++)
                c[i] = (b + i < b1) ? tile_counts[(b + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < kScanBatch; i++)
                if (b + i < b1) {
                    tile_counts[(b + i) * E + e] = run;
                    run += c[i];
                }
        }
    }
}

struct CountArgs {
    int64_t T;
    int E, k, TT, row_align, groups;
    int64_t tiles;
    uint32_t* ticket;
    int32_t* tile_counts;
    int32_t* tile_rank;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* group_offsets;
};

// Count + scan from a given routing table [T, k]. One block per tile (at
// least one block, which then only scans: T == 0 writes zero counts).
__global__ __launch_bounds__(1024) void k_count(const int32_t* __restrict__ topk_idx,
                                                CountArgs a) {
    extern __shared__ uint64_t s_mask[];   // [E]
    const int64_t tile = blockIdx.x;
    if (tile < a.tiles) {
        const int64_t t0 = tile * a.TT;
        const int n = (int)min((int64_t)a.TT, a.T - t0);
        const int32_t* ids = topk_idx + t0 * a.k;
        count_tile([ids](int p) { return ids[p]; }, n * a.k, a.k, a.E, tile, s_mask,
                   a.tile_counts, a.tile_rank + t0 * a.k);
    }
    if (last_block(a.ticket))
        scan_tiles(a.tile_counts, a.tiles, a.E, a.row_align, a.groups, a.expert_counts,
                   a.expert_offsets, a.group_offsets);
}

// Route + count + scan: the tile's TT tokens are routed first by TT * S
// threads (S lanes per token), their experts kept in LDS for the count.
template <int S, int K>
__global__ __launch_bounds__(1024) void k_route_count(const float* __restrict__ logits,
                                                      int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_w, CountArgs a) {
    extern __shared__ uint64_t s_mask[];   // [E], then the tile's experts [TT * k]
    int32_t* s_ids = reinterpret_cast<int32_t*>(s_mask + a.E);
    const int64_t tile = blockIdx.x;
    if (tile < a.tiles) {
        const int64_t t0 = tile * a.TT;
        const int n = (int)min((int64_t)a.TT, a.T - t0);
        if ((int)threadIdx.x < a.TT * S) {   // whole lane groups
            const int tl = threadIdx.x / S;
            const int g = threadIdx.x & (S - 1);
            const int64_t t = t0 + tl;
            const bool live = tl < n;
            double list[K];
            route_token<S, K>(logits + (live ? t : 0) * (int64_t)a.E, live, a.E, g, list);
            if (live)
                write_route<S, K>(list, g, t, tl, a.E, a.k, a.k, 0, 0.0f, topk_idx, topk_w, s_ids);
        }
        __syncthreads();
        count_tile([s_ids](int p) { return s_ids[p]; }, n * a.k, a.k, a.E, tile, s_mask,
                   a.tile_counts, a.tile_rank + t0 * a.k);
    }
    if (last_block(a.ticket))
        scan_tiles(a.tile_counts, a.tiles, a.E, a.row_align, a.groups, a.expert_counts,
                   a.expert_offsets, a.group_offsets);
}

// ---------------------------------------------------------------- K4

constexpr int kScatterThreads = 256;

// Zero the pad rows of one expert's segment, or the part of them this
// block owns (pad rows of expert e: [offsets[e] + counts[e], offsets[e+1])).
// Rows outside [0, max_rows) are never written, whatever the offsets say.
__device__ void zero_pad_rows(int pb, int pad_blocks_per_expert, int pad_rows_per_block, int H,
                              bool fp8, int64_t max_rows,
                              const int32_t* __restrict__ expert_counts,
                              const int32_t* __restrict__ expert_offsets,
                              unsigned char* __restrict__ out, float* __restrict__ scales,
                              int32_t* __restrict__ row_src) {
    const int e = pb / pad_blocks_per_expert;
    const int part = pb - e * pad_blocks_per_expert;
    const int64_t first = (int64_t)expert_offsets[e] + expert_counts[e];
    const int64_t npad = min((int64_t)expert_offsets[e + 1], max_rows) - first;
    const int lo = part * pad_rows_per_block;
    const int hi = (int)min(npad, (int64_t)lo + pad_rows_per_block);
    if (first < 0 || lo >= hi) return;
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
    int64_t T, int H, int E, int k, int TT, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row) {
    if ((int)blockIdx.x < pad_blocks) {
        zero_pad_rows(blockIdx.x, pad_blocks_per_expert, pad_rows_per_block, H, false, max_rows,
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
    const int32_t* tb = tile_base + (t / TT) * E;
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
    int64_t T, int H, int E, int k, int TT, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    float* __restrict__ scales, int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row) {
    extern __shared__ float s_scale[];             // [H / 128]
    if ((int)blockIdx.x < pad_blocks) {
        zero_pad_rows(blockIdx.x, pad_blocks_per_expert, pad_rows_per_block, H, true, max_rows,
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
    const int32_t* tb = tile_base + (t / TT) * E;

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

template <int S, int K>
static void launch_route_count_sk(const DispatchArgs& a, const CountArgs& c, int64_t grid,
                                  int threads, size_t lds, hipStream_t stream) {
    k_route_count<S, K><<<dim3((unsigned)grid), dim3(threads), lds, stream>>>(
        a.logits, const_cast<int32_t*>(a.topk_idx), a.topk_w, c);
}

template <int K>
static void launch_route_count_k(int S, const DispatchArgs& a, const CountArgs& c, int64_t grid,
                                 int threads, size_t lds, hipStream_t stream) {
    switch (S) {
        case 1: launch_route_count_sk<1, K>(a, c, grid, threads, lds, stream); break;
        case 2: launch_route_count_sk<2, K>(a, c, grid, threads, lds, stream); break;
        case 4: launch_route_count_sk<4, K>(a, c, grid, threads, lds, stream); break;
        case 8: launch_route_count_sk<8, K>(a, c, grid, threads, lds, stream); break;
        default: launch_route_count_sk<16, K>(a, c, grid, threads, lds, stream); break;
    }
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream, LaunchInfo info[3], int* n,
                           bool run) {
    const DispatchWorkspace ws = dispatch_workspace(a.T, a.E, a.k);
    const int TT = ws.tile_tokens;
    const int64_t tiles = ws.tiles;
    const int Ep = pow2_at_least(a.E);
    // routing inside the count kernel when the sorting-network path applies
    const bool fused = a.logits != nullptr && route_sort_applies(a.logits, a.E, a.k);
    const bool route_first = a.logits != nullptr && !fused;
    const int S = fused ? route_lanes(a.E) : 1;
    int count_threads = fused ? TT * S : 256;
    if (count_threads < Ep) count_threads = Ep;
    if (count_threads < kWave) count_threads = kWave;
    const size_t count_lds = (size_t)a.E * sizeof(uint64_t) +
                             (fused ? (size_t)TT * a.k * sizeof(int32_t) : 0);
    const int64_t count_grid = tiles > 0 ? tiles : 1;

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

    int nk = 0;
    LaunchInfo route_info;
    if (route_first)
        (void)launch_route_topk(a.logits, a.T, a.E, a.k, 0, 0.0f, const_cast<int32_t*>(a.topk_idx),
                                a.topk_w, stream, &route_info, false);
    if (info) {
        if (route_first) info[nk++] = route_info;
        info[nk++] = LaunchInfo{count_grid, count_threads, count_lds, fused ? S : TT};
        info[nk++] = a.fp8 ? LaunchInfo{scatter_blocks, fp8_threads,
                                        (size_t)(a.H / 128) * sizeof(float), fp8_waves}
                           : LaunchInfo{scatter_blocks, kScatterThreads, 0, bf16_waves_per_token};
    } else {
        nk = route_first ? 3 : 2;
    }
    if (n) *n = nk;
    if (!run) return hipSuccess;

    hipError_t err;
    if (route_first) {
        err = launch_route_topk(a.logits, a.T, a.E, a.k, 0, 0.0f, const_cast<int32_t*>(a.topk_idx),
                                a.topk_w, stream, nullptr);
        if (err != hipSuccess) return err;
    }
    const CountArgs c{a.T, a.E, a.k, TT, a.row_align, a.groups, tiles, a.ticket, a.tile_counts,
                      a.tile_rank, a.expert_counts, a.expert_offsets, a.group_offsets};
    if (fused) {
        switch (route_list_len(a.k)) {
            case 2: launch_route_count_k<2>(S, a, c, count_grid, count_threads, count_lds, stream); break;
            case 4: launch_route_count_k<4>(S, a, c, count_grid, count_threads, count_lds, stream); break;
            default: launch_route_count_k<8>(S, a, c, count_grid, count_threads, count_lds, stream); break;
        }
    } else {
        k_count<<<dim3((unsigned)count_grid), dim3(count_threads), count_lds, stream>>>(a.topk_idx,
                                                                                        c);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;

    // scatter: leading blocks zero pad rows, then the token work
    unsigned char* out = static_cast<unsigned char*>(a.out);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (scatter_blocks == 0) return hipSuccess;
    if (a.fp8) {
        const size_t lds = (size_t)(a.H / 128) * sizeof(float);
        k_scatter_fp8<<<dim3((unsigned)scatter_blocks), dim3(fp8_threads), lds, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_counts, a.expert_counts, a.expert_offsets, a.T,
            a.H, a.E, a.k, TT, a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block,
            out, a.out_scales, a.row_src, a.dst_row);
    } else {
        k_scatter_bf16<<<dim3((unsigned)scatter_blocks), dim3(kScatterThreads), 0, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_counts, a.expert_counts, a.expert_offsets, a.T,
            a.H, a.E, a.k, TT, a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block,
            out, a.row_src, a.dst_row);
    }
    return hipGetLastError();
}

}  // namespace moe
