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
//   count   one block per tile of TT tokens (TT = 16, 32 or 64 by T). The
//           block ORs one bit per (token, slot) into a 64-bit mask per expert
//           in LDS (atomic OR: a skewed expert costs no serialised counter)
//           and writes the tile's counts [tile, E] and, per slot, the token's
//           rank within the tile for its expert (popcount of the lower
//           tokens' bits). Both fit a byte: at most 64 tokens per tile. In
//           moe_route_dispatch the same block first routes its tokens (top-k
//           by sorting networks, topk_sort.h).
//   scan    up to 128 blocks, each owning a range of tiles. Every block brings
//           all byte counts into LDS in batches of 16-byte loads (chunks of
//           64 KiB), sums every expert's total and its prefix up to the
//           block's first tile, and scans the totals, padded to row_align,
//           over experts into offsets (the same in every block, so no block
//           waits for another; block 0 writes counts, offsets and group
//           offsets). Each block then writes, for its tiles, each tile's
//           first row inside the expert's segment (this makes the order
//           stable).
//   scatter one wave per (token, row chunk): row = segment offset + tile prefix
//           + in-tile rank; reads each x row once with 16-byte streaming loads
//           and stores it to its k rows (FP8: one quantisation per token, k
//           stores); the chunk-0 wave publishes dst_row / row_src. Leading
//           blocks zero the pad rows.
// Small batches (at most 64 tiles and 4096 tile counts, e.g. 128-token decode)
// skip the scan launch: every scatter block stages the byte counts itself and
// builds the tile prefixes and offsets in LDS while its x row is in flight
// (block 0 writes the count and offset outputs). In moe_route_dispatch, small
// batches with few experts (E <= 48) skip the counting launch as well: every
// scatter block routes the whole batch in LDS (route_block_small), so
// dispatch is one launch.
#include "moe_device.h"
#include "launch.h"
#include "topk_sort.h"

namespace moe {

int dispatch_tile_tokens(int64_t T) { return T <= 1024 ? 16 : T <= 4096 ? 32 : 64; }

int64_t dispatch_tiles(int64_t T) {
    const int TT = dispatch_tile_tokens(T);
    return (T + TT - 1) / TT;
}

static size_t round256(size_t n) { return (n + 255) / 256 * 256; }

static int count_row_bytes(int E) { return (E + 3) & ~3; }

DispatchWorkspace dispatch_workspace(int64_t T, int E, int k) {
    DispatchWorkspace w;
    w.tile_tokens = dispatch_tile_tokens(T);
    w.tiles = dispatch_tiles(T);
    w.counts_off = 0;
    w.base_off = round256((size_t)w.tiles * (size_t)count_row_bytes(E));
    w.rank_off = w.base_off + round256((size_t)w.tiles * (size_t)E * sizeof(int32_t));
    w.total = w.rank_off + round256((size_t)T * (size_t)k);
    return w;
}

// ---------------------------------------------------------------- count

// Tile histogram and in-tile ranks. ids(p) is the expert of pair p = tl * k + j
// of the tile (token tl, slot j), npairs = tokens in the tile * k. Writes the
// tile's counts counts[e] (the row padded with zeros to a multiple of 4
// bytes) and rank[p] (the tile's slice of the [T, k] rank array; 0xFF for a
// slot whose expert is outside [0, E), which the scatter never reads).
// With zeroed, the caller has already cleared s_mask and synchronised.
template <typename Ids>
__device__ __forceinline__ void count_tile(Ids ids, int npairs, int k, int E, uint64_t* s_mask,
                                           uint8_t* __restrict__ counts,
                                           uint8_t* __restrict__ rank, bool zeroed = false) {
    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    if (!zeroed) {
        for (int i = tid; i < E; i += NT) s_mask[i] = 0ull;
        __syncthreads();
    }
    for (int p = tid; p < npairs; p += NT) {
        const int e = ids(p);
        if ((unsigned)e < (unsigned)E) atomicOr(&s_mask[e], 1ull << (p / k));
    }
    __syncthreads();
    for (int i = tid; i < ((E + 3) & ~3); i += NT)
        counts[i] = i < E ? (uint8_t)__popcll(s_mask[i]) : (uint8_t)0;
    for (int p = tid; p < npairs; p += NT) {
        const int e = ids(p);
        int r = 0xFF;
        if ((unsigned)e < (unsigned)E) r = __popcll(s_mask[e] & ((1ull << (p / k)) - 1ull));
        rank[p] = (uint8_t)r;
    }
}

struct CountArgs {
    int64_t T;
    int E, k, TT;
    int64_t tiles;
    uint8_t* tile_counts;   // [tiles, E]
    uint8_t* tile_rank;     // [T, k]
};

// Counts from a given routing table [T, k]: one block per tile.
__global__ __launch_bounds__(1024) void k_count(const int32_t* __restrict__ topk_idx,
                                                CountArgs a) {
    extern __shared__ uint64_t s_mask[];   // [E]
    const int64_t tile = blockIdx.x;
    const int64_t t0 = tile * a.TT;
    const int n = (int)min((int64_t)a.TT, a.T - t0);
    const int32_t* ids = topk_idx + t0 * a.k;
    count_tile([ids](int p) { return ids[p]; }, n * a.k, a.k, a.E, s_mask,
               a.tile_counts + tile * ((a.E + 3) & ~3), a.tile_rank + t0 * a.k);
}

// Route + count: the tile's TT tokens are routed first by TT * S threads (S
// lanes per token), their experts kept in LDS for the count.
template <int S, int K>
__global__ __launch_bounds__(1024) void k_route_count(const float* __restrict__ logits,
                                                      int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_w, CountArgs a) {
    extern __shared__ uint64_t s_mask[];   // [E], then the tile's experts [TT * k]
    int32_t* s_ids = reinterpret_cast<int32_t*>(s_mask + a.E);
    const int64_t tile = blockIdx.x;
    const int64_t t0 = tile * a.TT;
    const int n = (int)min((int64_t)a.TT, a.T - t0);
    // clear the masks while the logits are in flight
    for (int i = threadIdx.x; i < a.E; i += blockDim.x) s_mask[i] = 0ull;
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
    count_tile([s_ids](int p) { return s_ids[p]; }, n * a.k, a.k, a.E, s_mask,
               a.tile_counts + tile * ((a.E + 3) & ~3), a.tile_rank + t0 * a.k, true);
}

// ---------------------------------------------------------------- scan

constexpr int kScanThreads = 1024;
constexpr int kScanLdsBytes = 64 * 1024;   // byte counts staged per chunk

// Byte i of word w.
__device__ __forceinline__ int byte_of(uint32_t w, int i) { return (int)((w >> (8 * i)) & 0xFFu); }

// Adds to acc[0..3] the columns 4q .. 4q+3 of rows [r0, r1) of the staged byte
// counts (one 32-bit word per row and column group, Q words per row),
// reading 8 rows at a time so that the LDS reads are in flight together.
__device__ __forceinline__ void column_sum4(const uint32_t* s_cnt, int r0, int r1, int Q, int q,
                                            int acc[4]) {
    int r = r0;
    for (; r + 8 <= r1; r += 8) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; i++) w[i] = s_cnt[(r + i) * Q + q];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int b = 0; b < 4; b++) acc[b] += byte_of(w[i], b);
    }
    for (; r < r1; r++) {
        const uint32_t w = s_cnt[r * Q + q];
#pragma unroll
        for (int b = 0; b < 4; b++) acc[b] += byte_of(w, b);
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

// Up to kScanBlocks blocks of 1024 threads. Thread tid = p * Qp + q handles
// the four experts 4q .. 4q+3 (Q = ceil(E / 4) groups, Qp = Q rounded up to a
// power of two), P = min(1024 / Qp, 4) threads sharing a group (the rest
// only take part in the expert scan; more sharers would cost more in the
// exchange of partial sums than they save in the column sums). Every block reads all
// byte counts (into LDS, in chunks of 64 KiB) and computes every expert's
// total and, for its own range of tiles, every expert's prefix at the range
// start; every block then scans the padded totals over experts (the same
// offsets in each block; block 0 writes them). Each block writes the tile
// prefixes (relative to the segment start) of its own range only, so the
// stores spread over the blocks and no block waits for another.
// 128 blocks measured faster than 16, 32, 64 or 256 at both prefill shapes.
// A block takes over half a CU's LDS, so one runs per CU: on a stream whose
// CU mask leaves fewer CUs the grid shrinks to one block per CU, as a second
// round of blocks would repeat the whole count read (3x the time on 32 CUs).
constexpr int kScanBlocks = 128;
constexpr int kScanShare = 4;   // at most this many threads per expert group

__global__ __launch_bounds__(kScanThreads) void k_scan(const uint8_t* __restrict__ tile_counts,
                                                       int64_t tiles, int E, int row_align,
                                                       int groups,
                                                       int32_t* __restrict__ tile_base,
                                                       int32_t* __restrict__ expert_counts,
                                                       int32_t* __restrict__ expert_offsets,
                                                       int32_t* __restrict__ group_offsets) {
    __shared__ __align__(16) uint32_t s_cnt[kScanLdsBytes / 4];
    __shared__ int32_t s_all[4][kScanThreads];
    __shared__ int32_t s_pre[4][kScanThreads];
    __shared__ int32_t s_off[kMaxExperts + 1];
    __shared__ int32_t s_wave[kScanThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int E4 = (E + 3) & ~3;   // bytes per count row
    const int Q = E4 / 4;
    int Qp = 1;
    while (Qp < Q) Qp <<= 1;
    const int P = kScanThreads / Qp < kScanShare ? kScanThreads / Qp : kScanShare;
    const int q = tid & (Qp - 1);
    const int p = tid / Qp;
    const bool real = q < Q && p < P;
    // this block's tiles
    const int64_t per_block = (tiles + gridDim.x - 1) / gridDim.x;
    const int64_t my0 = min(tiles, (int64_t)blockIdx.x * per_block);
    const int64_t my1 = min(tiles, my0 + per_block);
    // tiles per chunk: a multiple of 16, so every chunk starts 16-byte aligned
    const int64_t chunk = (int64_t)(kScanLdsBytes / E4) / 16 * 16;

    // stage tiles [c0, c0 + nt) of the byte counts; c0 is a multiple of 16,
    // so the source is 16-byte aligned, and the count array is padded to 256
    // bytes, so rounding the length up to 16 stays inside it (every load of
    // the chunk is issued before the first LDS store)
    auto stage = [&](int64_t c0, int nt) {
        constexpr int kIters = kScanLdsBytes / (16 * kScanThreads);
        const int n16 = (nt * E4 + 15) / 16;
        const uint4* src = reinterpret_cast<const uint4*>(tile_counts + c0 * E4);
        uint4* dst = reinterpret_cast<uint4*>(s_cnt);
        uint4 v[kIters];
#pragma unroll
        for (int j = 0; j < kIters; j++) {
            const int i = tid + j * kScanThreads;
            v[j] = i < n16 ? src[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int j = 0; j < kIters; j++) {
            const int i = tid + j * kScanThreads;
            if (i < n16) dst[i] = v[j];
        }
    };

    // pass 1: totals and the prefix at my0, over all tiles
    int all[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
    int64_t last_c0 = 0;
    int last_nt = 0;   // the chunk left in LDS
    for (int64_t c0 = 0; c0 < tiles; c0 += chunk) {
        const int nt = (int)min(chunk, tiles - c0);
        __syncthreads();
        stage(c0, nt);
        __syncthreads();
        const int per = (nt + P - 1) / P;
        const int r0 = min(nt, p * per);
        const int r1 = min(nt, r0 + per);
        if (real) {
            // rows of this chunk before my0 count into the prefix as well:
            // [r0, r1) splits at that point, each row is read once
            const int64_t before_mine = my0 - c0;
            const int rm = (int)max((int64_t)r0, min((int64_t)r1, before_mine));
            column_sum4(s_cnt, r0, rm, Q, q, pre);
            column_sum4(s_cnt, rm, r1, Q, q, all);
        }
        last_c0 = c0;
        last_nt = nt;
    }
    const bool staged_mine = last_c0 <= my0 && my1 <= last_c0 + last_nt;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        s_all[b][tid] = all[b] + pre[b];
        s_pre[b][tid] = pre[b];
    }
    __syncthreads();
    int cnt[4] = {0, 0, 0, 0}, start[4] = {0, 0, 0, 0};
    if (real)
#pragma unroll
        for (int pp = 0; pp < kScanShare; pp++)
            if (pp < P)
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    cnt[b] += s_all[b][pp * Qp + q];
                    start[b] += s_pre[b][pp * Qp + q];
                }
    int padded[4];
#pragma unroll
    for (int b = 0; b < 4; b++)
        padded[b] = (p == 0 && real && 4 * q + b < E)
                        ? (cnt[b] + row_align - 1) / row_align * row_align : 0;
    const int mine = padded[0] + padded[1] + padded[2] + padded[3];

    // exclusive scan of the padded totals over experts (only the p == 0
    // threads contribute; they come first, in expert order)
    const int incl = wave_inclusive_sum(mine);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int v = lane < kScanThreads / kWave ? s_wave[lane] : 0;
        const int vi = wave_inclusive_sum(v);
        if (lane < kScanThreads / kWave) s_wave[lane] = vi - v;
    }
    __syncthreads();
    if (p == 0 && real) {
        int off = s_wave[wave] + incl - mine;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int e = 4 * q + b;
            if (e < E) {
                s_off[e] = off;
                if (blockIdx.x == 0) {
                    expert_counts[e] = cnt[b];
                    expert_offsets[e] = off;
                }
                off += padded[b];
                if (e == E - 1) {
                    s_off[E] = off;
                    if (blockIdx.x == 0) expert_offsets[E] = off;
                }
            }
        }
    }
    __syncthreads();
    if (blockIdx.x == 0 && group_offsets != nullptr)
        for (int gi = tid; gi <= groups; gi += kScanThreads)
            group_offsets[gi] = s_off[gi * (E / groups)];

    // pass 2: the prefixes of my tiles. The P threads of a group split each
    // staged piece: thread p takes rows [r0, r1) and adds the rows before
    // them from LDS; every thread carries the piece's total into the next.
    int run[4] = {start[0], start[1], start[2], start[3]};
    int64_t c0 = my0;
    while (c0 < my1) {
        int64_t s0 = last_c0;   // staged range [s0, s0 + snt)
        int snt = last_nt;
        if (!staged_mine) {
            s0 = c0 & ~(int64_t)15;
            snt = (int)min(chunk, tiles - s0);
            __syncthreads();
            stage(s0, snt);
            __syncthreads();
        }
        const int nt = (int)min(my1 - c0, s0 + snt - c0);
        const int sr0 = (int)(c0 - s0);
        const int per = (nt + P - 1) / P;
        const int r0 = min(nt, p * per);
        const int r1 = min(nt, r0 + per);
        if (real) {
            int v[4] = {run[0], run[1], run[2], run[3]};
            column_sum4(s_cnt, sr0, sr0 + r0, Q, q, v);
            for (int r = r0; r < r1; r++) {
                const uint32_t w = s_cnt[(sr0 + r) * Q + q];
                int32_t* dst = tile_base + (c0 + r) * E + 4 * q;
#pragma unroll
                for (int b = 0; b < 4; b++)
                    if (4 * q + b < E) {
                        dst[b] = v[b];
                        v[b] += byte_of(w, b);
                    }
            }
            column_sum4(s_cnt, sr0, sr0 + nt, Q, q, run);
        }
        c0 += nt;
    }
}

// ---------------------------------------------------------------- scatter

// Inline scan for small batches: tiles <= kInlineTiles and tiles * E <=
// kInlineCells. Every thread of the block takes part (it holds barriers).
constexpr int kInlineTiles = 64;
constexpr int kInlineCells = 4096;

struct InlineLds {
    int32_t tb[kInlineCells];        // tile prefixes [tiles, E]
    int32_t off[kMaxExperts + 1];    // segment offsets
    int32_t tot[kMaxExperts];        // expert totals
    int32_t wave[1024 / kWave];
};

__device__ void inline_scan(const uint8_t* __restrict__ counts, int tiles, int E, int row_align,
                            int groups, bool write_out, int32_t* __restrict__ g_counts,
                            int32_t* __restrict__ g_offsets, int32_t* __restrict__ g_goffs,
                            InlineLds& L) {
    const int NT = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int E4 = (E + 3) & ~3;
    // stage the byte counts as 32-bit words (rows are padded to 4 bytes and
    // the array is 4-byte aligned), every load of a batch issued before any
    // LDS store, so that the staging costs one memory round trip
    constexpr int kBatch = 4;
    const uint32_t* words = reinterpret_cast<const uint32_t*>(counts);
    const int nwords = tiles * E4 / 4;
    for (int w0 = 0; w0 < nwords; w0 += kBatch * NT) {
        uint32_t v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
            const int w = w0 + i * NT + tid;
            v[i] = w < nwords ? words[w] : 0u;
        }
#pragma unroll
        for (int i = 0; i < kBatch; i++) {
            const int w = w0 + i * NT + tid;
            if (w < nwords) {
                const int b = (4 * w) / E4;
                const int c0 = 4 * w - b * E4;
#pragma unroll
                for (int q = 0; q < 4; q++)
                    if (c0 + q < E) L.tb[b * E + c0 + q] = byte_of(v[i], q);
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += NT) {
        int run = 0;
        for (int b = 0; b < tiles; b++) {
            const int c = L.tb[b * E + e];
            L.tb[b * E + e] = run;
            run += c;
        }
        L.tot[e] = run;
    }
    __syncthreads();
    // exclusive scan of the padded totals over experts: thread tid owns the
    // contiguous experts [e0, e1)
    const int per = (E + NT - 1) / NT;
    const int e0 = min(E, tid * per);
    const int e1 = min(E, e0 + per);
    int local = 0;
    for (int e = e0; e < e1; e++) local += (L.tot[e] + row_align - 1) / row_align * row_align;
    const int incl = wave_inclusive_sum(local);
    if (lane == kWave - 1) L.wave[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int v = lane < NT / kWave ? L.wave[lane] : 0;
        const int vi = wave_inclusive_sum(v);
        if (lane < NT / kWave) L.wave[lane] = vi - v;
    }
    __syncthreads();
    int run = L.wave[wave] + incl - local;
    for (int e = e0; e < e1; e++) {
        L.off[e] = run;
        run += (L.tot[e] + row_align - 1) / row_align * row_align;
        if (e == E - 1) L.off[E] = run;
    }
    __syncthreads();
    if (write_out) {
        for (int e = tid; e <= E; e += NT) {
            g_offsets[e] = L.off[e];
            if (e < E) g_counts[e] = L.tot[e];
        }
        if (g_goffs != nullptr)
            for (int gi = tid; gi <= groups; gi += NT) g_goffs[gi] = L.off[gi * (E / groups)];
    }
}

// Whole-batch routing inside one block, for decode batches with few experts
// (E <= 48, so one lane holds a token's whole logit row; T <= the block's
// threads; T * k <= kSmallPairs). Every block routes every token (a few
// hundred logits per block, served from L2 after the first block), keeps the
// experts in LDS, counts them per expert and scans the padded counts into
// segment offsets; block 0 writes topk_idx / topk_w, the counts and the
// offsets. A token's rank inside an expert's segment is the number of earlier
// (token, slot) pairs with that expert (the stable order), counted by the
// token's wave with ballots. Dispatch is then a single launch.
constexpr int kSmallExperts = 4 * kRouteChunks;   // 48
constexpr int kSmallTokens = 256;
constexpr int kSmallPairs = 1024;

struct SmallLds {
    int32_t ids[kSmallPairs];      // expert of pair t * k + j
    int32_t cnt[kWave];
    int32_t off[kWave + 1];
};

template <int K>
__device__ void route_block_small(const float* __restrict__ logits, int T, int E, int k,
                                  int row_align, int groups, bool write_out,
                                  int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                  int32_t* __restrict__ g_counts, int32_t* __restrict__ g_offsets,
                                  int32_t* __restrict__ g_goffs, SmallLds& L) {
    const int tid = threadIdx.x;
    if (tid < kWave) L.cnt[tid] = 0;
    __syncthreads();
    if (tid < T) {
        double list[K];
        route_token<1, K>(logits + (int64_t)tid * E, true, E, 0, list);
#pragma unroll
        for (int j = 0; j < K; j++)
            if (j < k) {
                const int e = cand_expert(list[j]);
                L.ids[tid * k + j] = e;
                atomicAdd(&L.cnt[e], 1);
            }
        if (write_out) write_route<1, K>(list, 0, tid, tid, E, k, k, 0, 0.0f, topk_idx, topk_w, nullptr);
    }
    __syncthreads();
    if (tid < kWave) {   // wave 0: exclusive scan of the padded counts over experts
        const int c = tid < E ? L.cnt[tid] : 0;
        const int padded = (c + row_align - 1) / row_align * row_align;
        const int incl = wave_inclusive_sum(padded);
        L.off[tid] = incl - padded;
        if (tid == kWave - 1) L.off[E] = incl;
        if (write_out && tid < E) {
            g_counts[tid] = c;
            g_offsets[tid] = incl - padded;
        }
        if (write_out && tid == kWave - 1) g_offsets[E] = incl;
    }
    __syncthreads();
    if (write_out && g_goffs != nullptr)
        for (int gi = tid; gi <= groups; gi += blockDim.x) g_goffs[gi] = L.off[gi * (E / groups)];
}

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

// Experts and in-tile ranks of slots j0 .. j0+7 of the token whose first
// slot is p0 (e = -1 past k). The token is wave-uniform; both loads are issued
// together, and the kernels issue them before the offsets are ready.
__device__ __forceinline__ void load_slots(const int32_t* __restrict__ topk_idx,
                                           const uint8_t* __restrict__ tile_rank, int64_t p0,
                                           int j0, int k, int e[8], int rk[8]) {
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
        const bool live = j0 + jj < k;
        e[jj] = live ? topk_idx[p0 + j0 + jj] : -1;
        rk[jj] = live ? tile_rank[p0 + j0 + jj] : 0;
    }
}

// Destination rows of slots j0 .. j0+7 of token t: the segment offset + the
// tile's first row in the segment (tb) + in-tile rank; -1 for dropped slots.
// The rank is read only for a live expert. (Loading experts and ranks
// together, as load_slots does, made the prefill-sized bf16 scatter 6 %
// slower.)
__device__ __forceinline__ void slot_rows(const int32_t* __restrict__ topk_idx,
                                          const uint8_t* __restrict__ tile_rank,
                                          const int32_t* __restrict__ offsets,
                                          const int32_t* __restrict__ tb, int64_t p0, int j0,
                                          int k, int E, int64_t max_rows, int r[8]) {
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
        r[jj] = -1;
        if (j0 + jj < k) {
            const int e = topk_idx[p0 + j0 + jj];
            if ((unsigned)e < (unsigned)E) {
                const int rr = offsets[e] + tb[e] + tile_rank[p0 + j0 + jj];
                r[jj] = (rr < 0 || rr >= max_rows) ? -1 : rr;   // never write outside
            }
        }
    }
}

// The same from experts and ranks already loaded (load_slots).
__device__ __forceinline__ void slot_rows(const int e[8], const int rk[8],
                                          const int32_t* __restrict__ offsets,
                                          const int32_t* __restrict__ tb, int E, int64_t max_rows,
                                          int r[8]) {
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
        r[jj] = -1;
        if ((unsigned)e[jj] < (unsigned)E) {
            const int rr = offsets[e[jj]] + tb[e[jj]] + rk[jj];
            r[jj] = (rr < 0 || rr >= max_rows) ? -1 : rr;   // never write outside
        }
    }
}

// Destination rows of slots j0 .. j0+7 of token t from the block-local
// routing: segment offset + the number of earlier pairs with the same expert.
// The whole wave takes part (t is wave-uniform).
__device__ __forceinline__ int row_small(const SmallLds& L, int p, int64_t max_rows) {
    const int lane = threadIdx.x & (kWave - 1);
    const int e = L.ids[p];
    int rank = 0;
    for (int q0 = 0; q0 < p; q0 += kWave) {
        const int q = q0 + lane;
        rank += __popcll(__ballot(q < p && L.ids[q] == e));
    }
    const int rr = L.off[e] + rank;
    return (rr < 0 || rr >= max_rows) ? -1 : rr;
}

__device__ __forceinline__ void slot_rows_small(const SmallLds& L, int64_t t, int j0, int k,
                                                int64_t max_rows, int r[8]) {
#pragma unroll
    for (int jj = 0; jj < 8; jj++)
        r[jj] = j0 + jj < k ? row_small(L, (int)t * k + j0 + jj, max_rows) : -1;
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
// Scan outputs as the scatter reads them: offsets [E+1], counts [E] and tile
// prefixes [tiles, E], from global memory (scan kernel) or from LDS (inline).
struct ScanView {
    const int32_t* off;
    const int32_t* cnt;
    const int32_t* tb;
};

// Where the scatter gets its rows from.
enum ScatterMode {
    kScanned = 0,   // the scan kernel ran: offsets and tile prefixes in global memory
    kInline = 1,    // the block scans the tile counts itself (small batches)
    kRouted = 2     // the block routes the whole batch itself (small batches, E <= 48)
};

// Routing inputs and outputs of the kRouted mode.
struct RouteArgs {
    const float* logits;
    int32_t* topk_idx;
    float* topk_w;
};

template <int MODE, int KL>
__global__ __launch_bounds__(kScatterThreads) void k_scatter_bf16(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const uint8_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_base,
    const uint8_t* __restrict__ tile_counts, int tiles, int row_align, int groups,
    int32_t* __restrict__ group_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int64_t T, int H, int E, int k, int TT, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row, RouteArgs ra) {
    const int lane = threadIdx.x & (kWave - 1);
    const int U = H / 8;                           // 16-byte units per row
    const int CW = (U + kWave - 1) / kWave;        // waves per token
    const bool pad_block = (int)blockIdx.x < pad_blocks;
    const int64_t gw = (int64_t)(blockIdx.x - pad_blocks) * kScatterWaves +
                       __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t t = pad_block ? T : gw / CW;
    const int chunk = (int)(gw - t * CW);
    const int u = chunk * kWave + lane;
    // the x row first, so that its load overlaps the scan or the routing
    uint4 a = make_uint4(0u, 0u, 0u, 0u);
    // experts and ranks of slots held .. held + 7; a small batch (inline scan)
    // loads the first eight before its scan, to overlap the two round trips
    // (in the prefill sizes, issuing them this early slowed the kernel)
    int e8[8], rk8[8], held = -1;
    if (t < T) {
        a = load16_nt(range_rsrc(x + t * (int64_t)H, 2 * H), 16 * u);
        if (MODE == kInline) {
            load_slots(topk_idx, tile_rank, t * k, 0, k, e8, rk8);
            held = 0;
        }
    }
    ScanView sv{expert_offsets, expert_counts, tile_base};
    __shared__ SmallLds Ls;
    if constexpr (MODE == kInline) {
        __shared__ InlineLds L;
        inline_scan(tile_counts, tiles, E, row_align, groups, blockIdx.x == 0, expert_counts,
                    expert_offsets, group_offsets, L);
        sv = ScanView{L.off, L.tot, L.tb};
    } else if constexpr (MODE == kRouted) {
        route_block_small<KL>(ra.logits, (int)T, E, k, row_align, groups, blockIdx.x == 0,
                              ra.topk_idx, ra.topk_w, expert_counts, expert_offsets,
                              group_offsets, Ls);
        sv = ScanView{Ls.off, Ls.cnt, nullptr};
    }
    if (pad_block) {
        zero_pad_rows(blockIdx.x, pad_blocks_per_expert, pad_rows_per_block, H, false, max_rows,
                      sv.cnt, sv.off, out, nullptr, row_src);
        return;
    }
    if (t >= T) return;
    const int64_t p0 = t * k;
    for (int j0 = 0; j0 < k; j0 += 8) {
        int r[8];
        if constexpr (MODE == kRouted) {
            slot_rows_small(Ls, t, j0, k, max_rows, r);
        } else {
            const int32_t* tb = sv.tb + (t / TT) * E;
            if constexpr (MODE == kInline) {
                if constexpr (MODE == kInline) {
                    if (j0 != held) {
                        load_slots(topk_idx, tile_rank, p0, j0, k, e8, rk8);
                        held = j0;
                    }
                    slot_rows(e8, rk8, sv.off, tb, E, max_rows, r);
                } else {
                    slot_rows(topk_idx, tile_rank, sv.off, tb, p0, j0, k, E, max_rows, r);
                }
            } else {
                slot_rows(topk_idx, tile_rank, sv.off, tb, p0, j0, k, E, max_rows, r);
            }
        }
        if (chunk == 0) publish_rows(lane, p0, j0, k, r, dst_row, row_src);
        if (u < U) {
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                if (r[jj] >= 0)
                    *reinterpret_cast<uint4*>(out + (int64_t)r[jj] * 2 * H + 16 * (int64_t)u) = a;
        }
    }
}

// Role of block b of a grid of T token blocks and P pad blocks: the pad
// blocks are spread evenly among the token blocks (one every D = (T + P) / P
// blocks), so that the pure writes of the pad rows mix with the reads and
// writes of the token rows instead of coming all at once. Returns the token
// index, or -1 - j for pad block j.
__device__ __forceinline__ int64_t block_role(int64_t b, int64_t T, int64_t P) {
    if (P == 0) return b;
    const int64_t D = (T + P) / P;
    if (b < P * D) return (b % D == D - 1) ? -1 - b / D : b - (b + 1) / D;
    return b - P;
}

// FP8 rows. One block per token, W waves; wave w handles row chunks w, w+W,
// ... of 64 lane units, a unit being 16 bf16 in (32 bytes) and 16 E4M3 codes
// out (16 bytes), so each aligned group of 8 lanes holds one 1x128 block and
// reduces its amax over DPP. The token is quantised once; its codes are stored
// to each destination row, and its 1x128 scales are staged in LDS and written
// to each row's scale segment with one contiguous store (instead of many small
// pieces from different waves, which cost HBM read-modify-write cycles).
template <int MODE, int KL>
__global__ __launch_bounds__(1024) void k_scatter_fp8(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ topk_idx,
    const uint8_t* __restrict__ tile_rank, const int32_t* __restrict__ tile_base,
    const uint8_t* __restrict__ tile_counts, int tiles, int row_align, int groups,
    int32_t* __restrict__ group_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ expert_offsets,
    int64_t T, int H, int E, int k, int TT, int64_t max_rows, int pad_blocks,
    int pad_blocks_per_expert, int pad_rows_per_block, unsigned char* __restrict__ out,
    float* __restrict__ scales, int32_t* __restrict__ row_src, int32_t* __restrict__ dst_row,
    RouteArgs ra) {
    extern __shared__ float s_scale[];             // [H / 128]
    const int64_t role = block_role(blockIdx.x, T, pad_blocks);
    const bool pad_block = role < 0;
    const int64_t t = pad_block ? 0 : role;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int W = blockDim.x / kWave;
    const int U = H / 16;                          // lane units per row
    const int CW = (U + kWave - 1) / kWave;
    const int nb = H / 128;
    const auto xr = range_rsrc(x + t * (int64_t)H, pad_block ? 0 : 2 * H);
    // the first chunk of the x row first, so that its load overlaps the scan
    // or the routing
    uint4 a0 = make_uint4(0u, 0u, 0u, 0u), b0 = a0;
    if (!pad_block && w < CW) {
        a0 = load16_nt(xr, 32 * (w * kWave + lane));
        b0 = load16_nt(xr, 32 * (w * kWave + lane) + 16);
    }
    // experts and ranks of slots held .. held + 7; a small batch (inline scan)
    // loads the first eight before its scan, to overlap the two round trips
    // (in the prefill sizes, issuing them this early slowed the kernel)
    int e8[8], rk8[8], held = -1;
    if (MODE == kInline && !pad_block) {
        load_slots(topk_idx, tile_rank, t * k, 0, k, e8, rk8);
        held = 0;
    }
    ScanView sv{expert_offsets, expert_counts, tile_base};
    __shared__ SmallLds Ls;
    if constexpr (MODE == kInline) {
        __shared__ InlineLds L;
        inline_scan(tile_counts, tiles, E, row_align, groups, blockIdx.x == 0, expert_counts,
                    expert_offsets, group_offsets, L);
        sv = ScanView{L.off, L.tot, L.tb};
    } else if constexpr (MODE == kRouted) {
        route_block_small<KL>(ra.logits, (int)T, E, k, row_align, groups, blockIdx.x == 0,
                              ra.topk_idx, ra.topk_w, expert_counts, expert_offsets,
                              group_offsets, Ls);
        sv = ScanView{Ls.off, Ls.cnt, nullptr};
    }
    if (pad_block) {
        zero_pad_rows((int)(-1 - role), pad_blocks_per_expert, pad_rows_per_block, H, true, max_rows,
                      sv.cnt, sv.off, out, scales, row_src);
        return;
    }
    const int64_t p0 = t * k;
    const int32_t* tb = MODE == kRouted ? nullptr : sv.tb + (t / TT) * E;

    for (int chunk = w; chunk < CW; chunk += W) {
        const int u = chunk * kWave + lane;
        const uint4 a = chunk == w ? a0 : load16_nt(xr, 32 * u);
        const uint4 b = chunk == w ? b0 : load16_nt(xr, 32 * u + 16);
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
            if constexpr (MODE == kRouted) {
                slot_rows_small(Ls, t, j0, k, max_rows, r);
            } else {
                if constexpr (MODE == kInline) {
                    if (j0 != held) {
                        load_slots(topk_idx, tile_rank, p0, j0, k, e8, rk8);
                        held = j0;
                    }
                    slot_rows(e8, rk8, sv.off, tb, E, max_rows, r);
                } else {
                    slot_rows(topk_idx, tile_rank, sv.off, tb, p0, j0, k, E, max_rows, r);
                }
            }
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
        int rr;
        if constexpr (MODE == kRouted) {
            rr = row_small(Ls, (int)p0 + j, max_rows);
        } else {
            const int e = topk_idx[p0 + j];
            if ((unsigned)e >= (unsigned)E) continue;
            rr = sv.off[e] + tb[e] + tile_rank[p0 + j];
        }
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

// CUs the stream may run on (its CU mask; every CU for a stream without
// one), or 0 if the runtime cannot say
static int stream_cus(hipStream_t stream) {
    uint32_t mask[32] = {};
    if (hipExtStreamGetCUMask(stream, 32, mask) != hipSuccess) {
        (void)hipGetLastError();   // a failed query is not the caller's error
        return 0;
    }
    int n = 0;
    for (uint32_t m : mask) n += __builtin_popcount(m);
    return n;
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream, LaunchInfo info[4], int* n,
                           bool run) {
    const DispatchWorkspace ws = dispatch_workspace(a.T, a.E, a.k);
    const int TT = ws.tile_tokens;
    const int64_t tiles = ws.tiles;
    // routing inside the count kernel when the sorting-network path applies
    const bool fused = a.logits != nullptr && route_sort_applies(a.logits, a.E, a.k);
    const bool route_first = a.logits != nullptr && !fused;
    const int S = fused ? route_lanes(a.T, a.E) : 1;
    int count_threads = fused ? TT * S : 256;
    if (count_threads < kWave) count_threads = kWave;
    const size_t count_lds = (size_t)a.E * sizeof(uint64_t) +
                             (fused ? (size_t)TT * a.k * sizeof(int32_t) : 0);
    // small batches scan inside the scatter (there must be scatter blocks)
    const bool inline_scan_ok = a.T > 0 && tiles <= kInlineTiles && tiles * a.E <= kInlineCells;
    int64_t scan_blocks = tiles < 1 ? 1 : tiles < kScanBlocks ? tiles : kScanBlocks;
    if (run && !inline_scan_ok && scan_blocks > 1) {
        const int cus = stream_cus(stream);
        if (cus > 0 && cus < scan_blocks) scan_blocks = cus;
    }
    // small batches with few experts: every scatter block routes the whole
    // batch, so dispatch is one launch (the scatter's blocks have at least
    // kSmallTokens threads)
    const bool routed = fused && a.T > 0 && a.E <= kSmallExperts && a.T <= kSmallTokens &&
                        a.T * a.k <= kSmallPairs;

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
    const char* scatter_name = routed ? "route+scan+scatter" : inline_scan_ok ? "scan+scatter" : "scatter";
    if (info) {
        if (route_first) info[nk++] = LaunchInfo{route_info.grid, route_info.block, route_info.lds,
                                                 route_info.param, "route"};
        if (!routed)
            info[nk++] = LaunchInfo{tiles, count_threads, count_lds, fused ? S : TT,
                                    fused ? "route_count" : "count"};
        if (!routed && !inline_scan_ok)
            info[nk++] = LaunchInfo{scan_blocks, kScanThreads, 0, tiles, "scan"};
        info[nk++] = a.fp8 ? LaunchInfo{scatter_blocks, fp8_threads,
                                        (size_t)(a.H / 128) * sizeof(float), fp8_waves,
                                        scatter_name}
                           : LaunchInfo{scatter_blocks, kScatterThreads, 0, bf16_waves_per_token,
                                        scatter_name};
    } else {
        nk = routed ? 1 : (route_first ? 1 : 0) + (inline_scan_ok ? 2 : 3);
    }
    if (n) *n = nk;
    if (!run) return hipSuccess;

    hipError_t err;
    if (route_first) {
        err = launch_route_topk(a.logits, a.T, a.E, a.k, 0, 0.0f, const_cast<int32_t*>(a.topk_idx),
                                a.topk_w, stream, nullptr);
        if (err != hipSuccess) return err;
    }
    const CountArgs c{a.T, a.E, a.k, TT, tiles, a.tile_counts, a.tile_rank};
    if (tiles > 0 && !routed) {
        if (fused) {
            switch (route_list_len(a.k)) {
                case 2: launch_route_count_k<2>(S, a, c, tiles, count_threads, count_lds, stream); break;
                case 4: launch_route_count_k<4>(S, a, c, tiles, count_threads, count_lds, stream); break;
                default: launch_route_count_k<8>(S, a, c, tiles, count_threads, count_lds, stream); break;
            }
        } else {
            k_count<<<dim3((unsigned)tiles), dim3(count_threads), count_lds, stream>>>(a.topk_idx, c);
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (!routed && !inline_scan_ok) {
        k_scan<<<dim3((unsigned)scan_blocks), kScanThreads, 0, stream>>>(
            a.tile_counts, tiles, a.E, a.row_align, a.groups, a.tile_base, a.expert_counts,
            a.expert_offsets, a.group_offsets);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }

    // scatter: leading blocks zero pad rows, then the token work
    unsigned char* out = static_cast<unsigned char*>(a.out);
    const uint16_t* x = static_cast<const uint16_t*>(a.x);
    if (scatter_blocks == 0) return hipSuccess;
    const RouteArgs ra{a.logits, const_cast<int32_t*>(a.topk_idx), a.topk_w};
    const int kl = route_list_len(a.k);
    if (a.fp8) {
        const size_t lds = (size_t)(a.H / 128) * sizeof(float);
        auto kern = routed ? (kl == 2 ? k_scatter_fp8<kRouted, 2>
                              : kl == 4 ? k_scatter_fp8<kRouted, 4> : k_scatter_fp8<kRouted, 8>)
                    : inline_scan_ok ? k_scatter_fp8<kInline, 2> : k_scatter_fp8<kScanned, 2>;
        kern<<<dim3((unsigned)scatter_blocks), dim3(fp8_threads), lds, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_base, a.tile_counts, (int)tiles, a.row_align,
            a.groups, a.group_offsets, a.expert_counts, a.expert_offsets, a.T, a.H, a.E, a.k, TT,
            a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block, out, a.out_scales,
            a.row_src, a.dst_row, ra);
    } else {
        auto kern = routed ? (kl == 2 ? k_scatter_bf16<kRouted, 2>
                              : kl == 4 ? k_scatter_bf16<kRouted, 4> : k_scatter_bf16<kRouted, 8>)
                    : inline_scan_ok ? k_scatter_bf16<kInline, 2> : k_scatter_bf16<kScanned, 2>;
        kern<<<dim3((unsigned)scatter_blocks), dim3(kScatterThreads), 0, stream>>>(
            x, a.topk_idx, a.tile_rank, a.tile_base, a.tile_counts, (int)tiles, a.row_align,
            a.groups, a.group_offsets, a.expert_counts, a.expert_offsets, a.T, a.H, a.E, a.k, TT,
            a.max_rows, (int)pad_blocks, pad_per_expert, pad_rows_per_block, out, a.row_src,
            a.dst_row, ra);
    }
    return hipGetLastError();
}

}  // namespace moe
