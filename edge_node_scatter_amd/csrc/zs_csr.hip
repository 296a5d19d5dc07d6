// Stable destination CSR for the GIE zonal scatter, gfx950.
//
// The fused forward walks each node's edges in the order index_add would add
// them, i.e. increasing edge id (deepmd-kit PR #6072, "fused Triton zonal
// scatter for the GIE head", section "What", last bullet).  This file builds
// that CSR with a deterministic counting sort; no result depends on the order
// in which atomics land:
//
//   1. count   one workgroup per edge tile histograms its destinations (LDS
//              bins when N fits, else the tile's own global row) and records
//              whether the tile held an out-of-range destination;
//   2. colscan per node, the exclusive scan of the per-tile counts over tiles
//              (tile-major offsets) and the node's degree; 8 threads share a
//              node's tiles, so the scan runs on N*8 threads;
//   3. scan    exclusive scan of degrees over nodes -> rowptr;
//   4. place   one wavefront per tile: running offsets rowptr[n] + offset of
//              the tile in node n's list start in LDS; the tile's edges are
//              taken 64 at a time (destinations prefetched 16 steps ahead);
//              lanes with equal keys are matched with ballots, ranked by lane
//              order, and the group's first lane advances the key's offset.
//              perm[offset + rank] = e.
//
// Every destination is range-checked; an out-of-range one is never used as an
// index and raises the validation flag.
#include "zs_internal.h"

namespace zs {

namespace {

constexpr int kCountThreads = 256;
constexpr int kScanThreads = 256;
constexpr int kScanItems = 16;
constexpr int kScanBlock = kScanThreads * kScanItems;   // elements per scan block
constexpr int64_t kLdsBinsMax = 16384;                 // 64 KiB of int32 bins
constexpr int64_t kTileEdgesMin = 2048;
constexpr int64_t kTilesMax = 1024;
constexpr int64_t kCountBudget = int64_t(1) << 24;     // max tiles * nodes entries

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = v;
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = v;
}

template <bool kLds>
__global__ __launch_bounds__(kCountThreads) void csr_count_kernel(
    const int64_t* __restrict__ dst, int64_t n_edges, int64_t n_nodes, int64_t tile_edges,
    int32_t* __restrict__ counts, int32_t* __restrict__ tile_bad) {
    extern __shared__ int32_t bins[];
    const int64_t t = blockIdx.x;
    const int64_t e0 = t * tile_edges;
    const int64_t e1 = e0 + tile_edges < n_edges ? e0 + tile_edges : n_edges;
    int32_t* row = counts + t * n_nodes;
    for (int64_t i = threadIdx.x; i < n_nodes; i += kCountThreads) {
        if (kLds)
            bins[i] = 0;
        else
            row[i] = 0;
    }
    __syncthreads();
    int bad = 0;
    for (int64_t e = e0 + threadIdx.x; e < e1; e += kCountThreads) {
        const int64_t key = dst[e];
        if (key >= 0 && key < n_nodes) {
            if (kLds)
                atomicAdd(&bins[key], 1);
            else
                atomicAdd(&row[key], 1);
        } else {
            bad = 1;
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) tile_bad[t] = bad;
    if (kLds)
        for (int64_t i = threadIdx.x; i < n_nodes; i += kCountThreads) row[i] = bins[i];
}

// Per node: counts[t][n] <- sum_{t' < t} counts[t'][n]; rowptr[n+1] <- degree.
// Workgroup = kColNodes nodes x kColChunks tile chunks.  Block 0 also folds the
// per-tile validation bits into the flag and sets rowptr[0].
constexpr int kColNodes = 32;
constexpr int kColChunks = 8;
__global__ __launch_bounds__(kColNodes * kColChunks) void csr_colscan_kernel(
    int32_t* __restrict__ counts, int64_t tiles, int64_t n_nodes, int32_t* __restrict__ rowptr,
    const int32_t* __restrict__ tile_bad, int32_t* __restrict__ flag) {
    __shared__ int32_t chunk_sum[kColChunks][kColNodes];
    const int i = threadIdx.x % kColNodes;
    const int c = threadIdx.x / kColNodes;
    const int64_t n = int64_t(blockIdx.x) * kColNodes + i;
    const int64_t t_lo = tiles * c / kColChunks;
    const int64_t t_hi = tiles * (c + 1) / kColChunks;
    int32_t sum = 0;
    if (n < n_nodes) {
        int64_t t = t_lo;
        for (; t + 8 <= t_hi; t += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = counts[(t + u) * n_nodes + n];
#pragma unroll
            for (int u = 0; u < 8; ++u) sum += v[u];
        }
        for (; t < t_hi; ++t) sum += counts[t * n_nodes + n];
    }
    chunk_sum[c][i] = sum;
    __syncthreads();
    int32_t run = 0, total = 0;
    for (int cc = 0; cc < kColChunks; ++cc) {
        if (cc < c) run += chunk_sum[cc][i];
        total += chunk_sum[cc][i];
    }
    if (n < n_nodes) {
        int64_t t = t_lo;
        for (; t + 8 <= t_hi; t += 8) {
            int32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = counts[(t + u) * n_nodes + n];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                counts[(t + u) * n_nodes + n] = run;
                run += v[u];
            }
        }
        for (; t < t_hi; ++t) {
            const int32_t v = counts[t * n_nodes + n];
            counts[t * n_nodes + n] = run;
            run += v;
        }
        if (c == 0) rowptr[n + 1] = total;
    }
    if (blockIdx.x == 0) {
        int bad = 0;
        for (int64_t t = threadIdx.x; t < tiles; t += blockDim.x) bad |= tile_bad[t];
        bad = __syncthreads_or(bad);
        if (threadIdx.x == 0) {
            *flag = bad ? 1 : 0;
            rowptr[0] = 0;
        }
    }
}

__device__ inline int32_t wave_inclusive_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// In-place inclusive scan of a[0..n) in blocks of kScanBlock; block totals to sums.
__global__ __launch_bounds__(kScanThreads) void scan_block_kernel(int32_t* __restrict__ a,
                                                                   int64_t n,
                                                                   int32_t* __restrict__ sums) {
    __shared__ int32_t wave_tot[kScanThreads / 64];
    const int64_t base = int64_t(blockIdx.x) * kScanBlock + int64_t(threadIdx.x) * kScanItems;
    int32_t v[kScanItems];
    int32_t run = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        v[i] = (base + i < n) ? a[base + i] : 0;
        run += v[i];
        v[i] = run;
    }
    const int32_t incl = wave_inclusive_scan(run);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += wave_tot[w];
    const int32_t excl = wave_off + incl - run;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i)
        if (base + i < n) a[base + i] = v[i] + excl;
    if (threadIdx.x == kScanThreads - 1) sums[blockIdx.x] = wave_off + incl;
}

// Single workgroup: exclusive scan of the block totals, in chunks with a carry.
__global__ __launch_bounds__(kScanThreads) void scan_sums_kernel(int32_t* __restrict__ sums,
                                                                  int64_t n) {
    __shared__ int32_t wave_tot[kScanThreads / 64];
    __shared__ int32_t carry_sh;
    if (threadIdx.x == 0) carry_sh = 0;
    __syncthreads();
    for (int64_t base = 0; base < n; base += kScanThreads) {
        const int64_t i = base + threadIdx.x;
        const int32_t x = i < n ? sums[i] : 0;
        const int32_t incl = wave_inclusive_scan(x);
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        int32_t off = carry_sh;
        int32_t tot = 0;
        for (int w = 0; w < kScanThreads / 64; ++w) {
            if (w < wave) off += wave_tot[w];
            tot += wave_tot[w];
        }
        if (i < n) sums[i] = off + incl - x;
        __syncthreads();
        if (threadIdx.x == 0) carry_sh += tot;
        __syncthreads();
    }
}

__global__ __launch_bounds__(kScanThreads) void scan_add_kernel(int32_t* __restrict__ a, int64_t n,
                                                                 const int32_t* __restrict__ sums) {
    const int32_t off = sums[blockIdx.x];
    const int64_t base = int64_t(blockIdx.x) * kScanBlock;
    for (int i = threadIdx.x; i < kScanBlock; i += kScanThreads)
        if (base + i < n) a[base + i] += off;
}

constexpr int kPlaceAhead = 16;   // 64-edge steps whose destinations are prefetched

template <bool kLds>
__global__ __launch_bounds__(64) void csr_place_kernel(
    const int64_t* __restrict__ dst, int64_t n_edges, int64_t n_nodes, int64_t tile_edges,
    int32_t* __restrict__ counts, const int32_t* __restrict__ rowptr, int32_t* __restrict__ perm,
    int32_t* __restrict__ dst32, int key_bits) {
    extern __shared__ int32_t run[];
    const int lane = threadIdx.x;
    const int64_t t = blockIdx.x;
    const int64_t e0 = t * tile_edges;
    const int64_t e1 = e0 + tile_edges < n_edges ? e0 + tile_edges : n_edges;
    int32_t* row = counts + t * n_nodes;
    if (kLds) {
        // running position of the next edge of node n inside this tile; the
        // loads of 8 strides are issued before any is consumed
        int64_t i0 = 0;
        for (; i0 + 8 * 64 <= n_nodes; i0 += 8 * 64) {
            int32_t a[8], c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                a[u] = rowptr[i0 + u * 64 + lane];
                c[u] = row[i0 + u * 64 + lane];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) run[i0 + u * 64 + lane] = a[u] + c[u];
        }
        for (int64_t i = i0 + lane; i < n_nodes; i += 64) run[i] = rowptr[i] + row[i];
        __syncthreads();
    }
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t chunk = e0; chunk < e1; chunk += 64 * kPlaceAhead) {
        int64_t keys[kPlaceAhead];
#pragma unroll
        for (int j = 0; j < kPlaceAhead; ++j) {
            const int64_t e = chunk + j * 64 + lane;
            keys[j] = e < e1 ? dst[e] : -1;
        }
#pragma unroll
        for (int j = 0; j < kPlaceAhead; ++j) {
            const int64_t e = chunk + j * 64 + lane;
            if (chunk + j * 64 >= e1) break;           // uniform
            const bool in = e < e1;
            const int64_t key64 = keys[j];
            const bool ok = in && key64 >= 0 && key64 < n_nodes;
            const int32_t key = ok ? int32_t(key64) : 0;
            if (in) dst32[e] = ok ? key : -1;
            uint64_t same = __ballot(ok);
            for (int b = 0; b < key_bits; ++b) {
                const bool bit = (key >> b) & 1;
                const uint64_t bal = __ballot(ok && bit);
                same &= bit ? bal : ~bal;
            }
            const int rank = __popcll(same & below);
            const int cnt = __popcll(same);
            const int leader = ok ? __ffsll((unsigned long long)same) - 1 : lane;
            int32_t base = 0;
            if (ok && rank == 0) {
                if (kLds) {
                    base = run[key];
                    run[key] = base + cnt;
                } else {
                    base = rowptr[key] + atomicAdd(&row[key], cnt);
                }
            }
            base = __shfl(base, leader, 64);
            const int64_t pos = int64_t(base) + rank;
            if (ok && pos >= 0 && pos < n_edges) perm[pos] = int32_t(e);
        }
    }
}

inline unsigned grid_for(int64_t n, int threads, int64_t cap = 1 << 20) {
    int64_t g = (n + threads - 1) / threads;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return unsigned(g);
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    fill_i32_kernel<<<grid_for(n, 256, 4096), 256, 0, stream>>>(p, n, v);
    return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    fill_f32_kernel<<<grid_for(n, 256, 4096), 256, 0, stream>>>(p, n, v);
    return hipGetLastError();
}

CsrPlan plan_csr(int64_t n_edges, int64_t n_nodes) {
    CsrPlan p{};
    int64_t tiles = (n_edges + kTileEdgesMin - 1) / kTileEdgesMin;
    if (tiles < 1) tiles = 1;
    if (tiles > kTilesMax) tiles = kTilesMax;
    const int64_t by_budget = kCountBudget / (n_nodes > 0 ? n_nodes : 1);
    if (tiles > by_budget) tiles = by_budget > 0 ? by_budget : 1;
    int64_t tile_edges = n_edges > 0 ? (n_edges + tiles - 1) / tiles : 1;
    if (n_edges > 0) tiles = (n_edges + tile_edges - 1) / tile_edges;
    p.tiles = tiles;
    p.tile_edges = tile_edges;
    p.lds_bins = n_nodes <= kLdsBinsMax;
    p.scan_blocks = (n_nodes + kScanBlock - 1) / kScanBlock;
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.off_flag = 0;
    p.off_tile_bad = 256;
    p.off_counts = align(p.off_tile_bad + size_t(tiles) * sizeof(int32_t));
    p.off_blocks = align(p.off_counts + size_t(tiles) * size_t(n_nodes) * sizeof(int32_t));
    p.bytes = align(p.off_blocks + size_t(p.scan_blocks > 0 ? p.scan_blocks : 1) * sizeof(int32_t));
    return p;
}

hipError_t launch_csr(const int64_t* dst, int64_t n_edges, int64_t n_nodes, int32_t* rowptr,
                      int32_t* perm, int32_t* dst32, void* workspace, const CsrPlan& plan,
                      int32_t* flag, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    if (!flag) flag = reinterpret_cast<int32_t*>(ws + plan.off_flag);
    int32_t* tile_bad = reinterpret_cast<int32_t*>(ws + plan.off_tile_bad);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + plan.off_counts);
    int32_t* sums = reinterpret_cast<int32_t*>(ws + plan.off_blocks);
    hipError_t err;
    const size_t lds = plan.lds_bins ? size_t(n_nodes) * sizeof(int32_t) : 0;
    if (plan.lds_bins)
        csr_count_kernel<true><<<unsigned(plan.tiles), kCountThreads, lds, stream>>>(
            dst, n_edges, n_nodes, plan.tile_edges, counts, tile_bad);
    else
        csr_count_kernel<false><<<unsigned(plan.tiles), kCountThreads, 0, stream>>>(
            dst, n_edges, n_nodes, plan.tile_edges, counts, tile_bad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    csr_colscan_kernel<<<grid_for(n_nodes, kColNodes, int64_t(1) << 30), kColNodes * kColChunks, 0,
                         stream>>>(counts, plan.tiles, n_nodes, rowptr, tile_bad, flag);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // inclusive scan of degrees in rowptr[1..N] -> rowptr[n+1] = edges with dst <= n
    scan_block_kernel<<<unsigned(plan.scan_blocks), kScanThreads, 0, stream>>>(rowptr + 1, n_nodes,
                                                                               sums);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (plan.scan_blocks > 1) {
        scan_sums_kernel<<<1, kScanThreads, 0, stream>>>(sums, plan.scan_blocks);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        scan_add_kernel<<<unsigned(plan.scan_blocks), kScanThreads, 0, stream>>>(rowptr + 1,
                                                                                 n_nodes, sums);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    int key_bits = 1;
    while (key_bits < 31 && (int64_t(1) << key_bits) < n_nodes) ++key_bits;
    if (plan.lds_bins)
        csr_place_kernel<true><<<unsigned(plan.tiles), 64, lds, stream>>>(
            dst, n_edges, n_nodes, plan.tile_edges, counts, rowptr, perm, dst32, key_bits);
    else
        csr_place_kernel<false><<<unsigned(plan.tiles), 64, 0, stream>>>(
            dst, n_edges, n_nodes, plan.tile_edges, counts, rowptr, perm, dst32, key_bits);
    return hipGetLastError();
}

}  // namespace zs
