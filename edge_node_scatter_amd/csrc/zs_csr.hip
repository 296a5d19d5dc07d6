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
//              (tile-major offsets) and the node's degree; 16 threads share a
//              node's tiles;
//   3. place   per tile: the workgroup scans the degrees into rowptr in LDS
//              (the first tile writes rowptr out) and adds the tile's offsets;
//              then one wavefront takes the tile's edges 64 at a time
//              (destinations prefetched 16 steps ahead); lanes with equal keys
//              are matched with ballots, ranked by lane order, and the group's
//              first lane advances the key's running offset.
//              perm[offset + rank] = e.
// When N is too large for LDS bins, the counts stay in global memory and a
// separate block scan produces rowptr before placement.
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
    constexpr int U = 8;   // loads issued before the first is consumed
    for (int64_t chunk = e0; chunk < e1; chunk += int64_t(kCountThreads) * U) {
        int64_t keys[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = chunk + int64_t(u) * kCountThreads + threadIdx.x;
            keys[u] = e < e1 ? dst[e] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = chunk + int64_t(u) * kCountThreads + threadIdx.x;
            if (e >= e1) continue;
            const int64_t key = keys[u];
            if (key >= 0 && key < n_nodes) {
                if (kLds)
                    atomicAdd(&bins[key], 1);
                else
                    atomicAdd(&row[key], 1);
            } else {
                bad = 1;
            }
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) tile_bad[t] = bad;
    if (kLds)
        for (int64_t i = threadIdx.x; i < n_nodes; i += kCountThreads) row[i] = bins[i];
}

// Per node: counts[t][n] <- sum_{t' < t} counts[t'][n] and deg[n] <- degree.
// Workgroup = kColNodes nodes x kColChunks tile chunks; each thread sums its
// chunk, the chunk sums are scanned in LDS, then the thread rewrites its chunk
// as exclusive offsets.  Block 0 also folds the per-tile out-of-range bits into
// the flag.
constexpr int kColNodes = 16;
constexpr int kColChunks = 16;
constexpr int kColMaxPer = int((kTilesMax + kColChunks - 1) / kColChunks);
__global__ __launch_bounds__(kColNodes * kColChunks) void csr_colscan_kernel(
    int32_t* __restrict__ counts, int64_t tiles, int64_t n_nodes, int32_t* __restrict__ deg,
    const int32_t* __restrict__ tile_bad, int32_t* __restrict__ flag) {
    __shared__ int32_t chunk_sum[kColChunks][kColNodes];
    const int i = threadIdx.x % kColNodes;
    const int c = threadIdx.x / kColNodes;
    const int64_t n = int64_t(blockIdx.x) * kColNodes + i;
    const int64_t t_lo = tiles * c / kColChunks;
    const int64_t t_hi = tiles * (c + 1) / kColChunks;
    // a thread's chunk (at most kColMaxPer tiles) is held in registers between
    // the two passes, and all its loads are issued before the first is used
    int32_t v[kColMaxPer];
    int32_t sum = 0;
#pragma unroll
    for (int u = 0; u < kColMaxPer; ++u) {
        const int64_t t = t_lo + u;
        v[u] = (n < n_nodes && t < t_hi) ? counts[t * n_nodes + n] : 0;
    }
#pragma unroll
    for (int u = 0; u < kColMaxPer; ++u) sum += v[u];
    chunk_sum[c][i] = sum;
    __syncthreads();
    int32_t run = 0, total = 0;
    for (int cc = 0; cc < kColChunks; ++cc) {
        if (cc < c) run += chunk_sum[cc][i];
        total += chunk_sum[cc][i];
    }
    if (n < n_nodes) {
#pragma unroll
        for (int u = 0; u < kColMaxPer; ++u) {
            const int64_t t = t_lo + u;
            if (t < t_hi) counts[t * n_nodes + n] = run;
            run += v[u];
        }
        if (c == 0) deg[n] = total;
    }
    if (blockIdx.x == 0) {
        int bad = 0;
        for (int64_t t = threadIdx.x; t < tiles; t += blockDim.x) bad |= tile_bad[t];
        bad = __syncthreads_or(bad);
        if (threadIdx.x == 0) *flag = bad ? 1 : 0;
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
constexpr int kPlaceThreads = 256; // threads of the set-up phase
constexpr int kPlaceMultiNodes = 4096;  // up to this N, 4 wavefronts place a tile

// run[i] (LDS) = src[i] (+ run[i] when ADD), i < n, by the whole workgroup;
// 16 strided loads per thread are issued before any is consumed.
template <bool ADD>
__device__ inline void lds_gather(int32_t* run, const int32_t* __restrict__ src, int64_t n) {
    constexpr int U = 16;
    for (int64_t base = 0; base < n; base += int64_t(kPlaceThreads) * U) {
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + int64_t(u) * kPlaceThreads + threadIdx.x;
            v[u] = i < n ? src[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + int64_t(u) * kPlaceThreads + threadIdx.x;
            if (i < n) run[i] = ADD ? run[i] + v[u] : v[u];
        }
    }
}

// In-place exclusive scan of run[0..n) (LDS) by the whole workgroup; returns
// the total.  Each thread scans a contiguous run of entries.
__device__ inline int32_t block_exclusive_scan_lds(int32_t* run, int64_t n) {
    __shared__ int32_t wave_tot[kPlaceThreads / 64];
    const int tid = threadIdx.x;
    const int64_t per = (n + kPlaceThreads - 1) / kPlaceThreads;
    const int64_t lo = tid * per < n ? tid * per : n;
    const int64_t hi = lo + per < n ? lo + per : n;
    int32_t local = 0;
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t d = run[i];
        run[i] = local;
        local += d;
    }
    const int32_t incl = wave_inclusive_scan(local);
    const int wave = tid >> 6, lane = tid & 63;
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t off = 0, total = 0;
    for (int w = 0; w < kPlaceThreads / 64; ++w) {
        if (w < wave) off += wave_tot[w];
        total += wave_tot[w];
    }
    off += incl - local;
    for (int64_t i = lo; i < hi; ++i) run[i] += off;
    __syncthreads();
    return total;
}

// LDS path (N <= kLdsBinsMax): rowptr is computed here from the degrees (the
// first tile's workgroup writes it out).  The tile is split into PW contiguous
// parts, one per wavefront; each part's running offsets start at
//   rowptr[n] + (offset of this tile in node n's list) + (edges of node n in
//   the tile's earlier parts),
// so the PW wavefronts place their parts independently and the result is the
// same as one wavefront walking the whole tile.  Global path (PW = 1): rowptr
// comes from the scan kernels and the running offsets live in the tile's row
// of counts.
template <bool kLds, int PW>
__global__ __launch_bounds__(kPlaceThreads) void csr_place_kernel(
    const int64_t* __restrict__ dst, int64_t n_edges, int64_t n_nodes, int64_t tile_edges,
    int32_t* __restrict__ counts, const int32_t* __restrict__ deg, int32_t* __restrict__ rowptr,
    int32_t* __restrict__ perm, int32_t* __restrict__ dst32, int key_bits) {
    extern __shared__ int32_t lds[];    // kLds: PW * n_nodes running offsets
    constexpr int kPerThread = (kPlaceMultiNodes + kPlaceThreads - 1) / kPlaceThreads;
    const int64_t t = blockIdx.x;
    const int64_t e0 = t * tile_edges;
    const int64_t e1 = e0 + tile_edges < n_edges ? e0 + tile_edges : n_edges;
    const int64_t part = (e1 - e0 + PW - 1) / PW;
    int32_t* row = counts + t * n_nodes;
    const int wave = threadIdx.x >> 6;
    if (kLds) {
        lds_gather<false>(lds, deg, n_nodes);
        __syncthreads();
        const int32_t total = block_exclusive_scan_lds(lds, n_nodes);
        if (t == 0) {
            for (int64_t i = threadIdx.x; i < n_nodes; i += kPlaceThreads) rowptr[i] = lds[i];
            if (threadIdx.x == 0) rowptr[n_nodes] = total;
        }
        __syncthreads();
        lds_gather<true>(lds, row, n_nodes);
        __syncthreads();
        if (PW > 1) {
            // per-part histograms, then per-part running offsets
            int32_t base[kPerThread];
#pragma unroll
            for (int u = 0; u < kPerThread; ++u) {
                const int64_t n = int64_t(u) * kPlaceThreads + threadIdx.x;
                base[u] = n < n_nodes ? lds[n] : 0;
            }
            __syncthreads();
            for (int64_t i = threadIdx.x; i < PW * n_nodes; i += kPlaceThreads) lds[i] = 0;
            __syncthreads();
            {
                const int64_t p0 = e0 + wave * part;
                const int64_t p1 = p0 + part < e1 ? p0 + part : e1;
                for (int64_t chunk = p0; chunk < p1; chunk += 64 * kPlaceAhead) {
                    int64_t keys[kPlaceAhead];
#pragma unroll
                    for (int j = 0; j < kPlaceAhead; ++j) {
                        const int64_t e = chunk + j * 64 + (threadIdx.x & 63);
                        keys[j] = e < p1 ? dst[e] : -1;
                    }
#pragma unroll
                    for (int j = 0; j < kPlaceAhead; ++j)
                        if (keys[j] >= 0 && keys[j] < n_nodes)
                            atomicAdd(&lds[wave * n_nodes + keys[j]], 1);
                }
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < kPerThread; ++u) {
                const int64_t n = int64_t(u) * kPlaceThreads + threadIdx.x;
                if (n < n_nodes) {
                    int32_t b = base[u];
#pragma unroll
                    for (int w = 0; w < PW; ++w) {
                        const int32_t c = lds[w * n_nodes + n];
                        lds[w * n_nodes + n] = b;
                        b += c;
                    }
                }
            }
            __syncthreads();
        }
    }
    if (wave >= PW) return;
    int32_t* run = lds + (PW > 1 ? wave * n_nodes : 0);
    const int lane = threadIdx.x & 63;
    const int64_t p0 = e0 + wave * part;
    const int64_t p1 = p0 + part < e1 ? p0 + part : e1;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t chunk = p0; chunk < p1; chunk += 64 * kPlaceAhead) {
        int64_t keys[kPlaceAhead];
#pragma unroll
        for (int j = 0; j < kPlaceAhead; ++j) {
            const int64_t e = chunk + j * 64 + lane;
            keys[j] = e < p1 ? dst[e] : -1;
        }
#pragma unroll
        for (int j = 0; j < kPlaceAhead; ++j) {
            const int64_t e = chunk + j * 64 + lane;
            if (chunk + j * 64 >= p1) break;           // uniform
            const bool in = e < p1;
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
            int32_t b0 = 0;
            if (ok && rank == 0) {
                if (kLds) {
                    b0 = run[key];
                    run[key] = b0 + cnt;
                } else {
                    b0 = rowptr[key] + atomicAdd(&row[key], cnt);
                }
            }
            b0 = __shfl(b0, leader, 64);
            const int64_t pos = int64_t(b0) + rank;
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
    p.off_deg = align(p.off_tile_bad + size_t(tiles) * sizeof(int32_t));
    p.off_counts = align(p.off_deg + size_t(n_nodes) * sizeof(int32_t));
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
    int32_t* deg = reinterpret_cast<int32_t*>(ws + plan.off_deg);
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
    // degrees go straight to rowptr[1..N] on the global path (scanned below)
    int32_t* deg_out = plan.lds_bins ? deg : rowptr + 1;
    csr_colscan_kernel<<<grid_for(n_nodes, kColNodes, int64_t(1) << 30), kColNodes * kColChunks, 0,
                         stream>>>(counts, plan.tiles, n_nodes, deg_out, tile_bad, flag);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    int key_bits = 1;
    while (key_bits < 31 && (int64_t(1) << key_bits) < n_nodes) ++key_bits;
    if (plan.lds_bins) {
        if (n_nodes <= kPlaceMultiNodes)
            csr_place_kernel<true, 4><<<unsigned(plan.tiles), kPlaceThreads, 4 * lds, stream>>>(
                dst, n_edges, n_nodes, plan.tile_edges, counts, deg, rowptr, perm, dst32,
                key_bits);
        else
            csr_place_kernel<true, 1><<<unsigned(plan.tiles), kPlaceThreads, lds, stream>>>(
                dst, n_edges, n_nodes, plan.tile_edges, counts, deg, rowptr, perm, dst32,
                key_bits);
        return hipGetLastError();
    }
    // global path: inclusive scan of degrees in rowptr[1..N]
    if ((err = launch_fill_i32(rowptr, 1, 0, stream)) != hipSuccess) return err;
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
    csr_place_kernel<false, 1><<<unsigned(plan.tiles), kPlaceThreads, 0, stream>>>(
        dst, n_edges, n_nodes, plan.tile_edges, counts, deg, rowptr, perm, dst32, key_bits);
    return hipGetLastError();
}

}  // namespace zs
