// Stable destination CSR for the GIE zonal scatter, gfx950.
//
// The fused forward walks each node's edges in the order index_add would add
// them, i.e. increasing edge id (deepmd-kit PR #6072, "fused Triton zonal
// scatter for the GIE head", section "What", last bullet).  This file builds
// that CSR with a deterministic two-level counting sort; no result depends on
// the order in which atomics land.
//
// Nodes are grouped into NB <= 1024 buckets of BN = 2^SB consecutive nodes
// (BN = 8 up to 8192 nodes).
//
//   1. bucket_count  one workgroup per edge tile histograms the tile's bucket
//                    ids in LDS and records whether the tile held an
//                    out-of-range destination;
//   2. bucket_scan   per bucket, the exclusive scan of the per-tile counts over
//                    tiles and the bucket's total; folds the out-of-range bits
//                    into the flag;
//   3. bucket_place  per tile: bucket starts (scan of the totals; tile 0 also
//                    writes them out) plus the tile's offsets give each
//                    bucket's running offset; the tile
//                    is split into 4 parts (one wavefront each, with per-part
//                    histograms so the parts start at the right offsets); lanes
//                    with equal bucket ids are matched with ballots and ranked
//                    by lane order.  Writes (destination, edge) pairs grouped by
//                    bucket, in increasing edge id within each bucket, and dst32;
//   4. node_place    one workgroup per bucket reads its contiguous run of pairs,
//                    histograms the local node ids (4 parts, per-part counts),
//                    writes rowptr for its nodes and places perm the same way.
//
// Both levels are stable, so perm lists each node's edges in increasing edge
// id.  Traffic is a few int32/int64 passes over the edges; the per-tile count
// matrix is tiles x NB entries, far smaller than tiles x N.
//
// Every destination is range-checked; an out-of-range one is never used as an
// index and raises the validation flag.
#include "zs_csr.h"

namespace zs {

namespace {

constexpr int kThreads = 256;                // every CSR kernel: 4 wavefronts
constexpr int kParts = kThreads / 64;        // wavefronts that place a tile / bucket
constexpr int kAhead = 8;                    // 64-edge steps whose keys are held at once
constexpr int64_t kTileEdgesMin = 1024;      // 4 steps per wavefront
constexpr int64_t kTilesMax = 4096;
constexpr int64_t kCountBudget = int64_t(1) << 21;   // tiles x buckets entries (8 MiB)
#ifndef ZS_CSR_BUCKET_BITS
#define ZS_CSR_BUCKET_BITS 10
#endif
constexpr int kBucketsMaxBits = ZS_CSR_BUCKET_BITS;   // NB <= 1024 (LDS tables <= 20 KiB)
constexpr int kBucketMinBits = 3;            // BN >= 8
constexpr int kNodeLdsMax = 2048;            // BN handled with LDS tables

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

__device__ inline int32_t wave_inclusive_scan(int32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// In-place exclusive scan of a[0..n) (LDS) by the whole workgroup; returns the
// total.  Each thread scans a contiguous run of entries.
__device__ inline int32_t block_exclusive_scan_lds(int32_t* a, int64_t n) {
    __shared__ int32_t wave_tot[kThreads / 64];
    const int tid = threadIdx.x;
    const int64_t per = (n + kThreads - 1) / kThreads;
    const int64_t lo = tid * per < n ? tid * per : n;
    const int64_t hi = lo + per < n ? lo + per : n;
    int32_t local = 0;
    for (int64_t i = lo; i < hi; ++i) {
        const int32_t d = a[i];
        a[i] = local;
        local += d;
    }
    const int32_t incl = wave_inclusive_scan(local);
    const int wave = tid >> 6, lane = tid & 63;
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int32_t off = 0, total = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
        if (w < wave) off += wave_tot[w];
        total += wave_tot[w];
    }
    off += incl - local;
    for (int64_t i = lo; i < hi; ++i) a[i] += off;
    __syncthreads();
    return total;
}

// dst[0..n) (LDS) <- src[0..n) (global), 16 loads per thread in flight.
__device__ inline void lds_load(int32_t* dst, const int32_t* __restrict__ src, int64_t n) {
    constexpr int U = 16;
    for (int64_t base = 0; base < n; base += int64_t(kThreads) * U) {
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + int64_t(u) * kThreads + threadIdx.x;
            v[u] = i < n ? src[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + int64_t(u) * kThreads + threadIdx.x;
            if (i < n) dst[i] = v[u];
        }
    }
}

// Lanes of the wavefront whose `key` (bits bits wide) equals this lane's,
// among the lanes with ok set.
__device__ inline uint64_t match_key(bool ok, int32_t key, int bits) {
    uint64_t same = __ballot(ok);
    for (int b = 0; b < bits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t bal = __ballot(ok && bit);
        same &= bit ? bal : ~bal;
    }
    return same;
}

// ---- level 1: buckets of BN consecutive nodes -------------------------------

__global__ __launch_bounds__(kThreads) void csr_bucket_count_kernel(
    const int64_t* __restrict__ dst, int64_t n_edges, int64_t n_nodes, int64_t tile_edges,
    int sb, int64_t n_buckets, int32_t* __restrict__ counts, int32_t* __restrict__ tile_bad) {
    extern __shared__ int32_t bins[];
    const int64_t t = blockIdx.x;
    const int64_t e0 = t * tile_edges;
    const int64_t e1 = e0 + tile_edges < n_edges ? e0 + tile_edges : n_edges;
    for (int64_t i = threadIdx.x; i < n_buckets; i += kThreads) bins[i] = 0;
    __syncthreads();
    int bad = 0;
    constexpr int U = 8;   // loads issued before the first is consumed
    for (int64_t chunk = e0; chunk < e1; chunk += int64_t(kThreads) * U) {
        int64_t keys[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = chunk + int64_t(u) * kThreads + threadIdx.x;
            keys[u] = e < e1 ? dst[e] : 0;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t e = chunk + int64_t(u) * kThreads + threadIdx.x;
            if (e >= e1) continue;
            const int64_t key = keys[u];
            if (key >= 0 && key < n_nodes)
                atomicAdd(&bins[key >> sb], 1);
            else
                bad = 1;
        }
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) tile_bad[t] = bad;
    int32_t* row = counts + t * n_buckets;
    for (int64_t i = threadIdx.x; i < n_buckets; i += kThreads) row[i] = bins[i];
}

// Per bucket: counts[t][b] <- sum_{t' < t} counts[t'][b] and tot[b] <- total.
// Workgroup = kColBuckets buckets x kColChunks tile chunks; each thread sums
// its chunk, the chunk sums are scanned in LDS, then the thread walks its
// chunk again (now from the cache) rewriting it as exclusive offsets.  Block 0
// also folds the per-tile out-of-range bits into the flag.  Up to
// kColFewTiles tiles, 4 buckets per workgroup (four times the workgroups for
// short columns: the 1000-node frame's whole build 25.2 vs 27.6 us, the
// 4096-node frames' within the run-to-run spread); longer columns keep 16 (the
// 16384-node frame's 2048 tiles: 81.6 us, against 102.9 us with 4).
constexpr int kColChunks = 64;
constexpr int64_t kColFewTiles = 1024;
template <int kColBuckets>
__global__ __launch_bounds__(kColBuckets * kColChunks) void csr_bucket_scan_kernel(
    int32_t* __restrict__ counts, int64_t tiles, int64_t n_buckets, int32_t* __restrict__ tot,
    const int32_t* __restrict__ tile_bad, int32_t* __restrict__ flag) {
    __shared__ int32_t chunk_sum[kColChunks][kColBuckets];
    const int i = threadIdx.x % kColBuckets;
    const int c = threadIdx.x / kColBuckets;
    const int64_t b = int64_t(blockIdx.x) * kColBuckets + i;
    const int64_t t_lo = tiles * c / kColChunks;
    const int64_t t_hi = tiles * (c + 1) / kColChunks;
    int32_t sum = 0;
    if (b < n_buckets) {
#pragma unroll 8
        for (int64_t t = t_lo; t < t_hi; ++t) sum += counts[t * n_buckets + b];
    }
    chunk_sum[c][i] = sum;
    __syncthreads();
    int32_t run = 0, total = 0;
    for (int cc = 0; cc < kColChunks; ++cc) {
        if (cc < c) run += chunk_sum[cc][i];
        total += chunk_sum[cc][i];
    }
    if (b < n_buckets) {
#pragma unroll 8
        for (int64_t t = t_lo; t < t_hi; ++t) {
            const int32_t v = counts[t * n_buckets + b];
            counts[t * n_buckets + b] = run;
            run += v;
        }
        if (c == 0) tot[b] = total;
    }
    if (blockIdx.x == 0) {
        int bad = 0;
        for (int64_t t = threadIdx.x; t < tiles; t += blockDim.x) bad |= tile_bad[t];
        bad = __syncthreads_or(bad);
        if (threadIdx.x == 0) *flag = bad ? 1 : 0;
    }
}

// Per tile: pairs[pos] = (dst, e) grouped by bucket; dst32[e].  LDS: the
// running offsets of the kParts parts, kParts x NB entries.  Part w of the
// tile starts, for bucket b, at
//   start[b] + (edges of b in earlier tiles) + (edges of b in parts < w).
__global__ __launch_bounds__(kThreads) void csr_bucket_place_kernel(
    const int64_t* __restrict__ dst, int64_t n_edges, int64_t n_nodes, int64_t tile_edges,
    int sb, int64_t n_buckets, int bucket_bits, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ tot, int2* __restrict__ pairs, int32_t* __restrict__ dst32,
    int32_t* __restrict__ starts) {
    extern __shared__ int32_t lds[];   // [0, NB): base; [NB, (1 + kParts) NB): parts
    int32_t* base = lds;
    int32_t* run_all = lds + n_buckets;
    const int64_t t = blockIdx.x;
    const int64_t e0 = t * tile_edges;
    const int64_t e1 = e0 + tile_edges < n_edges ? e0 + tile_edges : n_edges;
    const int64_t part = (e1 - e0 + kParts - 1) / kParts;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t p0 = e0 + wave * part < e1 ? e0 + wave * part : e1;
    const int64_t p1 = p0 + part < e1 ? p0 + part : e1;

    // this part's first keys are requested before anything else
    const bool single = p1 - p0 <= 64 * kAhead;
    int64_t keys[kAhead];
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
        const int64_t e = p0 + j * 64 + lane;
        keys[j] = e < p1 ? dst[e] : -1;
    }
    // bucket starts (tile 0 publishes them for the node level), plus this
    // tile's offsets within each bucket
    lds_load(base, tot, n_buckets);
    for (int64_t i = threadIdx.x; i < kParts * n_buckets; i += kThreads) run_all[i] = 0;
    __syncthreads();
    const int32_t total = block_exclusive_scan_lds(base, n_buckets);
    if (t == 0) {
        for (int64_t i = threadIdx.x; i < n_buckets; i += kThreads) starts[i] = base[i];
        if (threadIdx.x == 0) starts[n_buckets] = total;
    }
    {
        const int32_t* row = counts + t * n_buckets;
        constexpr int U = 16;
        for (int64_t b0 = 0; b0 < n_buckets; b0 += int64_t(kThreads) * U) {
            int32_t v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = b0 + int64_t(u) * kThreads + threadIdx.x;
                v[u] = i < n_buckets ? row[i] : 0;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = b0 + int64_t(u) * kThreads + threadIdx.x;
                if (i < n_buckets) base[i] += v[u];
            }
        }
    }
    // per-part histograms; a part of at most kAhead steps keeps its keys in
    // registers for the placement pass
    for (int64_t chunk = p0; chunk < p1; chunk += 64 * kAhead) {
        if (chunk != p0) {
#pragma unroll
            for (int j = 0; j < kAhead; ++j) {
                const int64_t e = chunk + j * 64 + lane;
                keys[j] = e < p1 ? dst[e] : -1;
            }
        }
#pragma unroll
        for (int j = 0; j < kAhead; ++j)
            if (keys[j] >= 0 && keys[j] < n_nodes)
                atomicAdd(&run_all[wave * n_buckets + (keys[j] >> sb)], 1);
    }
    __syncthreads();
    for (int64_t b = threadIdx.x; b < n_buckets; b += kThreads) {
        int32_t o = base[b];
#pragma unroll
        for (int w = 0; w < kParts; ++w) {
            const int32_t c = run_all[w * n_buckets + b];
            run_all[w * n_buckets + b] = o;
            o += c;
        }
    }
    __syncthreads();

    int32_t* run = run_all + wave * n_buckets;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t chunk = p0; chunk < p1; chunk += 64 * kAhead) {
        if (!single) {
#pragma unroll
            for (int j = 0; j < kAhead; ++j) {
                const int64_t e = chunk + j * 64 + lane;
                keys[j] = e < p1 ? dst[e] : -1;
            }
        }
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            if (chunk + j * 64 >= p1) break;           // uniform
            const int64_t e = chunk + j * 64 + lane;
            const bool in = e < p1;
            const int64_t key64 = keys[j];
            const bool ok = in && key64 >= 0 && key64 < n_nodes;
            const int32_t key = ok ? int32_t(key64) : 0;
            if (in) dst32[e] = ok ? key : -1;
            const int32_t bucket = key >> sb;
            const uint64_t same = match_key(ok, bucket, bucket_bits);
            const int rank = __popcll(same & below);
            const int cnt = __popcll(same);
            const int leader = ok ? __ffsll((unsigned long long)same) - 1 : lane;
            int32_t o = 0;
            wave_lds_sync();   // the previous step's leaders wrote run[] entries read here
            if (ok && rank == 0) {
                o = run[bucket];
                run[bucket] = o + cnt;
            }
            o = __shfl(o, leader, 64);
            const int64_t pos = int64_t(o) + rank;
            if (ok && pos >= 0 && pos < n_edges) pairs[pos] = make_int2(key, int32_t(e));
        }
    }
}

// ---- level 2: nodes within a bucket -------------------------------------------

// One workgroup per bucket b (nodes [b*BN, min(N, (b+1)*BN))).  Its pairs are
// the contiguous run [starts[b], starts[b + 1]) in increasing edge id.
// LDS path (BN <= kNodeLdsMax): per-part histograms and running offsets in LDS,
// kParts wavefronts.  Global path: one wavefront, running offsets in `scratch`
// (the bucket's own BN entries of an N-entry workspace array).
template <bool kLds>
__global__ __launch_bounds__(kThreads) void csr_node_place_kernel(
    const int2* __restrict__ pairs, int64_t n_edges, int64_t n_nodes, int sb, int64_t n_buckets,
    const int32_t* __restrict__ starts, int32_t* __restrict__ rowptr, int32_t* __restrict__ perm,
    int32_t* __restrict__ scratch) {
    extern __shared__ int32_t lds[];   // kLds: [0, BN): node offsets; then kParts x BN
    const int64_t b = blockIdx.x;
    const int64_t bn = int64_t(1) << sb;
    const int64_t n0 = b * bn;
    const int64_t nn = n0 + bn < n_nodes ? bn : n_nodes - n0;   // nodes in this bucket
    const int32_t s0 = starts[b];                                 // the bucket's run of pairs
    const int64_t r0 = s0, r1 = starts[b + 1];
    constexpr int PW = kLds ? kParts : 1;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t part = (r1 - r0 + PW - 1) / PW;
    const int64_t p0 = r0 + wave * part < r1 ? r0 + wave * part : r1;
    const int64_t p1 = p0 + part < r1 ? p0 + part : r1;
    int32_t* node_off = kLds ? lds : scratch + n0;
    int32_t* run_all = lds + bn;

    // per-part histograms of the local node ids
    if (kLds) {
        for (int64_t i = threadIdx.x; i < (1 + PW) * bn; i += kThreads) lds[i] = 0;
    } else {
        for (int64_t i = threadIdx.x; i < nn; i += kThreads) node_off[i] = 0;
    }
    __syncthreads();
    // a part of at most kAhead2 steps keeps its pairs in registers for the
    // placement pass
    constexpr int kAhead2 = 16;
    const bool single = p1 - p0 <= 64 * kAhead2;
    int2 pr[kAhead2];
    if (wave < PW) {
        for (int64_t chunk = p0; chunk < p1; chunk += 64 * kAhead2) {
#pragma unroll
            for (int j = 0; j < kAhead2; ++j) {
                const int64_t k = chunk + j * 64 + lane;
                pr[j] = k < p1 ? pairs[k] : make_int2(-1, -1);
            }
#pragma unroll
            for (int j = 0; j < kAhead2; ++j) {
                const int64_t loc = int64_t(pr[j].x) - n0;
                if (pr[j].x >= 0 && loc >= 0 && loc < nn) {
                    if (kLds)
                        atomicAdd(&run_all[wave * bn + loc], 1);
                    else
                        atomicAdd(&node_off[loc], 1);
                }
            }
        }
    }
    __syncthreads();
    // node offsets: exclusive scan over the bucket's nodes of their totals
    if (kLds) {
        for (int64_t i = threadIdx.x; i < nn; i += kThreads) {
            int32_t s = 0;
#pragma unroll
            for (int w = 0; w < PW; ++w) s += run_all[w * bn + i];
            node_off[i] = s;
        }
        __syncthreads();
        block_exclusive_scan_lds(node_off, nn);
    } else if (threadIdx.x < 64) {
        int32_t carry = 0;
        for (int64_t base = 0; base < nn; base += 64) {
            const int64_t i = base + lane;
            const int32_t x = i < nn ? node_off[i] : 0;
            const int32_t incl = wave_inclusive_scan(x);
            if (i < nn) node_off[i] = carry + incl - x;
            carry += __shfl(incl, 63, 64);
        }
    }
    __syncthreads();
    for (int64_t i = threadIdx.x; i < nn; i += kThreads) rowptr[n0 + i] = s0 + node_off[i];
    if (b == n_buckets - 1 && threadIdx.x == 0) rowptr[n_nodes] = int32_t(r1);
    if (kLds) {
        for (int64_t i = threadIdx.x; i < nn; i += kThreads) {
            int32_t o = s0 + node_off[i];
#pragma unroll
            for (int w = 0; w < PW; ++w) {
                const int32_t c = run_all[w * bn + i];
                run_all[w * bn + i] = o;
                o += c;
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < nn; i += kThreads) node_off[i] += s0;
    }
    __syncthreads();
    if (wave >= PW) return;

    int32_t* run = kLds ? run_all + wave * bn : node_off;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    for (int64_t chunk = p0; chunk < p1; chunk += 64 * kAhead2) {
        if (!single) {
#pragma unroll
            for (int j = 0; j < kAhead2; ++j) {
                const int64_t k = chunk + j * 64 + lane;
                pr[j] = k < p1 ? pairs[k] : make_int2(-1, -1);
            }
        }
#pragma unroll
        for (int j = 0; j < kAhead2; ++j) {
            if (chunk + j * 64 >= p1) break;           // uniform
            const int64_t loc64 = int64_t(pr[j].x) - n0;
            const bool ok = pr[j].x >= 0 && loc64 >= 0 && loc64 < nn;
            const int32_t loc = ok ? int32_t(loc64) : 0;
            const uint64_t same = match_key(ok, loc, sb);
            const int rank = __popcll(same & below);
            const int cnt = __popcll(same);
            const int leader = ok ? __ffsll((unsigned long long)same) - 1 : lane;
            int32_t o = 0;
            if (kLds) wave_lds_sync();   // the previous step's leaders wrote run[] entries read here
            if (ok && rank == 0) {
                if (kLds) {
                    o = run[loc];
                    run[loc] = o + cnt;
                } else {
                    o = atomicAdd(&run[loc], cnt);   // returns the running offset
                }
            }
            o = __shfl(o, leader, 64);
            const int64_t pos = int64_t(o) + rank;
            if (ok && pos >= 0 && pos < n_edges) perm[pos] = pr[j].y;
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
    int node_bits = 0;
    while (node_bits < 62 && (int64_t(1) << node_bits) < n_nodes) ++node_bits;
    p.bucket_shift = node_bits - kBucketsMaxBits > kBucketMinBits ? node_bits - kBucketsMaxBits
                                                                   : kBucketMinBits;
    p.buckets = (n_nodes + (int64_t(1) << p.bucket_shift) - 1) >> p.bucket_shift;
    p.bucket_bits = 0;
    while ((int64_t(1) << p.bucket_bits) < p.buckets) ++p.bucket_bits;
    p.node_lds = (int64_t(1) << p.bucket_shift) <= kNodeLdsMax;
    // tiles: as many 1024-edge tiles as the count matrix budget allows
    int64_t max_tiles = kCountBudget / p.buckets;
    if (max_tiles > kTilesMax) max_tiles = kTilesMax;
    if (max_tiles < 1) max_tiles = 1;
    int64_t tile_edges = (n_edges + max_tiles - 1) / max_tiles;
    if (tile_edges < kTileEdgesMin) tile_edges = kTileEdgesMin;
    p.tile_edges = tile_edges;
    p.tiles = n_edges > 0 ? (n_edges + tile_edges - 1) / tile_edges : 1;
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.off_flag = 0;
    p.off_tile_bad = 256;
    p.off_counts = align(p.off_tile_bad + size_t(p.tiles) * sizeof(int32_t));
    p.off_tot = align(p.off_counts + size_t(p.tiles) * size_t(p.buckets) * sizeof(int32_t));
    p.off_starts = align(p.off_tot + size_t(p.buckets) * sizeof(int32_t));
    p.off_pairs = align(p.off_starts + size_t(p.buckets + 1) * sizeof(int32_t));
    p.off_scratch = align(p.off_pairs + size_t(n_edges > 0 ? n_edges : 1) * sizeof(int2));
    p.bytes = align(p.off_scratch + (p.node_lds ? size_t(0) : size_t(n_nodes) * sizeof(int32_t)));
    return p;
}

hipError_t launch_csr(const int64_t* dst, int64_t n_edges, int64_t n_nodes, int32_t* rowptr,
                      int32_t* perm, int32_t* dst32, void* workspace, const CsrPlan& plan,
                      int32_t* flag, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    if (!flag) flag = reinterpret_cast<int32_t*>(ws + plan.off_flag);
    int32_t* tile_bad = reinterpret_cast<int32_t*>(ws + plan.off_tile_bad);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + plan.off_counts);
    int32_t* tot = reinterpret_cast<int32_t*>(ws + plan.off_tot);
    int32_t* starts = reinterpret_cast<int32_t*>(ws + plan.off_starts);
    int2* pairs = reinterpret_cast<int2*>(ws + plan.off_pairs);
    int32_t* scratch = reinterpret_cast<int32_t*>(ws + plan.off_scratch);
    const int sb = plan.bucket_shift;
    const int64_t nb = plan.buckets;
    hipError_t err;
    csr_bucket_count_kernel<<<unsigned(plan.tiles), kThreads, size_t(nb) * sizeof(int32_t),
                              stream>>>(dst, n_edges, n_nodes, plan.tile_edges, sb, nb, counts,
                                        tile_bad);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (plan.tiles <= kColFewTiles)
        csr_bucket_scan_kernel<4><<<grid_for(nb, 4, int64_t(1) << 30), 4 * kColChunks, 0,
                                    stream>>>(counts, plan.tiles, nb, tot, tile_bad, flag);
    else
        csr_bucket_scan_kernel<16><<<grid_for(nb, 16, int64_t(1) << 30), 16 * kColChunks, 0,
                                     stream>>>(counts, plan.tiles, nb, tot, tile_bad, flag);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    csr_bucket_place_kernel<<<unsigned(plan.tiles), kThreads,
                              size_t(1 + kParts) * size_t(nb) * sizeof(int32_t), stream>>>(
        dst, n_edges, n_nodes, plan.tile_edges, sb, nb, plan.bucket_bits, counts, tot, pairs,
        dst32, starts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t bn = int64_t(1) << sb;
    if (plan.node_lds)
        csr_node_place_kernel<true><<<unsigned(nb), kThreads,
                                      size_t(1 + kParts) * size_t(bn) * sizeof(int32_t), stream>>>(
            pairs, n_edges, n_nodes, sb, nb, starts, rowptr, perm, scratch);
    else
        csr_node_place_kernel<false><<<unsigned(nb), kThreads, 0, stream>>>(
            pairs, n_edges, n_nodes, sb, nb, starts, rowptr, perm, scratch);
    return hipGetLastError();
}

}  // namespace zs
