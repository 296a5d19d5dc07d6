// Stable destination CSR for the GIE zonal scatter, gfx950.
//
// The fused forward walks each node's edges in the order index_add would add
// them, i.e. increasing edge id (deepmd-kit PR #6072, "fused Triton zonal
// scatter for the GIE head", section "What", last bullet).  This file builds
// that CSR with a deterministic two-level counting sort in two kernels; no
// result depends on the order in which atomics land.
//
// Nodes are grouped into NB <= 1024 buckets of BN = 2^SB consecutive nodes
// (NB <= 256 while a bucket's node tables fit in LDS), the edges into W
// chunks of consecutive edge ids.
//
//   1. chunk_sort   one 1024-thread workgroup per chunk: validates the
//                   destinations (dst32 = -1 where out of range), sorts the
//                   chunk's edges stably by bucket inside the chunk's own
//                   region of the pairs array (16 parts, one wavefront each;
//                   per-part histograms give each part its offsets; lanes with
//                   equal bucket ids are matched with ballots and ranked by
//                   lane order) and writes the offset of every bucket's run in
//                   the chunk, loff[b][c] (loff[NB][c] = the chunk's valid
//                   edges; bucket-major, so a bucket's entries are contiguous).
//   2. bucket_place one workgroup per bucket b: its edges, in increasing edge
//                   id, are the runs [loff[b][c], loff[b + 1][c]) of chunks
//                   c = 0, 1, ... in turn, and the bucket's first CSR position
//                   is sum over c of loff[b][c] (every valid edge of a lower
//                   bucket sits before b's run in its chunk).  The workgroup
//                   gathers its runs, histograms the local node ids, writes
//                   rowptr for its nodes and places perm stably the same way.
//
// Neither kernel reads more than two rows of the NB x W offset table, so
// every workgroup is a few memory round trips deep.
//
// Node order (optional output): a permutation of the nodes that the forward
// uses as the order in which it hands nodes to wavefronts (results do not
// depend on it).  Each bucket_place workgroup ranks its own bucket's nodes by
// decreasing degree (ties by node id) and writes them rank-major: slot
// r * NBf + ((b + r) mod NBf) for rank r of full bucket b (NBf full buckets),
// the partial last bucket's nodes after them in rank order.  So the first
// NBf slots hold every bucket's highest-degree node, the next NBf every
// bucket's second, and so on: heavy nodes are handed out first, and each band
// of NBf consecutive slots, which the dispatcher spreads over the compute
// units, draws from all buckets.  Frames with buckets of more than 64 nodes
// (above 16384 nodes) get the identity order.
//
// Every destination is range-checked; an out-of-range one is never used as an
// index and raises the validation flag.
#include "zs_csr.h"

namespace zs {

namespace {

#ifndef ZS_CSR_THREADS
#define ZS_CSR_THREADS 1024
#endif
#ifndef ZS_CSR_CHUNK
#define ZS_CSR_CHUNK 0   // 0: by frame size (below)
#endif
#ifndef ZS_CSR_BUCKET_BITS
#define ZS_CSR_BUCKET_BITS 8
#endif
constexpr int kThreads = ZS_CSR_THREADS;     // both kernels' LDS path
constexpr int kParts = kThreads / 64;        // wavefronts that sort a chunk / place a bucket
constexpr int kGlobalThreads = 256;          // bucket_place with node tables in global memory
constexpr int kAhead = 8;                    // 64-edge steps whose keys are held at once
// Chunk length: 4096 edges from 2^19 edges on (measured, per build: the
// 4096-node frames 26 vs 28 us, the 16384-node frame 75 vs 81 us against
// 2048), 2048 below (the 1000-node frame 18 vs 19 us); longer when the frame
// has more than kChunksMax such chunks.
constexpr int64_t kChunkEdgesSmall = ZS_CSR_CHUNK > 0 ? ZS_CSR_CHUNK : 2048;
constexpr int64_t kChunkEdgesLarge = ZS_CSR_CHUNK > 0 ? ZS_CSR_CHUNK : 4096;
constexpr int64_t kChunkLargeFrom = int64_t(1) << 19;
constexpr int64_t kChunksMax = 4096;
constexpr int kBucketBitsSmall = ZS_CSR_BUCKET_BITS;   // NB <= 2^this while BN fits the LDS tables
constexpr int kBucketBitsMax = 10;           // NB <= 1024
constexpr int kNodeLdsMax = 512;             // BN handled with LDS tables

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

// Inclusive scan over the wavefront with DPP lane moves: shifts by 1, 2, 4
// and 8 inside each 16-lane row (lanes past the row's start read 0), then
// row 0's and row 1's last lanes broadcast into the rows above them.
__device__ inline int32_t wave_inclusive_scan(int32_t v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
    return v;
}

// In-place exclusive scan of a[0..n) (LDS) by the whole workgroup of TH
// threads; returns the total.  Each thread scans a contiguous run of entries.
template <int TH>
__device__ inline int32_t block_exclusive_scan_lds(int32_t* a, int64_t n) {
    __shared__ int32_t wave_tot[TH / 64];
    const int tid = threadIdx.x;
    const int64_t per = (n + TH - 1) / TH;
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
    // every lane reads one wavefront total; their scan gives each wavefront
    // its offset (entry wave - 1) and the total (entry TH/64 - 1)
    const int32_t tots = wave_inclusive_scan(lane < TH / 64 ? wave_tot[lane] : 0);
    const int32_t total = __builtin_amdgcn_readlane(tots, TH / 64 - 1);
    int32_t off = wave > 0 ? __builtin_amdgcn_readlane(tots, wave - 1) : 0;
    off += incl - local;
    for (int64_t i = lo; i < hi; ++i) a[i] += off;
    __syncthreads();
    return total;
}

// Sum of v over the workgroup of TH threads (every thread gets it).
template <int TH>
__device__ inline int64_t block_sum(int64_t v) {
    __shared__ int64_t part[TH / 64];
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) v += __shfl_xor(v, h, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    int64_t s = 0;
    for (int w = 0; w < TH / 64; ++w) s += part[w];
    __syncthreads();
    return s;
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

// One 64-edge step of a stable placement: the lanes with ok set and equal
// key (bits wide) are ranked in lane order and take consecutive positions from
// run[key], which the step advances.  Returns the lane's position (unused when
// !ok).  run is this wavefront's own LDS table, or with kAtomic a table in
// global memory that only this wavefront updates.
template <bool kAtomic>
__device__ __attribute__((always_inline)) inline int64_t place_step(bool ok, int32_t key, int bits,
                                                                    int32_t* run) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const uint64_t same = match_key(ok, key, bits);
    const int rank = __popcll(same & below);
    const int cnt = __popcll(same);
    const int leader = ok ? __ffsll((unsigned long long)same) - 1 : lane;
    int32_t o = 0;
    if (!kAtomic) wave_lds_sync();   // the previous step's leaders wrote run[] entries read here
    if (ok && rank == 0) {
        if (kAtomic) {
            o = atomicAdd(&run[key], cnt);   // returns the running offset
        } else {
            o = run[key];
            run[key] = o + cnt;
        }
    }
    o = __shfl(o, leader, 64);
    return int64_t(o) + rank;
}

// ---- node order --------------------------------------------------------------

constexpr int kOrderBucketMax = 64;   // bucket sizes that get a ranked order (one wavefront)

// Slot of the node of rank `rank` (0 = highest degree) in bucket b: rank-major
// over the nf full buckets, rotated by the rank, and the partial bucket nf
// (if any) after all of them.
__device__ __attribute__((always_inline)) inline int64_t order_slot(int64_t b, int64_t rank,
                                                                    int64_t nf, int64_t bn) {
    return b < nf ? rank * nf + (b + rank) % nf : nf * bn + rank;
}

// ---- kernel 1: sort each chunk by bucket ------------------------------------

// LDS: per-part bucket counts, then running offsets (kParts x NB), and the
// chunk's bucket offsets (NB).  Part w of chunk c starts, for bucket b, at
//   loff[b][c] + (edges of b in parts < w of c).
__global__ __launch_bounds__(kThreads) void csr_chunk_sort_kernel(
    const int64_t* __restrict__ dst, int64_t n_edges, int64_t n_nodes, int64_t chunk_edges,
    int sb, int64_t n_buckets, int bucket_bits, int32_t* __restrict__ dst32,
    int32_t* __restrict__ loff, int32_t* __restrict__ chunk_bad, int2* __restrict__ pairs) {
    extern __shared__ int32_t lds[];
    int32_t* run_all = lds;
    int32_t* boff = lds + kParts * n_buckets;
    const int64_t c = blockIdx.x;
    const int64_t e0 = c * chunk_edges;
    const int64_t e1 = e0 + chunk_edges < n_edges ? e0 + chunk_edges : n_edges;
    const int64_t part = (e1 - e0 + kParts - 1) / kParts;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t p0 = e0 + wave * part < e1 ? e0 + wave * part : e1;
    const int64_t p1 = p0 + part < e1 ? p0 + part : e1;

    // keys of edges [at, at + 64 * kAhead) of this part (-1: none or out of range)
    int32_t keys[kAhead];
    int bad = 0;
    auto load = [&](int64_t at, bool write) {
        int64_t d[kAhead];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            const int64_t e = at + j * 64 + lane;
            d[j] = e < p1 ? dst[e] : -1;
        }
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            const int64_t e = at + j * 64 + lane;
            const bool in = e < p1;
            const bool ok = in && d[j] >= 0 && d[j] < n_nodes;
            keys[j] = ok ? int32_t(d[j]) : -1;
            if (write && in) {
                dst32[e] = keys[j];
                bad |= !ok;
            }
        }
    };
    const bool single = p1 - p0 <= 64 * kAhead;
    load(p0, true);
    for (int64_t i = tid; i < kParts * n_buckets; i += kThreads) run_all[i] = 0;
    __syncthreads();
    // per-part histograms
    for (int64_t at = p0; at < p1; at += 64 * kAhead) {
        if (at != p0) load(at, true);
#pragma unroll
        for (int j = 0; j < kAhead; ++j)
            if (keys[j] >= 0) atomicAdd(&run_all[wave * n_buckets + (keys[j] >> sb)], 1);
    }
    __syncthreads();
    for (int64_t b = tid; b < n_buckets; b += kThreads) {
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < kParts; ++w) s += run_all[w * n_buckets + b];
        boff[b] = s;
    }
    __syncthreads();
    const int32_t valid = block_exclusive_scan_lds<kThreads>(boff, n_buckets);
    const int64_t W = gridDim.x;   // chunks
    for (int64_t b = tid; b < n_buckets; b += kThreads) {
        int32_t o = boff[b];
        loff[b * W + c] = o;
#pragma unroll
        for (int w = 0; w < kParts; ++w) {
            const int32_t n = run_all[w * n_buckets + b];
            run_all[w * n_buckets + b] = o;
            o += n;
        }
    }
    if (tid == 0) loff[n_buckets * W + c] = valid;
    bad = __syncthreads_or(bad);
    if (tid == 0) chunk_bad[c] = bad;

    int32_t* run = run_all + wave * n_buckets;
    int2* out = pairs + e0;
    const int64_t len = e1 - e0;
    for (int64_t at = p0; at < p1; at += 64 * kAhead) {
        if (!single) load(at, false);
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            if (at + j * 64 >= p1) break;              // uniform
            const int64_t e = at + j * 64 + lane;
            const bool ok = keys[j] >= 0;
            const int32_t key = ok ? keys[j] : 0;
            const int64_t pos = place_step<false>(ok, key >> sb, bucket_bits, run);
            if (ok && pos >= 0 && pos < len) out[pos] = make_int2(key, int32_t(e));
        }
    }
}

// ---- kernel 2: place each bucket's edges by node ----------------------------

// The bucket's edge sequence (increasing edge id) is the concatenation over
// chunks of their runs.  runpre[c] = first sequence index of chunk c's run
// (runpre[W] = the bucket's size), runoff[c] = the run's offset in its chunk.
struct BucketRuns {
    const int32_t* runpre;
    const int32_t* runoff;
    int64_t chunks;
    int64_t chunk_edges;
    const int2* pairs;

    // Pairs at K sequence indices at once; only the first nv (uniform over
    // the wavefront) are looked up, and entries with ok[k] false get
    // (-1, -1).  Binary lifting from chunk 0 by the powers of two from top
    // (the largest one below chunks) down, the indices stepping together so
    // that the LDS reads of a step are in flight at the same time.  Finds,
    // like at(), the largest c with runpre[c] <= i (runs are < 2^31 long).
    template <int K>
    __device__ __attribute__((always_inline)) void at_k(const int64_t (&i)[K], const bool (&ok)[K],
                                                        int nv, int32_t top, int2 (&out)[K]) const {
        int32_t c[K], ii[K];
#pragma unroll
        for (int k = 0; k < K; ++k) {
            c[k] = 0;
            ii[k] = int32_t(i[k]);
        }
        const int32_t nch = int32_t(chunks);
        for (int32_t step = top; step > 0; step >>= 1) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                if (k >= nv) break;   // uniform
                const int32_t cand = c[k] + step;
                if (cand < nch && runpre[cand] <= ii[k]) c[k] = cand;
            }
        }
#pragma unroll
        for (int k = 0; k < K; ++k)
            out[k] = k < nv && ok[k]
                         ? pairs[int64_t(c[k]) * chunk_edges + runoff[c[k]] + (ii[k] - runpre[c[k]])]
                         : make_int2(-1, -1);
    }

    // pair at sequence index i (0 <= i < runpre[W])
    __device__ __attribute__((always_inline)) int2 at(int64_t i) const {
        int64_t lo = 0, hi = chunks - 1;      // largest c with runpre[c] <= i
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            if (runpre[mid] <= i) lo = mid; else hi = mid - 1;
        }
        return pairs[lo * chunk_edges + runoff[lo] + (i - runpre[lo])];
    }
};

// Collects the bucket's runs into LDS (runpre, runoff: W + 1 and W entries)
// and returns the bucket's first CSR position; runpre[W] holds its size.
template <int TH>
__device__ __attribute__((always_inline)) inline int64_t bucket_runs(
    const int32_t* __restrict__ loff, int64_t chunks, int64_t n_buckets, int64_t b,
    int32_t* runpre, int32_t* runoff) {
    int64_t before = 0;
    for (int64_t c = threadIdx.x; c < chunks; c += TH) {
        const int32_t lo = loff[b * chunks + c], hi = loff[(b + 1) * chunks + c];
        runoff[c] = lo;
        runpre[c] = hi - lo;
        before += lo;
    }
    const int64_t start = block_sum<TH>(before);   // (its barriers order the LDS writes)
    const int32_t size = block_exclusive_scan_lds<TH>(runpre, chunks);
    if (threadIdx.x == 0) runpre[chunks] = size;
    __syncthreads();
    return start;
}

// Folds the per-chunk out-of-range bits into the flag (one workgroup).
template <int TH>
__device__ __attribute__((always_inline)) inline void fold_flag(
    const int32_t* __restrict__ chunk_bad, int64_t chunks, int32_t* __restrict__ flag) {
    int bad = 0;
    for (int64_t c = threadIdx.x; c < chunks; c += TH) bad |= chunk_bad[c];
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) *flag = bad ? 1 : 0;
}

// LDS path (BN <= kNodeLdsMax).  LDS: runpre (W + 1), runoff (W), per-part
// node counts then running offsets (kParts x BN), node offsets (BN).
__global__ __launch_bounds__(kThreads) void csr_bucket_place_kernel(
    const int2* __restrict__ pairs, const int32_t* __restrict__ loff,
    const int32_t* __restrict__ chunk_bad, int64_t chunks, int64_t chunk_edges, int64_t n_edges,
    int64_t n_nodes, int sb, int64_t n_buckets, int32_t* __restrict__ flag,
    int32_t* __restrict__ rowptr, int32_t* __restrict__ perm, int32_t* __restrict__ order) {
    extern __shared__ int32_t lds[];
    const int64_t bn = int64_t(1) << sb;
    int32_t* runpre = lds;
    int32_t* runoff = lds + chunks + 1;
    int32_t* run_all = runoff + chunks;
    int32_t* noff = run_all + kParts * bn;
    const int64_t b = blockIdx.x;
    const int64_t n0 = b * bn;
    const int64_t nn = n0 + bn < n_nodes ? bn : n_nodes - n0;   // nodes in this bucket
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    if (b == 0) fold_flag<kThreads>(chunk_bad, chunks, flag);
    for (int64_t i = tid; i < kParts * bn; i += kThreads) run_all[i] = 0;
    const int64_t start = bucket_runs<kThreads>(loff, chunks, n_buckets, b, runpre, runoff);
    const BucketRuns seq{runpre, runoff, chunks, chunk_edges, pairs};
    const int64_t size = runpre[chunks];
    const int64_t part = (size + kParts - 1) / kParts;
    const int64_t p0 = wave * part < size ? wave * part : size;
    const int64_t p1 = p0 + part < size ? p0 + part : size;

    const bool single = p1 - p0 <= 64 * kAhead;
    int32_t top = 0;   // largest power of two below chunks (0 for one chunk)
    while (chunks > 1 && int64_t(top) * 2 < chunks) top = top ? top * 2 : 1;
    int2 pr[kAhead];
    auto load = [&](int64_t at) {
        int64_t idx[kAhead];
        bool ok[kAhead];
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            idx[j] = at + j * 64 + lane;
            ok[j] = idx[j] < p1;
        }
        const int64_t left = (p1 - at + 63) / 64;
        seq.at_k<kAhead>(idx, ok, int(left < kAhead ? left : kAhead), top, pr);
    };
    for (int64_t at = p0; at < p1; at += 64 * kAhead) {
        load(at);
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            const int64_t loc = int64_t(pr[j].x) - n0;
            if (pr[j].x >= 0 && loc >= 0 && loc < nn) atomicAdd(&run_all[wave * bn + loc], 1);
        }
    }
    __syncthreads();
    int32_t my_deg = 0;   // degree of node n0 + tid
    for (int64_t n = tid; n < nn; n += kThreads) {
        int32_t s = 0;
#pragma unroll
        for (int w = 0; w < kParts; ++w) s += run_all[w * bn + n];
        noff[n] = s;
        if (n == tid) my_deg = s;
    }
    if (order != nullptr) {
        if (bn <= kOrderBucketMax) {
            // wavefront 0 holds the bucket's nodes, one per lane: rank by
            // decreasing degree, ties by node id
            if (wave == 0) {
                int64_t rank = 0;
                for (int k = 0; k < int(nn); ++k) {
                    const int32_t dk = __builtin_amdgcn_readlane(my_deg, k);
                    rank += dk > my_deg || (dk == my_deg && k < lane);
                }
                if (lane < nn) order[order_slot(b, rank, n_nodes >> sb, bn)] = int32_t(n0 + lane);
            }
        } else {
            for (int64_t n = tid; n < nn; n += kThreads) order[n0 + n] = int32_t(n0 + n);
        }
    }
    __syncthreads();
    block_exclusive_scan_lds<kThreads>(noff, nn);
    for (int64_t n = tid; n < nn; n += kThreads) {
        int32_t o = int32_t(start) + noff[n];
        rowptr[n0 + n] = o;
#pragma unroll
        for (int w = 0; w < kParts; ++w) {
            const int32_t k = run_all[w * bn + n];
            run_all[w * bn + n] = o;
            o += k;
        }
    }
    if (b == n_buckets - 1 && tid == 0) rowptr[n_nodes] = int32_t(start + size);
    __syncthreads();

    int32_t* run = run_all + wave * bn;
    for (int64_t at = p0; at < p1; at += 64 * kAhead) {
        if (!single) load(at);
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            if (at + j * 64 >= p1) break;              // uniform
            const int64_t loc64 = int64_t(pr[j].x) - n0;
            const bool ok = pr[j].x >= 0 && loc64 >= 0 && loc64 < nn;
            const int64_t pos = place_step<false>(ok, ok ? int32_t(loc64) : 0, sb, run);
            if (ok && pos >= 0 && pos < n_edges) perm[pos] = pr[j].y;
        }
    }
}

// Global path (BN > kNodeLdsMax): node counts and running offsets in
// `scratch` (the bucket's own BN entries of an N-entry workspace array); all
// wavefronts count, wavefront 0 scans and places (in sequence order, so the
// placement is stable).  LDS: runpre (W + 1), runoff (W).
__global__ __launch_bounds__(kGlobalThreads) void csr_bucket_place_global_kernel(
    const int2* __restrict__ pairs, const int32_t* __restrict__ loff,
    const int32_t* __restrict__ chunk_bad, int64_t chunks, int64_t chunk_edges, int64_t n_edges,
    int64_t n_nodes, int sb, int64_t n_buckets, int32_t* __restrict__ flag,
    int32_t* __restrict__ rowptr, int32_t* __restrict__ perm, int32_t* __restrict__ scratch,
    int32_t* __restrict__ order) {
    extern __shared__ int32_t lds[];
    const int64_t bn = int64_t(1) << sb;
    int32_t* runpre = lds;
    int32_t* runoff = lds + chunks + 1;
    const int64_t b = blockIdx.x;
    const int64_t n0 = b * bn;
    const int64_t nn = n0 + bn < n_nodes ? bn : n_nodes - n0;
    int32_t* node_off = scratch + n0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    if (b == 0) fold_flag<kGlobalThreads>(chunk_bad, chunks, flag);
    for (int64_t n = tid; n < nn; n += kGlobalThreads) node_off[n] = 0;
    const int64_t start = bucket_runs<kGlobalThreads>(loff, chunks, n_buckets, b, runpre,
                                                      runoff);
    const BucketRuns seq{runpre, runoff, chunks, chunk_edges, pairs};
    const int64_t size = runpre[chunks];
    for (int64_t i = tid; i < size; i += kGlobalThreads) {
        const int2 p = seq.at(i);
        const int64_t loc = int64_t(p.x) - n0;
        if (p.x >= 0 && loc >= 0 && loc < nn) atomicAdd(&node_off[loc], 1);
    }
    __threadfence();
    __syncthreads();
    if (tid < 64) {
        int32_t carry = int32_t(start);
        for (int64_t base = 0; base < nn; base += 64) {
            const int64_t n = base + lane;
            const int32_t x = n < nn ? node_off[n] : 0;
            const int32_t incl = wave_inclusive_scan(x);
            if (n < nn) {
                node_off[n] = carry + incl - x;
                rowptr[n0 + n] = carry + incl - x;
            }
            carry += __shfl(incl, 63, 64);
        }
        if (b == n_buckets - 1 && lane == 0) rowptr[n_nodes] = int32_t(start + size);
    }
    __threadfence();
    __syncthreads();
    if (order != nullptr)   // buckets of more than kOrderBucketMax nodes: identity
        for (int64_t n = tid; n < nn; n += kGlobalThreads) order[n0 + n] = int32_t(n0 + n);
    if (tid >= 64) return;
    for (int64_t base = 0; base < size; base += 64) {
        const int64_t i = base + lane;
        const int2 p = i < size ? seq.at(i) : make_int2(-1, -1);
        const int64_t loc64 = int64_t(p.x) - n0;
        const bool ok = p.x >= 0 && loc64 >= 0 && loc64 < nn;
        const int64_t pos = place_step<true>(ok, ok ? int32_t(loc64) : 0, sb, node_off);
        if (ok && pos >= 0 && pos < n_edges) perm[pos] = p.y;
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

__global__ void iota_i32_kernel(int32_t* __restrict__ p, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += int64_t(gridDim.x) * blockDim.x)
        p[i] = int32_t(i);
}

hipError_t launch_iota_i32(int32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    iota_i32_kernel<<<grid_for(n, 256, 4096), 256, 0, stream>>>(p, n);
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
    // at most 256 buckets while a bucket's nodes fit the LDS tables, else up
    // to 1024 (then, past 2^19 nodes, node tables in global memory)
    int sb = node_bits > kBucketBitsSmall ? node_bits - kBucketBitsSmall : 0;
    if ((int64_t(1) << sb) > kNodeLdsMax)
        sb = node_bits > kBucketBitsMax ? node_bits - kBucketBitsMax : 0;
    p.bucket_shift = sb;
    p.buckets = (n_nodes + (int64_t(1) << sb) - 1) >> sb;
    p.bucket_bits = 0;
    while ((int64_t(1) << p.bucket_bits) < p.buckets) ++p.bucket_bits;
    p.node_lds = (int64_t(1) << sb) <= kNodeLdsMax;
    int64_t chunk = (n_edges + kChunksMax - 1) / kChunksMax;
    const int64_t chunk_min = n_edges >= kChunkLargeFrom ? kChunkEdgesLarge : kChunkEdgesSmall;
    if (chunk < chunk_min) chunk = chunk_min;
    p.chunk_edges = chunk;
    p.chunks = n_edges > 0 ? (n_edges + chunk - 1) / chunk : 1;
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    p.off_flag = 0;
    p.off_chunk_bad = 256;
    p.off_loff = align(p.off_chunk_bad + size_t(p.chunks) * sizeof(int32_t));
    p.off_pairs =
        align(p.off_loff + size_t(p.chunks) * size_t(p.buckets + 1) * sizeof(int32_t));
    p.off_scratch = align(p.off_pairs + size_t(n_edges > 0 ? n_edges : 1) * sizeof(int2));
    p.bytes = align(p.off_scratch + (p.node_lds ? size_t(0) : size_t(n_nodes) * sizeof(int32_t)));
    return p;
}

hipError_t launch_csr(const int64_t* dst, int64_t n_edges, int64_t n_nodes, int32_t* rowptr,
                      int32_t* perm, int32_t* dst32, int32_t* order, void* workspace,
                      const CsrPlan& plan, int32_t* flag, hipStream_t stream) {
    char* ws = static_cast<char*>(workspace);
    if (!flag) flag = reinterpret_cast<int32_t*>(ws + plan.off_flag);
    int32_t* chunk_bad = reinterpret_cast<int32_t*>(ws + plan.off_chunk_bad);
    int32_t* loff = reinterpret_cast<int32_t*>(ws + plan.off_loff);
    int2* pairs = reinterpret_cast<int2*>(ws + plan.off_pairs);
    int32_t* scratch = reinterpret_cast<int32_t*>(ws + plan.off_scratch);
    const int sb = plan.bucket_shift;
    const int64_t nb = plan.buckets;
    const int64_t W = plan.chunks;
    hipError_t err;
    csr_chunk_sort_kernel<<<unsigned(W), kThreads,
                            size_t(kParts + 1) * size_t(nb) * sizeof(int32_t), stream>>>(
        dst, n_edges, n_nodes, plan.chunk_edges, sb, nb, plan.bucket_bits, dst32, loff, chunk_bad,
        pairs);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t runs_lds = size_t(2 * W + 1) * sizeof(int32_t);
    const int64_t bn = int64_t(1) << sb;
    if (plan.node_lds) {
        csr_bucket_place_kernel<<<unsigned(nb), kThreads,
                                  runs_lds + size_t(kParts + 1) * size_t(bn) * sizeof(int32_t),
                                  stream>>>(pairs, loff, chunk_bad, W, plan.chunk_edges, n_edges,
                                            n_nodes, sb, nb, flag, rowptr, perm, order);
    } else {
        csr_bucket_place_global_kernel<<<unsigned(nb), kGlobalThreads, runs_lds, stream>>>(
            pairs, loff, chunk_bad, W, plan.chunk_edges, n_edges, n_nodes, sb, nb, flag, rowptr,
            perm, scratch, order);
    }
    return hipGetLastError();
}

}  // namespace zs
