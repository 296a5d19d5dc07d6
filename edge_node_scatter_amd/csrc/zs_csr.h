// Internal declarations of the CSR build (zs_csr.hip), used by the C ABI.
// Not part of the public ABI (that is include/zs.h).
#pragma once

#include "zs_internal.h"

namespace zs {

// ---- CSR build ------------------------------------------------------------
struct CsrPlan {
    int64_t chunks;       // W: edge chunks sorted by the first kernel
    int64_t chunk_edges;  // edges per chunk (the last may be shorter)
    int bucket_shift;     // SB: a bucket holds 2^SB consecutive nodes
    int bucket_bits;      // ceil(log2(buckets))
    int64_t buckets;      // NB
    bool node_lds;        // per-bucket node tables fit in LDS
    size_t off_flag;      // int32 error flag
    size_t off_chunk_bad; // int32 [W] per-chunk out-of-range indicator
    size_t off_loff;      // int32 [NB + 1][W] offset of each bucket's run in each chunk
    size_t off_pairs;     // int2 [n_edges] (destination, edge), chunk-major, bucket runs
    size_t off_scratch;   // int32 [n_nodes] node offsets (only without node_lds)
    size_t bytes;         // total workspace bytes
};
CsrPlan plan_csr(int64_t n_edges, int64_t n_nodes);
// flag: device int32 that receives the out-of-range indicator; NULL selects
// the one inside the workspace (at plan.off_flag).  order: NULL, or n_nodes
// int32 that receive the node order (the forward's schedule).
hipError_t launch_csr(const int64_t* dst, int64_t n_edges, int64_t n_nodes, int32_t* rowptr,
                      int32_t* perm, int32_t* dst32, int32_t* order, void* workspace,
                      const CsrPlan& plan, int32_t* flag, hipStream_t stream);
// order[i] = i for i < n (the node order of a frame without edges).
hipError_t launch_iota_i32(int32_t* p, int64_t n, hipStream_t stream);

}  // namespace zs
