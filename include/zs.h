/*
 * zs.h -- C ABI of the GIE zonal-scatter library for AMD Instinct MI355X
 * (gfx950): the forward and backward of the geometric initial embedding's
 * zonal scatter of the SeZM/DPA4 descriptor, plus the stable destination CSR
 * both passes walk.
 *
 * Source of the operation: deepmd-kit PR #6072 ("fused Triton zonal scatter
 * for the GIE head"), sections "What" and "Boundary and layout contract".
 * With lmax = 3 the padded node layout has (lmax+1)^2 = 16 rows; row
 * r = l*l + l + m (m = -l..l) belongs to degree l, giving row groups of 3/5/7
 * rows for l = 1/2/3, and row 0 (l = 0) is the scalar row, always zero.
 *
 *   message[e][r][c] = coupling[e][r-1] * radial[e][l(r)-1][c]
 *   out[n][r][c]     = sum over edges e with dst[e] == n of message[e][r][c]
 *
 * The fused operator never materialises the (E, 15, C) message surface.
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or retains them, and keeps no global state apart
 *    from zs_build_csr_noalloc's fixed per-device scratch (below).
 *  - Kernels run on the calling thread's current HIP device; every buffer and
 *    the stream must belong to that device.
 *  - Arrays are dense, row-major and contiguous; fp32 arrays must be 4-byte
 *    aligned (16-byte alignment and C % 4 == 0 select the vector kernels).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream), except the CSR builds without a bad_flag, which synchronize
 *    `stream` once at the end to read back their index-validation flag.
 *  - Inputs are never written.  Outputs must not overlap inputs or each other.
 *  - Sizes: 0 <= n_edges <= ZS_MAX_EDGES, 1 <= n_nodes <= ZS_MAX_NODES,
 *    1 <= channels <= ZS_MAX_CHANNELS.  n_edges == 0 is valid.
 *  - Errors are negative return codes (zs_status); nothing is written when an
 *    argument check fails.  Argument checks run on the host before any HIP
 *    call, so a failing check touches no device state.
 */
#ifndef ZS_H_
#define ZS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZS_LMAX 3
#define ZS_ROWS 16          /* (ZS_LMAX + 1)^2 padded rows per node          */
#define ZS_ZONAL 15         /* rows 1..15, one coupling column each           */
#define ZS_SLOTS 3          /* radial slots, one per degree l = 1..ZS_LMAX    */
#define ZS_MAX_CHANNELS 1024
#define ZS_MAX_EDGES 2147483647LL  /* perm and rowptr hold int32 positions     */
#define ZS_MAX_NODES 2147483646LL

typedef enum zs_status {
    ZS_OK = 0,
    ZS_ERR_NULL = -1,        /* a required pointer is NULL                      */
    ZS_ERR_SHAPE = -2,       /* a size is outside the ranges above              */
    ZS_ERR_INDEX = -3,       /* a destination index is outside [0, n_nodes)     */
    ZS_ERR_UNSUPPORTED = -4, /* an fp32/int32 pointer is not 4-byte aligned     */
    ZS_ERR_ALIAS = -5,       /* an output overlaps an input or another output   */
    ZS_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required         */
    ZS_ERR_HIP = -7,         /* a HIP runtime call (launch, copy, sync) failed  */
    ZS_ERR_SCRATCH = -8      /* the sizes need more scratch than the library's
                                fixed device buffer holds (zs_build_csr_noalloc) */
} zs_status;

/* Static, human-readable text for a status code; never NULL. */
const char *zs_status_string(int status);

/* Workspace bytes zs_build_csr needs for these sizes (0 if the sizes are out
 * of range).  The workspace is scratch only; its contents need not be
 * preserved between calls. */
size_t zs_csr_workspace_bytes(int64_t n_edges, int64_t n_nodes);

/*
 * zs_build_csr -- stable destination CSR (same page, "What", last bullet: the
 * fused forward walks the stable-sort CSR, whose per-node order is the edge
 * order index_add uses).
 *
 *   dst      [n_edges]     int64  destination node of each edge (input)
 *   rowptr   [n_nodes + 1] int32  rowptr[n] = #edges with dst < n (output)
 *   perm     [n_edges]     int32  perm[k] = edge at sorted position k, edges of
 *                                 equal dst in increasing edge id (output)
 *   dst32    [n_edges]     int32  int32 copy of dst, -1 where out of range (output;
 *                                 zs_backward_normalized reads it)
 *   order    [n_nodes]     int32  node schedule for the forward (output; may be
 *                                 NULL): a permutation of the nodes.  The nodes are
 *                                 split into buckets of B consecutive nodes, B the
 *                                 smallest power of two >= n_nodes / 256 (B = 1
 *                                 below 257 nodes), and ranked inside each bucket
 *                                 by decreasing degree (equal degrees: increasing
 *                                 id).  With F = floor(n_nodes / B) full buckets,
 *                                 rank r of full bucket b is at order[r*F + (b + r)
 *                                 mod F], rank r of the partial last bucket at
 *                                 order[F*B + r].  Frames with B > 64 (more than
 *                                 16384 nodes) get order[i] = i.  A scheduling aid
 *                                 only: the forward's results do not depend on it.
 *   workspace, workspace_bytes >= zs_csr_workspace_bytes(n_edges, n_nodes),
 *                                 256-byte aligned device scratch
 *   bad_flag                      NULL: synchronous index check -- the call
 *                                 synchronizes `stream` and returns ZS_ERR_INDEX
 *                                 when any dst is outside [0, n_nodes).
 *                                 Non-NULL (device int32): asynchronous -- the call
 *                                 returns after enqueueing; when the stream
 *                                 reaches the end of the build, *bad_flag is 0 if
 *                                 every dst was in range and nonzero otherwise.
 *
 * Out-of-range destinations are never used as indices: the outputs are then
 * unspecified, but no memory outside them, the workspace and bad_flag is
 * written.
 */
int zs_build_csr(const int64_t *dst, int64_t n_edges, int64_t n_nodes,
                 int32_t *rowptr, int32_t *perm, int32_t *dst32, int32_t *order,
                 void *workspace, size_t workspace_bytes, int32_t *bad_flag,
                 void *stream);

/*
 * zs_build_csr_noalloc -- zs_build_csr for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the build's scratch is a fixed buffer of
 * ZS_NOALLOC_SCRATCH_BYTES inside the library, one per device, held from the
 * first call on that device until the process ends.  The call allocates and
 * frees nothing; the caller still passes the inputs and outputs.
 *
 *   dst, n_edges, n_nodes, rowptr, perm, dst32, order, bad_flag, stream
 *       as in zs_build_csr (same kernels, bitwise the same outputs).  The
 *       buffers and the stream must belong to the calling thread's current
 *       device.
 *
 * Returns ZS_ERR_SCRATCH, before any device work, when
 * zs_csr_workspace_bytes(n_edges, n_nodes) > ZS_NOALLOC_SCRATCH_BYTES (about
 * 4 million edges fit at 1000 to 16384 nodes; the 2.6 million-edge,
 * 16384-node frame needs 20.5 MiB).  Nothing in the buffer has to start at zero: every
 * entry a build reads was written earlier in the same build.  All calls on
 * one device share its buffer, so calls whose work overlaps on that device
 * (other streams, other threads) race: serialize them.
 */
#define ZS_NOALLOC_SCRATCH_BYTES (32u << 20)

int zs_build_csr_noalloc(const int64_t *dst, int64_t n_edges, int64_t n_nodes,
                         int32_t *rowptr, int32_t *perm, int32_t *dst32,
                         int32_t *order, int32_t *bad_flag, void *stream);

/*
 * zs_forward -- fused zonal scatter forward (same page, "What", Forward
 * bullet): one wavefront per node walks the node's CSR range in order and
 * accumulates in registers.
 *
 *   coupling [n_edges][15]             fp32  zonal coupling (input)
 *   radial   [n_edges][3][channels]    fp32  radial features, slot l-1 (input)
 *   rowptr, perm                       from zs_build_csr for the same dst
 *   order    [n_nodes]                 int32 node schedule from the same
 *                                            zs_build_csr call, or NULL (nodes in
 *                                            index order).  It decides only which
 *                                            wavefront sums which node and when
 *                                            (every bucket's highest-degree nodes
 *                                            first, spread over the compute units):
 *                                            any permutation of 0..n_nodes-1 gives
 *                                            bitwise the same out.
 *   out      [n_nodes][16][channels]   fp32  fully overwritten (output)
 *
 * out[n][0][:] = +0; out[n][r][c] adds fp32(coupling*radial) products over the
 * node's edges in increasing edge id, starting from +0, with separate fp32
 * multiply and add (no fused multiply-add): bitwise the fp32 result of the
 * materialised message followed by index_add.  Run-to-run deterministic.
 * A CSR that zs_build_csr did not produce gives unspecified values but no
 * out-of-bounds access (positions and edge ids are range-checked); an order
 * entry outside [0, n_nodes) is skipped, so the nodes such an order leaves
 * out keep their previous out rows.
 */
int zs_forward(const float *coupling, const float *radial,
               const int32_t *rowptr, const int32_t *perm, const int32_t *order,
               int64_t n_nodes, int64_t n_edges, int64_t channels, float *out,
               void *stream);

/*
 * zs_backward -- fused zonal scatter backward (same page, "What", Backward
 * bullet): both operand gradients in a single edge-parallel pass, with no
 * materialised message gradient.  Edges are visited grouped by destination
 * (CSR order) so each node's upstream gradient rows are read once.
 *
 *   grad_out      [n_nodes][16][channels]  fp32  upstream gradient (row 0 unused)
 *   coupling, radial                       as in zs_forward
 *   dst32, rowptr, perm                    from zs_build_csr for the same dst; dst32
 *                                          is checked (non-NULL, 4-byte aligned, not
 *                                          overlapping the outputs) but the current
 *                                          CSR-ordered kernels do not read it: it is
 *                                          part of the signature so that an
 *                                          edge-ordered traversal needs no ABI change
 *   grad_coupling [n_edges][15]            fp32  fully overwritten (output)
 *   grad_radial   [n_edges][3][channels]   fp32  fully overwritten (output)
 *
 * grad_radial[e][l-1][c] = sum over the rows r of degree l, in increasing r,
 *   of fp32(grad_out[dst[e]][r][c] * coupling[e][r-1]), fp32 adds from +0.
 * grad_coupling[e][r-1] = sum over c of grad_out[dst[e]][r][c] *
 *   radial[e][l(r)-1][c], with exact products accumulated in fp64 and rounded
 *   to fp32 once (equal to the correctly rounded sum except in rare near-ties,
 *   where it may differ by one fp32 ulp).  Run-to-run deterministic.
 */
int zs_backward(const float *grad_out, const float *coupling,
                const float *radial, const int32_t *dst32,
                const int32_t *rowptr, const int32_t *perm, int64_t n_nodes,
                int64_t n_edges, int64_t channels, float *grad_coupling,
                float *grad_radial, void *stream);

/*
 * zs_forward_strided / zs_backward_strided -- the same operations on strided
 * views of the two edge inputs, so callers need not copy them to contiguous
 * buffers first.  The GIE page's test suite feeds the operator sliced views of
 * the radial features (section "Tests"), and the band page (deepmd-kit PR
 * #6071, "banded Wigner-D storage for the fused inference consumers",
 * Summary) stores each edge's rotation as a packed (E, 3D-2) band whose
 * m = 0 segment is the zonal coupling, i.e. a coupling view with an edge
 * stride of 46 floats.
 *
 *   coupling[e][j]   is read at coupling[e * coupling_edge_stride + j]
 *   radial[e][s][c]  is read at radial[e * radial_edge_stride +
 *                                      s * radial_slot_stride + c]
 *
 * Strides are in floats and must be >= 0, with each view spanning at most
 * 2^60 floats ((n_edges - 1) * edge stride plus its last row), else
 * ZS_ERR_SHAPE; inputs are only read, so overlapping or broadcast (stride 0)
 * rows are allowed.  Outputs
 * are contiguous as in zs_forward/zs_backward, must not overlap the strided
 * inputs' extents, and results are identical to those calls on contiguous
 * copies of the views.
 * Radial strides that are multiples of 4 (with a 16-byte aligned base) keep
 * the vector kernels.
 */
int zs_forward_strided(const float *coupling, int64_t coupling_edge_stride,
                       const float *radial, int64_t radial_edge_stride,
                       int64_t radial_slot_stride, const int32_t *rowptr,
                       const int32_t *perm, const int32_t *order, int64_t n_nodes,
                       int64_t n_edges, int64_t channels, float *out,
                       void *stream);

int zs_backward_strided(const float *grad_out, const float *coupling,
                        int64_t coupling_edge_stride, const float *radial,
                        int64_t radial_edge_stride, int64_t radial_slot_stride,
                        const int32_t *dst32, const int32_t *rowptr,
                        const int32_t *perm, int64_t n_nodes, int64_t n_edges,
                        int64_t channels, float *grad_coupling,
                        float *grad_radial, void *stream);

/*
 * zs_forward_normalized -- the scatter followed by the inverse-square-root
 * degree normalisation the GIE page keeps after it ("What", third bullet; last
 * step of the sequence diagram), fused into the same node-parallel pass.  The
 * degree is the sum of the edges' cutoff-envelope factors.
 *
 *   coupling, radial, rowptr, perm, order, n_nodes, n_edges, channels
 *                                    as in zs_forward
 *   env   [n_edges]                  fp32  cutoff-envelope factor per edge (input)
 *   y     [n_nodes][16][channels]    fp32  normalised output (output)
 *   out   [n_nodes][16][channels]    fp32  unnormalised scatter, bitwise the
 *                                          zs_forward result (output; may be
 *                                          NULL when not needed)
 *   norm  [n_nodes]                  fp32  per-node factor (output)
 *
 * deg[n] = fp32 sum of env over the node's edges in increasing edge id, from +0;
 * norm[n] = 1 / sqrt(deg[n]) (correctly rounded fp32 square root, then fp32
 * division), or 0 when deg[n] <= 0 (no edges, or NaN);
 * y[n][r][c] = out[n][r][c] * norm[n] (fp32).  Inputs must be contiguous; the
 * outputs must not overlap each other or any input.  Run-to-run deterministic.
 */
int zs_forward_normalized(const float *coupling, const float *radial,
                          const float *env, const int32_t *rowptr,
                          const int32_t *perm, const int32_t *order,
                          int64_t n_nodes, int64_t n_edges, int64_t channels,
                          float *y, float *out, float *norm, void *stream);

/*
 * zs_backward_normalized -- gradients through the normalised scatter (same
 * page and passage: the normalisation keeps its own cotangent because the
 * degree depends on geometry through the envelope).
 *
 *   grad_y  [n_nodes][16][channels]  fp32  upstream gradient of y (row 0 unused)
 *   out, norm                              from zs_forward_normalized (inputs)
 *   coupling, radial, dst32, rowptr, perm  as in zs_backward
 *   grad_coupling, grad_radial             as in zs_backward, computed with
 *                                          grad_out[n][r][c] = fp32(grad_y *
 *                                          norm[n]) (outputs)
 *   grad_env [n_edges]  fp32  gradient of env (output)
 *   grad_deg [n_nodes]  fp32  gradient of deg (output; also the per-node table
 *                             grad_env is gathered from)
 *
 * grad_deg[n] = -1/2 * t * t * t * s, t = norm[n], evaluated in fp64 from the
 * left, s = sum over rows 1..15 and channels of grad_y * out (exact products,
 * fp64 sum), rounded to fp32 once; 0 when norm[n] == 0.
 * grad_env[e] = grad_deg[dst32[e]] (0 where dst32[e] < 0).  When n_edges == 0
 * only grad_deg is written and the edge pointers may be NULL.  Inputs must be
 * contiguous; outputs must not overlap each other or any input.
 */
int zs_backward_normalized(const float *grad_y, const float *out,
                           const float *norm, const float *coupling,
                           const float *radial, const int32_t *dst32,
                           const int32_t *rowptr, const int32_t *perm,
                           int64_t n_nodes, int64_t n_edges, int64_t channels,
                           float *grad_coupling, float *grad_radial,
                           float *grad_env, float *grad_deg, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ZS_H_ */
