/*
 * Oracle for the GIE zonal scatter (lmax = 3) -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path (the HIP library) never calls it and
 * shares no code, header or table with it.
 *
 * Plain, single-threaded, sequential C.  Built with -O2 -ffp-contract=off and
 * no fast-math, so every float operation below is one IEEE-754 operation
 * rounded to nearest-even, in exactly the order the loops state.
 *
 * What is computed (deepmd-kit PR #6072, "fused Triton zonal scatter for the
 * GIE head", section "What" and section "Boundary and layout contract"):
 *
 *   The padded node layout has (lmax+1)^2 = 16 rows.  Row r of degree l and
 *   order m is r = l*l + l + m, m = -l..l, so degree l owns the contiguous
 *   block of 2l+1 rows starting at l*l (sizes 3/5/7 for l = 1/2/3).  Row 0
 *   (l = 0, the scalar row) receives nothing and is identically +0.
 *
 *   coupling (E, 15): column r-1 is the zonal coupling of edge e for row r.
 *   radial   (E, 3, C): slot l-1 holds the radial features of degree l.
 *   The per-edge message is message[e][r][c] = coupling[e][r-1] *
 *   radial[e][l(r)-1][c]; the reference composition materialises it and then
 *   index-adds it onto dst[e].  index_add applies edges in increasing edge
 *   order, which is also the order of the stable destination-sorted CSR the
 *   fused kernel walks (same page, "What", last bullet).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the message is a materialised fp32 tensor, so each product is rounded to
 *     fp32 before it is added (no fused multiply-add);
 *   - accumulators start at +0.0f and every edge is added, in edge order;
 *   - grad_radial[e][l-1][c] adds the products g[n][r][c]*coupling[e][r-1]
 *     over the rows of degree l in increasing r, fp32 multiply then add, from
 *     +0.0f;
 *   - grad_coupling[e][r-1] = sum over c of g[n][r][c]*radial[e][l-1][c]: each
 *     fp32 x fp32 product is exact in fp64, the sum is accumulated in fp64 in
 *     increasing c and rounded to fp32 once;
 *   - upstream gradient row 0 has no effect (row 0 does not depend on inputs);
 *   - a destination outside [0, N) is an error (index_add raises).
 *
 * Flat layouts (row-major, contiguous):
 *   coupling[e*15 + (r-1)], radial[(e*3 + (l-1))*C + c], out[(n*16 + r)*C + c].
 * The radial offset is the one pinned by the GIE page's review thread on
 * masking the backward's padded channel loads: a (777, 3, 40) radial tensor
 * holds 93,240 floats and the last edge's degree-3 row starts at float 93,200.
 *
 * Return values: 0 on success, -3 when a destination index is out of range.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ZS_ORACLE_ROWS 16
#define ZS_ORACLE_ZONAL 15
#define ZS_ORACLE_LMAX 3

static int check_dst(const int64_t *dst, int64_t E, int64_t N)
{
    for (int64_t e = 0; e < E; ++e)
        if (dst[e] < 0 || dst[e] >= N)
            return -3;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Forward, fp32, original edge order (the pages' reference composition).    */
/* ------------------------------------------------------------------------- */
int zs_oracle_forward_f32(const float *coupling, const float *radial,
                          const int64_t *dst, int64_t E, int64_t N, int64_t C,
                          float *out)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t i = 0; i < N * ZS_ORACLE_ROWS * C; ++i)
        out[i] = 0.0f;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t n = dst[e];
        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {
            const float *rad = radial + (e * 3 + (l - 1)) * C;
            for (int m = -l; m <= l; ++m) {
                const int r = l * l + l + m;
                const float w = coupling[e * ZS_ORACLE_ZONAL + (r - 1)];
                float *o = out + (n * ZS_ORACLE_ROWS + r) * C;
                for (int64_t c = 0; c < C; ++c) {
                    const float msg = w * rad[c];
                    o[c] = o[c] + msg;
                }
            }
        }
    }
    return 0;
}

/* Forward for a sample of nodes only: rows[i] receives out[nodes[i]] (16*C
 * floats).  Same arithmetic and order as zs_oracle_forward_f32, restricted to
 * the sampled destinations, for workloads too large to compute in full. */
int zs_oracle_forward_nodes_f32(const float *coupling, const float *radial,
                                const int64_t *dst, int64_t E, int64_t N,
                                int64_t C, const int64_t *nodes,
                                int64_t n_sample, float *rows)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t i = 0; i < n_sample; ++i) {
        const int64_t n = nodes[i];
        float *o_node = rows + i * ZS_ORACLE_ROWS * C;
        for (int64_t j = 0; j < ZS_ORACLE_ROWS * C; ++j)
            o_node[j] = 0.0f;
        if (n < 0 || n >= N)
            return -3;
        for (int64_t e = 0; e < E; ++e) {
            if (dst[e] != n)
                continue;
            for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {
                const float *rad = radial + (e * 3 + (l - 1)) * C;
                for (int m = -l; m <= l; ++m) {
                    const int r = l * l + l + m;
                    const float w = coupling[e * ZS_ORACLE_ZONAL + (r - 1)];
                    float *o = o_node + r * C;
                    for (int64_t c = 0; c < C; ++c) {
                        const float msg = w * rad[c];
                        o[c] = o[c] + msg;
                    }
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Backward, fp32 outputs.                                                   */
/* ------------------------------------------------------------------------- */
static void backward_one_edge_f32(const float *grad_out, const float *coupling,
                                  const float *radial, int64_t e, int64_t n,
                                  int64_t C, float *gc_row, float *gr_row)
{
    for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {
        const float *rad = radial + (e * 3 + (l - 1)) * C;
        /* grad_radial: rows of degree l in increasing r, fp32 mul then add. */
        for (int64_t c = 0; c < C; ++c) {
            float acc = 0.0f;
            for (int m = -l; m <= l; ++m) {
                const int r = l * l + l + m;
                const float p = grad_out[(n * ZS_ORACLE_ROWS + r) * C + c] *
                                coupling[e * ZS_ORACLE_ZONAL + (r - 1)];
                acc = acc + p;
            }
            gr_row[(l - 1) * C + c] = acc;
        }
        /* grad_coupling: exact products, fp64 sum in increasing c, one rounding. */
        for (int m = -l; m <= l; ++m) {
            const int r = l * l + l + m;
            const float *g = grad_out + (n * ZS_ORACLE_ROWS + r) * C;
            double s = 0.0;
            for (int64_t c = 0; c < C; ++c)
                s = s + (double)g[c] * (double)rad[c];
            gc_row[r - 1] = (float)s;
        }
    }
}

int zs_oracle_backward_f32(const float *grad_out, const float *coupling,
                           const float *radial, const int64_t *dst, int64_t E,
                           int64_t N, int64_t C, float *grad_coupling,
                           float *grad_radial)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t e = 0; e < E; ++e)
        backward_one_edge_f32(grad_out, coupling, radial, e, dst[e], C,
                              grad_coupling + e * ZS_ORACLE_ZONAL,
                              grad_radial + e * 3 * C);
    return 0;
}

/* Backward for a sample of edges: gc[i] / gr[i] receive the gradients of
 * edge edges[i] (15 and 3*C floats).  Each edge's gradients depend only on
 * that edge, so this is the full computation restricted to the sample. */
int zs_oracle_backward_edges_f32(const float *grad_out, const float *coupling,
                                 const float *radial, const int64_t *dst,
                                 int64_t E, int64_t N, int64_t C,
                                 const int64_t *edges, int64_t n_sample,
                                 float *gc, float *gr)
{
    for (int64_t i = 0; i < n_sample; ++i) {
        const int64_t e = edges[i];
        if (e < 0 || e >= E || dst[e] < 0 || dst[e] >= N)
            return -3;
        backward_one_edge_f32(grad_out, coupling, radial, e, dst[e], C,
                              gc + i * ZS_ORACLE_ZONAL, gr + i * 3 * C);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* fp64 versions: the same definitions evaluated in double from fp32 inputs.  */
/* Used by the tests to pin the fp32 oracle against error bounds.            */
/* ------------------------------------------------------------------------- */
int zs_oracle_forward_f64(const float *coupling, const float *radial,
                          const int64_t *dst, int64_t E, int64_t N, int64_t C,
                          double *out)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t i = 0; i < N * ZS_ORACLE_ROWS * C; ++i)
        out[i] = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t n = dst[e];
        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {
            const float *rad = radial + (e * 3 + (l - 1)) * C;
            for (int m = -l; m <= l; ++m) {
                const int r = l * l + l + m;
                const double w = coupling[e * ZS_ORACLE_ZONAL + (r - 1)];
                double *o = out + (n * ZS_ORACLE_ROWS + r) * C;
                for (int64_t c = 0; c < C; ++c)
                    o[c] = o[c] + w * (double)rad[c];
            }
        }
    }
    return 0;
}

int zs_oracle_backward_f64(const float *grad_out, const float *coupling,
                           const float *radial, const int64_t *dst, int64_t E,
                           int64_t N, int64_t C, double *grad_coupling,
                           double *grad_radial)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t n = dst[e];
        for (int l = 1; l <= ZS_ORACLE_LMAX; ++l) {
            const float *rad = radial + (e * 3 + (l - 1)) * C;
            for (int64_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int m = -l; m <= l; ++m) {
                    const int r = l * l + l + m;
                    acc = acc + (double)grad_out[(n * ZS_ORACLE_ROWS + r) * C + c] *
                                (double)coupling[e * ZS_ORACLE_ZONAL + (r - 1)];
                }
                grad_radial[(e * 3 + (l - 1)) * C + c] = acc;
            }
            for (int m = -l; m <= l; ++m) {
                const int r = l * l + l + m;
                const float *g = grad_out + (n * ZS_ORACLE_ROWS + r) * C;
                double s = 0.0;
                for (int64_t c = 0; c < C; ++c)
                    s = s + (double)g[c] * (double)rad[c];
                grad_coupling[e * ZS_ORACLE_ZONAL + (r - 1)] = s;
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Stable destination CSR (same page, "What", last bullet): counting sort of  */
/* edges by dst that keeps equal keys in increasing edge order.              */
/*   rowptr[n] = number of edges with dst < n  (N+1 entries)                 */
/*   perm[k]   = the edge at sorted position k                               */
/* ------------------------------------------------------------------------- */
int zs_oracle_csr(const int64_t *dst, int64_t E, int64_t N, int32_t *rowptr,
                  int32_t *perm, int32_t *cursor /* N ints of scratch */)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t n = 0; n <= N; ++n)
        rowptr[n] = 0;
    for (int64_t e = 0; e < E; ++e)
        rowptr[dst[e] + 1] += 1;            /* degree of dst[e], shifted by one */
    for (int64_t n = 0; n < N; ++n)
        rowptr[n + 1] += rowptr[n];          /* inclusive scan => exclusive starts */
    for (int64_t n = 0; n < N; ++n)
        cursor[n] = rowptr[n];
    for (int64_t e = 0; e < E; ++e)          /* increasing e keeps ties stable */
        perm[cursor[dst[e]]++] = (int32_t)e;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Degree normalisation applied after the scatter.                           */
/*                                                                           */
/* The GIE page keeps an inverse-square-root degree normalisation right      */
/* after the scatter, with its own cotangent because the degree depends on   */
/* the cutoff envelope, i.e. on geometry ("What", third bullet; last step of */
/* the sequence diagram).  Reading used here:                                */
/*   deg[n]  = sum of env[e] over the edges of n (fp32, edge order, from +0) */
/*   norm[n] = 1 / sqrt(deg[n])  (fp32 sqrt, then fp32 division),            */
/*             0 when deg[n] <= 0                                            */
/*   y[n][r][c] = out[n][r][c] * norm[n]  (fp32)                             */
/* Backward, gy being the upstream gradient of y:                            */
/*   g_out[n][r][c] = gy[n][r][c] * norm[n]  (fp32), then the scatter        */
/*                    backward above with g_out as upstream gradient         */
/*   ddeg[n] = -1/2 * t*t*t * s, t = norm[n] (fp64, left to right), where    */
/*             s = sum over r = 1..15, c of gy[n][r][c] * out[n][r][c]       */
/*             (exact products, fp64 sum over r then c); rounded to fp32     */
/*             once; 0 when norm[n] == 0                                     */
/*   grad_env[e] = ddeg[dst[e]]                                              */
/* ------------------------------------------------------------------------- */
int zs_oracle_forward_norm_f32(const float *coupling, const float *radial,
                               const float *env, const int64_t *dst, int64_t E,
                               int64_t N, int64_t C, float *y, float *out,
                               float *norm)
{
    const int rc = zs_oracle_forward_f32(coupling, radial, dst, E, N, C, out);
    if (rc)
        return rc;
    for (int64_t n = 0; n < N; ++n)
        norm[n] = 0.0f;                      /* used as the degree accumulator */
    for (int64_t e = 0; e < E; ++e)
        norm[dst[e]] = norm[dst[e]] + env[e];
    for (int64_t n = 0; n < N; ++n) {
        const float deg = norm[n];
        if (deg > 0.0f) {
            const float root = sqrtf(deg);
            norm[n] = 1.0f / root;
        } else {
            norm[n] = 0.0f;
        }
    }
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < ZS_ORACLE_ROWS * C; ++i)
            y[n * ZS_ORACLE_ROWS * C + i] = out[n * ZS_ORACLE_ROWS * C + i] * norm[n];
    return 0;
}

int zs_oracle_backward_norm_f32(const float *grad_y, const float *out,
                                const float *norm, const float *coupling,
                                const float *radial, const int64_t *dst,
                                int64_t E, int64_t N, int64_t C,
                                float *grad_coupling, float *grad_radial,
                                float *grad_env, float *grad_out_scratch)
{
    if (check_dst(dst, E, N))
        return -3;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < ZS_ORACLE_ROWS * C; ++i)
            grad_out_scratch[n * ZS_ORACLE_ROWS * C + i] =
                grad_y[n * ZS_ORACLE_ROWS * C + i] * norm[n];
    const int rc = zs_oracle_backward_f32(grad_out_scratch, coupling, radial, dst,
                                          E, N, C, grad_coupling, grad_radial);
    if (rc)
        return rc;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t n = dst[e];
        double s = 0.0;
        for (int r = 1; r < ZS_ORACLE_ROWS; ++r)
            for (int64_t c = 0; c < C; ++c) {
                const int64_t i = (n * ZS_ORACLE_ROWS + r) * C + c;
                s = s + (double)grad_y[i] * (double)out[i];
            }
        const double t = norm[n];
        grad_env[e] = t == 0.0 ? 0.0f : (float)(-0.5 * t * t * t * s);
    }
    return 0;
}

/* fp64 versions for the pins: the same reading with every step in double. */
int zs_oracle_forward_norm_f64(const float *coupling, const float *radial,
                               const float *env, const int64_t *dst, int64_t E,
                               int64_t N, int64_t C, double *y, double *norm)
{
    const int rc = zs_oracle_forward_f64(coupling, radial, dst, E, N, C, y);
    if (rc)
        return rc;
    for (int64_t n = 0; n < N; ++n)
        norm[n] = 0.0;
    for (int64_t e = 0; e < E; ++e)
        norm[dst[e]] = norm[dst[e]] + (double)env[e];
    for (int64_t n = 0; n < N; ++n)
        norm[n] = norm[n] > 0.0 ? 1.0 / sqrt(norm[n]) : 0.0;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t i = 0; i < ZS_ORACLE_ROWS * C; ++i)
            y[n * ZS_ORACLE_ROWS * C + i] = y[n * ZS_ORACLE_ROWS * C + i] * norm[n];
    return 0;
}
