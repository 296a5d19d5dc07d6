/*
 * K-thread variant of the oracle -- TEST INFRASTRUCTURE ONLY (the benchmark's
 * all-cores CPU baseline and its tests).  Not the oracle the parity tests
 * compare against, and never loaded by the product path.
 *
 * It includes zs_oracle.c (the backward's per-edge function, the index check)
 * and adds the forward's per-edge loop of zs_oracle_forward_f32 written for
 * one destination block, with the work split over threads so that no result
 * changes:
 *   forward:  nodes are split between threads; each node's edges are added
 *             in increasing edge id (the oracle's stable CSR), the order in
 *             which the sequential oracle adds them to that node;
 *   backward: edges are split between threads; each edge's gradients depend
 *             on that edge and its destination's upstream rows only.
 * Results are bitwise those of zs_oracle_forward_f32 / zs_oracle_backward_f32.
 */
#include "zs_oracle.c"

/* Adds edge e's message into its destination's 16 x C block o_node: each
 * product rounded to fp32, then added (zs_oracle_forward_f32's inner loops). */
static void mt_forward_one_edge_f32(const float *coupling, const float *radial,
                                    int64_t e, int64_t C, float *o_node)
{
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

int zs_oracle_mt_forward_f32(const float *coupling, const float *radial,
                             const int32_t *rowptr, const int32_t *perm,
                             int64_t N, int64_t C, float *out, int64_t threads)
{
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 64) num_threads((int)threads) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        float *o_node = out + n * ZS_ORACLE_ROWS * C;
        for (int64_t j = 0; j < ZS_ORACLE_ROWS * C; ++j)
            o_node[j] = 0.0f;
        if (rowptr[n] > rowptr[n + 1]) {
            bad = 1;
            continue;
        }
        for (int64_t k = rowptr[n]; k < rowptr[n + 1]; ++k)
            mt_forward_one_edge_f32(coupling, radial, perm[k], C, o_node);
    }
    return bad ? -3 : 0;
}

int zs_oracle_mt_backward_f32(const float *grad_out, const float *coupling,
                              const float *radial, const int64_t *dst, int64_t E,
                              int64_t N, int64_t C, float *grad_coupling,
                              float *grad_radial, int64_t threads)
{
    if (check_dst(dst, E, N))
        return -3;
#pragma omp parallel for schedule(static) num_threads((int)threads)
    for (int64_t e = 0; e < E; ++e)
        backward_one_edge_f32(grad_out, coupling, radial, e, dst[e], C,
                              grad_coupling + e * ZS_ORACLE_ZONAL,
                              grad_radial + e * 3 * C);
    return 0;
}
