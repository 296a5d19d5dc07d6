// Fused GIE zonal scatter, forward, gfx950.
//
// deepmd-kit PR #6072 ("fused Triton zonal scatter for the GIE head"), section
// "What", Forward bullet: a node-parallel kernel walks the stable destination
// CSR, keeps the node's message sum in registers and writes the padded
// (N, 16, C) layout with a zero scalar row; the (E, 15, C) message surface is
// never formed.
//
// Mapping (one 64-lane wavefront per node and channel tile):
//   lane = j * NQ + q.  q picks VEC consecutive channels (tile width NQ*VEC),
//   j picks a slot of RPS consecutive padded rows (rows j*RPS+1 .. j*RPS+RPS;
//   the one past row 15 stands for the scalar row 0 and is written as +0).
//   Every edge of the node is visited in CSR order (= increasing edge id); the
//   wavefront prefetches U edges' perm entries, radial vectors and coupling
//   values before accumulating them in order, so U edges' loads are in flight.
//   A lane needs the radial slots of its rows only: at most two distinct slots
//   (rows 3,4 straddle degrees 1 and 2), so it issues one or two vector loads
//   per edge.
//
// Arithmetic: acc = acc + fp32(w * x), separately rounded (the library is
// compiled with -ffp-contract=off), starting from +0 and in edge order -- the
// fp32 result of materialising the message and index-adding it.
#include "zs_internal.h"

namespace zs {

namespace {

template <int VEC, int NQ, int U>
__global__ __launch_bounds__(64) void zs_fwd_kernel(const float* __restrict__ coupling,
                                                    const float* __restrict__ radial,
                                                    const int32_t* __restrict__ rowptr,
                                                    const int32_t* __restrict__ perm,
                                                    int64_t n_nodes, int64_t n_edges, int64_t C,
                                                    float* __restrict__ out) {
    using V = VecT<VEC>;
    using VT = typename V::T;
    constexpr int NS = 64 / NQ;
    constexpr int RPS = kRows / NS;
    static_assert(NS * RPS == kRows, "row slots must tile the 16 padded rows");

    const int lane = threadIdx.x;
    const int q = lane % NQ;
    const int j = lane / NQ;
    const int r_first = j * RPS + 1;
    const int r_last = (j * RPS + RPS) < kZonal ? (j * RPS + RPS) : kZonal;
    const int sA = row_slot(r_first);
    const int sB = row_slot(r_last);
    const bool two_slots = sA != sB;
    const int64_t c0 = (int64_t(blockIdx.y) * NQ + q) * VEC;
    const bool act = c0 < C;
    const int64_t row_stride = int64_t(kSlots) * C;

    for (int64_t node = blockIdx.x; node < n_nodes; node += gridDim.x) {
        int64_t k0 = rowptr[node];
        int64_t k1 = rowptr[node + 1];
        k0 = k0 < 0 ? 0 : (k0 > n_edges ? n_edges : k0);
        k1 = k1 < k0 ? k0 : (k1 > n_edges ? n_edges : k1);

        float acc[RPS][VEC];
#pragma unroll
        for (int i = 0; i < RPS; ++i)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[i][v] = 0.0f;

        for (int64_t k = k0; k < k1; k += U) {
            int32_t e[U];
#pragma unroll
            for (int b = 0; b < U; ++b) {
                const int32_t pe = (k + b < k1) ? perm[k + b] : -1;
                e[b] = (pe >= 0 && pe < n_edges) ? pe : -1;
            }
            VT xa[U], xb[U];
            float w[U][RPS];
#pragma unroll
            for (int b = 0; b < U; ++b) {
                if (e[b] >= 0 && act) {
                    const float* rrow = radial + int64_t(e[b]) * row_stride + c0;
                    xa[b] = V::load(rrow + sA * C);
                    xb[b] = two_slots ? V::load(rrow + sB * C) : xa[b];
                    const float* crow = coupling + int64_t(e[b]) * kZonal;
#pragma unroll
                    for (int i = 0; i < RPS; ++i) {
                        const int r = r_first + i;
                        w[b][i] = r <= kZonal ? crow[r - 1] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < U; ++b) {
                if (e[b] >= 0 && act) {
#pragma unroll
                    for (int i = 0; i < RPS; ++i) {
                        const int r = r_first + i;
                        if (r <= kZonal) {
                            const VT x = row_slot(r) == sA ? xa[b] : xb[b];
#pragma unroll
                            for (int v = 0; v < VEC; ++v) {
                                const float m = w[b][i] * V::get(x, v);
                                acc[i][v] = acc[i][v] + m;
                            }
                        }
                    }
                }
            }
        }

        if (act) {
            float* onode = out + node * kRows * C + c0;
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                const int r = r_first + i;
                if (r <= kZonal) {
                    V::store(onode + int64_t(r) * C, acc[i]);
                } else {
                    float z[VEC];
#pragma unroll
                    for (int v = 0; v < VEC; ++v) z[v] = 0.0f;
                    V::store(onode, z);   // scalar row 0
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_forward(const float* coupling, const float* radial, const int32_t* rowptr,
                          const int32_t* perm, int64_t n_nodes, int64_t n_edges, int64_t channels,
                          float* out, bool vec4, hipStream_t stream) {
    constexpr int64_t kGridCap = 1 << 20;
    const unsigned gx = unsigned(n_nodes < kGridCap ? n_nodes : kGridCap);
    if (vec4) {
        constexpr int NQ = 8, VEC = 4;
        const unsigned gy = unsigned((channels + NQ * VEC - 1) / (NQ * VEC));
        zs_fwd_kernel<VEC, NQ, 8><<<dim3(gx, gy), 64, 0, stream>>>(coupling, radial, rowptr, perm,
                                                                   n_nodes, n_edges, channels, out);
    } else {
        constexpr int NQ = 16, VEC = 1;
        const unsigned gy = unsigned((channels + NQ * VEC - 1) / (NQ * VEC));
        zs_fwd_kernel<VEC, NQ, 8><<<dim3(gx, gy), 64, 0, stream>>>(coupling, radial, rowptr, perm,
                                                                   n_nodes, n_edges, channels, out);
    }
    return hipGetLastError();
}

}  // namespace zs
