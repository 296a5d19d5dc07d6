// Envelope gradient of the inverse-square-root degree normalisation, gfx950.
//
// deepmd-kit PR #6072 ("fused Triton zonal scatter for the GIE head"), section
// "What", third bullet, and the last step of its sequence diagram: the degree
// normalisation after the scatter stays outside the fused scatter and keeps
// its own cotangent, because the degree is a sum of cutoff-envelope factors
// and so depends on geometry.  With deg[n] = sum of env over the node's edges,
// norm = deg^(-1/2) and y = out * norm:
//   dL/ddeg[n] = -1/2 * norm^3 * sum_{r = 1..15, c} gy[n][r][c] * out[n][r][c]
//   dL/denv[e] = dL/ddeg[dst[e]]
// (row 0 of out is zero, so it is left out of the sum).
//
// Two kernels (the staged backward in zs_bwd.hip forms grad_deg itself while
// it stages the upstream rows; zs_norm_deg_kernel serves the other layouts):
//   zs_norm_deg_kernel: one wavefront per node streams its 15*C upstream and
//     output values (coalesced; 16-byte loads when C % 4 == 0), forms the exact
//     fp32 x fp32 products in fp64, reduces them across the wavefront with a
//     fixed butterfly and rounds -1/2 t^3 s to fp32 once (0 when norm == 0).
//   zs_norm_env_kernel: edge-parallel gather grad_env[e] = grad_deg[dst32[e]],
//     four edges per thread; the per-node table is small and stays in the
//     caches, so this is one coalesced read of dst32 and one coalesced write
//     per edge.
#include "zs_internal.h"

namespace zs {

namespace {

constexpr int kNormWaves = 4;   // nodes per 256-thread block

template <int VEC>
__global__ __launch_bounds__(256) void zs_norm_deg_kernel(const float* __restrict__ grad_y,
                                                          const float* __restrict__ out,
                                                          const float* __restrict__ norm,
                                                          int64_t n_nodes, int64_t C,
                                                          float* __restrict__ grad_deg) {
    using V = VecT<VEC>;
    using VT = typename V::T;
    const int lane = threadIdx.x & 63;
    const int64_t count = int64_t(kZonal) * C / VEC;   // vectors in rows 1..15
    for (int64_t node = int64_t(blockIdx.x) * kNormWaves + (threadIdx.x >> 6); node < n_nodes;
         node += int64_t(gridDim.x) * kNormWaves) {
        const int64_t base = (node * kRows + 1) * C;
        const float* gp = grad_y + base;
        const float* op = out + base;
        double s = 0.0;
        for (int64_t i = lane; i < count; i += 64) {
            const VT g = V::load(gp + i * VEC);
            const VT o = V::load(op + i * VEC);
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                s = __builtin_fma(double(V::get(g, v)), double(V::get(o, v)), s);
        }
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) s = s + __shfl_xor(s, h, 64);
        if (lane == 0) {
            const double t = norm[node];
            grad_deg[node] = t == 0.0 ? 0.0f : float(-0.5 * t * t * t * s);
        }
    }
}

// Four consecutive edges per thread (16-byte loads and stores when both
// arrays are 16-byte aligned, which VEC4 asserts), so each thread has four
// independent table loads in flight.
template <bool VEC4>
__global__ __launch_bounds__(256) void zs_norm_env_kernel(const int32_t* __restrict__ dst32,
                                                          const float* __restrict__ grad_deg,
                                                          int64_t n_nodes, int64_t n_edges,
                                                          float* __restrict__ grad_env) {
    for (int64_t e = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4; e < n_edges;
         e += int64_t(gridDim.x) * 256 * 4) {
        if (VEC4 && e + 4 <= n_edges) {
            const int4 d = *reinterpret_cast<const int4*>(dst32 + e);
            float4 g;
            g.x = (d.x >= 0 && d.x < n_nodes) ? grad_deg[d.x] : 0.0f;
            g.y = (d.y >= 0 && d.y < n_nodes) ? grad_deg[d.y] : 0.0f;
            g.z = (d.z >= 0 && d.z < n_nodes) ? grad_deg[d.z] : 0.0f;
            g.w = (d.w >= 0 && d.w < n_nodes) ? grad_deg[d.w] : 0.0f;
            *reinterpret_cast<float4*>(grad_env + e) = g;
        } else {
            for (int64_t k = e; k < e + 4 && k < n_edges; ++k) {
                const int32_t d = dst32[k];
                grad_env[k] = (d >= 0 && d < n_nodes) ? grad_deg[d] : 0.0f;
            }
        }
    }
}

}  // namespace

hipError_t launch_norm_grad(const float* grad_y, const float* out, const float* norm,
                            const int32_t* dst32, int64_t n_nodes, int64_t n_edges,
                            int64_t channels, float* grad_deg, float* grad_env, bool deg_done,
                            hipStream_t stream) {
    constexpr int64_t kGridCap = 1 << 20;
    const int64_t node_blocks = (n_nodes + kNormWaves - 1) / kNormWaves;
    const unsigned gn = unsigned(node_blocks < kGridCap ? node_blocks : kGridCap);
    const bool vec4 = channels % 4 == 0 && reinterpret_cast<uintptr_t>(grad_y) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(out) % 16 == 0;
    if (deg_done) {
        // formed by the staged backward while it staged the rows
    } else if (vec4) {
        zs_norm_deg_kernel<4><<<gn, 256, 0, stream>>>(grad_y, out, norm, n_nodes, channels,
                                                      grad_deg);
    } else {
        zs_norm_deg_kernel<1><<<gn, 256, 0, stream>>>(grad_y, out, norm, n_nodes, channels,
                                                      grad_deg);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || n_edges == 0) return err;
    const int64_t edge_blocks = (n_edges + 1023) / 1024;
    const unsigned ge = unsigned(edge_blocks < kGridCap ? edge_blocks : kGridCap);
    if (reinterpret_cast<uintptr_t>(dst32) % 16 == 0 && reinterpret_cast<uintptr_t>(grad_env) % 16 == 0)
        zs_norm_env_kernel<true><<<ge, 256, 0, stream>>>(dst32, grad_deg, n_nodes, n_edges,
                                                         grad_env);
    else
        zs_norm_env_kernel<false><<<ge, 256, 0, stream>>>(dst32, grad_deg, n_nodes, n_edges,
                                                          grad_env);
    return hipGetLastError();
}

}  // namespace zs
