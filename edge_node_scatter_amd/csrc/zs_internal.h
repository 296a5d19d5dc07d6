// Internal declarations shared by the HIP translation units of libzs.
// Not part of the public ABI (that is include/zs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace zs {

// Degree-slot of padded row r (1..15) for lmax = 3: the rows of degree l are
// l*l .. l*l + 2l, so rows 1-3 -> slot 0, 4-8 -> slot 1, 9-15 -> slot 2.
__host__ __device__ constexpr int row_slot(int r) { return r < 4 ? 0 : (r < 9 ? 1 : 2); }

constexpr int kRows = 16;
constexpr int kZonal = 15;
constexpr int kSlots = 3;

// Orders LDS accesses between the lanes of one wavefront.  A lane that reads
// what another lane of its wavefront wrote to LDS, or overwrites what another
// lane still has to read, relies on the accesses on either side of this
// point staying on their side: the release fence keeps earlier accesses
// before it, the acquire fence keeps later ones after it, and the wave
// barrier keeps the two fences together.  At wavefront scope none of the
// three emits an instruction (a wavefront's LDS operations complete in issue
// order); they only bind the compiler.
__device__ __attribute__((always_inline)) inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Vector of VEC consecutive fp32 channels (VEC = 4: one 16-byte access).
template <int VEC>
struct VecT;
template <>
struct VecT<4> {
    using T = float4;
    __device__ static T load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static void store(float* p, const float (&v)[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
    __device__ static float get(const T& v, int i) {
        return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
    }
};
template <>
struct VecT<1> {
    using T = float;
    __device__ static T load(const float* p) { return *p; }
    __device__ static void store(float* p, const float (&v)[1]) { *p = v[0]; }
    __device__ static float get(const T& v, int) { return v; }
};

// Read-once / write-once 16-byte accesses of radial and grad_radial rows.
// NT = true marks them non-temporal (streamed past the caches), which keeps
// the L2 and the memory-side cache for the data that is reused (coupling
// lines shared by neighbouring edges, the upstream rows of a node).
typedef float zs_f4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __attribute__((always_inline)) inline float4 load_stream4(const float* p) {
    if (NT) {
        const zs_f4 v = __builtin_nontemporal_load(reinterpret_cast<const zs_f4*>(p));
        return make_float4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const float4*>(p);
}
template <bool NT>
__device__ __attribute__((always_inline)) inline void store_stream4(float* p, float4 v) {
    if (NT) {
        zs_f4 t = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(t, reinterpret_cast<zs_f4*>(p));
    } else {
        *reinterpret_cast<float4*>(p) = v;
    }
}

// Build-time tuning knobs (defaults are the measured best on MI355X).
#ifndef ZS_FWD_NT
#define ZS_FWD_NT 1
#endif
#ifndef ZS_BWD_NT
#define ZS_BWD_NT 1
#endif

// ---- forward / backward -----------------------------------------------------
// Strides (in floats) of the two edge inputs.  Coupling columns and radial
// channels are unit-stride; a contiguous layout is {15, 3*C, C}.
struct InLayout {
    int64_t cpl_edge;   // coupling: edge -> edge
    int64_t rad_edge;   // radial: edge -> edge
    int64_t rad_slot;   // radial: slot -> slot
};

// Inverse-square-root degree normalisation fused into the scatter.  Forward:
// env [n_edges] is read, y [n_nodes][16][C] = out * norm and norm [n_nodes] are
// written (out itself only when non-null).  Backward: norm [n_nodes] scales the
// upstream rows before they are used.  y == nullptr selects the plain scatter
// (env may be null when there are no edges).
struct NormIO {
    const float* env;
    float* y;
    float* norm;
};

// order: NULL (grid position = node) or the node order from the CSR build
// (the node handed to each grid position).
hipError_t launch_forward(const float* coupling, const float* radial, InLayout L,
                          const int32_t* rowptr, const int32_t* perm, const int32_t* order,
                          int64_t n_nodes, int64_t n_edges, int64_t channels, float* out,
                          bool vec4, NormIO nio, hipStream_t stream);

// Normalised backward.  norm == nullptr: plain backward.  Otherwise grad_out is
// the gradient of y and is multiplied by norm[dst] (fp32) on load, and when
// out and grad_deg are non-null the staged kernel also forms the degree
// gradient grad_deg[n] = -1/2 t^3 sum_{r>=1,c} grad_out * out (t = norm[n])
// while it stages the node's rows.
struct NormGrad {
    const float* norm;
    const float* out;
    float* grad_deg;
};

// *deg_done (may be null) is set when grad_deg was written.
hipError_t launch_backward(const float* grad_out, const float* coupling, const float* radial,
                           InLayout L, const int32_t* rowptr, const int32_t* perm,
                           int64_t n_nodes, int64_t n_edges,
                           int64_t channels, float* grad_coupling, float* grad_radial, bool vec4,
                           NormGrad ng, bool* deg_done, hipStream_t stream);

// Envelope gradient of the normalisation: grad_deg[n] (fp32, per node) from
// grad_y, out and norm unless deg_done, then grad_env[e] = grad_deg[dst32[e]]
// (0 for dst32 < 0).
hipError_t launch_norm_grad(const float* grad_y, const float* out, const float* norm,
                            const int32_t* dst32, int64_t n_nodes, int64_t n_edges,
                            int64_t channels, float* grad_deg, float* grad_env, bool deg_done,
                            hipStream_t stream);

// Small fill kernel (used instead of hipMemsetAsync so the calls stay
// capturable in HIP graphs).
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t stream);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t stream);

}  // namespace zs
