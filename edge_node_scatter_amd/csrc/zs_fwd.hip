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

// NORM: as zs_fwd_staged_kernel below (envelope sum, y, norm, optional out).
template <int VEC, int NQ, int U, bool NORM>
__global__ __launch_bounds__(64) void zs_fwd_kernel(const float* __restrict__ coupling,
                                                    const float* __restrict__ radial, InLayout L,
                                                    const int32_t* __restrict__ rowptr,
                                                    const int32_t* __restrict__ perm,
                                                    int64_t n_nodes, int64_t n_edges, int64_t C,
                                                    float* __restrict__ out, NormIO nio) {
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
        float deg = 0.0f;

        for (int64_t k = k0; k < k1; k += U) {
            int32_t e[U];
#pragma unroll
            for (int b = 0; b < U; ++b) {
                const int32_t pe = (k + b < k1) ? perm[k + b] : -1;
                e[b] = (pe >= 0 && pe < n_edges) ? pe : -1;
            }
            VT xa[U], xb[U];
            float w[U][RPS];
            float ev[U];
            if (NORM) {
#pragma unroll
                for (int b = 0; b < U; ++b) ev[b] = e[b] >= 0 ? nio.env[e[b]] : 0.0f;
            }
#pragma unroll
            for (int b = 0; b < U; ++b) {
                if (e[b] >= 0 && act) {
                    const float* rrow = radial + int64_t(e[b]) * L.rad_edge + c0;
                    xa[b] = V::load(rrow + sA * L.rad_slot);
                    xb[b] = two_slots ? V::load(rrow + sB * L.rad_slot) : xa[b];
                    const float* crow = coupling + int64_t(e[b]) * L.cpl_edge;
#pragma unroll
                    for (int i = 0; i < RPS; ++i) {
                        const int r = r_first + i;
                        w[b][i] = r <= kZonal ? crow[r - 1] : 0.0f;
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < U; ++b) {
                if (NORM && e[b] >= 0) deg = deg + ev[b];
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

        float nrm = 1.0f;
        if (NORM) {
            nrm = deg > 0.0f ? 1.0f / sqrtf(deg) : 0.0f;
            if (lane == 0 && blockIdx.y == 0) nio.norm[node] = nrm;
        }
#pragma unroll
        for (int pass = 0; pass < (NORM ? 2 : 1); ++pass) {
            // NORM: pass 0 writes y, pass 1 the unnormalised out (if requested)
            float* base = (NORM && pass == 0) ? nio.y : out;
            if (!act || base == nullptr) continue;
            float* onode = base + node * kRows * C + c0;
#pragma unroll
            for (int i = 0; i < RPS; ++i) {
                const int r = r_first + i;
                float v[VEC];
#pragma unroll
                for (int u = 0; u < VEC; ++u)
                    v[u] = r > kZonal ? 0.0f : ((NORM && pass == 0) ? acc[i][u] * nrm : acc[i][u]);
                V::store(r <= kZonal ? onode + int64_t(r) * C : onode, v);   // row 0 is +0
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Staged forward for C % 4 == 0 with 16-byte aligned radial and out.
//
// Same lane mapping as above with VEC = 4, NQ = 8 (lane = j*8 + q: rows 2j+1,
// 2j+2 and channels 4q..4q+3 of a 32-channel tile).  The edges of a node are
// taken 16 at a time (a batch).  A batch's radial rows (16 x 3 x 32 floats)
// and coupling rows (16 x 15 floats) are fetched with coalesced, all-distinct
// 16-byte / 4-byte loads (six float4 and up to four floats per lane), kept in
// registers while the previous batch is being accumulated, then written to
// LDS from where each lane reads the float4 and two weights it needs per edge.
// The perm entries of a batch are fetched two batches ahead and every load is
// unconditional (absent edges read a valid substitute), so each data load is
// issued one batch before it is consumed and no load waits on another.
// Accumulation order and arithmetic are the same as in zs_fwd_kernel.
// ---------------------------------------------------------------------------
#ifndef ZS_FWD_BATCH
#define ZS_FWD_BATCH 8
#endif
constexpr int kFwdBatch = ZS_FWD_BATCH;
constexpr int kFwdRadVec = kFwdBatch * kSlots * 8 / 64;   // float4 per lane per batch (6)
constexpr int kFwdCplVec = (kFwdBatch * kZonal + 63) / 64; // floats per lane per batch (4)

struct FwdRegs {
    float4 r[kFwdRadVec];
    float w[kFwdCplVec];
};

// Lane mapping of the coalesced batch fetch (i = fetch slot, lane = 0..63):
//   radial float4 f = i*64 + lane -> batch edge f / 24, slot (f % 24) / 8, quad f % 8
//   coupling float idx = i*64 + lane -> batch edge idx / 15, column idx % 15 (idx < 240)
__device__ __attribute__((always_inline)) inline int fwd_rad_edge(int i, int lane) {
    return (i * 64 + lane) / (kSlots * 8);
}
__device__ __attribute__((always_inline)) inline int fwd_rad_rem(int i, int lane) {
    return (i * 64 + lane) % (kSlots * 8);
}
__device__ __attribute__((always_inline)) inline int fwd_cpl_idx(int i, int lane) {
    return i * 64 + lane;
}

// A batch's perm entries, fetched one batch before they are used.  Every lane
// issues its load from a valid position (clamped to the node's last edge) and
// the entry is range-checked only when it is used, so the load never forces an
// early wait.  Lane L < span carries the entry of edge k + L.
struct PermRaw {
    int32_t raw;
    bool valid;
};

__device__ __attribute__((always_inline)) inline PermRaw perm_issue(
    const int32_t* __restrict__ perm, int64_t k, int64_t k1, int lane, int span) {
    const int64_t kk = k + lane;
    PermRaw p;
    p.valid = lane < span && kk < k1;
    p.raw = perm[p.valid ? kk : k1 - 1];
    return p;
}

__device__ __attribute__((always_inline)) inline int perm_resolve(PermRaw p, int64_t n_edges) {
    return (p.valid && p.raw >= 0 && p.raw < n_edges) ? p.raw : -1;
}

// Loads of one batch, all unconditional: absent edges and channels past C read
// a valid substitute (edge 0, the tile's first channel) that is never used.
// With NORM, the fetch slots after the batch's 15 * kFwdBatch coupling floats
// carry the edges' envelope factors (one per edge).
template <bool NORM>
__device__ __attribute__((always_inline)) inline void fwd_fetch(FwdRegs& R, int lane, int pe,
                                                                 const float* __restrict__ coupling,
                                                                 const float* __restrict__ radial,
                                                                 const float* __restrict__ env,
                                                                 const InLayout& L, int64_t C,
                                                                 int64_t cbase) {
#pragma unroll
    for (int i = 0; i < kFwdRadVec; ++i) {
        const int rem = fwd_rad_rem(i, lane);
        const int64_t ch = cbase + (rem & 7) * 4;
        const int e = __shfl(pe, fwd_rad_edge(i, lane), 64);
        const int64_t es = e >= 0 ? e : 0;
        const int64_t cs = ch < C ? ch : cbase;
        R.r[i] = load_stream4<ZS_FWD_NT != 0>(radial + es * L.rad_edge + (rem >> 3) * L.rad_slot +
                                              cs);
    }
#pragma unroll
    for (int i = 0; i < kFwdCplVec; ++i) {
        const int idx = fwd_cpl_idx(i, lane);
        const bool in = idx < kFwdBatch * kZonal;
        const bool in_env = NORM && !in && idx < kFwdBatch * (kZonal + 1);
        const int b = in ? idx / kZonal : (in_env ? idx - kFwdBatch * kZonal : 0);
        const int e = __shfl(pe, b, 64);
        const int64_t es = e >= 0 ? e : 0;
        R.w[i] = in_env ? env[es] : coupling[es * L.cpl_edge + (in ? idx % kZonal : 0)];
    }
}

// With NORM the envelope factor of batch edge b sits in csh[b * 16 + 15] and
// deg accumulates the envelopes in edge order (fp32 adds from +0).
template <bool NORM>
__device__ __attribute__((always_inline)) inline void fwd_stage_accumulate(
    const FwdRegs& R, float4* rsh, float* csh, int cnt, int lane, int q, int j, int sA, int sB,
    float (&acc0)[4], float (&acc1)[4], float& deg) {
#pragma unroll
    for (int i = 0; i < kFwdRadVec; ++i) rsh[i * 64 + lane] = R.r[i];
#pragma unroll
    for (int i = 0; i < kFwdCplVec; ++i) {
        const int idx = fwd_cpl_idx(i, lane);
        if (idx < kFwdBatch * kZonal)
            csh[(idx / kZonal) * 16 + idx % kZonal] = R.w[i];
        else if (NORM && idx < kFwdBatch * (kZonal + 1))
            csh[(idx - kFwdBatch * kZonal) * 16 + 15] = R.w[i];
    }
    auto edge = [&](int b) {
        if (NORM) deg = deg + csh[b * 16 + 15];
        const float4 xa = rsh[b * (kSlots * 8) + sA * 8 + q];
        const float4 xb = rsh[b * (kSlots * 8) + sB * 8 + q];
        const float w0 = csh[b * 16 + 2 * j];
        const float w1 = csh[b * 16 + 2 * j + 1];
        float m;
        m = w0 * xa.x; acc0[0] = acc0[0] + m;
        m = w0 * xa.y; acc0[1] = acc0[1] + m;
        m = w0 * xa.z; acc0[2] = acc0[2] + m;
        m = w0 * xa.w; acc0[3] = acc0[3] + m;
        m = w1 * xb.x; acc1[0] = acc1[0] + m;
        m = w1 * xb.y; acc1[1] = acc1[1] + m;
        m = w1 * xb.z; acc1[2] = acc1[2] + m;
        m = w1 * xb.w; acc1[3] = acc1[3] + m;
    };
    if (cnt == kFwdBatch) {
        // full batch: unrolled so the LDS reads of all its edges are in flight
#pragma unroll
        for (int b = 0; b < kFwdBatch; ++b) edge(b);
    } else {
        for (int b = 0; b < cnt; ++b) edge(b);
    }
}

// NORM: also accumulate each node's envelope sum deg in edge order and write
// y = out * norm with norm = 1/sqrt(deg) (0 for deg <= 0); out (the
// unnormalised sum) is written only when the pointer is non-null.
template <bool NORM>
__global__ __launch_bounds__(64) void zs_fwd_staged_kernel(const float* __restrict__ coupling,
                                                           const float* __restrict__ radial,
                                                           InLayout L,
                                                           const int32_t* __restrict__ rowptr,
                                                           const int32_t* __restrict__ perm,
                                                           int64_t n_nodes, int64_t n_edges,
                                                           int64_t C, float* __restrict__ out,
                                                           NormIO nio) {
    static_assert(kFwdCplVec * 64 >= kFwdBatch * (kZonal + 1), "envelope slots");
    __shared__ float4 rsh[kFwdBatch * kSlots * 8];
    __shared__ float csh[kFwdBatch * 16];

    const int lane = threadIdx.x;
    const int q = lane & 7;
    const int j = lane >> 3;
    const int rA = 2 * j + 1;                 // rows rA, rA + 1 (rA + 1 == 16 is row 0)
    const int sA = row_slot(rA);
    const int sB = row_slot(rA + 1 <= kZonal ? rA + 1 : kZonal);
    const int64_t cbase = int64_t(blockIdx.y) * 32;
    const int64_t c0 = cbase + q * 4;
    const bool act = c0 < C;

    if (lane < kFwdBatch) csh[lane * 16 + 15] = 0.0f;   // pad column, never fetched

    for (int64_t node = blockIdx.x; node < n_nodes; node += gridDim.x) {
        int64_t k0 = rowptr[node];
        int64_t k1 = rowptr[node + 1];
        k0 = k0 < 0 ? 0 : (k0 > n_edges ? n_edges : k0);
        k1 = k1 < k0 ? k0 : (k1 > n_edges ? n_edges : k1);
        const int64_t nb = (k1 - k0 + kFwdBatch - 1) / kFwdBatch;

        float acc0[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float acc1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float deg = 0.0f;
        auto batch_count = [k0, k1](int64_t t) {
            const int64_t kb = k0 + t * kFwdBatch;
            return int(k1 - kb < kFwdBatch ? k1 - kb : kFwdBatch);
        };

        if (nb > 0) {
            FwdRegs RA, RB;
            PermRaw rA = perm_issue(perm, k0, k1, lane, kFwdBatch);
            PermRaw rB = perm_issue(perm, k0 + kFwdBatch, k1, lane, kFwdBatch);
            fwd_fetch<NORM>(RA, lane, perm_resolve(rA, n_edges), coupling, radial, nio.env, L, C,
                            cbase);
            for (int64_t t = 0; t < nb; t += 2) {
                const PermRaw rN = perm_issue(perm, k0 + (t + 2) * kFwdBatch, k1, lane, kFwdBatch);
                fwd_fetch<NORM>(RB, lane, perm_resolve(rB, n_edges), coupling, radial, nio.env, L,
                                C, cbase);
                fwd_stage_accumulate<NORM>(RA, rsh, csh, batch_count(t), lane, q, j, sA, sB, acc0,
                                           acc1, deg);
                if (t + 1 >= nb) break;
                rB = perm_issue(perm, k0 + (t + 3) * kFwdBatch, k1, lane, kFwdBatch);
                fwd_fetch<NORM>(RA, lane, perm_resolve(rN, n_edges), coupling, radial, nio.env, L,
                                C, cbase);
                fwd_stage_accumulate<NORM>(RB, rsh, csh, batch_count(t + 1), lane, q, j, sA, sB,
                                           acc0, acc1, deg);
            }
        }

        if (NORM) {
            const float nrm = deg > 0.0f ? 1.0f / sqrtf(deg) : 0.0f;
            if (lane == 0 && blockIdx.y == 0) nio.norm[node] = nrm;
            if (act) {
                float* ynode = nio.y + node * kRows * C + c0;
                float4 v0, v1;
                v0.x = acc0[0] * nrm; v0.y = acc0[1] * nrm; v0.z = acc0[2] * nrm; v0.w = acc0[3] * nrm;
                v1.x = acc1[0] * nrm; v1.y = acc1[1] * nrm; v1.z = acc1[2] * nrm; v1.w = acc1[3] * nrm;
                *reinterpret_cast<float4*>(ynode + int64_t(rA) * C) = v0;
                if (rA + 1 <= kZonal)
                    *reinterpret_cast<float4*>(ynode + int64_t(rA + 1) * C) = v1;
                else
                    *reinterpret_cast<float4*>(ynode) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
        }
        if (act && (!NORM || out != nullptr)) {
            float* onode = out + node * kRows * C + c0;
            *reinterpret_cast<float4*>(onode + int64_t(rA) * C) =
                make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
            if (rA + 1 <= kZonal)
                *reinterpret_cast<float4*>(onode + int64_t(rA + 1) * C) =
                    make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
            else
                *reinterpret_cast<float4*>(onode) = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }
}

}  // namespace

hipError_t launch_forward(const float* coupling, const float* radial, InLayout L,
                          const int32_t* rowptr, const int32_t* perm, int64_t n_nodes,
                          int64_t n_edges, int64_t channels, float* out, bool vec4,
                          NormIO nio, hipStream_t stream) {
    constexpr int64_t kGridCap = 1 << 20;
    const unsigned gx = unsigned(n_nodes < kGridCap ? n_nodes : kGridCap);
    const bool norm = nio.y != nullptr;   // env may be NULL when there are no edges
    if (vec4) {
        const unsigned gy = unsigned((channels + 31) / 32);
        if (norm)
            zs_fwd_staged_kernel<true><<<dim3(gx, gy), 64, 0, stream>>>(
                coupling, radial, L, rowptr, perm, n_nodes, n_edges, channels, out, nio);
        else
            zs_fwd_staged_kernel<false><<<dim3(gx, gy), 64, 0, stream>>>(
                coupling, radial, L, rowptr, perm, n_nodes, n_edges, channels, out, nio);
    } else {
        constexpr int NQ = 16, VEC = 1;
        const unsigned gy = unsigned((channels + NQ * VEC - 1) / (NQ * VEC));
        if (norm)
            zs_fwd_kernel<VEC, NQ, 8, true><<<dim3(gx, gy), 64, 0, stream>>>(
                coupling, radial, L, rowptr, perm, n_nodes, n_edges, channels, out, nio);
        else
            zs_fwd_kernel<VEC, NQ, 8, false><<<dim3(gx, gy), 64, 0, stream>>>(
                coupling, radial, L, rowptr, perm, n_nodes, n_edges, channels, out, nio);
    }
    return hipGetLastError();
}

}  // namespace zs
