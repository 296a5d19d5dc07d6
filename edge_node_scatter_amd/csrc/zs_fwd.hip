// Fused GIE zonal scatter, forward, gfx950.
//
// Operation: deepmd-kit PR #6072 ("fused Triton zonal scatter for the GIE
// head"), section "What", Forward bullet.  Each node's output rows are summed
// by the wavefront that owns the node: it visits the node's incoming edges in
// destination-sorted order, multiplies each edge's coupling weight into its
// radial features on the fly and adds the product into registers.  Per-edge
// products therefore never exist in memory; the only write is the node's
// 16-row block, whose row 0 is stored as zeros.
//
// Three kernels, chosen per launch: zs_fwd_staged_kernel (one wavefront per
// node and channel tile, C % 4 == 0, aligned), zs_fwd_slot_kernel (three
// wavefronts per node and tile, one per radial slot, for launches with few
// nodes) and zs_fwd_kernel (any C and alignment).  All three accumulate the
// same products in the same order, so their results are bitwise equal.
//
// Grid position s sums node order[s] when the caller passes the node schedule
// the CSR build produces (every bucket's highest-degree nodes first, each band
// spread over the compute units), else node s.  When a launch's wavefronts are
// all resident at once the dispatcher's placement is fixed by position, so the
// schedule is what spreads high-degree nodes evenly: on the skewed 4096-node
// frame the forward takes 65.5 instead of 72.6 us.
//
// Mapping of zs_fwd_kernel (one 64-lane wavefront per node and channel tile):
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

// Node handled at grid position slot: order[slot] when a node order is given
// (-1, skipped, when the entry is not a node), else slot itself.  The order
// only decides which wavefront sums which node, and when; every node's sums
// are the same either way.
__device__ __attribute__((always_inline)) inline int64_t node_at(const int32_t* __restrict__ order,
                                                                 int64_t slot, int64_t n_nodes) {
    if (order == nullptr) return slot;
    const int64_t n = order[slot];
    return n >= 0 && n < n_nodes ? n : -1;
}

// NORM: as zs_fwd_staged_kernel below (envelope sum, y, norm, optional out).
template <int VEC, int NQ, int U, bool NORM>
__global__ __launch_bounds__(64) void zs_fwd_kernel(const float* __restrict__ coupling,
                                                    const float* __restrict__ radial, InLayout L,
                                                    const int32_t* __restrict__ rowptr,
                                                    const int32_t* __restrict__ perm,
                                                    const int32_t* __restrict__ order,
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

    for (int64_t slot = blockIdx.x; slot < n_nodes; slot += gridDim.x) {
        const int64_t node = node_at(order, slot, n_nodes);
        if (node < 0) continue;
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
// One 64-lane wavefront per (node, channel tile of T = 8*VEC channels);
// lane = j*8 + q owns padded rows 2j+1, 2j+2 (the one past row 15 stands for
// row 0) and channels q*VEC .. q*VEC+VEC-1 of the tile, so one wavefront
// covers up to 64 channels and the node's perm entries and coupling rows are
// read once per tile.  The edges of a node are taken B at a time (a batch).
// A batch's radial rows (B x 3 x T floats) and coupling rows (B x 15 floats,
// plus B envelope factors when normalising) are fetched with coalesced,
// all-distinct 16-byte / 4-byte loads, kept in registers while the previous
// batch is accumulated, then written to LDS, from where each lane reads the
// VEC values of each of its two radial slots and its two weights per edge.
// The perm entries of a batch are fetched two batches ahead and every load is
// unconditional (absent edges and channels read a valid substitute), so each
// data load is issued one batch before it is consumed and no load waits on
// another.  Accumulation order and arithmetic are those of zs_fwd_kernel.
// ---------------------------------------------------------------------------
template <int VEC, int B>
struct FwdShape {
    static constexpr int T = 8 * VEC;                   // channels per tile
    static constexpr int F4 = T / 4;                    // float4 per slot row of a tile
    static constexpr int RAD = B * kSlots * F4;         // radial float4 per batch
    static constexpr int RV = (RAD + 63) / 64;          // radial float4 per lane
    static constexpr int CV = (B * (kZonal + 1) + 63) / 64;   // coupling/env floats per lane
};

template <int VEC, int B>
struct FwdRegs {
    float4 r[FwdShape<VEC, B>::RV];
    float w[FwdShape<VEC, B>::CV];
};

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

// Loads of one batch, all unconditional: absent edges, channels past C and
// fetch slots past the batch read a valid substitute (edge 0, the tile's
// first channel) that is never used.  Radial float4 f = i*64 + lane is batch
// edge f / (3*F4), slot (f % (3*F4)) / F4, float4 f % F4 of the tile; coupling
// float idx = i*64 + lane is batch edge idx / 15, column idx % 15 for
// idx < 15*B, and with NORM the envelope factor of batch edge idx - 15*B for
// the next B slots.
template <int VEC, int B, bool NORM>
__device__ __attribute__((always_inline)) inline void fwd_fetch(
    FwdRegs<VEC, B>& R, int lane, int pe, const float* __restrict__ coupling,
    const float* __restrict__ radial, const float* __restrict__ env, const InLayout& L, int64_t C,
    int64_t cbase) {
    using S = FwdShape<VEC, B>;
#pragma unroll
    for (int i = 0; i < S::RV; ++i) {
        const int f = i * 64 + lane;
        const int rem = f % (kSlots * S::F4);
        const int64_t ch = cbase + (rem % S::F4) * 4;
        const int e = __shfl(pe, f < S::RAD ? f / (kSlots * S::F4) : 0, 64);
        const int64_t es = e >= 0 ? e : 0;
        const int64_t cs = ch < C ? ch : cbase;
        R.r[i] = load_stream4<ZS_FWD_NT != 0>(radial + es * L.rad_edge +
                                              (rem / S::F4) * L.rad_slot + cs);
    }
#pragma unroll
    for (int i = 0; i < S::CV; ++i) {
        const int idx = i * 64 + lane;
        const bool in = idx < B * kZonal;
        const bool in_env = NORM && !in && idx < B * (kZonal + 1);
        const int b = in ? idx / kZonal : (in_env ? idx - B * kZonal : 0);
        const int e = __shfl(pe, b, 64);
        const int64_t es = e >= 0 ? e : 0;
        R.w[i] = in_env ? env[es] : coupling[es * L.cpl_edge + (in ? idx % kZonal : 0)];
    }
}

// VEC consecutive floats from LDS with the widest accesses their alignment
// allows (q*VEC floats into a 32-byte aligned row).
template <int VEC>
__device__ __attribute__((always_inline)) inline void lds_read(const float* p, float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            const float4 t = reinterpret_cast<const float4*>(p)[i];
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
    } else if constexpr (VEC % 2 == 0) {
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) {
            const float2 t = reinterpret_cast<const float2*>(p)[i];
            v[2 * i] = t.x; v[2 * i + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = p[i];
    }
}

// Stores VEC consecutive floats of an output row; n_valid < VEC masks the
// channels past C.  Rows are 16-byte aligned (C % 4 == 0).
template <int VEC>
__device__ __attribute__((always_inline)) inline void row_store(float* p, const float (&v)[VEC],
                                                                int n_valid) {
    if (n_valid >= VEC) {
        if constexpr (VEC % 4 == 0) {
#pragma unroll
            for (int i = 0; i < VEC / 4; ++i)
                reinterpret_cast<float4*>(p)[i] =
                    make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
        } else if constexpr (VEC % 2 == 0) {
#pragma unroll
            for (int i = 0; i < VEC / 2; ++i)
                reinterpret_cast<float2*>(p)[i] = make_float2(v[2 * i], v[2 * i + 1]);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i) p[i] = v[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            if (i < n_valid) p[i] = v[i];
    }
}

// With NORM the envelope factor of batch edge b sits in csh[b * 16 + 15] and
// deg accumulates the envelopes in edge order (fp32 adds from +0).
template <int VEC, int B, bool NORM>
__device__ __attribute__((always_inline)) inline void fwd_stage_accumulate(
    const FwdRegs<VEC, B>& R, float4* rsh, float* csh, int cnt, int lane, int q, int j, int sA,
    int sB, float (&acc0)[VEC], float (&acc1)[VEC], float& deg) {
    using S = FwdShape<VEC, B>;
    wave_lds_sync();   // the previous batch's reads come before these writes
#pragma unroll
    for (int i = 0; i < S::RV; ++i)
        if (S::RAD % 64 == 0 || i * 64 + lane < S::RAD) rsh[i * 64 + lane] = R.r[i];
#pragma unroll
    for (int i = 0; i < S::CV; ++i) {
        const int idx = i * 64 + lane;
        if (idx < B * kZonal)
            csh[(idx / kZonal) * 16 + idx % kZonal] = R.w[i];
        else if (NORM && idx < B * (kZonal + 1))
            csh[(idx - B * kZonal) * 16 + 15] = R.w[i];
    }
    wave_lds_sync();   // every lane reads values other lanes staged
    const float* rf = reinterpret_cast<const float*>(rsh);
    auto edge = [&](int b) {
        if (NORM) deg = deg + csh[b * 16 + 15];
        float xa[VEC], xb[VEC];
        lds_read<VEC>(rf + (b * kSlots + sA) * S::T + q * VEC, xa);
        lds_read<VEC>(rf + (b * kSlots + sB) * S::T + q * VEC, xb);
        const float w0 = csh[b * 16 + 2 * j];
        const float w1 = csh[b * 16 + 2 * j + 1];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            float m = w0 * xa[v];
            acc0[v] = acc0[v] + m;
            m = w1 * xb[v];
            acc1[v] = acc1[v] + m;
        }
    };
    if (cnt == B) {
        // full batch: unrolled so the LDS reads of all its edges are in flight
#pragma unroll
        for (int b = 0; b < B; ++b) edge(b);
    } else {
        for (int b = 0; b < cnt; ++b) edge(b);
    }
}

// One node of the staged forward, by the calling wavefront (lanes as above;
// channel tile blockIdx.y).  rsh / csh: this wavefront's LDS staging
// (FwdShape<VEC, B>::RAD float4 and B*16 floats).
// NORM: also accumulate the node's envelope sum deg in edge order and write
// y = out * norm with norm = 1/sqrt(deg) (0 for deg <= 0); out (the
// unnormalised sum) is written only when the pointer is non-null.
// The pad column csh[b*16 + 15] is read only as the weight of the lanes that
// own the slot past row 15, whose sums are never stored (those lanes store
// zeros into row 0), and carries the envelope factors with NORM.
template <int VEC, int B, bool NORM>
__device__ __attribute__((always_inline)) inline void fwd_staged_node(
    int64_t node, int64_t k0, int64_t k1, const float* __restrict__ coupling,
    const float* __restrict__ radial, const InLayout& L, const int32_t* __restrict__ perm,
    int64_t n_edges, int64_t C, float* __restrict__ out, const NormIO& nio, float4* rsh,
    float* csh) {
    using S = FwdShape<VEC, B>;
    static_assert(S::CV * 64 >= B * (kZonal + 1), "coupling and envelope slots");
    static_assert(B <= 64, "one perm entry per lane");
    const int lane = threadIdx.x & 63;
    const int q = lane & 7;
    const int j = lane >> 3;
    const int rA = 2 * j + 1;                 // rows rA, rA + 1 (rA + 1 == 16 is row 0)
    const int sA = row_slot(rA);
    const int sB = row_slot(rA + 1 <= kZonal ? rA + 1 : kZonal);
    const int64_t cbase = int64_t(blockIdx.y) * S::T;
    const int64_t c0 = cbase + q * VEC;
    const int n_valid = c0 >= C ? 0 : (C - c0 < VEC ? int(C - c0) : VEC);
    const int64_t nb = (k1 - k0 + B - 1) / B;

    float acc0[VEC], acc1[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc0[v] = acc1[v] = 0.0f;
    float deg = 0.0f;
    auto batch_count = [k0, k1](int64_t t) {
        const int64_t kb = k0 + t * B;
        return int(k1 - kb < B ? k1 - kb : B);
    };

    if (nb > 0) {
        FwdRegs<VEC, B> RA, RB;
        PermRaw pA = perm_issue(perm, k0, k1, lane, B);
        PermRaw pB = perm_issue(perm, k0 + B, k1, lane, B);
        fwd_fetch<VEC, B, NORM>(RA, lane, perm_resolve(pA, n_edges), coupling, radial, nio.env,
                                L, C, cbase);
        for (int64_t t = 0; t < nb; t += 2) {
            const PermRaw pN = perm_issue(perm, k0 + (t + 2) * B, k1, lane, B);
            fwd_fetch<VEC, B, NORM>(RB, lane, perm_resolve(pB, n_edges), coupling, radial,
                                    nio.env, L, C, cbase);
            fwd_stage_accumulate<VEC, B, NORM>(RA, rsh, csh, batch_count(t), lane, q, j, sA, sB,
                                               acc0, acc1, deg);
            if (t + 1 >= nb) break;
            pB = perm_issue(perm, k0 + (t + 3) * B, k1, lane, B);
            fwd_fetch<VEC, B, NORM>(RA, lane, perm_resolve(pN, n_edges), coupling, radial,
                                    nio.env, L, C, cbase);
            fwd_stage_accumulate<VEC, B, NORM>(RB, rsh, csh, batch_count(t + 1), lane, q, j, sA,
                                               sB, acc0, acc1, deg);
        }
    }

    float zero[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) zero[v] = 0.0f;
    if (NORM) {
        const float nrm = deg > 0.0f ? 1.0f / sqrtf(deg) : 0.0f;
        if (lane == 0 && blockIdx.y == 0) nio.norm[node] = nrm;
        float y0[VEC], y1[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            y0[v] = acc0[v] * nrm;
            y1[v] = acc1[v] * nrm;
        }
        float* ynode = nio.y + node * kRows * C + c0;
        row_store<VEC>(ynode + int64_t(rA) * C, y0, n_valid);
        if (rA + 1 <= kZonal)
            row_store<VEC>(ynode + int64_t(rA + 1) * C, y1, n_valid);
        else
            row_store<VEC>(ynode, zero, n_valid);
    }
    if (!NORM || out != nullptr) {
        float* onode = out + node * kRows * C + c0;
        row_store<VEC>(onode + int64_t(rA) * C, acc0, n_valid);
        if (rA + 1 <= kZonal)
            row_store<VEC>(onode + int64_t(rA + 1) * C, acc1, n_valid);
        else
            row_store<VEC>(onode, zero, n_valid);
    }
}

// A node's CSR range [k0, k1), clamped to [0, n_edges].
__device__ __attribute__((always_inline)) inline void node_range(const int32_t* __restrict__ rowptr,
                                                                 int64_t node, int64_t n_edges,
                                                                 int64_t& k0, int64_t& k1) {
    k0 = rowptr[node];
    k1 = rowptr[node + 1];
    k0 = k0 < 0 ? 0 : (k0 > n_edges ? n_edges : k0);
    k1 = k1 < k0 ? k0 : (k1 > n_edges ? n_edges : k1);
}

// Nodes of degree above `heavy` take batches of BH = 8 edges when the launch
// uses 4 (VEC <= 4): twice the bytes in flight for the nodes that finish
// last; the others keep B.  Both paths add the same products in the same
// order.
template <int VEC, int B, bool NORM>
__global__ __launch_bounds__(64) void zs_fwd_staged_kernel(const float* __restrict__ coupling,
                                                           const float* __restrict__ radial,
                                                           InLayout L,
                                                           const int32_t* __restrict__ rowptr,
                                                           const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ order,
                                                           int64_t heavy, int64_t n_nodes,
                                                           int64_t n_edges, int64_t C,
                                                           float* __restrict__ out, NormIO nio) {
    constexpr int BH = (B == 4 && VEC <= 4) ? 8 : B;
    __shared__ float4 rsh[FwdShape<VEC, BH>::RAD];
    __shared__ float csh[BH * 16];
    if (threadIdx.x < BH) csh[threadIdx.x * 16 + 15] = 0.0f;   // pad column, never fetched
    for (int64_t slot = blockIdx.x; slot < n_nodes; slot += gridDim.x) {
        const int64_t node = node_at(order, slot, n_nodes);
        if (node < 0) continue;
        int64_t k0, k1;
        node_range(rowptr, node, n_edges, k0, k1);
        if (BH != B && k1 - k0 > heavy)
            fwd_staged_node<VEC, BH, NORM>(node, k0, k1, coupling, radial, L, perm, n_edges, C,
                                           out, nio, rsh, csh);
        else
            fwd_staged_node<VEC, B, NORM>(node, k0, k1, coupling, radial, L, perm, n_edges, C,
                                          out, nio, rsh, csh);
    }
}

// ---------------------------------------------------------------------------
// Slot-split forward: a workgroup of three wavefronts per (node, channel tile
// of T = 8*VEC channels).  Wavefront s accumulates the rows of degree
// l = s + 1 (rows l*l .. l*l + 2l, 2l + 1 of them), so it reads only radial
// slot s of each edge (whole 128-byte lines at C = 32) and coupling columns
// l*l - 1 .. l*l + 2l - 1.  Lane = j*8 + q owns row l*l + j (j < 2l + 1) and
// channels q*VEC .. q*VEC+VEC-1 of the tile.  Each wavefront walks the node's
// edges in CSR order with the staged kernel's pipeline (perm entries two
// batches ahead, data one batch ahead, unconditional loads, LDS staging);
// the three wavefronts share the CU's caches for the node's perm entries and
// coupling lines and need no barrier: each stages into its own LDS slice.
// Accumulation order and arithmetic are those of zs_fwd_kernel, so results
// are bitwise those of the other forward kernels.
// ---------------------------------------------------------------------------
template <int VEC, int B>
struct SlotShape {
    static constexpr int T = 8 * VEC;          // channels per tile
    static constexpr int F4 = T / 4;           // float4 per slot row of a tile
    static constexpr int RAD = B * F4;         // radial float4 per batch
    static constexpr int RV = (RAD + 63) / 64;
    static constexpr int CW = B * 8;           // coupling floats per batch: 8 per edge
    static constexpr int CV = (CW + 63) / 64;
};

// One node's slot s (rows of degree s + 1) of the slot-split forward, by the
// calling wavefront (lane = j*8 + q; channel tile blockIdx.y).  rsh / csh:
// this wavefront's LDS staging (SlotShape<VEC, B>::RAD float4 and ::CW
// floats).
template <int VEC, int B, bool NORM>
__device__ __attribute__((always_inline)) inline void fwd_slot_node(
    int64_t node, int s, int64_t k0, int64_t k1, const float* __restrict__ coupling,
    const float* __restrict__ radial, const InLayout& L, const int32_t* __restrict__ perm,
    int64_t n_edges, int64_t C, float* __restrict__ out, const NormIO& nio, float4* rsh,
    float* csh) {
    using S = SlotShape<VEC, B>;
    static_assert(B <= 64, "one perm entry per lane");
    const int lane = threadIdx.x & 63;
    const int l = s + 1;
    const int r0 = l * l;                      // first row of the slot
    const int nr = 2 * l + 1;                  // rows of the slot
    const int q = lane & 7;
    const int j = lane >> 3;
    const int64_t cbase = int64_t(blockIdx.y) * S::T;
    const int64_t c0 = cbase + q * VEC;
    const int n_valid = c0 >= C ? 0 : (C - c0 < VEC ? int(C - c0) : VEC);
    const int64_t slot_off = int64_t(s) * L.rad_slot;
    const int64_t nb = (k1 - k0 + B - 1) / B;

    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
    float deg = 0.0f;

    // Loads of one batch: radial float4 f = i*64 + lane is batch edge
    // f / F4, float4 f % F4 of the tile's slot row; coupling float
    // idx = i*64 + lane is batch edge idx / 8, column idx % 8 of the slot
    // (column 7, never a row of the slot, carries the envelope factor
    // with NORM).  Absent edges, channels and columns read a valid
    // substitute (edge 0, the tile's first channel, the slot's first
    // column) that is never used.
    auto fetch = [&](float4 (&rr)[S::RV], float (&ww)[S::CV], int pe) {
#pragma unroll
        for (int i = 0; i < S::RV; ++i) {
            const int f = i * 64 + lane;
            const int e = __shfl(pe, f < S::RAD ? f / S::F4 : 0, 64);
            const int64_t es = e >= 0 ? e : 0;
            const int64_t ch = cbase + (f % S::F4) * 4;
            const int64_t cs = ch < C ? ch : cbase;
            rr[i] = load_stream4<ZS_FWD_NT != 0>(radial + es * L.rad_edge + slot_off + cs);
        }
#pragma unroll
        for (int i = 0; i < S::CV; ++i) {
            const int idx = i * 64 + lane;
            const int b = idx < S::CW ? idx >> 3 : 0;
            const int col = idx & 7;
            const int e = __shfl(pe, b, 64);
            const int64_t es = e >= 0 ? e : 0;
            const bool in_env = NORM && col == 7;
            ww[i] = in_env ? nio.env[es]
                           : coupling[es * L.cpl_edge + (r0 - 1) + (col < nr ? col : 0)];
        }
    };
    auto stage_accumulate = [&](const float4 (&rr)[S::RV], const float (&ww)[S::CV], int cnt) {
        wave_lds_sync();   // the previous batch's reads come before these writes
#pragma unroll
        for (int i = 0; i < S::RV; ++i)
            if (S::RAD % 64 == 0 || i * 64 + lane < S::RAD) rsh[i * 64 + lane] = rr[i];
#pragma unroll
        for (int i = 0; i < S::CV; ++i)
            if (S::CW % 64 == 0 || i * 64 + lane < S::CW) csh[i * 64 + lane] = ww[i];
        wave_lds_sync();   // every lane reads values other lanes staged
        const float* rf = reinterpret_cast<const float*>(rsh);
        const int jw = j < nr ? j : 0;
        auto edge = [&](int b) {
            if (NORM) deg = deg + csh[b * 8 + 7];
            float x[VEC];
            lds_read<VEC>(rf + b * S::T + q * VEC, x);
            const float w = csh[b * 8 + jw];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float m = w * x[v];
                acc[v] = acc[v] + m;
            }
        };
        if (cnt == B) {
#pragma unroll
            for (int b = 0; b < B; ++b) edge(b);
        } else {
            for (int b = 0; b < cnt; ++b) edge(b);
        }
    };
    auto batch_count = [k0, k1](int64_t t) {
        const int64_t kb = k0 + t * B;
        return int(k1 - kb < B ? k1 - kb : B);
    };

    if (nb > 0) {
        float4 RA[S::RV], RB[S::RV];
        float WA[S::CV], WB[S::CV];
        PermRaw pA = perm_issue(perm, k0, k1, lane, B);
        PermRaw pB = perm_issue(perm, k0 + B, k1, lane, B);
        fetch(RA, WA, perm_resolve(pA, n_edges));
        for (int64_t t = 0; t < nb; t += 2) {
            const PermRaw pN = perm_issue(perm, k0 + (t + 2) * B, k1, lane, B);
            fetch(RB, WB, perm_resolve(pB, n_edges));
            stage_accumulate(RA, WA, batch_count(t));
            if (t + 1 >= nb) break;
            pB = perm_issue(perm, k0 + (t + 3) * B, k1, lane, B);
            fetch(RA, WA, perm_resolve(pN, n_edges));
            stage_accumulate(RB, WB, batch_count(t + 1));
        }
    }

    float zero[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) zero[v] = 0.0f;
    const int64_t row_off = node * kRows * C + c0;
    if (NORM) {
        const float nrm = deg > 0.0f ? 1.0f / sqrtf(deg) : 0.0f;
        if (s == 0 && lane == 0 && blockIdx.y == 0) nio.norm[node] = nrm;
        float y[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) y[v] = acc[v] * nrm;
        if (j < nr) row_store<VEC>(nio.y + row_off + int64_t(r0 + j) * C, y, n_valid);
        else if (s == 0 && j == nr) row_store<VEC>(nio.y + row_off, zero, n_valid);
    }
    if (!NORM || out != nullptr) {
        if (j < nr) row_store<VEC>(out + row_off + int64_t(r0 + j) * C, acc, n_valid);
        else if (s == 0 && j == nr) row_store<VEC>(out + row_off, zero, n_valid);
    }
}

template <int VEC, int B, bool NORM>
__global__ __launch_bounds__(192) void zs_fwd_slot_kernel(const float* __restrict__ coupling,
                                                          const float* __restrict__ radial,
                                                          InLayout L,
                                                          const int32_t* __restrict__ rowptr,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ order,
                                                          int64_t n_nodes, int64_t n_edges,
                                                          int64_t C, float* __restrict__ out,
                                                          NormIO nio) {
    using S = SlotShape<VEC, B>;
    __shared__ float4 rsh_all[kSlots][S::RAD];
    __shared__ float csh_all[kSlots][S::CW];
    const int s = threadIdx.x >> 6;            // slot of this wavefront
    for (int64_t slot = blockIdx.x; slot < n_nodes; slot += gridDim.x) {
        const int64_t node = node_at(order, slot, n_nodes);
        if (node < 0) continue;
        int64_t k0, k1;
        node_range(rowptr, node, n_edges, k0, k1);
        fwd_slot_node<VEC, B, NORM>(node, s, k0, k1, coupling, radial, L, perm, n_edges, C, out,
                                    nio, rsh_all[s], csh_all[s]);
    }
}

template <int VEC, int B>
void launch_slot(const float* coupling, const float* radial, InLayout L, const int32_t* rowptr,
                 const int32_t* perm, const int32_t* order, int64_t n_nodes, int64_t n_edges,
                 int64_t channels, float* out, NormIO nio, unsigned gx, hipStream_t stream) {
    const unsigned gy = unsigned((channels + 8 * VEC - 1) / (8 * VEC));
    if (nio.y != nullptr)
        zs_fwd_slot_kernel<VEC, B, true><<<dim3(gx, gy), 192, 0, stream>>>(
            coupling, radial, L, rowptr, perm, order, n_nodes, n_edges, channels, out, nio);
    else
        zs_fwd_slot_kernel<VEC, B, false><<<dim3(gx, gy), 192, 0, stream>>>(
            coupling, radial, L, rowptr, perm, order, n_nodes, n_edges, channels, out, nio);
}

// Degree above which the staged kernel's 4-edge launches give a node 8-edge
// batches: 5/4 of the mean degree.  Measured (forward, read-flushed caches) on
// the skewed 4096-node frame with the CSR build's node schedule: 69.3 ->
// 65.5 us, and 59.4 -> 58.6 us on a frame of i.i.d. uniform destinations.
// Without a schedule the heavy nodes crowd some compute units and the wider
// batches gain nothing (71.7 us either way).
int64_t heavy_degree(int64_t n_edges, int64_t n_nodes) {
    return n_nodes > 0 ? (5 * n_edges) / (4 * n_nodes) : 0;
}

template <int VEC, int B>
void launch_staged(const float* coupling, const float* radial, InLayout L, const int32_t* rowptr,
                   const int32_t* perm, const int32_t* order, int64_t n_nodes, int64_t n_edges,
                   int64_t channels, float* out, NormIO nio, unsigned gx, hipStream_t stream) {
    const unsigned gy = unsigned((channels + 8 * VEC - 1) / (8 * VEC));
    const int64_t heavy = heavy_degree(n_edges, n_nodes);
    if (nio.y != nullptr)   // env may be NULL when there are no edges
        zs_fwd_staged_kernel<VEC, B, true><<<dim3(gx, gy), 64, 0, stream>>>(
            coupling, radial, L, rowptr, perm, order, heavy, n_nodes, n_edges, channels, out, nio);
    else
        zs_fwd_staged_kernel<VEC, B, false><<<dim3(gx, gy), 64, 0, stream>>>(
            coupling, radial, L, rowptr, perm, order, heavy, n_nodes, n_edges, channels, out, nio);
}

// Edges per batch of the staged kernel, from the number of wavefronts the
// launch provides.  With at least 4 per SIMD (4096), other wavefronts hide
// each one's latency and 4 is best (4096-node frame, C = 32: 55 us, 8 edges
// 57 us, 16 edges slower).  With fewer, a wavefront's own batches must keep
// its loads in flight (8 edges; smaller launches go to the slot-split kernel,
// below).  Batches above 4 edges are used at <= 4 channels per lane, to bound
// the registers.
int forward_batch(int64_t waves, int vec) {
    return (vec > 4 || waves >= 4096) ? 4 : 8;
}

// When a frame gives the one-wavefront-per-tile kernel too few wavefronts to
// keep the memory system busy, the slot-split kernel's three per tile win:
// measured warm on one GPU at 158 edges per node, C = 32: 500 nodes
// 21.1 -> 14.8 us, 1000 nodes 22.7 -> 18.3 us (16-edge batches), 1500 nodes
// 27.1 -> 24.9 us, 2000 nodes 33.6 -> 31.6 us (8-edge batches), 2500 nodes
// and more slower (39.4 -> 40.6 us); C = 64, 1000 nodes 41.2 -> 29.0 us,
// 2000 nodes slower.  Returns the slot kernel's batch, or 0 for the staged
// kernel.
int forward_slot_batch(int64_t waves, int vec) {
    if (waves < 1280) return vec > 4 ? 8 : 16;
    if (vec <= 4 && waves < 2048) return 8;
    return 0;
}

// Channel tiling of the staged forward: one tile of VEC = ceil(C / 8)
// channels per lane up to 64 channels; beyond that, tiles of 64 channels, so
// every tile starts on a 256-byte boundary of a radial row (narrower tiles
// would split 128-byte lines between two wavefronts).
int forward_tile_vec(int64_t channels) {
    return channels > 64 ? 8 : int((channels + 7) / 8);
}

}  // namespace

hipError_t launch_forward(const float* coupling, const float* radial, InLayout L,
                          const int32_t* rowptr, const int32_t* perm, const int32_t* order,
                          int64_t n_nodes, int64_t n_edges, int64_t channels, float* out,
                          bool vec4, NormIO nio, hipStream_t stream) {
    constexpr int64_t kGridCap = 1 << 20;
    const unsigned gx = unsigned(n_nodes < kGridCap ? n_nodes : kGridCap);
    if (vec4) {
#define ZS_FWD_STAGED(V, BB)                                                                     \
    launch_staged<V, BB>(coupling, radial, L, rowptr, perm, order, n_nodes, n_edges, channels, out, \
                         nio, gx, stream)
#define ZS_FWD_STAGED_B(V)                         \
    switch (batch) {                               \
        case 8: ZS_FWD_STAGED(V, 8); break;        \
        default: ZS_FWD_STAGED(V, 4); break;       \
    }
        const int vec = forward_tile_vec(channels);
        const int64_t tiles = (channels + 8 * vec - 1) / (8 * vec);
        const int batch = forward_batch(int64_t(gx) * tiles, vec);
        const int slot_batch = forward_slot_batch(int64_t(gx) * tiles, vec);
        if (slot_batch > 0) {
#define ZS_FWD_SLOT(V)                                                                         \
    do {                                                                                         \
        if (slot_batch == 16)                                                                    \
            launch_slot<V, 16>(coupling, radial, L, rowptr, perm, order, n_nodes, n_edges,      \
                               channels, out, nio, gx, stream);                                  \
        else                                                                                     \
            launch_slot<V, 8>(coupling, radial, L, rowptr, perm, order, n_nodes, n_edges,       \
                              channels, out, nio, gx, stream);                                   \
    } while (0)
            switch (vec) {
                case 1: ZS_FWD_SLOT(1); break;
                case 2: ZS_FWD_SLOT(2); break;
                case 3: ZS_FWD_SLOT(3); break;
                case 4: ZS_FWD_SLOT(4); break;
                case 5: ZS_FWD_SLOT(5); break;
                case 6: ZS_FWD_SLOT(6); break;
                case 7: ZS_FWD_SLOT(7); break;
                default: ZS_FWD_SLOT(8); break;
            }
#undef ZS_FWD_SLOT
            return hipGetLastError();
        }
        switch (vec) {
            case 1: ZS_FWD_STAGED_B(1); break;
            case 2: ZS_FWD_STAGED_B(2); break;
            case 3: ZS_FWD_STAGED_B(3); break;
            case 4: ZS_FWD_STAGED_B(4); break;
            case 5: ZS_FWD_STAGED(5, 4); break;
            case 6: ZS_FWD_STAGED(6, 4); break;
            case 7: ZS_FWD_STAGED(7, 4); break;
            default: ZS_FWD_STAGED(8, 4); break;
        }
#undef ZS_FWD_STAGED_B
#undef ZS_FWD_STAGED
    } else {
        constexpr int NQ = 16, VEC = 1;
        const unsigned gy = unsigned((channels + NQ * VEC - 1) / (NQ * VEC));
        if (nio.y != nullptr)
            zs_fwd_kernel<VEC, NQ, 8, true><<<dim3(gx, gy), 64, 0, stream>>>(
                coupling, radial, L, rowptr, perm, order, n_nodes, n_edges, channels, out, nio);
        else
            zs_fwd_kernel<VEC, NQ, 8, false><<<dim3(gx, gy), 64, 0, stream>>>(
                coupling, radial, L, rowptr, perm, order, n_nodes, n_edges, channels, out, nio);
    }
    return hipGetLastError();
}

}  // namespace zs
