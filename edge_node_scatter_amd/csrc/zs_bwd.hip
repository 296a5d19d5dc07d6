// Fused GIE zonal scatter, backward, gfx950.
//
// deepmd-kit PR #6072 ("fused Triton zonal scatter for the GIE head"), section
// "What", Backward bullet: one edge-parallel kernel returns both operand
// gradients, (E, 15) for the coupling and (E, 3, C) for the radial features,
// without gathering a materialised message gradient.  For edge e with
// n = dst[e] and upstream gradient g = grad_out[n]:
//
//   grad_radial[e][l-1][c] = sum over rows r of degree l of g[r][c] * coupling[e][r-1]
//   grad_coupling[e][r-1]  = sum over c of g[r][c] * radial[e][l(r)-1][c]
//
// Edges are visited grouped by destination (one wavefront per work item, a
// node or a consecutive part of its CSR range), so g[n] is read once per work
// item instead of once per edge.  Within a wavefront, lane = b * NQ + q: b picks one of
// EPW = 64/NQ edges processed side by side, q picks VEC consecutive channels.
// Each lane holds g[n][1..15] for its channels.
//
//  - grad_radial: lane-local, rows of each degree in increasing r, fp32
//    multiply then add from +0 (compiled with -ffp-contract=off).
//  - grad_coupling: the exact fp32 x fp32 products are accumulated in fp64
//    (fma), first over the lane's channels, then across the NQ lanes of the
//    edge by recursive halving (each step trades half of the 16 row sums with
//    the partner lane), and rounded to fp32 once.
#include "zs_internal.h"

namespace zs {

namespace {

// Recursive-halving reduction of 16 row partials over the NQ lanes of an edge.
// Step with partner distance H: the lane keeps the upper or lower half of its
// CNT values (upper when bit H of q is set), sends the other half to lane
// q ^ H and adds what it receives.  After all steps the lane owns rows
// [base, base + 16/NQ), each summed over the NQ lanes in a fixed order.
template <int H, int CNT>
struct Halving {
    __device__ static void run(double (&v)[16], int q, int& base) {
        constexpr int half = CNT / 2;
        const bool up = (q & H) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const double keep = up ? v[i + half] : v[i];
            const double send = up ? v[i] : v[i + half];
            const double recv = __shfl_xor(send, H, 64);
            v[i] = keep + recv;
        }
        if (up) base += half;
        Halving<H / 2, half>::run(v, q, base);
    }
};
template <int CNT>
struct Halving<0, CNT> {
    __device__ static void run(double (&)[16], int, int&) {}
};

template <int NQ>
__device__ inline int reduce_rows(double (&v)[16], int q) {
    int base = 0;
    Halving<NQ / 2, 16>::run(v, q, base);
    return base;
}

template <int VEC, int NQ, bool GREG>
__global__ __launch_bounds__(256) void zs_bwd_kernel(
    const float* __restrict__ grad_out, const float* __restrict__ coupling,
    const float* __restrict__ radial, InLayout L, const int32_t* __restrict__ rowptr,
    const int32_t* __restrict__ perm, int64_t n_nodes, int64_t n_edges, int64_t C,
    float* __restrict__ grad_coupling, float* __restrict__ grad_radial,
    const float* __restrict__ norm) {
    using V = VecT<VEC>;
    using VT = typename V::T;
    constexpr int EPW = 64 / NQ;
    constexpr int WAVES = 4;
    constexpr int STEP = EPW * WAVES;
    constexpr int TW = NQ * VEC;
    constexpr int KEEP = 16 / NQ;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int q = lane % NQ;
    const int b = lane / NQ;
    const int64_t n_tiles = GREG ? 1 : (C + TW - 1) / TW;
    const int64_t row_stride = int64_t(kSlots) * C;

    for (int64_t node = blockIdx.x; node < n_nodes; node += gridDim.x) {
        int64_t k0 = rowptr[node];
        int64_t k1 = rowptr[node + 1];
        k0 = k0 < 0 ? 0 : (k0 > n_edges ? n_edges : k0);
        k1 = k1 < k0 ? k0 : (k1 > n_edges ? n_edges : k1);
        if (k0 >= k1) continue;
        const float* gnode = grad_out + node * kRows * C;
        // upstream rows are grad_out * norm[node] (fp32) when normalised;
        // multiplying by 1.0f otherwise leaves them bit-identical
        const float gs = norm != nullptr ? norm[node] : 1.0f;

        float greg[kZonal][VEC];
        if (GREG) {
            const int64_t c0 = int64_t(q) * VEC;
#pragma unroll
            for (int r = 1; r <= kZonal; ++r) {
                VT t{};
                if (c0 < C) t = V::load(gnode + int64_t(r) * C + c0);
#pragma unroll
                for (int v = 0; v < VEC; ++v) greg[r - 1][v] = c0 < C ? V::get(t, v) * gs : 0.0f;
            }
        }

        for (int64_t kb = k0 + int64_t(wave) * EPW; kb < k1; kb += STEP) {
            const int64_t k = kb + b;
            int32_t e = k < k1 ? perm[k] : -1;
            const bool ok = e >= 0 && e < n_edges;
            if (!ok) e = 0;

            float w[kZonal];
            const float* crow = coupling + int64_t(e) * L.cpl_edge;
#pragma unroll
            for (int i = 0; i < kZonal; ++i) w[i] = ok ? crow[i] : 0.0f;

            double part[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) part[i] = 0.0;

            for (int64_t t = 0; t < n_tiles; ++t) {
                const int64_t c0 = t * TW + int64_t(q) * VEC;
                const bool act = ok && c0 < C;
                float g[kZonal][VEC];
                if (GREG) {
#pragma unroll
                    for (int r = 0; r < kZonal; ++r)
#pragma unroll
                        for (int v = 0; v < VEC; ++v) g[r][v] = greg[r][v];
                } else {
#pragma unroll
                    for (int r = 1; r <= kZonal; ++r) {
                        VT tv{};
                        if (act) tv = V::load(gnode + int64_t(r) * C + c0);
#pragma unroll
                        for (int v = 0; v < VEC; ++v) g[r - 1][v] = act ? V::get(tv, v) * gs : 0.0f;
                    }
                }
                float x[kSlots][VEC];
                const float* rrow = radial + int64_t(e) * L.rad_edge + c0;
#pragma unroll
                for (int s = 0; s < kSlots; ++s) {
                    VT tv{};
                    if (act) tv = V::load(rrow + s * L.rad_slot);
#pragma unroll
                    for (int v = 0; v < VEC; ++v) x[s][v] = act ? V::get(tv, v) : 0.0f;
                }

                // grad_radial: rows of each degree in increasing r.
                float acc[kSlots][VEC];
#pragma unroll
                for (int s = 0; s < kSlots; ++s)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) acc[s][v] = 0.0f;
#pragma unroll
                for (int r = 1; r <= kZonal; ++r)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const float p = g[r - 1][v] * w[r - 1];
                        acc[row_slot(r)][v] = acc[row_slot(r)][v] + p;
                    }
                if (act) {
#pragma unroll
                    for (int s = 0; s < kSlots; ++s)
                        V::store(grad_radial + int64_t(e) * row_stride + s * C + c0, acc[s]);
                }

                // grad_coupling partials: exact products, fp64 accumulation.
#pragma unroll
                for (int r = 1; r <= kZonal; ++r)
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        part[r - 1] = __builtin_fma(double(g[r - 1][v]),
                                                    double(x[row_slot(r)][v]), part[r - 1]);
            }

            const int base = reduce_rows<NQ>(part, q);
            if (ok) {
#pragma unroll
                for (int i = 0; i < KEEP; ++i) {
                    const int idx = base + i;
                    if (idx < kZonal) grad_coupling[int64_t(e) * kZonal + idx] = float(part[i]);
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// Staged backward for C % 4 == 0 with 16-byte aligned grad_out, radial and
// grad_radial, and C <= NQ*VEC with VEC dividing C.  One wavefront per node;
// lane = b*NQ + q handles channels q*VEC .. q*VEC+VEC-1 of edge slot b
// (EPW = 64/NQ edges per step); lanes with q*VEC >= C hold no channels.
//
//  - The node's upstream rows g[n][1..15] are staged in LDS once and re-read
//    every step (holding them and their fp64 conversions in registers across
//    steps would need ~180 registers).
//  - Each step's perm entries are fetched two steps ahead; its radial values
//    (3 x VEC per lane) and its coupling rows (EPW x 15 floats, fetched with
//    coalesced all-distinct loads, at most two per lane) one step ahead into
//    one of two register buffers, so loads overlap the previous step's math.
//    Every load is unconditional (absent edges read a valid substitute), so
//    within a step the compiler waits only for the buffer it consumes; at the
//    head of the step loop it still waits for all loads, because address
//    temporaries reuse registers the prefetch writes (measured harmless at four
//    wavefronts per SIMD, where the other wavefronts keep the memory busy).
//    The coupling floats go through LDS so every lane of an edge gets the
//    edge's 15 weights.
//  - The 15 row sums of grad_coupling are reduced in two rounds (rows 1-8 of
//    degrees 1 and 2, then rows 9-15 of degree 3), 8 values each, by
//    recursive halving with DPP lane exchanges inside each 8- or 16-lane
//    edge group.
// Arithmetic is that of zs_bwd_kernel.
// ---------------------------------------------------------------------------
template <int NQ, int VEC>
struct BwdRegs {
    static constexpr int EPW = 64 / NQ;
    static constexpr int CPL = (EPW * kZonal + 63) / 64;   // coupling floats per lane
    float x[kSlots][VEC];
    float w[CPL];
};

// A step's perm entry (lane's edge slot b), fetched one step before it is
// used.  The load is issued from a valid position (clamped to the node's last
// edge) and range-checked only when used, so it never forces an early wait.
struct PermRaw {
    int32_t raw;
    bool valid;
};

__device__ __attribute__((always_inline)) inline PermRaw bwd_perm_issue(
    const int32_t* __restrict__ perm, int64_t k, int64_t k1) {
    PermRaw p;
    p.valid = k < k1;
    p.raw = perm[p.valid ? k : k1 - 1];
    return p;
}

__device__ __attribute__((always_inline)) inline int bwd_perm_resolve(PermRaw p, int64_t n_edges) {
    return (p.valid && p.raw >= 0 && p.raw < n_edges) ? p.raw : -1;
}

// VEC consecutive read-once floats (radial) with the widest accesses their
// alignment allows; q*VEC floats into 16-byte aligned rows.
template <int VEC, bool NT>
__device__ __attribute__((always_inline)) inline void load_stream_vec(const float* p,
                                                                     float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i) {
            const float4 t = load_stream4<NT>(p + 4 * i);
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
    } else if constexpr (VEC % 2 == 0) {
        typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) {
            const f2 t = NT ? __builtin_nontemporal_load(reinterpret_cast<const f2*>(p) + i)
                            : reinterpret_cast<const f2*>(p)[i];
            v[2 * i] = t.x; v[2 * i + 1] = t.y;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) v[i] = NT ? __builtin_nontemporal_load(p + i) : p[i];
    }
}

template <int VEC, bool NT>
__device__ __attribute__((always_inline)) inline void store_stream_vec(float* p,
                                                                      const float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int i = 0; i < VEC / 4; ++i)
            store_stream4<NT>(p + 4 * i, make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2],
                                                     v[4 * i + 3]));
    } else if constexpr (VEC % 2 == 0) {
        typedef float f2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int i = 0; i < VEC / 2; ++i) {
            f2 t = {v[2 * i], v[2 * i + 1]};
            if (NT)
                __builtin_nontemporal_store(t, reinterpret_cast<f2*>(p) + i);
            else
                reinterpret_cast<f2*>(p)[i] = t;
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            if (NT)
                __builtin_nontemporal_store(v[i], p + i);
            else
                p[i] = v[i];
        }
    }
}

template <int VEC>
__device__ __attribute__((always_inline)) inline void lds_read_vec(const float* p,
                                                                  float (&v)[VEC]) {
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

// Loads of one step, all unconditional: absent edges read edge 0 and lanes
// without channels read channel 0; such values are zeroed (channels) or never
// stored (edges), so they cannot reach a result.
template <int NQ, int VEC>
__device__ __attribute__((always_inline)) inline void bwd_fetch(BwdRegs<NQ, VEC>& R, int e,
                                                                 int lane, bool cact, int64_t c0,
                                                                 const float* __restrict__ coupling,
                                                                 const float* __restrict__ radial,
                                                                 const InLayout& L) {
    constexpr int EPW = BwdRegs<NQ, VEC>::EPW;
    const int64_t es = e >= 0 ? e : 0;
    const int64_t cs = cact ? c0 : 0;
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
        load_stream_vec<VEC, ZS_BWD_NT != 0>(radial + es * L.rad_edge + s * L.rad_slot + cs,
                                             R.x[s]);
#pragma unroll
    for (int i = 0; i < BwdRegs<NQ, VEC>::CPL; ++i) {
        const int idx = i * 64 + lane;               // coupling float of this step
        const bool in = idx < EPW * kZonal;
        const int owner = (in ? idx / kZonal : 0) * NQ;   // a lane of that edge slot
        const int ee = __shfl(e, owner, 64);
        const int64_t ees = ee >= 0 ? ee : 0;
        R.w[i] = coupling[ees * L.cpl_edge + (in ? idx % kZonal : 0)];
    }
}

// Lane exchange of a double inside a 16-lane DPP row.
template <int CTRL>
__device__ __attribute__((always_inline)) inline double dpp_f64(double v) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// DPP controls: partner of lane q (within its aligned group) at halving step H.
//   H = 8: row_mirror (q <-> 15 - q), H = 4: row_half_mirror (q <-> 7 - q),
//   H = 2: quad_perm [2,3,0,1] (q ^ 2), H = 1: quad_perm [1,0,3,2] (q ^ 1).
// Each pairs a lane with bit H set with one that has it clear, so "up" = q & H.
template <int H>
struct PartnerCtrl;
template <> struct PartnerCtrl<8> { static constexpr int v = 0x140; };
template <> struct PartnerCtrl<4> { static constexpr int v = 0x141; };
template <> struct PartnerCtrl<2> { static constexpr int v = 0x4E; };   // [2,3,0,1]
template <> struct PartnerCtrl<1> { static constexpr int v = 0xB1; };   // [1,0,3,2]

template <int H, int CNT>
struct Halving8 {
    __device__ __attribute__((always_inline)) static void run(double (&v)[8], int q, int& base) {
        constexpr int half = CNT / 2;
        const bool up = (q & H) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const double keep = up ? v[i + half] : v[i];
            const double send = up ? v[i] : v[i + half];
            v[i] = keep + dpp_f64<PartnerCtrl<H>::v>(send);
        }
        if (up) base += half;
        Halving8<H / 2, half>::run(v, q, base);
    }
};
template <int CNT>
struct Halving8<0, CNT> {
    __device__ static void run(double (&)[8], int, int&) {}
};

// 8 fp64 row partials -> one row sum per lane, over the NQ lanes of an edge.
template <int NQ>
__device__ __attribute__((always_inline)) inline double reduce8(double (&v)[8], int q, int& base) {
    base = 0;
    if (NQ == 16) {
        Halving8<8, 8>::run(v, q, base);                  // steps 8, 4, 2
        return v[0] + dpp_f64<PartnerCtrl<1>::v>(v[0]);   // both of a pair hold the sum
    } else {
        Halving8<4, 8>::run(v, q, base);                  // steps 4, 2, 1
        return v[0];
    }
}

// grad_radial stores are non-temporal, except with 8 lanes per edge and
// fewer than 4 channels per lane: there each store instruction writes
// 4- or 8-byte pieces of 8 edges' rows, and plain stores, which the L2 merges
// into whole lines, measured faster (4096-node frame, warm / caches flushed:
// C = 24 151 -> 129 / 189 -> 158 us, C = 12 121 -> 114 / 158 -> 128 us,
// C = 8 97 -> 98 / 129 -> 106 us); with 16 lanes per edge (C = 48) they were
// slower (190 -> 224 us warm).
template <int NQ, int VEC>
constexpr bool kBwdStoreNT = ZS_BWD_NT != 0 && (NQ != 8 || VEC % 4 == 0);

// gsh: the node's upstream rows 1..15, T = NQ*VEC floats each (zero past C).
template <int NQ, int VEC, bool FULL>
__device__ __attribute__((always_inline)) inline void bwd_compute(
    const BwdRegs<NQ, VEC>& R, int e, int lane, int b, bool cact, int64_t c0, int q,
    const float* gsh, float* wsh, int64_t C, float* __restrict__ grad_coupling,
    float* __restrict__ grad_radial) {
    constexpr int EPW = BwdRegs<NQ, VEC>::EPW;
    constexpr int T = NQ * VEC;
    // stage this step's coupling rows, then read the 15 weights of edge slot b
    wave_lds_sync();   // the previous step's reads come before these writes
#pragma unroll
    for (int i = 0; i < BwdRegs<NQ, VEC>::CPL; ++i) {
        const int idx = i * 64 + lane;
        if (idx < EPW * kZonal) wsh[(idx / kZonal) * 16 + idx % kZonal] = R.w[i];
    }
    wave_lds_sync();   // each lane reads the rows other lanes staged
    float w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 t = reinterpret_cast<const float4*>(wsh + b * 16)[i];
        w[4 * i] = t.x; w[4 * i + 1] = t.y; w[4 * i + 2] = t.z; w[4 * i + 3] = t.w;
    }
    const bool ok = e >= 0;
    const bool act = ok && cact;
    const int64_t row_stride = int64_t(kSlots) * C;
    float x[kSlots][VEC];   // lanes without channels contribute exact zeros to the channel sums
#pragma unroll
    for (int s = 0; s < kSlots; ++s)
#pragma unroll
        for (int v = 0; v < VEC; ++v) x[s][v] = (FULL || cact) ? R.x[s][v] : 0.0f;
    float* grow = grad_radial + int64_t(ok ? e : 0) * row_stride + c0;
    float* gcrow = grad_coupling + int64_t(ok ? e : 0) * kZonal;
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        // Re-read the staged rows every step (see above).
        __asm__ volatile("" ::: "memory");
        const int r_lo = round == 0 ? 1 : 9;
        const int r_hi = round == 0 ? 8 : 15;
        double part[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) part[i] = 0.0;
        float acc[kSlots][VEC];
#pragma unroll
        for (int s = 0; s < kSlots; ++s)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[s][v] = 0.0f;
#pragma unroll
        for (int r = r_lo; r <= r_hi; ++r) {
            float g[VEC];
            lds_read_vec<VEC>(gsh + (r - 1) * T + q * VEC, g);
            const int s = row_slot(r);
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const float p = g[v] * w[r - 1];
                acc[s][v] = acc[s][v] + p;
                part[r - r_lo] = __builtin_fma(double(g[v]), double(x[s][v]), part[r - r_lo]);
            }
        }
        if (act) {
#pragma unroll
            for (int s = 0; s < kSlots; ++s)
                if (row_slot(r_lo) <= s && s <= row_slot(r_hi))
                    store_stream_vec<VEC, kBwdStoreNT<NQ, VEC>>(grow + s * C, acc[s]);
        }
        int base;
        const double sum = reduce8<NQ>(part, q, base);
        const int col = r_lo - 1 + base;
        if (ok && col <= r_hi - 1 && (NQ == 8 || (q & 1) == 0)) gcrow[col] = float(sum);
    }
}

// Occupancy request for the staged backward: 4 wavefronts per SIMD (<= 128
// VGPRs) for the common shapes whose registers fit; the others are left to
// the compiler rather than spill.
#ifndef ZS_BWD_WAVES_PER_EU
#define ZS_BWD_WAVES_PER_EU 4
#endif

template <int NQ, int VEC, bool FULL>
struct BwdOccupancy {
    static constexpr int v = (FULL && VEC <= 4) ? ZS_BWD_WAVES_PER_EU : 1;
};

// Largest number of work items a node is split into, and the edges per item
// that a split aims at (both compile-time, so their divisions are cheap).  Measured (backward alone, same GPU, warm / flushed):
// skewed degrees 157 -> 137 us, 1000-node frame 41 -> 36 us, 16384-node frame
// 966 -> 932 us, uniform 4096-node frame 122 -> 123 us warm and 150 -> 146 us
// cold, against no splitting.
#ifndef ZS_BWD_MAX_PARTS
#define ZS_BWD_MAX_PARTS 4
#endif
constexpr int kBwdMaxParts = ZS_BWD_MAX_PARTS;
#ifndef ZS_BWD_PART_EDGES
#define ZS_BWD_PART_EDGES 40
#endif
constexpr uint32_t kBwdPartEdges = ZS_BWD_PART_EDGES;
// Slots between consecutive parts of a node (see the work-item loop).  When
// the grid is resident at once, the dispatcher places workgroups on compute
// units in a fixed round-robin, so with parts numbered part-major a node's
// parts would share slot position and compute unit, and a compute unit's load
// would be the summed degrees of its own few nodes, four times over.  Shifting
// each part by 8 slots (a multiple of the XCD count, so the node's upstream
// rows stay in one XCD's L2) gives each compute unit four different node sets.
// Measured (backward alone, warm / read-flushed): skewed degrees
// 136.5 / 136.4 -> 127.6 / 127.8 us; uniform 4096- and 1000-node frames
// unchanged.  A shift of 1 (parts on different XCDs) gives the skewed frame
// 129 us and costs the 1000-node frame 1.5 us (upstream rows fetched by
// several XCDs).
constexpr int64_t kBwdPartShift = 8;

// Start of part p of a node's len edges split into `parts` (p = parts: len),
// in whole steps of STEP edges (the edges one step of the wavefront takes):
// the node's ceil(len / STEP) steps are dealt so that the first (steps mod
// parts) parts take one step more than the others.  Interior points are
// multiples of STEP, so only the last part ends with a partly filled step,
// and since parts are dispatched part-major, a node's shorter parts are the
// ones that run last (a per-item timeline of the Poisson-degree frame showed
// the kernel ending on late 6-step last parts).  32-bit divisions by constants.
template <uint32_t STEP>
__device__ __attribute__((always_inline)) inline uint32_t split_point(uint32_t len, uint32_t p,
                                                                      uint32_t parts) {
    if (p == 0) return 0;
    if (p >= parts) return len;
    const uint32_t steps = (len + STEP - 1) / STEP;
    uint32_t q, r;
    switch (parts) {
        case 2: q = steps / 2; r = steps % 2; break;
        case 3: q = steps / 3; r = steps % 3; break;
        case 4: q = steps / 4; r = steps % 4; break;
        default: q = steps / parts; r = steps % parts; break;
    }
    const uint32_t at = (p * q + (p < r ? p : r)) * STEP;
    return at < len ? at : len;
}

// FULL: C == NQ*VEC, every lane holds real channels (no channel masking).
template <int NQ, int VEC, bool FULL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(BwdOccupancy<NQ, VEC, FULL>::v)))
void zs_bwd_staged_kernel(
    const float* __restrict__ grad_out, const float* __restrict__ coupling,
    const float* __restrict__ radial, InLayout L, const int32_t* __restrict__ rowptr,
    const int32_t* __restrict__ perm, int64_t n_nodes, int64_t n_edges, int64_t C,
    float* __restrict__ grad_coupling, float* __restrict__ grad_radial, NormGrad ng) {
    constexpr int EPW = 64 / NQ;
    constexpr int T = NQ * VEC;
    static_assert(T % 4 == 0, "the upstream rows are staged as float4");
    __shared__ float4 gsh4[kZonal * T / 4];
    __shared__ float4 wsh4[EPW * 4];
    float* gsh = reinterpret_cast<float*>(gsh4);
    float* wsh = reinterpret_cast<float*>(wsh4);
    const int lane = threadIdx.x;
    const int q = lane % NQ;
    const int b = lane / NQ;
    const int64_t c0 = int64_t(q) * VEC;
    const bool cact = FULL || c0 < C;
    if (lane < EPW) wsh[lane * 16 + 15] = 0.0f;     // pad column, never fetched

    // Work item = (node, part), kBwdMaxParts items per node: a node of degree
    // d is split into min(kBwdMaxParts, ceil(d / kBwdPartEdges)) consecutive
    // pieces (edges are independent here) and the items past that exit at
    // once.  High-degree nodes so become several work items of similar size,
    // which the dispatcher balances across the SIMDs.  Items are numbered
    // part-major (item = part * N + slot): workgroups are handed to the XCDs
    // round-robin, so consecutive items must not share a part index.  Slot s
    // of part p takes node (s + kBwdPartShift * p) mod N, a bijection per part.
    for (int64_t item = blockIdx.x; item < n_nodes * kBwdMaxParts; item += gridDim.x) {
        int64_t node = item;
        int part = 0;
        while (node >= n_nodes) {   // at most kBwdMaxParts - 1 steps
            node -= n_nodes;
            ++part;
        }
        node += int64_t(part) * kBwdPartShift;
        if (node >= n_nodes) node %= n_nodes;
        int64_t k0 = rowptr[node];
        int64_t k1 = rowptr[node + 1];
        k0 = k0 < 0 ? 0 : (k0 > n_edges ? n_edges : k0);
        k1 = k1 < k0 ? k0 : (k1 > n_edges ? n_edges : k1);
        {
            // 32-bit arithmetic (CSR positions are int32) with constant divisors
            const uint32_t len = uint32_t(k1 - k0);
            uint32_t parts = len / kBwdPartEdges + (len % kBwdPartEdges != 0);
            parts = parts < 1 ? 1 : (parts > kBwdMaxParts ? kBwdMaxParts : parts);
            if (uint32_t(part) >= parts) continue;
            const int64_t base = k0;
            k0 = base + split_point<EPW>(len, uint32_t(part), parts);
            k1 = base + split_point<EPW>(len, uint32_t(part) + 1, parts);
        }
        const bool deg = ng.grad_deg != nullptr && part == 0;   // also form the degree gradient
        if (k0 >= k1 && !deg) continue;
        const float* gnode = grad_out + node * kRows * C;
        const float gs = ng.norm != nullptr ? ng.norm[node] : 1.0f;   // see zs_bwd_kernel
        // Prologue in issue order: the first two steps' perm entries, then the
        // node's upstream rows (rows 1..15 of the tile, float4 i = u*64 + lane,
        // into registers), then the first step's operands; only then are the
        // rows written to LDS, so the three round trips overlap (the degree
        // gradient's out rows are read while the rows are written).  Lanes
        // past the rows or channels load row 1's first float4 (always present)
        // and stage zeros.
        const bool has_edges = k0 < k1;
        PermRaw qA{0, false}, qB{0, false};
        if (has_edges) {
            qA = bwd_perm_issue(perm, k0 + b, k1);
            qB = bwd_perm_issue(perm, k0 + EPW + b, k1);
        }
        constexpr int kStageF4 = kZonal * T / 4;
        constexpr int kStage = (kStageF4 + 63) / 64;
        float4 gv[kStage];
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const int i = u * 64 + lane;
            const int64_t c = int64_t(i % (T / 4)) * 4;
            const bool ok = i < kStageF4 && c < C;
            gv[u] = *reinterpret_cast<const float4*>(
                gnode + (ok ? int64_t(i / (T / 4) + 1) * C + c : C));
        }
        BwdRegs<NQ, VEC> A, B;
        int eA = -1;
        if (has_edges) {
            eA = bwd_perm_resolve(qA, n_edges);
            bwd_fetch<NQ, VEC>(A, eA, lane, cact, c0, coupling, radial, L);
        }
        double s = 0.0;   // degree gradient: sum of grad_out * out over rows 1..15
        wave_lds_sync();   // the previous item's reads of the rows come before these writes
#pragma unroll
        for (int u = 0; u < kStage; ++u) {
            const int i = u * 64 + lane;
            if (kStageF4 % 64 != 0 && i >= kStageF4) continue;
            const int64_t c = int64_t(i % (T / 4)) * 4;
            float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (c < C) {
                v = gv[u];
                if (deg) {
                    const float4 o = *reinterpret_cast<const float4*>(
                        ng.out + (node * kRows + i / (T / 4) + 1) * C + c);
                    s = __builtin_fma(double(v.x), double(o.x), s);
                    s = __builtin_fma(double(v.y), double(o.y), s);
                    s = __builtin_fma(double(v.z), double(o.z), s);
                    s = __builtin_fma(double(v.w), double(o.w), s);
                }
                v.x = v.x * gs; v.y = v.y * gs; v.z = v.z * gs; v.w = v.w * gs;
            }
            gsh4[i] = v;
        }
        wave_lds_sync();   // every lane reads rows other lanes staged
        if (deg) {
#pragma unroll
            for (int h = 32; h >= 1; h >>= 1) s = s + __shfl_xor(s, h, 64);
            if (lane == 0) {
                const double t = ng.norm[node];
                ng.grad_deg[node] = t == 0.0 ? 0.0f : float(-0.5 * t * t * t * s);
            }
        }
        if (!has_edges) continue;
        const int64_t nsteps = (k1 - k0 + EPW - 1) / EPW;
        for (int64_t t = 0; t < nsteps; t += 2) {
            const PermRaw qN = bwd_perm_issue(perm, k0 + (t + 2) * EPW + b, k1);
            const int eB = bwd_perm_resolve(qB, n_edges);
            bwd_fetch<NQ, VEC>(B, eB, lane, cact, c0, coupling, radial, L);
            bwd_compute<NQ, VEC, FULL>(A, eA, lane, b, cact, c0, q, gsh, wsh, C, grad_coupling,
                                       grad_radial);
            if (t + 1 >= nsteps) break;
            qB = bwd_perm_issue(perm, k0 + (t + 3) * EPW + b, k1);
            eA = bwd_perm_resolve(qN, n_edges);
            bwd_fetch<NQ, VEC>(A, eA, lane, cact, c0, coupling, radial, L);
            bwd_compute<NQ, VEC, FULL>(B, eB, lane, b, cact, c0, q, gsh, wsh, C, grad_coupling,
                                       grad_radial);
        }
    }
}

// Lane layout of the staged backward for a channel count (C % 4 == 0):
// NQ lanes per edge and VEC channels per lane with VEC dividing C, so every
// lane holds all or none of its channels.  Layouts with at most 4 channels
// per lane come first (8 lanes per edge, then 16): wider lanes need more than
// 128 registers, and the lower occupancy costs more than idle lanes do.
// Returns false when C needs more than 16 lanes of at most 8 channels.
bool backward_layout(int64_t C, int& nq, int& vec) {
    for (int n : {8, 16})
        for (int v = 1; v <= 4; ++v)
            if (n * v >= C && C % v == 0) {
                nq = n;
                vec = v;
                return true;
            }
    for (int v = 5; v <= 8; ++v)
        if (16 * v >= C && C % v == 0) {
            nq = 16;
            vec = v;
            return true;
        }
    return false;
}

}  // namespace

hipError_t launch_backward(const float* grad_out, const float* coupling, const float* radial,
                           InLayout L, const int32_t* rowptr, const int32_t* perm,
                           int64_t n_nodes, int64_t n_edges,
                           int64_t channels, float* grad_coupling, float* grad_radial, bool vec4,
                           NormGrad ng, bool* deg_done, hipStream_t stream) {
    const float* norm = ng.norm;
    if (deg_done) *deg_done = false;
    constexpr int64_t kGridCap = 1 << 20;
    const unsigned gx = unsigned(n_nodes < kGridCap ? n_nodes : kGridCap);
#define ZS_BWD_LAUNCH(VEC, NQ, GREG)                                                            \
    zs_bwd_kernel<VEC, NQ, GREG><<<gx, 256, 0, stream>>>(grad_out, coupling, radial, L, rowptr,  \
                                                         perm, n_nodes, n_edges, channels,       \
                                                         grad_coupling, grad_radial, norm)
#define ZS_BWD_STAGED(NQ, VEC)                                                                  \
    do {                                                                                         \
        if (channels == (NQ) * (VEC))                                                            \
            zs_bwd_staged_kernel<NQ, VEC, true><<<gxp, 64, 0, stream>>>(                         \
                grad_out, coupling, radial, L, rowptr, perm, n_nodes, n_edges, channels,         \
                grad_coupling, grad_radial, ng);                                          \
        else                                                                                     \
            zs_bwd_staged_kernel<NQ, VEC, false><<<gxp, 64, 0, stream>>>(                        \
                grad_out, coupling, radial, L, rowptr, perm, n_nodes, n_edges, channels,         \
                grad_coupling, grad_radial, ng);                                          \
        if (deg_done) *deg_done = ng.grad_deg != nullptr;                                        \
    } while (0)
    const int64_t items = n_nodes * kBwdMaxParts;
    const unsigned gxp = unsigned(items < kGridCap ? items : kGridCap);
    int nq = 0, vec = 0;
    if (vec4 && backward_layout(channels, nq, vec)) {
        switch (nq * 16 + vec) {
            case 8 * 16 + 1: ZS_BWD_STAGED(8, 1); break;
            case 8 * 16 + 2: ZS_BWD_STAGED(8, 2); break;
            case 8 * 16 + 3: ZS_BWD_STAGED(8, 3); break;
            case 8 * 16 + 4: ZS_BWD_STAGED(8, 4); break;
            case 16 * 16 + 3: ZS_BWD_STAGED(16, 3); break;
            case 16 * 16 + 4: ZS_BWD_STAGED(16, 4); break;
            case 16 * 16 + 5: ZS_BWD_STAGED(16, 5); break;
            case 16 * 16 + 6: ZS_BWD_STAGED(16, 6); break;
            case 16 * 16 + 7: ZS_BWD_STAGED(16, 7); break;
            default: ZS_BWD_STAGED(16, 8); break;
        }
    } else if (vec4) {
        ZS_BWD_LAUNCH(4, 16, false);
    } else {
        if (channels <= 16)
            ZS_BWD_LAUNCH(1, 16, true);
        else
            ZS_BWD_LAUNCH(1, 16, false);
    }
#undef ZS_BWD_STAGED
#undef ZS_BWD_LAUNCH
    return hipGetLastError();
}

}  // namespace zs
