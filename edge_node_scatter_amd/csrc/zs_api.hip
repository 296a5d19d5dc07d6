// C ABI of libzs (declared in include/zs.h): argument checks on the host, then
// kernel dispatch.  Every check runs before the first HIP call, so a rejected
// call leaves device state untouched.
#include "zs.h"

#include <mutex>

#include "zs_csr.h"
#include "zs_internal.h"

namespace {

// Scratch of zs_build_csr_noalloc: one copy per device, created with the code
// object.  Host code never uses this name as an address (on the host it is a
// stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[ZS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // guarded by g_scratch_mutex

// Device address of the current device's scratch; NULL if HIP fails.
void* noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

struct Range {
    uintptr_t lo, hi;   // [lo, hi)
};

Range span(const void* p, int64_t count, size_t elem) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + uintptr_t(count) * elem};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool sizes_ok(int64_t n_edges, int64_t n_nodes) {
    return n_edges >= 0 && n_edges <= ZS_MAX_EDGES && n_nodes >= 1 && n_nodes <= ZS_MAX_NODES;
}

bool channels_ok(int64_t c) { return c >= 1 && c <= ZS_MAX_CHANNELS; }

int hip_status(hipError_t e) { return e == hipSuccess ? ZS_OK : ZS_ERR_HIP; }

}  // namespace

extern "C" {

const char* zs_status_string(int status) {
    switch (status) {
        case ZS_OK: return "ok";
        case ZS_ERR_NULL: return "a required pointer is NULL";
        case ZS_ERR_SHAPE: return "a size is out of the supported range";
        case ZS_ERR_INDEX: return "a destination index is outside [0, n_nodes)";
        case ZS_ERR_UNSUPPORTED: return "a pointer is not aligned to its element size";
        case ZS_ERR_ALIAS: return "an output overlaps an input or another output";
        case ZS_ERR_WORKSPACE: return "workspace is NULL or too small";
        case ZS_ERR_HIP: return "a HIP runtime call failed";
        case ZS_ERR_SCRATCH:
            return "the sizes need more scratch than the library's fixed device buffer holds";
        default: return "unknown status";
    }
}

size_t zs_csr_workspace_bytes(int64_t n_edges, int64_t n_nodes) {
    if (!sizes_ok(n_edges, n_nodes)) return 0;
    return zs::plan_csr(n_edges, n_nodes).bytes;
}

}  // extern "C"

namespace {

// Host-side checks of the CSR build's buffers (not the workspace).
int csr_args(const int64_t* dst, int64_t n_edges, int64_t n_nodes, const int32_t* rowptr,
             const int32_t* perm, const int32_t* dst32, const int32_t* order,
             const int32_t* bad_flag) {
    if (!sizes_ok(n_edges, n_nodes)) return ZS_ERR_SHAPE;
    if (!rowptr || (n_edges > 0 && (!dst || !perm || !dst32))) return ZS_ERR_NULL;
    if (!aligned(rowptr, 4) || (n_edges > 0 && (!aligned(dst, 8) || !aligned(perm, 4) ||
                                                !aligned(dst32, 4))))
        return ZS_ERR_UNSUPPORTED;
    if ((bad_flag && !aligned(bad_flag, 4)) || (order && !aligned(order, 4)))
        return ZS_ERR_UNSUPPORTED;
    const Range r_dst = span(dst, n_edges, 8), r_rowptr = span(rowptr, n_nodes + 1, 4),
                r_perm = span(perm, n_edges, 4), r_dst32 = span(dst32, n_edges, 4),
                r_flag = span(bad_flag, bad_flag ? 1 : 0, 4),
                r_order = span(order, order ? n_nodes : 0, 4);
    if (overlap(r_rowptr, r_dst) || overlap(r_perm, r_dst) || overlap(r_dst32, r_dst) ||
        overlap(r_rowptr, r_perm) || overlap(r_rowptr, r_dst32) || overlap(r_perm, r_dst32) ||
        overlap(r_flag, r_dst) || overlap(r_flag, r_rowptr) || overlap(r_flag, r_perm) ||
        overlap(r_flag, r_dst32) || overlap(r_order, r_dst) || overlap(r_order, r_rowptr) ||
        overlap(r_order, r_perm) || overlap(r_order, r_dst32) || overlap(r_order, r_flag))
        return ZS_ERR_ALIAS;
    return ZS_OK;
}

// The build on checked arguments.  With n_edges > 0 the workspace holds at
// least plan.bytes and overlaps none of the buffers.
int csr_run(const int64_t* dst, int64_t n_edges, int64_t n_nodes, int32_t* rowptr,
            int32_t* perm, int32_t* dst32, int32_t* order, void* workspace, int32_t* bad_flag,
            hipStream_t s) {
    if (n_edges == 0) {
        hipError_t err = zs::launch_fill_i32(rowptr, n_nodes + 1, 0, s);
        if (err == hipSuccess && bad_flag) err = zs::launch_fill_i32(bad_flag, 1, 0, s);
        if (err == hipSuccess && order) err = zs::launch_iota_i32(order, n_nodes, s);
        return hip_status(err);
    }
    const zs::CsrPlan plan = zs::plan_csr(n_edges, n_nodes);
    hipError_t err = zs::launch_csr(dst, n_edges, n_nodes, rowptr, perm, dst32, order, workspace,
                                    plan, bad_flag, s);
    if (err != hipSuccess) return ZS_ERR_HIP;
    if (bad_flag) return ZS_OK;
    int32_t flag = 0;
    const int32_t* dflag = reinterpret_cast<const int32_t*>(static_cast<char*>(workspace) +
                                                            plan.off_flag);
    if (hipMemcpyAsync(&flag, dflag, sizeof(flag), hipMemcpyDeviceToHost, s) != hipSuccess)
        return ZS_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return ZS_ERR_HIP;
    return flag ? ZS_ERR_INDEX : ZS_OK;
}

}  // namespace

extern "C" {

int zs_build_csr(const int64_t* dst, int64_t n_edges, int64_t n_nodes, int32_t* rowptr,
                 int32_t* perm, int32_t* dst32, int32_t* order, void* workspace,
                 size_t workspace_bytes, int32_t* bad_flag, void* stream) {
    const int st = csr_args(dst, n_edges, n_nodes, rowptr, perm, dst32, order, bad_flag);
    if (st != ZS_OK) return st;
    if (n_edges > 0) {
        const zs::CsrPlan plan = zs::plan_csr(n_edges, n_nodes);
        if (!workspace || workspace_bytes < plan.bytes) return ZS_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return ZS_ERR_UNSUPPORTED;
        const Range r_ws = span(workspace, int64_t(plan.bytes), 1);
        if (overlap(r_ws, span(dst, n_edges, 8)) || overlap(r_ws, span(rowptr, n_nodes + 1, 4)) ||
            overlap(r_ws, span(perm, n_edges, 4)) || overlap(r_ws, span(dst32, n_edges, 4)) ||
            overlap(r_ws, span(bad_flag, bad_flag ? 1 : 0, 4)) ||
            overlap(r_ws, span(order, order ? n_nodes : 0, 4)))
            return ZS_ERR_ALIAS;
    }
    return csr_run(dst, n_edges, n_nodes, rowptr, perm, dst32, order, workspace, bad_flag,
                   static_cast<hipStream_t>(stream));
}

int zs_build_csr_noalloc(const int64_t* dst, int64_t n_edges, int64_t n_nodes,
                         int32_t* rowptr, int32_t* perm, int32_t* dst32, int32_t* order,
                         int32_t* bad_flag, void* stream) {
    const int st = csr_args(dst, n_edges, n_nodes, rowptr, perm, dst32, order, bad_flag);
    if (st != ZS_OK) return st;
    void* ws = nullptr;
    if (n_edges > 0) {
        if (zs::plan_csr(n_edges, n_nodes).bytes > size_t(ZS_NOALLOC_SCRATCH_BYTES))
            return ZS_ERR_SCRATCH;
        ws = noalloc_scratch();   // first call on this device: symbol lookup, no allocation
        if (ws == nullptr) return ZS_ERR_HIP;
    }
    return csr_run(dst, n_edges, n_nodes, rowptr, perm, dst32, order, ws, bad_flag,
                   static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// Largest extent, in floats, of a strided input view (2^60: the view's byte
// extent and every index the kernels form stay far inside int64).
constexpr int64_t kMaxExtent = int64_t(1) << 60;

// Floats spanned by E edges of the strided inputs, or -1 when that extent
// overflows or exceeds kMaxExtent.
int64_t view_extent(int64_t E, int64_t edge_stride, int64_t tail) {
    if (E <= 0) return 0;
    int64_t x = 0;
    if (__builtin_mul_overflow(E - 1, edge_stride, &x) || __builtin_add_overflow(x, tail, &x) ||
        x > kMaxExtent)
        return -1;
    return x;
}
int64_t cpl_extent(int64_t E, int64_t cs) { return view_extent(E, cs, zs::kZonal); }
int64_t rad_extent(int64_t E, int64_t re, int64_t rs, int64_t C) {
    if (rs > kMaxExtent) return -1;
    return view_extent(E, re, 2 * rs + C);
}

// Strided input layouts: any non-negative strides (inputs are only read, so
// overlapping or broadcast rows are harmless) whose views span at most
// kMaxExtent floats.
bool layout_ok(int64_t E, int64_t cs, int64_t re, int64_t rs, int64_t C) {
    return cs >= 0 && re >= 0 && rs >= 0 && cpl_extent(E, cs) >= 0 &&
           rad_extent(E, re, rs, C) >= 0;
}

int forward_impl(const float* coupling, int64_t cs, const float* radial, int64_t re, int64_t rs,
                 const int32_t* rowptr, const int32_t* perm, const int32_t* order,
                 int64_t n_nodes, int64_t n_edges, int64_t channels, float* out, void* stream) {
    if (!sizes_ok(n_edges, n_nodes) || !channels_ok(channels)) return ZS_ERR_SHAPE;
    if (!layout_ok(n_edges, cs, re, rs, channels)) return ZS_ERR_SHAPE;
    if (!out || !rowptr || (n_edges > 0 && (!coupling || !radial || !perm))) return ZS_ERR_NULL;
    if (!aligned(out, 4) || !aligned(rowptr, 4) || (order && !aligned(order, 4)) ||
        (n_edges > 0 && (!aligned(coupling, 4) || !aligned(radial, 4) || !aligned(perm, 4))))
        return ZS_ERR_UNSUPPORTED;
    const Range r_out = span(out, n_nodes * zs::kRows * channels, 4);
    if (overlap(r_out, span(coupling, cpl_extent(n_edges, cs), 4)) ||
        overlap(r_out, span(radial, rad_extent(n_edges, re, rs, channels), 4)) ||
        overlap(r_out, span(rowptr, n_nodes + 1, 4)) || overlap(r_out, span(perm, n_edges, 4)) ||
        overlap(r_out, span(order, order ? n_nodes : 0, 4)))
        return ZS_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool vec4 = channels % 4 == 0 && aligned(out, 16) &&
                      (n_edges == 0 || (aligned(radial, 16) && re % 4 == 0 && rs % 4 == 0));
    return hip_status(zs::launch_forward(coupling, radial, zs::InLayout{cs, re, rs}, rowptr, perm,
                                         order, n_nodes, n_edges, channels, out, vec4,
                                         zs::NormIO{nullptr, nullptr, nullptr}, s));
}

int backward_impl(const float* grad_out, const float* coupling, int64_t cs, const float* radial,
                  int64_t re, int64_t rs, const int32_t* dst32, const int32_t* rowptr,
                  const int32_t* perm, int64_t n_nodes, int64_t n_edges, int64_t channels,
                  float* grad_coupling, float* grad_radial, void* stream) {
    if (!sizes_ok(n_edges, n_nodes) || !channels_ok(channels)) return ZS_ERR_SHAPE;
    if (!layout_ok(n_edges, cs, re, rs, channels)) return ZS_ERR_SHAPE;
    if (n_edges == 0) return ZS_OK;   // both gradients are empty
    if (!grad_out || !coupling || !radial || !dst32 || !rowptr || !perm || !grad_coupling ||
        !grad_radial)
        return ZS_ERR_NULL;
    if (!aligned(grad_out, 4) || !aligned(coupling, 4) || !aligned(radial, 4) ||
        !aligned(dst32, 4) || !aligned(rowptr, 4) || !aligned(perm, 4) ||
        !aligned(grad_coupling, 4) || !aligned(grad_radial, 4))
        return ZS_ERR_UNSUPPORTED;
    const Range r_gc = span(grad_coupling, n_edges * zs::kZonal, 4);
    const Range r_gr = span(grad_radial, n_edges * zs::kSlots * channels, 4);
    const Range ins[] = {span(grad_out, n_nodes * zs::kRows * channels, 4),
                         span(coupling, cpl_extent(n_edges, cs), 4),
                         span(radial, rad_extent(n_edges, re, rs, channels), 4),
                         span(dst32, n_edges, 4), span(rowptr, n_nodes + 1, 4),
                         span(perm, n_edges, 4)};
    if (overlap(r_gc, r_gr)) return ZS_ERR_ALIAS;
    for (const Range& in : ins)
        if (overlap(r_gc, in) || overlap(r_gr, in)) return ZS_ERR_ALIAS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool vec4 = channels % 4 == 0 && aligned(grad_out, 16) && aligned(radial, 16) &&
                      aligned(grad_radial, 16) && re % 4 == 0 && rs % 4 == 0;
    return hip_status(zs::launch_backward(grad_out, coupling, radial, zs::InLayout{cs, re, rs},
                                          rowptr, perm, n_nodes, n_edges, channels,
                                          grad_coupling, grad_radial, vec4,
                                          zs::NormGrad{nullptr, nullptr, nullptr}, nullptr, s));
}

}  // namespace

extern "C" {

int zs_forward(const float* coupling, const float* radial, const int32_t* rowptr,
               const int32_t* perm, const int32_t* order, int64_t n_nodes, int64_t n_edges,
               int64_t channels, float* out, void* stream) {
    return forward_impl(coupling, zs::kZonal, radial, zs::kSlots * channels, channels, rowptr,
                        perm, order, n_nodes, n_edges, channels, out, stream);
}

int zs_forward_strided(const float* coupling, int64_t coupling_edge_stride, const float* radial,
                       int64_t radial_edge_stride, int64_t radial_slot_stride,
                       const int32_t* rowptr, const int32_t* perm, const int32_t* order,
                       int64_t n_nodes, int64_t n_edges, int64_t channels, float* out,
                       void* stream) {
    return forward_impl(coupling, coupling_edge_stride, radial, radial_edge_stride,
                        radial_slot_stride, rowptr, perm, order, n_nodes, n_edges, channels, out,
                        stream);
}

int zs_backward(const float* grad_out, const float* coupling, const float* radial,
                const int32_t* dst32, const int32_t* rowptr, const int32_t* perm, int64_t n_nodes,
                int64_t n_edges, int64_t channels, float* grad_coupling, float* grad_radial,
                void* stream) {
    return backward_impl(grad_out, coupling, zs::kZonal, radial, zs::kSlots * channels, channels,
                         dst32, rowptr, perm, n_nodes, n_edges, channels, grad_coupling,
                         grad_radial, stream);
}

int zs_backward_strided(const float* grad_out, const float* coupling,
                        int64_t coupling_edge_stride, const float* radial,
                        int64_t radial_edge_stride, int64_t radial_slot_stride,
                        const int32_t* dst32, const int32_t* rowptr, const int32_t* perm,
                        int64_t n_nodes, int64_t n_edges, int64_t channels, float* grad_coupling,
                        float* grad_radial, void* stream) {
    return backward_impl(grad_out, coupling, coupling_edge_stride, radial, radial_edge_stride,
                         radial_slot_stride, dst32, rowptr, perm, n_nodes, n_edges, channels,
                         grad_coupling, grad_radial, stream);
}

int zs_forward_normalized(const float* coupling, const float* radial, const float* env,
                          const int32_t* rowptr, const int32_t* perm, const int32_t* order,
                          int64_t n_nodes, int64_t n_edges, int64_t channels, float* y,
                          float* out, float* norm, void* stream) {
    if (!sizes_ok(n_edges, n_nodes) || !channels_ok(channels)) return ZS_ERR_SHAPE;
    if (!y || !norm || !rowptr || (n_edges > 0 && (!coupling || !radial || !env || !perm)))
        return ZS_ERR_NULL;
    if (!aligned(y, 4) || !aligned(norm, 4) || (out && !aligned(out, 4)) || !aligned(rowptr, 4) ||
        (order && !aligned(order, 4)) ||
        (n_edges > 0 && (!aligned(coupling, 4) || !aligned(radial, 4) || !aligned(env, 4) ||
                         !aligned(perm, 4))))
        return ZS_ERR_UNSUPPORTED;
    const int64_t node_floats = n_nodes * zs::kRows * channels;
    const Range outs[] = {span(y, node_floats, 4), span(out, out ? node_floats : 0, 4),
                          span(norm, n_nodes, 4)};
    const Range ins[] = {span(coupling, n_edges * zs::kZonal, 4),
                         span(radial, n_edges * zs::kSlots * channels, 4),
                         span(env, n_edges, 4), span(rowptr, n_nodes + 1, 4),
                         span(perm, n_edges, 4), span(order, order ? n_nodes : 0, 4)};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return ZS_ERR_ALIAS;
        for (const Range& in : ins)
            if (overlap(outs[i], in)) return ZS_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool vec4 = channels % 4 == 0 && aligned(y, 16) && (!out || aligned(out, 16)) &&
                      (n_edges == 0 || aligned(radial, 16));
    return hip_status(zs::launch_forward(coupling, radial,
                                         zs::InLayout{zs::kZonal, zs::kSlots * channels, channels},
                                         rowptr, perm, order, n_nodes, n_edges, channels, out,
                                         vec4, zs::NormIO{env, y, norm}, s));
}

int zs_backward_normalized(const float* grad_y, const float* out, const float* norm,
                           const float* coupling, const float* radial, const int32_t* dst32,
                           const int32_t* rowptr, const int32_t* perm, int64_t n_nodes,
                           int64_t n_edges, int64_t channels, float* grad_coupling,
                           float* grad_radial, float* grad_env, float* grad_deg, void* stream) {
    if (!sizes_ok(n_edges, n_nodes) || !channels_ok(channels)) return ZS_ERR_SHAPE;
    if (!grad_y || !out || !norm || !grad_deg) return ZS_ERR_NULL;
    if (n_edges > 0 && (!coupling || !radial || !dst32 || !rowptr || !perm || !grad_coupling ||
                        !grad_radial || !grad_env))
        return ZS_ERR_NULL;
    if (!aligned(grad_y, 4) || !aligned(out, 4) || !aligned(norm, 4) || !aligned(grad_deg, 4))
        return ZS_ERR_UNSUPPORTED;
    if (n_edges > 0 &&
        (!aligned(coupling, 4) || !aligned(radial, 4) || !aligned(dst32, 4) ||
         !aligned(rowptr, 4) || !aligned(perm, 4) || !aligned(grad_coupling, 4) ||
         !aligned(grad_radial, 4) || !aligned(grad_env, 4)))
        return ZS_ERR_UNSUPPORTED;
    const int64_t node_floats = n_nodes * zs::kRows * channels;
    const int64_t e_in = n_edges > 0 ? n_edges : 0;
    const Range outs[] = {span(grad_coupling, e_in * zs::kZonal, 4),
                          span(grad_radial, e_in * zs::kSlots * channels, 4),
                          span(grad_env, e_in, 4), span(grad_deg, n_nodes, 4)};
    const Range ins[] = {span(grad_y, node_floats, 4), span(out, node_floats, 4),
                         span(norm, n_nodes, 4), span(coupling, e_in * zs::kZonal, 4),
                         span(radial, e_in * zs::kSlots * channels, 4), span(dst32, e_in, 4),
                         span(rowptr, n_edges > 0 ? n_nodes + 1 : 0, 4), span(perm, e_in, 4)};
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return ZS_ERR_ALIAS;
        for (const Range& in : ins)
            if (overlap(outs[i], in)) return ZS_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool deg_done = false;
    if (n_edges > 0) {
        const bool vec4 = channels % 4 == 0 && aligned(grad_y, 16) && aligned(radial, 16) &&
                          aligned(grad_radial, 16);
        // the degree gradient is formed inside the backward when out can be
        // read in 16-byte pieces beside grad_y
        const bool fuse = aligned(out, 16);
        const hipError_t err = zs::launch_backward(
            grad_y, coupling, radial, zs::InLayout{zs::kZonal, zs::kSlots * channels, channels},
            rowptr, perm, n_nodes, n_edges, channels, grad_coupling, grad_radial, vec4,
            zs::NormGrad{norm, fuse ? out : nullptr, fuse ? grad_deg : nullptr}, &deg_done, s);
        if (err != hipSuccess) return ZS_ERR_HIP;
    }
    return hip_status(zs::launch_norm_grad(grad_y, out, norm, dst32, n_nodes, n_edges, channels,
                                           grad_deg, grad_env, deg_done, s));
}

}  // extern "C"
