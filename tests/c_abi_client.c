/*
 * Plain C client of libzs (include/zs.h): no Python, no torch.  It reads a
 * problem from a binary file, runs the stable CSR build, the forward and the
 * backward on the default HIP stream, and writes the results to a binary file.
 *
 * Input file (little endian):  int64 N, E, C; int64 dst[E]; float coupling[E][15];
 *                              float radial[E][3][C]; float grad_out[N][16][C]
 * Output file:                 int32 rowptr[N+1]; int32 perm[E]; float out[N][16][C];
 *                              float grad_coupling[E][15]; float grad_radial[E][3][C]
 *
 * Exit status 0 on success; otherwise the failing call and its status text go
 * to stderr.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "zs.h"

static int fail_hip(const char *what, hipError_t e)
{
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 2;
}

static int fail_zs(const char *what, int s)
{
    fprintf(stderr, "%s: %s (%d)\n", what, zs_status_string(s), s);
    return 3;
}

static void *read_block(FILE *f, size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (p && bytes && fread(p, 1, bytes, f) != bytes) {
        free(p);
        return NULL;
    }
    return p;
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s INPUT OUTPUT\n", argv[0]);
        return 1;
    }
    FILE *f = fopen(argv[1], "rb");
    if (!f) {
        perror(argv[1]);
        return 1;
    }
    int64_t hdr[3];
    if (fread(hdr, sizeof hdr, 1, f) != 1) {
        fprintf(stderr, "short header\n");
        return 1;
    }
    const int64_t N = hdr[0], E = hdr[1], C = hdr[2];
    const size_t b_dst = (size_t)E * 8, b_cpl = (size_t)E * 15 * 4;
    const size_t b_rad = (size_t)E * 3 * C * 4, b_node = (size_t)N * 16 * C * 4;
    int64_t *dst = read_block(f, b_dst);
    float *cpl = read_block(f, b_cpl), *rad = read_block(f, b_rad), *g = read_block(f, b_node);
    fclose(f);
    if (!dst || !cpl || !rad || !g) {
        fprintf(stderr, "short input\n");
        return 1;
    }

    void *d_dst, *d_cpl, *d_rad, *d_g, *d_rowptr, *d_perm, *d_dst32, *d_ws, *d_out, *d_gc, *d_gr,
        *d_order;
    const size_t ws_bytes = zs_csr_workspace_bytes(E, N);
    hipError_t e;
    void **bufs[] = {&d_dst, &d_cpl, &d_rad, &d_g, &d_rowptr, &d_perm, &d_dst32, &d_ws,
                     &d_out, &d_gc, &d_gr, &d_order};
    const size_t sizes[] = {b_dst, b_cpl, b_rad, b_node, (size_t)(N + 1) * 4, (size_t)E * 4,
                            (size_t)E * 4, ws_bytes, b_node, b_cpl, b_rad, (size_t)N * 4};
    for (int i = 0; i < 12; ++i)
        if ((e = hipMalloc(bufs[i], sizes[i] ? sizes[i] : 256)) != hipSuccess)
            return fail_hip("hipMalloc", e);
    if ((e = hipMemcpy(d_dst, dst, b_dst, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(d_cpl, cpl, b_cpl, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(d_rad, rad, b_rad, hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(d_g, g, b_node, hipMemcpyHostToDevice)) != hipSuccess)
        return fail_hip("hipMemcpy to device", e);

    int s = zs_build_csr(d_dst, E, N, d_rowptr, d_perm, d_dst32, d_order, d_ws, ws_bytes, NULL,
                         NULL);
    if (s != ZS_OK)
        return fail_zs("zs_build_csr", s);
    s = zs_forward(d_cpl, d_rad, d_rowptr, d_perm, d_order, N, E, C, d_out, NULL);
    if (s != ZS_OK)
        return fail_zs("zs_forward", s);
    s = zs_backward(d_g, d_cpl, d_rad, d_dst32, d_rowptr, d_perm, N, E, C, d_gc, d_gr, NULL);
    if (s != ZS_OK)
        return fail_zs("zs_backward", s);
    if ((e = hipDeviceSynchronize()) != hipSuccess)
        return fail_hip("hipDeviceSynchronize", e);

    int32_t *rowptr = malloc((size_t)(N + 1) * 4), *perm = malloc((size_t)E * 4 + 4);
    float *out = malloc(b_node), *gc = malloc(b_cpl + 4), *gr = malloc(b_rad + 4);
    if ((e = hipMemcpy(rowptr, d_rowptr, (size_t)(N + 1) * 4, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(perm, d_perm, (size_t)E * 4, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(out, d_out, b_node, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(gc, d_gc, b_cpl, hipMemcpyDeviceToHost)) != hipSuccess ||
        (e = hipMemcpy(gr, d_gr, b_rad, hipMemcpyDeviceToHost)) != hipSuccess)
        return fail_hip("hipMemcpy to host", e);
    FILE *o = fopen(argv[2], "wb");
    if (!o) {
        perror(argv[2]);
        return 1;
    }
    fwrite(rowptr, 4, (size_t)(N + 1), o);
    fwrite(perm, 4, (size_t)E, o);
    fwrite(out, 1, b_node, o);
    fwrite(gc, 1, b_cpl, o);
    fwrite(gr, 1, b_rad, o);
    fclose(o);
    for (int i = 0; i < 12; ++i)
        hipFree(*bufs[i]);
    free(dst); free(cpl); free(rad); free(g);
    free(rowptr); free(perm); free(out); free(gc); free(gr);
    return 0;
}
