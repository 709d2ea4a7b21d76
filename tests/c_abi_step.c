/* One fused attention step driven from plain C through the library's C
 * ABI: device buffers from hipMalloc, the calls on the default stream, the
 * raster output copied back.  tests/test_gpu_parity.py builds it with gcc
 * (against include/sva.h and the HIP runtime's C API), runs it on inputs it
 * writes and compares the output with the Python binding's, bit for bit.
 *
 * The same step is then run as one sva_forward call and must give the same
 * bytes.
 *
 * usage: c_abi_step B H T Hh W d block sparsity flags in.bin out.bin
 * in.bin: q, k, v as [B, N, H, d] bf16 (raw), then wq, wk as [H, d] fp32.
 * out.bin: O as [B, N, H, d] bf16. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "sva.h"

#define SVA_TRY(x)                                                            \
    do {                                                                      \
        const int rc_ = (x);                                                  \
        if (rc_ != SVA_OK) {                                                  \
            fprintf(stderr, "%s -> %d (%s): %s\n", #x, rc_,                   \
                    sva_status_string(rc_), sva_last_error());                \
            return 1;                                                         \
        }                                                                     \
    } while (0)
#define HIP_TRY(x)                                                            \
    do {                                                                      \
        const hipError_t e_ = (x);                                            \
        if (e_ != hipSuccess) {                                               \
            fprintf(stderr, "%s -> %s\n", #x, hipGetErrorString(e_));         \
            return 1;                                                         \
        }                                                                     \
    } while (0)

int main(int argc, char** argv) {
    if (argc != 12) {
        fprintf(stderr, "usage: %s B H T Hh W d block sparsity flags in.bin out.bin\n", argv[0]);
        return 2;
    }
    const int B = atoi(argv[1]), H = atoi(argv[2]), T = atoi(argv[3]), Hh = atoi(argv[4]);
    const int W = atoi(argv[5]), d = atoi(argv[6]), block = atoi(argv[7]);
    const double sparsity = atof(argv[8]);
    const unsigned flags = (unsigned)atoi(argv[9]);

    sva_plan plan;
    sva_plan_info info;
    SVA_TRY(sva_plan_create(&plan, B, H, T, Hh, W, d, block, sparsity, flags));
    SVA_TRY(sva_plan_get_info(plan, &info));

    const size_t raster = (size_t)B * (size_t)info.N * (size_t)H * (size_t)d;  /* elements */
    const size_t tiled = (size_t)B * (size_t)H * (size_t)info.Np * (size_t)d;
    const size_t wsz = (size_t)H * (size_t)d;
    const size_t in_bytes = 3 * raster * 2 + 2 * wsz * 4;
    unsigned char* host = malloc(in_bytes);
    if (!host) return 1;
    FILE* f = fopen(argv[10], "rb");
    if (!f || fread(host, 1, in_bytes, f) != in_bytes) {
        fprintf(stderr, "cannot read %s\n", argv[10]);
        return 1;
    }
    fclose(f);

    void *q, *k, *v, *wq, *wk, *q_r, *k_t, *v_t, *ws, *o;
    int32_t* col = NULL;
    const size_t ws_bytes = info.select_workspace_bytes > 0 ? info.select_workspace_bytes : 16;
    HIP_TRY(hipMalloc(&q, raster * 2));
    HIP_TRY(hipMalloc(&k, raster * 2));
    HIP_TRY(hipMalloc(&v, raster * 2));
    HIP_TRY(hipMalloc(&wq, wsz * 4));
    HIP_TRY(hipMalloc(&wk, wsz * 4));
    HIP_TRY(hipMalloc(&q_r, tiled * 2));
    HIP_TRY(hipMalloc(&k_t, tiled * 2));
    HIP_TRY(hipMalloc(&v_t, tiled * 2));
    HIP_TRY(hipMalloc(&ws, ws_bytes));
    HIP_TRY(hipMalloc(&o, raster * 2));
    if (!info.dense) HIP_TRY(hipMalloc((void**)&col, (size_t)info.nnz * sizeof(int32_t)));
    HIP_TRY(hipMemcpy(q, host, raster * 2, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(k, host + raster * 2, raster * 2, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(v, host + 2 * raster * 2, raster * 2, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(wq, host + 3 * raster * 2, wsz * 4, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(wk, host + 3 * raster * 2 + wsz * 4, wsz * 4, hipMemcpyHostToDevice));

    /* the fused step: Q' in tile order, K' as K tiles and the block means;
     * V tiles; the top-k from the means; O straight to raster order */
    SVA_TRY(sva_qk_norm_rope_tiled(plan, q, k, wq, wk, q_r, k_t, info.dense ? NULL : ws,
                                   info.dense ? 0 : ws_bytes, NULL));
    SVA_TRY(sva_reorder(plan, v, v_t, SVA_FORWARD_VT, NULL));
    if (!info.dense) SVA_TRY(sva_select_blocks(plan, NULL, NULL, ws, ws_bytes, col, NULL));
    SVA_TRY(sva_attention_ex(plan, q_r, k_t, v_t, col, NULL, NULL, o, SVA_LAYOUT_RASTER, NULL));
    HIP_TRY(hipDeviceSynchronize());

    HIP_TRY(hipMemcpy(host, o, raster * 2, hipMemcpyDeviceToHost));

    /* the same step as one sva_forward call, into a second output: the
     * two must agree bit for bit */
    void* o2;
    HIP_TRY(hipMalloc(&o2, raster * 2));
    sva_step_buffers sb = {0};
    sb.q = q; sb.k = k; sb.v = v; sb.wq = wq; sb.wk = wk;
    sb.q_r = q_r; sb.k_t = k_t; sb.v_t = v_t;
    sb.select_ws = ws; sb.select_ws_bytes = ws_bytes; sb.col = col;
    sb.o = o2;
    SVA_TRY(sva_forward(plan, &sb, NULL, NULL));
    HIP_TRY(hipDeviceSynchronize());
    unsigned char* host2 = malloc(raster * 2);
    if (!host2) return 1;
    HIP_TRY(hipMemcpy(host2, o2, raster * 2, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < raster * 2; ++i)
        if (host2[i] != host[i]) {
            fprintf(stderr, "sva_forward differs from the separate calls at byte %zu\n", i);
            return 1;
        }
    free(host2);
    hipFree(o2);

    f = fopen(argv[11], "wb");
    if (!f || fwrite(host, 1, raster * 2, f) != raster * 2) {
        fprintf(stderr, "cannot write %s\n", argv[11]);
        return 1;
    }
    fclose(f);
    hipFree(q); hipFree(k); hipFree(v); hipFree(wq); hipFree(wk);
    hipFree(q_r); hipFree(k_t); hipFree(v_t); hipFree(ws); hipFree(o);
    if (col) hipFree(col);
    SVA_TRY(sva_destroy(plan));
    free(host);
    printf("ok\n");
    return 0;
}
