/* The whole hot path from plain C (C99 + the HIP runtime API, no Python, no
 * torch): the caller allocates every device buffer, the library plans
 * nothing on the device it was not given, and the reorder is folded into the
 * two calls (gather form).
 *
 *   path_demo DIR B Hq Hkv N D block_q block_k causal window sink_front sink_back
 *             tau theta sparsity lambda
 *
 * DIR holds q.bin (bf16 [B,Hq,N,D]), k.bin and v.bin (bf16 [B,Hkv,N,D]) and
 * perm.bin (int32 [N], the token order of sa_plan_permutation).  "none" leaves
 * tau, theta, sparsity or lambda unset.  Writes o.bin (fp32 [B,Hq,N,D], the
 * original token order), row_ptr.bin, col_idx.bin and counters.bin to DIR and
 * prints the two status words and the kept block count. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sparse_attn.h"

#define HIP_OK(x)                                                                   \
    do {                                                                            \
        hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                     \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
            return 10;                                                              \
        }                                                                           \
    } while (0)

static void* load(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    if (!f) return NULL;
    void* p = malloc(bytes ? bytes : 1);
    if (p && fread(p, 1, bytes, f) != bytes) {
        free(p);
        p = NULL;
    }
    fclose(f);
    return p;
}

static int save(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f) return 1;
    const int bad = fwrite(p, 1, bytes, f) != bytes;
    return fclose(f) != 0 || bad;
}

static double opt(const char* s, double unset) { return strcmp(s, "none") == 0 ? unset : atof(s); }

int main(int argc, char** argv) {
    if (argc != 17) {
        fprintf(stderr, "usage: %s DIR B Hq Hkv N D block_q block_k causal window sink_front sink_back "
                        "tau theta sparsity lambda\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    sa_mask_params mp;
    memset(&mp, 0, sizeof mp);
    mp.B = atoi(argv[2]);
    mp.Hq = atoi(argv[3]);
    mp.Hkv = atoi(argv[4]);
    mp.N = atoll(argv[5]);
    mp.D = atoi(argv[6]);
    mp.block_q = atoi(argv[7]);
    mp.block_k = atoi(argv[8]);
    mp.causal = atoi(argv[9]);
    mp.window = atoll(argv[10]);
    mp.sink_front = atoll(argv[11]);
    mp.sink_back = atoll(argv[12]);
    mp.tau = opt(argv[13], -1.0);
    mp.theta = opt(argv[14], 0.0);
    mp.sparsity = opt(argv[15], -1.0);
    const size_t ws_bytes = sa_predict_workspace_bytes(&mp);
    if (ws_bytes == 0) {
        fprintf(stderr, "invalid mask parameters\n");
        return 3;
    }
    sa_attn_params ap;
    memset(&ap, 0, sizeof ap);
    ap.B = mp.B; ap.Hq = mp.Hq; ap.Hkv = mp.Hkv; ap.D = mp.D; ap.Dv = mp.D;
    ap.block_q = mp.block_q; ap.block_k = mp.block_k; ap.N = mp.N; ap.causal = mp.causal;
    ap.lambda = (float)opt(argv[16], -INFINITY);

    const int64_t n_qb = (mp.N + mp.block_q - 1) / mp.block_q, n_kb = (mp.N + mp.block_k - 1) / mp.block_k;
    const int64_t rows = (int64_t)mp.B * mp.Hq * n_qb, cap = rows * n_kb;
    const int64_t groups = (mp.block_q + SA_PV_GROUP_ROWS - 1) / SA_PV_GROUP_ROWS;
    ap.col_cap = cap;
    const size_t q_bytes = (size_t)mp.B * mp.Hq * mp.N * mp.D * 2, kv_bytes = (size_t)mp.B * mp.Hkv * mp.N * mp.D * 2;
    const size_t o_bytes = (size_t)mp.B * mp.Hq * mp.N * mp.D * 4;

    void* hq = load(dir, "q.bin", q_bytes);
    void* hk = load(dir, "k.bin", kv_bytes);
    void* hv = load(dir, "v.bin", kv_bytes);
    void* hp = load(dir, "perm.bin", (size_t)mp.N * 4);
    if (!hq || !hk || !hv || !hp) {
        fprintf(stderr, "missing or short input files in %s\n", dir);
        return 4;
    }
    void *q, *k, *v, *perm, *ws, *row_ptr, *col_idx, *status, *o, *counters, *skip;
    HIP_OK(hipMalloc(&q, q_bytes));
    HIP_OK(hipMalloc(&k, kv_bytes));
    HIP_OK(hipMalloc(&v, kv_bytes));
    HIP_OK(hipMalloc(&perm, (size_t)mp.N * 4));
    HIP_OK(hipMalloc(&ws, ws_bytes));
    HIP_OK(hipMalloc(&row_ptr, (size_t)(rows + 1) * 4));
    HIP_OK(hipMalloc(&col_idx, (size_t)cap * 4));
    HIP_OK(hipMalloc(&status, 8));
    HIP_OK(hipMalloc(&o, o_bytes));
    HIP_OK(hipMalloc(&counters, 24));
    HIP_OK(hipMalloc(&skip, (size_t)cap * groups));
    HIP_OK(hipMemcpy(q, hq, q_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(k, hk, kv_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(v, hv, kv_bytes, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(perm, hp, (size_t)mp.N * 4, hipMemcpyHostToDevice));

    int32_t* st = (int32_t*)status;
    int rc = sa_predict_mask_gather((const uint16_t*)q, (const uint16_t*)k, (const int32_t*)perm, &mp, ws, ws_bytes,
                                    (int32_t*)row_ptr, (int32_t*)col_idx, cap, NULL, NULL, NULL, st, NULL);
    if (rc != SA_OK) {
        fprintf(stderr, "sa_predict_mask_gather: %s\n", sa_status_string(rc));
        return 5;
    }
    rc = sa_sparse_attn_fwd_gather((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const int32_t*)perm,
                                   (float*)o, &ap, (const int32_t*)row_ptr, (const int32_t*)col_idx, (uint8_t*)skip,
                                   (int64_t*)counters, st + 1, NULL);
    if (rc != SA_OK) {
        fprintf(stderr, "sa_sparse_attn_fwd_gather: %s\n", sa_status_string(rc));
        return 6;
    }
    HIP_OK(hipDeviceSynchronize());

    int32_t hst[2];
    HIP_OK(hipMemcpy(hst, status, 8, hipMemcpyDeviceToHost));
    int32_t* hrp = (int32_t*)malloc((size_t)(rows + 1) * 4);
    float* ho = (float*)malloc(o_bytes);
    int64_t hcnt[3];
    if (!hrp || !ho) return 7;
    HIP_OK(hipMemcpy(hrp, row_ptr, (size_t)(rows + 1) * 4, hipMemcpyDeviceToHost));
    const int64_t nnz = hrp[rows] < cap ? hrp[rows] : cap;
    int32_t* hci = (int32_t*)malloc((size_t)(nnz ? nnz : 1) * 4);
    if (!hci) return 7;
    HIP_OK(hipMemcpy(hci, col_idx, (size_t)nnz * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ho, o, o_bytes, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hcnt, counters, 24, hipMemcpyDeviceToHost));
    if (save(dir, "o.bin", ho, o_bytes) || save(dir, "row_ptr.bin", hrp, (size_t)(rows + 1) * 4) ||
        save(dir, "col_idx.bin", hci, (size_t)nnz * 4) || save(dir, "counters.bin", hcnt, 24))
        return 8;
    printf("status %d %d nnz %lld\n", hst[0], hst[1], (long long)nnz);
    hipFree(q); hipFree(k); hipFree(v); hipFree(perm); hipFree(ws); hipFree(row_ptr);
    hipFree(col_idx); hipFree(status); hipFree(o); hipFree(counters); hipFree(skip);
    free(hq); free(hk); free(hv); free(hp); free(hrp); free(ho); free(hci);
    return 0;
}
