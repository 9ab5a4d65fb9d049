/* A plain C99 caller of the library's host-only entry points: it plans the
 * window and Hilbert token orders of a small video layout, sizes the mask
 * prediction workspace, and prints the results for the test to compare with
 * the oracle.  Nothing here touches a GPU. */
#include <stdio.h>
#include <stdlib.h>

#include "sparse_attn.h"

static int plan(int order, int t, int h, int w, int txt, int sink) {
    sa_layout L;
    L.n_tokens = (int64_t)txt + (int64_t)t * h * w;
    L.order = order;
    L.t = t; L.h = h; L.w = w;
    L.win_t = 2; L.win_h = 4; L.win_w = 4;
    L.txt_len = txt;
    L.first_frame_sink = sink;
    int32_t* perm = (int32_t*)malloc((size_t)L.n_tokens * sizeof(int32_t));
    if (!perm) return 1;
    const int st = sa_plan_permutation(&L, perm, L.n_tokens);
    printf("perm %d %lld", st, (long long)L.n_tokens);
    for (int64_t i = 0; i < L.n_tokens; ++i) printf(" %d", perm[i]);
    printf("\n");
    free(perm);
    return st;
}

int main(void) {
    printf("status %s|%s\n", sa_status_string(SA_OK), sa_status_string(SA_ERR_UNSUPPORTED));
    if (plan(SA_ORDER_WINDOW, 3, 5, 7, 6, 1) != SA_OK) return 2;
    if (plan(SA_ORDER_HILBERT, 3, 5, 7, 0, 0) != SA_OK) return 3;
    sa_mask_params p = {0};
    p.B = 1; p.Hq = 4; p.Hkv = 2; p.N = 1000; p.D = 128; p.block_q = 128; p.block_k = 64;
    p.tau = 0.9; p.theta = 0.0; p.sparsity = -1.0;
    printf("ws %zu\n", sa_predict_workspace_bytes(&p));
    p.D = 96;  /* not compiled */
    printf("ws_bad %zu\n", sa_predict_workspace_bytes(&p));
    return 0;
}
