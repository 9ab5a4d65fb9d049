// Internal declarations shared by the C-ABI layer and the kernel translation
// units.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sparse_attn.h"

namespace sa {

// Geometry of one predict call, derived from sa_mask_params.
struct PredictShape {
    int B, Hq, Hkv, D;
    int64_t N;
    int bq, bk;
    int64_t n_qb, n_kb;
    int64_t Nk;    // keys per sequence
    int64_t rows;  // B * Hq * n_qb
    int64_t off[6];
    size_t bytes;
};

// Fills s from p; returns SA_OK or an error code.  Pure host arithmetic.
int predict_shape(const sa_mask_params* p, PredictShape* s);
int validate_predict(const sa_mask_params* p);
int validate_attn(const sa_attn_params* p);

// Kernel launchers (each enqueues on `stream`; returns hipError_t).
hipError_t launch_permute(const void* x, int x_dtype, uint16_t* y, const int32_t* perm,
                          int64_t rows_bh, int64_t N, int D, hipStream_t stream);
hipError_t launch_unpermute(const float* y, float* x, const int32_t* perm, int64_t rows_bh,
                            int64_t N, int Dv, hipStream_t stream);

struct TopCdfArgs {
    const float* qbar;
    const float* kbar;
    const float* simq;
    const float* simk;
    uint8_t* mask;
    int32_t* counts;
    int32_t* group_tot;  // kept blocks per group of query blocks (topcdf_group_rows)
    int32_t* super_tot;  // kept blocks per kSuperGroups consecutive groups (zeroed beforehand)
    const uint8_t* forced;  // [n_qb][n_kb] forced block pattern shared by all heads, or null
    int B, Hq, Hkv, D;
    int64_t N;
    int bq, bk;
    int n_qb, n_kb;
    int causal;
    int64_t Nk;  // keys per sequence (N unless they differ)
    int64_t window, sink_front, sink_back;
    int64_t sink_rows;  // query blocks touching tokens [0, sink_rows) keep their whole valid row
    float tau;       // < 0: unset
    double tau_d;    // tau as given, for the >= 1 test
    float theta;     // <= 0: off
    double sparsity;  // < 0: unset
    float scale;
};

// FP8 codes and scales the block statistics pass writes as well (sa_predict_mask_qk8):
// q8 [B,Hq,N,D] with q_scale [B,Hq,n_qb]; k8 [B,Hkv,N_k,D] with k_scale [B,Hkv,n_kt],
// n_kt = ceil(N_k / kKeyQuantRows)
struct Quant8 {
    uint8_t* q8;
    float* q_scale;
    uint8_t* k8;
    float* k_scale;
    int64_t n_kt;
};

// perm: token permutation (q and k in the original order), or null; qz: null, or the
// FP8 outputs to write in the same pass (block_q <= kQuantMaxBlock, block_k 64 or 128)
hipError_t launch_block_stats(const uint16_t* q, const uint16_t* k, const int32_t* perm, const PredictShape& s,
                              float* qbar, float* kbar, float* simq, float* simk,
                              int32_t* dev_status, int32_t* super_tot, int n_super, const Quant8* qz,
                              hipStream_t stream);
hipError_t launch_topcdf(const TopCdfArgs& a, hipStream_t stream);
// Number of TopCdf groups (8..16 consecutive query blocks of one head).
int64_t topcdf_groups(int64_t bh, int64_t n_qb);
// Groups per super-group of the CSR offsets.
constexpr int kSuperGroups = 256;
hipError_t launch_csr(const uint8_t* mask, const int32_t* counts, const int32_t* group_tot, int64_t bh,
                      int n_qb, int n_kb, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                      int32_t* dev_status, hipStream_t stream);

// Largest block (rows) of the FP8 quantizer.
constexpr int kQuantMaxBlock = 128;
// Rows per K quantization block of the FP8 attention path (the 64-key tile).
constexpr int kKeyQuantRows = 64;
// Most 64-key tiles per sequence on the FP8 attention path (their scales sit in LDS).
constexpr int kMaxKeyTiles = 4096;

// x: bf16 [BH, N, D]; perm: token permutation or null; codes: E4M3 [BH, N, D];
// scales: fp32 [BH, ceil(N / block)].  D is 64 or 128, block 1..kQuantMaxBlock.
hipError_t launch_quant_fp8(const uint16_t* x, const int32_t* perm, int64_t BH, int64_t N, int D, int block,
                            uint8_t* codes, float* scales, hipStream_t stream);

struct FlashArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    // FP8 QK path (q8 non-null): E4M3 codes of Q and K in place of q and k, with
    // one scale per query block (q_scale [B,Hq,n_qb]) and per 64-key tile
    // (k_scale [B,Hkv,n_kt])
    const uint8_t* q8;
    const uint8_t* k8;
    const float* q_scale;
    const float* k_scale;
    int n_kt;
    float* o;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const int32_t* perm;  // token permutation (q, k, v, o in the original order), or null
    uint8_t* pv_skip;
    unsigned long long* counters;
    int32_t* dev_status;
    int B, Hq, Hkv, D;
    int64_t N;
    int64_t Nk;  // keys per sequence (N unless they differ)
    int bq, bk;
    int n_qb, n_kb;
    int64_t col_cap;
    int causal;
    float lambda;  // -inf: off
    float scale;
};

hipError_t launch_flash(const FlashArgs& a, hipStream_t stream);

// The body of the sa_predict_mask* entry points: argument checks, workspace
// carving and the three prediction launches (perm, forced: optional).
int predict_mask_impl(const uint16_t* q, const uint16_t* k, const int32_t* perm, const uint8_t* forced,
                      const sa_mask_params* p, void* ws, size_t ws_bytes, int32_t* row_ptr, int32_t* col_idx,
                      int64_t col_cap, uint8_t* mask_out, float* sim_q, float* sim_k, int32_t* dev_status,
                      void* stream, const Quant8* qz = nullptr);

}  // namespace sa
