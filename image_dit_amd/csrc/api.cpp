// C-ABI entry points: synchronous host-side argument checks, workspace
// carving and kernel orchestration.  No HIP runtime call happens before every
// argument has been checked, so invalid calls are rejected on any machine.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "sa_internal.h"

namespace sa {

namespace {
constexpr int64_t kAlign = 256;
int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool head_dim_ok(int d) { return d == 64 || d == 128; }
}  // namespace

int validate_predict(const sa_mask_params* p) {
    if (!p) return SA_ERR_INVALID_ARGUMENT;
    if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Hq % p->Hkv != 0) return SA_ERR_INVALID_ARGUMENT;
    if (p->N <= 0 || p->N > INT32_MAX) return SA_ERR_INVALID_ARGUMENT;
    if (p->block_q <= 0 || p->block_k <= 0 || p->block_q > 256 || p->block_k > 256)
        return SA_ERR_INVALID_ARGUMENT;
    if (p->causal != 0 && p->causal != 1) return SA_ERR_INVALID_ARGUMENT;
    if (p->n_keys < 0 || (p->n_keys != 0 && p->n_keys != p->N && p->causal)) return SA_ERR_INVALID_ARGUMENT;
    if (p->sink_rows < 0 || p->sink_rows > p->N) return SA_ERR_INVALID_ARGUMENT;
    if (p->window < 0 || (p->window > 0 && !p->causal)) return SA_ERR_INVALID_ARGUMENT;
    const int64_t nk = p->n_keys > 0 ? p->n_keys : p->N;
    if (p->sink_front < 0 || p->sink_back < 0 || p->sink_front > nk || p->sink_back > nk)
        return SA_ERR_INVALID_ARGUMENT;
    const bool tau_set = p->tau >= 0.0;
    const bool s_set = p->sparsity >= 0.0;
    if (std::isnan(p->tau) || std::isnan(p->sparsity) || std::isnan(p->theta))
        return SA_ERR_INVALID_ARGUMENT;
    if (tau_set && !(p->tau > 0.0 && p->tau <= 1.0)) return SA_ERR_INVALID_ARGUMENT;
    if (s_set && !(p->sparsity < 1.0)) return SA_ERR_INVALID_ARGUMENT;
    if (!tau_set && !s_set) return SA_ERR_INVALID_ARGUMENT;  // nothing would select blocks
    if (!(p->theta <= 1.0) || std::isinf(p->theta)) return SA_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(p->scale) || p->scale < 0.0f) return SA_ERR_INVALID_ARGUMENT;
    if (!head_dim_ok(p->D)) return SA_ERR_UNSUPPORTED;
    const int64_t n_kb = (nk + p->block_k - 1) / p->block_k;
    if (n_kb > SA_MAX_KEY_BLOCKS) return SA_ERR_UNSUPPORTED;
    // row_ptr entries are int32
    if (int64_t(p->B) * p->Hq * ((p->N + p->block_q - 1) / p->block_q) + 1 > INT32_MAX) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

int predict_shape(const sa_mask_params* p, PredictShape* s) {
    const int st = validate_predict(p);
    if (st != SA_OK) return st;
    s->B = p->B;
    s->Hq = p->Hq;
    s->Hkv = p->Hkv;
    s->D = p->D;
    s->N = p->N;
    s->bq = p->block_q;
    s->bk = p->block_k;
    s->n_qb = (p->N + p->block_q - 1) / p->block_q;
    s->Nk = p->n_keys > 0 ? p->n_keys : p->N;
    s->n_kb = (s->Nk + p->block_k - 1) / p->block_k;
    s->rows = int64_t(p->B) * p->Hq * s->n_qb;
    const int64_t qblk = int64_t(p->B) * p->Hq * s->n_qb;
    const int64_t kblk = int64_t(p->B) * p->Hkv * s->n_kb;
    int64_t o = 0;
    s->off[0] = o; o = align_up(o + qblk * p->D * 4);
    s->off[1] = o; o = align_up(o + kblk * p->D * 4);
    s->off[2] = o; o = align_up(o + qblk * 4);
    s->off[3] = o; o = align_up(o + kblk * 4);
    s->off[4] = o; o = align_up(o + qblk * s->n_kb);
    // row counts, group totals, super-group totals
    const int64_t groups = topcdf_groups(int64_t(p->B) * p->Hq, s->n_qb);
    s->off[5] = o; o = align_up(o + (qblk + groups + (groups + kSuperGroups - 1) / kSuperGroups) * 4);
    s->bytes = size_t(o);
    return SA_OK;
}

int validate_attn(const sa_attn_params* p) {
    if (!p) return SA_ERR_INVALID_ARGUMENT;
    if (p->B <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Hq % p->Hkv != 0) return SA_ERR_INVALID_ARGUMENT;
    if (p->N <= 0 || p->N > INT32_MAX) return SA_ERR_INVALID_ARGUMENT;
    if (p->causal != 0 && p->causal != 1) return SA_ERR_INVALID_ARGUMENT;
    if (p->block_q <= 0 || p->block_k <= 0) return SA_ERR_INVALID_ARGUMENT;
    if (std::isnan(p->lambda) || (p->lambda >= 0.0f)) return SA_ERR_INVALID_ARGUMENT;
    if (p->col_cap < 0) return SA_ERR_INVALID_ARGUMENT;
    if (!std::isfinite(p->scale) || p->scale < 0.0f) return SA_ERR_INVALID_ARGUMENT;
    if (p->D != p->Dv || !head_dim_ok(p->D)) return SA_ERR_UNSUPPORTED;
    if (p->n_keys < 0 || p->n_keys > INT32_MAX || (p->n_keys != 0 && p->n_keys != p->N && p->causal))
        return SA_ERR_INVALID_ARGUMENT;
    // one head of q, k or v is addressed with 32-bit byte offsets below 2^31
    const int64_t nk = p->n_keys > 0 ? p->n_keys : p->N;
    if (std::max(p->N, nk) * p->D * 2 >= (int64_t(1) << 31)) return SA_ERR_UNSUPPORTED;
    const bool pair_ok = (p->block_q == 16 && p->block_k == 16) ||
                         (p->block_q == 128 && (p->block_k == 64 || p->block_k == 128));
    if (!pair_ok) return SA_ERR_UNSUPPORTED;
    // rows (one workgroup each) and row_ptr entries are int32
    const int64_t rows = int64_t(p->B) * p->Hq * ((p->N + p->block_q - 1) / p->block_q);
    if (rows + 1 > INT32_MAX) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

}  // namespace sa

using namespace sa;

extern "C" const char* sa_status_string(int code) {
    switch (code) {
        case SA_OK: return "ok";
        case SA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SA_ERR_UNSUPPORTED: return "unsupported shape (head dim or block sizes not compiled)";
        case SA_ERR_CAPACITY: return "col_idx capacity exceeded";
        case SA_ERR_EMPTY_ROW: return "a query block keeps no key block";
        case SA_ERR_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

extern "C" int sa_permute(const void* x, int x_dtype, uint16_t* y, const int32_t* perm,
                          int32_t B, int32_t H, int64_t N, int32_t D, void* stream) {
    if (!x || !y || !perm || B <= 0 || H <= 0 || N <= 0 || N > INT32_MAX || D <= 0 || D % 8 != 0)
        return SA_ERR_INVALID_ARGUMENT;
    if (x_dtype != SA_BF16 && x_dtype != SA_F32) return SA_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) return SA_ERR_INVALID_ARGUMENT;
    if (N * (D / 8) > INT32_MAX) return SA_ERR_UNSUPPORTED;  // one (row, chunk) index per thread, int32
    const hipError_t e = launch_permute(x, x_dtype, y, perm, int64_t(B) * H, N, D,
                                        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" int sa_unpermute(const float* y, float* x, const int32_t* perm, int32_t B, int32_t H,
                            int64_t N, int32_t Dv, void* stream) {
    if (!x || !y || !perm || B <= 0 || H <= 0 || N <= 0 || N > INT32_MAX || Dv <= 0 || Dv % 4 != 0)
        return SA_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15) return SA_ERR_INVALID_ARGUMENT;
    if (N * (Dv / 4) > INT32_MAX) return SA_ERR_UNSUPPORTED;  // one (row, chunk) index per thread, int32
    const hipError_t e = launch_unpermute(y, x, perm, int64_t(B) * H, N, Dv,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" size_t sa_predict_workspace_bytes(const sa_mask_params* p) {
    PredictShape s;
    return predict_shape(p, &s) == SA_OK ? s.bytes : 0;
}

extern "C" int sa_predict_workspace_offsets(const sa_mask_params* p, int64_t off[6]) {
    PredictShape s;
    const int st = predict_shape(p, &s);
    if (st != SA_OK) return st;
    if (!off) return SA_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 6; ++i) off[i] = s.off[i];
    return SA_OK;
}

namespace sa {

int predict_mask_impl(const uint16_t* q, const uint16_t* k, const int32_t* perm, const uint8_t* forced,
                 const sa_mask_params* p, void* ws, size_t ws_bytes, int32_t* row_ptr, int32_t* col_idx,
                 int64_t col_cap, uint8_t* mask_out, float* sim_q, float* sim_k, int32_t* dev_status,
                 void* stream, const Quant8* qz) {
    PredictShape s;
    const int st = predict_shape(p, &s);
    if (st != SA_OK) return st;
    if (perm && s.Nk != s.N) return SA_ERR_UNSUPPORTED;  // one permutation for queries and keys
    if (!q || !k || !ws || !row_ptr || !dev_status || col_cap < 0 || (col_cap > 0 && !col_idx))
        return SA_ERR_INVALID_ARGUMENT;
    if (ws_bytes < s.bytes || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1))) return SA_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k)) & 15) return SA_ERR_INVALID_ARGUMENT;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    char* base = static_cast<char*>(ws);
    float* qbar = reinterpret_cast<float*>(base + s.off[0]);
    float* kbar = reinterpret_cast<float*>(base + s.off[1]);
    float* simq = reinterpret_cast<float*>(base + s.off[2]);
    float* simk = reinterpret_cast<float*>(base + s.off[3]);
    uint8_t* mask = reinterpret_cast<uint8_t*>(base + s.off[4]);
    int32_t* counts = reinterpret_cast<int32_t*>(base + s.off[5]);

    const int64_t n_groups = topcdf_groups(int64_t(s.B) * s.Hq, s.n_qb);
    const int64_t n_super = (n_groups + kSuperGroups - 1) / kSuperGroups;
    int32_t* super_tot = counts + s.rows + n_groups;
    Quant8 z;
    if (qz) {
        z = *qz;
        z.n_kt = (s.Nk + kKeyQuantRows - 1) / kKeyQuantRows;
    }
    hipError_t e = launch_block_stats(q, k, perm, s, qbar, kbar, simq, simk, dev_status, super_tot, int(n_super),
                                      qz ? &z : nullptr, hs);
    if (e != hipSuccess) return SA_ERR_HIP;

    TopCdfArgs a;
    a.qbar = qbar; a.kbar = kbar; a.simq = simq; a.simk = simk;
    a.mask = mask; a.counts = counts; a.group_tot = counts + s.rows; a.forced = forced;
    a.super_tot = super_tot;
    a.B = s.B; a.Hq = s.Hq; a.Hkv = s.Hkv; a.D = s.D; a.N = s.N;
    a.bq = s.bq; a.bk = s.bk; a.n_qb = int(s.n_qb); a.n_kb = int(s.n_kb); a.Nk = s.Nk;
    a.causal = p->causal; a.window = p->window;
    a.sink_front = p->sink_front; a.sink_back = p->sink_back; a.sink_rows = p->sink_rows;
    a.tau_d = p->tau;
    a.tau = float(p->tau);
    a.theta = p->theta > 0.0 ? float(p->theta) : 0.0f;
    a.sparsity = p->sparsity;
    a.scale = p->scale > 0.0f ? p->scale : float(1.0 / std::sqrt(double(p->D)));
    e = launch_topcdf(a, hs);
    if (e != hipSuccess) return SA_ERR_HIP;

    e = launch_csr(mask, counts, a.group_tot, int64_t(s.B) * s.Hq, int(s.n_qb), int(s.n_kb), row_ptr, col_idx,
                   col_cap, dev_status, hs);
    if (e != hipSuccess) return SA_ERR_HIP;

    if (mask_out) {
        e = hipMemcpyAsync(mask_out, mask, size_t(s.rows) * s.n_kb, hipMemcpyDeviceToDevice, hs);
        if (e != hipSuccess) return SA_ERR_HIP;
    }
    if (sim_q) {
        e = hipMemcpyAsync(sim_q, simq, size_t(s.rows) * 4, hipMemcpyDeviceToDevice, hs);
        if (e != hipSuccess) return SA_ERR_HIP;
    }
    if (sim_k) {
        e = hipMemcpyAsync(sim_k, simk, size_t(s.B) * s.Hkv * s.n_kb * 4, hipMemcpyDeviceToDevice, hs);
        if (e != hipSuccess) return SA_ERR_HIP;
    }
    return SA_OK;
}

}  // namespace sa

namespace {

// FP8 QK operands of sa_sparse_attn_fwd_qk8 (all null on the bf16 path)
struct QK8 {
    const uint8_t* q8 = nullptr;
    const float* q_scale = nullptr;
    const uint8_t* k8 = nullptr;
    const float* k_scale = nullptr;
};

int sparse_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* perm, float* o,
                    const sa_attn_params* p, const int32_t* row_ptr, const int32_t* col_idx, uint8_t* pv_skip,
                    int64_t* counters, int32_t* dev_status, void* stream, const QK8& f8 = QK8{}) {
    const int st = validate_attn(p);
    if (st != SA_OK) return st;
    const bool fp8 = f8.q8 != nullptr;
    if (fp8) {
        if (!f8.k8 || !f8.q_scale || !f8.k_scale) return SA_ERR_INVALID_ARGUMENT;
        if ((reinterpret_cast<uintptr_t>(f8.q8) | reinterpret_cast<uintptr_t>(f8.k8)) & 15 ||
            (reinterpret_cast<uintptr_t>(f8.q_scale) | reinterpret_cast<uintptr_t>(f8.k_scale)) & 3)
            return SA_ERR_INVALID_ARGUMENT;
        const int64_t nk = p->n_keys > 0 ? p->n_keys : p->N;
        if (p->D != 128 || p->block_q != 128 || !(p->block_k == 64 || p->block_k == 128)) return SA_ERR_UNSUPPORTED;
        if ((nk + kKeyQuantRows - 1) / kKeyQuantRows >= kMaxKeyTiles) return SA_ERR_UNSUPPORTED;
        q = k = nullptr;
    } else if (!q || !k) {
        return SA_ERR_INVALID_ARGUMENT;
    }
    if (!v || !o || !row_ptr || !col_idx || !dev_status) return SA_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
         reinterpret_cast<uintptr_t>(o)) & 15)
        return SA_ERR_INVALID_ARGUMENT;
    FlashArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.q8 = f8.q8; a.k8 = f8.k8; a.q_scale = f8.q_scale; a.k_scale = f8.k_scale;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.perm = perm; a.pv_skip = pv_skip;
    a.counters = reinterpret_cast<unsigned long long*>(counters);
    a.dev_status = dev_status;
    a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.D = p->D; a.N = p->N;
    a.Nk = p->n_keys > 0 ? p->n_keys : p->N;
    if (perm && a.Nk != a.N) return SA_ERR_UNSUPPORTED;  // one permutation for queries and keys
    a.bq = p->block_q; a.bk = p->block_k;
    a.n_qb = int((p->N + p->block_q - 1) / p->block_q);
    a.n_kb = int((a.Nk + p->block_k - 1) / p->block_k);
    a.n_kt = int((a.Nk + kKeyQuantRows - 1) / kKeyQuantRows);
    a.col_cap = p->col_cap;
    a.causal = p->causal;
    a.lambda = p->lambda;
    a.scale = p->scale > 0.0f ? p->scale : float(1.0 / std::sqrt(double(p->D)));
    const hipError_t e = launch_flash(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

}  // namespace

extern "C" int sa_predict_mask(const uint16_t* q, const uint16_t* k, const sa_mask_params* p,
                               void* ws, size_t ws_bytes, int32_t* row_ptr, int32_t* col_idx,
                               int64_t col_cap, uint8_t* mask_out, float* sim_q, float* sim_k,
                               int32_t* dev_status, void* stream) {
    return predict_mask_impl(q, k, nullptr, nullptr, p, ws, ws_bytes, row_ptr, col_idx, col_cap, mask_out, sim_q, sim_k,
                        dev_status, stream);
}

extern "C" int sa_predict_mask_gather(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                                      const sa_mask_params* p, void* ws, size_t ws_bytes, int32_t* row_ptr,
                                      int32_t* col_idx, int64_t col_cap, uint8_t* mask_out, float* sim_q,
                                      float* sim_k, int32_t* dev_status, void* stream) {
    if (!perm_dev) return SA_ERR_INVALID_ARGUMENT;
    return predict_mask_impl(q, k, perm_dev, nullptr, p, ws, ws_bytes, row_ptr, col_idx, col_cap, mask_out, sim_q, sim_k,
                        dev_status, stream);
}

extern "C" int sa_predict_mask_ex(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                                  const uint8_t* forced_dev, const sa_mask_params* p, void* ws, size_t ws_bytes,
                                  int32_t* row_ptr, int32_t* col_idx, int64_t col_cap, uint8_t* mask_out,
                                  float* sim_q, float* sim_k, int32_t* dev_status, void* stream) {
    return predict_mask_impl(q, k, perm_dev, forced_dev, p, ws, ws_bytes, row_ptr, col_idx, col_cap, mask_out,
                        sim_q, sim_k, dev_status, stream);
}

extern "C" int sa_sparse_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, float* o,
                                  const sa_attn_params* p, const int32_t* row_ptr,
                                  const int32_t* col_idx, uint8_t* pv_skip, int64_t* counters,
                                  int32_t* dev_status, void* stream) {
    return sparse_attn_fwd(q, k, v, nullptr, o, p, row_ptr, col_idx, pv_skip, counters, dev_status, stream);
}

extern "C" int sa_sparse_attn_fwd_gather(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* perm_dev, float* o, const sa_attn_params* p,
                                         const int32_t* row_ptr, const int32_t* col_idx, uint8_t* pv_skip,
                                         int64_t* counters, int32_t* dev_status, void* stream) {
    if (!perm_dev) return SA_ERR_INVALID_ARGUMENT;
    return sparse_attn_fwd(q, k, v, perm_dev, o, p, row_ptr, col_idx, pv_skip, counters, dev_status, stream);
}

extern "C" int sa_quantize_fp8(const uint16_t* x, const int32_t* perm_dev, int32_t B, int32_t H, int64_t N,
                               int32_t D, int32_t block, uint8_t* codes, float* scales, void* stream) {
    if (!x || !codes || !scales || B <= 0 || H <= 0 || N <= 0 || N > INT32_MAX) return SA_ERR_INVALID_ARGUMENT;
    if (block <= 0 || block > kQuantMaxBlock) return SA_ERR_INVALID_ARGUMENT;
    if (!head_dim_ok(D)) return SA_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(codes) & 7) ||
        (reinterpret_cast<uintptr_t>(scales) & 3))
        return SA_ERR_INVALID_ARGUMENT;
    const hipError_t e = launch_quant_fp8(x, perm_dev, int64_t(B) * H, N, D, block, codes, scales,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SA_OK : SA_ERR_HIP;
}

extern "C" int sa_sparse_attn_fwd_qk8(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                                      const float* k_scale, const uint16_t* v, const int32_t* perm_dev, float* o,
                                      const sa_attn_params* p, const int32_t* row_ptr, const int32_t* col_idx,
                                      uint8_t* pv_skip, int64_t* counters, int32_t* dev_status, void* stream) {
    if (!q8) return SA_ERR_INVALID_ARGUMENT;
    QK8 f8;
    f8.q8 = q8; f8.q_scale = q_scale; f8.k8 = k8; f8.k_scale = k_scale;
    return sparse_attn_fwd(nullptr, nullptr, v, perm_dev, o, p, row_ptr, col_idx, pv_skip, counters, dev_status,
                           stream, f8);
}

extern "C" int sa_predict_mask_qk8(const uint16_t* q, const uint16_t* k, const int32_t* perm_dev,
                                   const sa_mask_params* p, void* ws, size_t ws_bytes, int32_t* row_ptr,
                                   int32_t* col_idx, int64_t col_cap, uint8_t* q8, float* q_scale, uint8_t* k8,
                                   float* k_scale, int32_t* dev_status, void* stream) {
    const int st = validate_predict(p);
    if (st != SA_OK) return st;
    if (!q8 || !q_scale || !k8 || !k_scale) return SA_ERR_INVALID_ARGUMENT;
    if (((reinterpret_cast<uintptr_t>(q8) | reinterpret_cast<uintptr_t>(k8)) & 7) ||
        ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale)) & 3))
        return SA_ERR_INVALID_ARGUMENT;
    if (p->block_q > kQuantMaxBlock || !(p->block_k == kKeyQuantRows || p->block_k == 2 * kKeyQuantRows))
        return SA_ERR_UNSUPPORTED;
    Quant8 z{q8, q_scale, k8, k_scale, 0};
    return predict_mask_impl(q, k, perm_dev, nullptr, p, ws, ws_bytes, row_ptr, col_idx, col_cap, nullptr, nullptr,
                             nullptr, dev_status, stream, &z);
}
