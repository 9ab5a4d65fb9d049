// Block-mask prediction kernels (SpargeAttn notes, section 2.2, selective
// token compression; MindIE-SD "稀疏" page, rf_v2 block representatives and
// sinks; "44. Local Sliding and Sparse Attention", Step 2 causal window).
//
//   k_block_stats  one streaming pass over Q and K: per block the mean token
//                  and the mean pairwise cosine ||mean_t x_t/||x_t||||^2.
//                  HBM-bound: every byte of Q and K is read exactly once.
//   k_topcdf       per query block: compressed scores against every key-block
//                  mean, guard/sink/window forcing, softmax over the
//                  candidates, an LDS bitonic sort on (probability desc, index
//                  asc), an exclusive scan for TopCdf, the keep floor, and the
//                  dense mask row plus its kept count.
//   k_csr_scan     exclusive scan of the row counts -> row_ptr.
//   k_csr_fill     ascending column lists from the mask rows (ballot compaction).
#include <cfloat>

#include "sa_internal.h"

namespace sa {
namespace {

__device__ inline float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
__device__ inline int wave_sum_i(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// ---------------------------------------------------------------- block stats
// One workgroup (256 threads) per block.  A token row of D bf16 is split in
// D/8 chunks of 16 bytes; CH = D/8 consecutive lanes hold one row, 256/CH rows
// are in flight per pass.  Row norms are reduced across the CH lanes with
// shuffles; the per-row-slot partial sums are then reduced through LDS.
template <int D>
__global__ __launch_bounds__(256) void k_block_stats(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k, int64_t N,
                                                     int bq, int bk, int64_t q_blocks, int n_qb,
                                                     int n_kb, float* __restrict__ qbar,
                                                     float* __restrict__ kbar, float* __restrict__ simq,
                                                     float* __restrict__ simk, int32_t* dev_status) {
    constexpr int CH = D / 8;
    constexpr int RPP = 256 / CH;
    __shared__ float sx[RPP][D + 1];
    __shared__ float su[RPP][D + 1];
    __shared__ float red[4];

    if (blockIdx.x == 0 && threadIdx.x == 0) *dev_status = SA_OK;

    const int64_t blk = blockIdx.x;
    const bool is_q = blk < q_blocks;
    const int64_t local = is_q ? blk : blk - q_blocks;
    const int nb = is_q ? n_qb : n_kb;
    const int b = is_q ? bq : bk;
    const int64_t bh = local / nb;
    const int j = int(local - bh * nb);
    const int64_t t0 = int64_t(j) * b;
    const int len = int(min(int64_t(b), N - t0));
    const uint16_t* src = (is_q ? q : k) + (bh * N + t0) * D;

    const int tid = threadIdx.x;
    const int ch = tid % CH;
    const int slot = tid / CH;

    float ax[8], au[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ax[e] = au[e] = 0.f;

    for (int r0 = 0; r0 < len; r0 += 4 * RPP) {
        uint4 raw[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int r = r0 + s * RPP + slot;
            raw[s] = r < len ? *(reinterpret_cast<const uint4*>(src + int64_t(r) * D) + ch)
                             : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            float v[8];
            v[0] = bf16f(raw[s].x & 0xffffu); v[1] = bf16f(raw[s].x >> 16);
            v[2] = bf16f(raw[s].y & 0xffffu); v[3] = bf16f(raw[s].y >> 16);
            v[4] = bf16f(raw[s].z & 0xffffu); v[5] = bf16f(raw[s].z >> 16);
            v[6] = bf16f(raw[s].w & 0xffffu); v[7] = bf16f(raw[s].w >> 16);
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
            for (int m = CH / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
            const float inv = ss > 0.f ? 1.0f / sqrtf(ss) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ax[e] += v[e];
                au[e] = fmaf(v[e], inv, au[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sx[slot][ch * 8 + e] = ax[e];
        su[slot][ch * 8 + e] = au[e];
    }
    __syncthreads();
    float um2 = 0.f;
    if (tid < D) {
        float tx = 0.f, tu = 0.f;
#pragma unroll 8
        for (int s = 0; s < RPP; ++s) {
            tx += sx[s][tid];
            tu += su[s][tid];
        }
        const float inv_len = 1.0f / float(len);
        const float mean = tx * inv_len;
        const float um = tu * inv_len;
        um2 = um * um;
        float* outm = (is_q ? qbar : kbar) + local * D;
        outm[tid] = mean;
    }
    um2 = wave_sum(um2);
    if ((tid & 63) == 0 && tid < D) red[tid >> 6] = um2;
    __syncthreads();
    if (tid == 0) {
        float sim = 0.f;
        for (int w = 0; w < D / 64; ++w) sim += red[w];
        (is_q ? simq : simk)[local] = sim;
    }
}

// ---------------------------------------------------------------- TopCdf
constexpr int kRowsPerWG = 4;  // one query block per wavefront

struct RowGeom {
    int nv;        // valid key blocks (prefix 0..nv-1)
    int64_t q_first, q_end;
};

__device__ inline RowGeom row_geom(const TopCdfArgs& a, int i) {
    RowGeom g;
    g.q_first = int64_t(i) * a.bq;
    g.q_end = min(g.q_first + a.bq, a.N);
    if (a.causal) {
        const int64_t last_q = g.q_end - 1;
        g.nv = int(min(int64_t(a.n_kb), last_q / a.bk + 1));
    } else {
        g.nv = a.n_kb;
    }
    return g;
}

__device__ inline bool forced_block(const TopCdfArgs& a, const RowGeom& g, int j, float sk) {
    const int64_t k_first = int64_t(j) * a.bk;
    const int64_t k_end = min(k_first + a.bk, a.N);
    bool f = (a.theta > 0.f) && (sk < a.theta);
    f |= (a.sink_front > 0) && (k_first < a.sink_front);
    f |= (a.sink_back > 0) && (k_end > a.N - a.sink_back);
    if (a.causal) {
        f |= (a.window > 0) && (k_end - 1 >= g.q_first - a.window + 1);
        f |= (k_first < g.q_end) && (k_end > g.q_first);
    }
    return f;
}

// Dynamic LDS: qs[4][D] f32 | logits[4][n_kb] f32 | keys[4][S] u64 | mrow[4][n_kb] u8
template <int D>
__global__ __launch_bounds__(256) void k_topcdf(TopCdfArgs a, int S) {
    extern __shared__ __align__(16) unsigned char smem[];
    float* qs = reinterpret_cast<float*>(smem);
    float* logits = qs + kRowsPerWG * D;
    const int nkb_pad = (a.n_kb + 3) & ~3;
    unsigned long long* keys_all =
        reinterpret_cast<unsigned long long*>(logits + kRowsPerWG * nkb_pad + ((kRowsPerWG * nkb_pad) & 1));
    uint8_t* mrow_all = reinterpret_cast<uint8_t*>(keys_all + kRowsPerWG * S);

    const int groups = (a.n_qb + kRowsPerWG - 1) / kRowsPerWG;
    const int bh = blockIdx.x / groups;  // b * Hq + hq
    const int i0 = (blockIdx.x - bh * groups) * kRowsPerWG;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int64_t kvh = int64_t(b) * a.Hkv + hk;
    const float* kbar = a.kbar + kvh * a.n_kb * D;
    const float* simk = a.simk + kvh * a.n_kb;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    // query-block means of the WG's rows
    for (int t = tid; t < kRowsPerWG * D; t += 256) {
        const int r = t / D;
        const int i = i0 + r;
        qs[t] = i < a.n_qb ? a.qbar[(int64_t(bh) * a.n_qb + i) * D + (t - r * D)] : 0.f;
    }
    // columns any of the WG's rows can see
    const int i_last = min(i0 + kRowsPerWG, a.n_qb) - 1;
    const int ncols = row_geom(a, i_last).nv;
    __syncthreads();

    // compressed scores: thread per key block, all rows at once (kbar read once per WG)
    for (int j = tid; j < ncols; j += 256) {
        float acc[kRowsPerWG];
#pragma unroll
        for (int r = 0; r < kRowsPerWG; ++r) acc[r] = 0.f;
        const float4* kr = reinterpret_cast<const float4*>(kbar + int64_t(j) * D);
#pragma unroll 4
        for (int d4 = 0; d4 < D / 4; ++d4) {
            const float4 kv = kr[d4];
#pragma unroll
            for (int r = 0; r < kRowsPerWG; ++r) {
                const float4 qv = reinterpret_cast<const float4*>(qs + r * D)[d4];
                acc[r] = fmaf(qv.x, kv.x, acc[r]);
                acc[r] = fmaf(qv.y, kv.y, acc[r]);
                acc[r] = fmaf(qv.z, kv.z, acc[r]);
                acc[r] = fmaf(qv.w, kv.w, acc[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < kRowsPerWG; ++r) logits[r * nkb_pad + j] = acc[r] * a.scale;
    }
    __syncthreads();

    // ---- per-row selection: wavefront `wave` owns row i
    const int i = i0 + wave;
    const bool row_ok = i < a.n_qb;
    const RowGeom g = row_geom(a, row_ok ? i : i_last);
    const float* lrow = logits + wave * nkb_pad;
    unsigned long long* keys = keys_all + wave * S;
    uint8_t* mrow = mrow_all + wave * nkb_pad;
    const int64_t row = int64_t(bh) * a.n_qb + (row_ok ? i : 0);
    const bool forced_row = row_ok && a.theta > 0.f && a.simq[row] < a.theta;

    // forced flags, candidate max and counts
    float cmax = -FLT_MAX;
    int n_forced = 0, n_cand = 0;
    for (int j = lane; j < a.n_kb; j += 64) {
        uint8_t f = 0;
        if (j < g.nv) {
            f = forced_block(a, g, j, simk[j]) ? 1 : 0;
            n_forced += f;
            if (!f) {
                ++n_cand;
                cmax = fmaxf(cmax, lrow[j]);
            }
        }
        mrow[j] = f;
    }
    cmax = wave_max(cmax);
    n_forced = wave_sum_i(n_forced);
    n_cand = wave_sum_i(n_cand);

    float esum = 0.f;
    for (int j = lane; j < g.nv; j += 64)
        if (!mrow[j]) esum += expf(lrow[j] - cmax);
    esum = wave_sum(esum);
    const float inv_sum = 1.0f / esum;
    // sort keys: (probability bits, ~index) descending; non-candidates are 0
    for (int j = lane; j < S; j += 64) {
        unsigned long long key = 0ull;
        if (j < g.nv && !mrow[j]) {
            const float p = expf(lrow[j] - cmax) * inv_sum;
            key = (static_cast<unsigned long long>(__float_as_uint(p)) << 32) |
                  static_cast<unsigned long long>(0xffffffffu - uint32_t(j));
        }
        keys[j] = key;
    }
    __syncthreads();
    for (int kk = 2; kk <= S; kk <<= 1) {
        for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            for (int t = lane; t < (S >> 1); t += 64) {
                const int lo = ((t & ~(jj - 1)) << 1) | (t & (jj - 1));
                const int hi = lo + jj;
                const unsigned long long x = keys[lo], y = keys[hi];
                const bool desc = (lo & kk) == 0;
                if (desc ? (x < y) : (x > y)) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }

    // TopCdf: count positions whose exclusive prefix mass is below tau
    int k_cdf = 0;
    if (a.tau_d >= 1.0) {
        k_cdf = n_cand;
    } else if (a.tau_d > 0.0) {
        const int E = S >= 64 ? S / 64 : 1;
        const int p0 = lane * E;
        float part = 0.f;
        for (int e = 0; e < E; ++e) {
            const int r = p0 + e;
            if (r < n_cand) part += __uint_as_float(uint32_t(keys[r] >> 32));
        }
        // exclusive wave scan of the lane partials, in lane order
        float incl = part;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const float o = __shfl_up(incl, m);
            if (lane >= m) incl += o;
        }
        float run = __shfl_up(incl, 1);
        if (lane == 0) run = 0.f;
        int cnt = 0;
        for (int e = 0; e < E; ++e) {
            const int r = p0 + e;
            if (r < n_cand) {
                if (double(run) < a.tau_d) ++cnt;
                run += __uint_as_float(uint32_t(keys[r] >> 32));
            }
        }
        k_cdf = wave_sum_i(cnt);
    }
    int extra = 0;
    if (a.sparsity >= 0.0) {
        const double floor_keep = ceil((1.0 - a.sparsity) * double(g.nv));
        extra = max(0, int(floor_keep) - n_forced);
    }
    int keep = min(n_cand, max(k_cdf, extra));
    if (forced_row) keep = 0;
    for (int r = lane; r < keep; r += 64) {
        const int j = int(0xffffffffu - uint32_t(keys[r] & 0xffffffffull));
        mrow[j] = 1;
    }
    if (forced_row)
        for (int j = lane; j < g.nv; j += 64) mrow[j] = 1;
    __syncthreads();
    if (row_ok) {
        uint8_t* out = a.mask + row * a.n_kb;
        for (int j = lane; j < a.n_kb; j += 64) out[j] = mrow[j];
        if (lane == 0) a.counts[row] = forced_row ? g.nv : n_forced + keep;
    }
}

// ---------------------------------------------------------------- CSR
__global__ __launch_bounds__(1024) void k_csr_scan(const int32_t* __restrict__ counts, int64_t rows,
                                                   int32_t* __restrict__ row_ptr, int64_t col_cap,
                                                   int32_t* dev_status) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    const int64_t per = (rows + 1023) / 1024;
    const int64_t r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
    int64_t s = 0;
    for (int64_t r = r0; r < r1; ++r) s += counts[r];
    part[tid] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int64_t v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int64_t run = part[tid] - s;
    for (int64_t r = r0; r < r1; ++r) {
        row_ptr[r] = int32_t(run);
        run += counts[r];
    }
    if (tid == 1023) {
        row_ptr[rows] = int32_t(part[1023]);
        if (part[1023] > col_cap) *dev_status = SA_ERR_CAPACITY;
    }
}

__global__ __launch_bounds__(256) void k_csr_fill(const uint8_t* __restrict__ mask, int64_t rows, int n_kb,
                                                  const int32_t* __restrict__ row_ptr,
                                                  int32_t* __restrict__ col_idx, int64_t col_cap) {
    const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    const uint8_t* m = mask + row * n_kb;
    int64_t base = row_ptr[row];
    for (int j0 = 0; j0 < n_kb; j0 += 64) {
        const int j = j0 + lane;
        const bool on = j < n_kb && m[j];
        const unsigned long long bal = __ballot(on);
        const int before = __popcll(bal & ((1ull << lane) - 1ull));
        const int64_t pos = base + before;
        if (on && pos < col_cap) col_idx[pos] = j;
        base += __popcll(bal);
    }
}

int pow2_at_least(int v) {
    int s = 1;
    while (s < v) s <<= 1;
    return s;
}

}  // namespace

hipError_t launch_block_stats(const uint16_t* q, const uint16_t* k, const PredictShape& s, float* qbar,
                              float* kbar, float* simq, float* simk, int32_t* dev_status,
                              hipStream_t stream) {
    const int64_t qb = int64_t(s.B) * s.Hq * s.n_qb;
    const int64_t kb = int64_t(s.B) * s.Hkv * s.n_kb;
    if (qb + kb > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid(unsigned(qb + kb));
    if (s.D == 128)
        hipLaunchKernelGGL(k_block_stats<128>, grid, dim3(256), 0, stream, q, k, s.N, s.bq, s.bk, qb,
                           int(s.n_qb), int(s.n_kb), qbar, kbar, simq, simk, dev_status);
    else
        hipLaunchKernelGGL(k_block_stats<64>, grid, dim3(256), 0, stream, q, k, s.N, s.bq, s.bk, qb,
                           int(s.n_qb), int(s.n_kb), qbar, kbar, simq, simk, dev_status);
    return hipGetLastError();
}

hipError_t launch_topcdf(const TopCdfArgs& a, hipStream_t stream) {
    const int S = max(2, pow2_at_least(a.n_kb));
    const int nkb_pad = (a.n_kb + 3) & ~3;
    const size_t lds = size_t(kRowsPerWG) * a.D * 4 + size_t(kRowsPerWG) * nkb_pad * 4 + 8 +
                       size_t(kRowsPerWG) * S * 8 + size_t(kRowsPerWG) * nkb_pad;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int groups = (a.n_qb + kRowsPerWG - 1) / kRowsPerWG;
    const int64_t nwg = int64_t(a.B) * a.Hq * groups;
    if (nwg > INT32_MAX) return hipErrorInvalidValue;
    if (a.D == 128)
        hipLaunchKernelGGL(k_topcdf<128>, dim3(unsigned(nwg)), dim3(256), lds, stream, a, S);
    else
        hipLaunchKernelGGL(k_topcdf<64>, dim3(unsigned(nwg)), dim3(256), lds, stream, a, S);
    return hipGetLastError();
}

hipError_t launch_csr(const uint8_t* mask, const int32_t* counts, int64_t rows, int n_kb, int32_t* row_ptr,
                      int32_t* col_idx, int64_t col_cap, int32_t* dev_status, hipStream_t stream) {
    hipLaunchKernelGGL(k_csr_scan, dim3(1), dim3(1024), 0, stream, counts, rows, row_ptr, col_cap, dev_status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nwg = (rows + 3) / 4;
    hipLaunchKernelGGL(k_csr_fill, dim3(unsigned(nwg)), dim3(256), 0, stream, mask, rows, n_kb, row_ptr,
                       col_idx, col_cap);
    return hipGetLastError();
}

}  // namespace sa
