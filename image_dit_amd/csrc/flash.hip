// Block-sparse FlashAttention-style forward (SpargeAttn notes, section 2.1:
// online softmax with running max m, running sum l and unnormalised output O;
// blocks outside the mask skip both QK^T and PV; section 2.3: PV skip when
// the running-max gap of a row group is below lambda).
//
// k_flash_mfma<D, BK>: one workgroup of 4 wavefronts per 128-row query block;
// wavefront w owns query rows 32w..32w+31 and is the PV-skip group.  Scores
// are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 so that
// every accumulator a lane holds belongs to ONE query row (lane & 31): row
// max/sum need no cross-lane work beyond one exchange with lane ^ 32, and the
// output rescale is one scalar per lane.  O^T = V^T P^T reuses the score
// registers directly as the B operand (the key order inside a 16-key MFMA
// step only has to agree between the two operands).  K is staged row-major in
// LDS (padded rows), V transposed (padded rows) so both MFMA operands are
// contiguous LDS reads.
//
// k_flash_small<D>: the 16x16-block case (tiny workloads), plain fp32 ALU.
#include <cmath>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__global__ void k_attn_init(int32_t* status, unsigned long long* counters) {
    *status = SA_OK;
    if (counters) counters[0] = counters[1] = counters[2] = 0ull;
}

template <int D, int BK>
__global__ __launch_bounds__(256) void k_flash_mfma(FlashArgs a) {
    constexpr int BQ = 128;
    constexpr int KSTR = D + 8;   // bf16 per K row in LDS (16-byte pad: conflict-free 16-B reads)
    constexpr int VSTR = BK + 4;  // bf16 per V^T row in LDS (8-byte pad)
    constexpr int NT = D / 32;    // output tiles (32 dv each)
    constexpr int KS = D / 16;    // MFMA k-steps over the head dim
    constexpr int MT = BK / 32;   // score tiles (32 keys each)
    constexpr int PS = BK / 16;   // MFMA k-steps over keys
    __shared__ __align__(16) uint16_t Ks[BK * KSTR];
    __shared__ __align__(16) uint16_t Vt[D * VSTR];

    const int row = blockIdx.x;
    const int qb = row % a.n_qb;
    const int bh = row / a.n_qb;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int64_t N = a.N;
    const uint16_t* Qh = a.q + int64_t(bh) * N * D;
    const uint16_t* Kh = a.k + (int64_t(b) * a.Hkv + hk) * N * D;
    const uint16_t* Vh = a.v + (int64_t(b) * a.Hkv + hk) * N * D;
    float* Oh = a.o + int64_t(bh) * N * D;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int64_t wrow0 = int64_t(qb) * BQ + wave * 32;
    const int64_t qrow = wrow0 + l32;
    const bool row_valid = qrow < N;
    const bool wave_rows = wrow0 < N;

    bf16x8_t qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (row_valid) u = *reinterpret_cast<const uint4*>(Qh + qrow * D + ks * 16 + half * 8);
        qf[ks] = as_bf16x8(u);
    }

    floatx16 oacc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
    float m_run = -INFINITY;
    float l_part = 0.f;
    const float c2 = a.scale * kLog2e;
    const bool lam_on = a.lambda > -INFINITY;
    const float lam2 = a.lambda * kLog2e;
    int n_exec = 0, n_skip = 0;

    const int e0 = a.row_ptr[row];
    int e1 = a.row_ptr[row + 1];
    if (e1 > a.col_cap) {
        if (tid == 0) *a.dev_status = SA_ERR_CAPACITY;
        e1 = int(a.col_cap);
    }
    for (int e = e0; e < e1; ++e) {
        const int jblk = a.col_idx[e];
        if (jblk < 0 || jblk >= a.n_kb) {  // uniform across the workgroup
            if (tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;
            continue;
        }
        const int64_t kb0 = int64_t(jblk) * BK;
        __syncthreads();  // previous block's LDS reads are done
        // ---- K tile, row-major
        constexpr int KCH = D / 8;
#pragma unroll
        for (int c = tid; c < BK * KCH; c += 256) {
            const int rr = c / KCH, cc = c % KCH;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (kb0 + rr < N) u = *reinterpret_cast<const uint4*>(Kh + (kb0 + rr) * D + cc * 8);
            *reinterpret_cast<uint4*>(Ks + rr * KSTR + cc * 8) = u;
        }
        // ---- V tile, transposed through 4x4 register blocks
        constexpr int DB4 = D / 4;
#pragma unroll
        for (int c = tid; c < (BK / 4) * DB4; c += 256) {
            const int kb4 = c / DB4, db4 = c % DB4;
            uint2 rv[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int64_t key = kb0 + kb4 * 4 + rr;
                rv[rr] = key < N ? *reinterpret_cast<const uint2*>(Vh + key * D + db4 * 4) : make_uint2(0, 0);
            }
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int sh = (cc & 1) * 16;
                const uint32_t x0 = ((cc < 2 ? rv[0].x : rv[0].y) >> sh) & 0xffffu;
                const uint32_t x1 = ((cc < 2 ? rv[1].x : rv[1].y) >> sh) & 0xffffu;
                const uint32_t x2 = ((cc < 2 ? rv[2].x : rv[2].y) >> sh) & 0xffffu;
                const uint32_t x3 = ((cc < 2 ? rv[3].x : rv[3].y) >> sh) & 0xffffu;
                *reinterpret_cast<uint2*>(Vt + (db4 * 4 + cc) * VSTR + kb4 * 4) =
                    make_uint2(x0 | (x1 << 16), x2 | (x3 << 16));
            }
        }
        __syncthreads();
        if (!wave_rows) {
            if (a.pv_skip && lane == 0) a.pv_skip[int64_t(e) * 4 + wave] = 0;
            continue;
        }

        // ---- S^T = K Q^T (keys x queries)
        floatx16 sacc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(Ks + (32 * mt + l32) * KSTR + ks * 16 + half * 8);
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
            }
        }
        // ---- online softmax for query row qrow (log2 domain)
        float smax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t key = kb0 + 32 * mt + 8 * (i >> 2) + 4 * half + (i & 3);
                const bool ok = key < N && (!a.causal || key <= qrow);
                const float s = ok ? sacc[mt][i] * c2 : -INFINITY;
                sacc[mt][i] = s;
                smax = fmaxf(smax, s);
            }
        smax = fmaxf(smax, __shfl_xor(smax, 32));
        const float m_new = fmaxf(m_run, smax);
        bool skip = false;
        if (lam_on) {
            float gap = (row_valid && smax > -INFINITY) ? smax - m_new : -INFINITY;
            gap = wave_max(gap);
            skip = gap < lam2;
        }
        const float msafe = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - msafe);
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(sacc[mt][i] - msafe);
                sacc[mt][i] = p;
                psum += p;
            }
        l_part = l_part * alpha + psum;
        m_run = m_new;
        if (a.pv_skip && lane == 0) a.pv_skip[int64_t(e) * 4 + wave] = skip ? 1 : 0;
        if (skip) {
            ++n_skip;
            continue;
        }
        ++n_exec;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[t][i] *= alpha;
        bf16x8_t pb[PS];
#pragma unroll
        for (int ps = 0; ps < PS; ++ps)
#pragma unroll
            for (int x = 0; x < 8; ++x) pb[ps][x] = (__bf16)sacc[ps >> 1][8 * (ps & 1) + x];
        // ---- O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int ps = 0; ps < PS; ++ps) {
                const uint16_t* vp = Vt + (32 * t + l32) * VSTR + ps * 16 + 4 * half;
                const uint2 lo = *reinterpret_cast<const uint2*>(vp);
                const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
                const bf16x8_t vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[ps], oacc[t], 0, 0, 0);
            }
    }

    // ---- epilogue: O / l
    const float l_tot = l_part + __shfl_xor(l_part, 32);
    if (row_valid) {
        const float inv = 1.0f / l_tot;  // l = 0 (no key) -> 0 * inf = NaN
        if (l_tot == 0.f) *a.dev_status = SA_ERR_EMPTY_ROW;
        float* orow = Oh + qrow * D;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float4 v;
                v.x = oacc[t][4 * g + 0] * inv;
                v.y = oacc[t][4 * g + 1] * inv;
                v.z = oacc[t][4 * g + 2] * inv;
                v.w = oacc[t][4 * g + 3] * inv;
                *reinterpret_cast<float4*>(orow + 32 * t + 8 * g + 4 * half) = v;
            }
    }
    if (a.counters) {
        if (tid == 0) atomicAdd(&a.counters[0], (unsigned long long)(e1 > e0 ? e1 - e0 : 0));
        if (lane == 0 && wave_rows) {
            atomicAdd(&a.counters[1], (unsigned long long)n_exec);
            atomicAdd(&a.counters[2], (unsigned long long)n_skip);
        }
    }
}

// 16x16 blocks: thread (r, c) owns query row r of the block and output
// columns c, c+16, ...; scores go through LDS.  The whole 16-row block is one
// PV-skip group.
template <int D>
__global__ __launch_bounds__(256) void k_flash_small(FlashArgs a) {
    constexpr int B = 16;
    __shared__ float Qs[B][D + 1];
    __shared__ float Ks[B][D + 1];
    __shared__ float Vs[B][D + 1];
    __shared__ float Ss[B][B + 1];
    __shared__ float gaps[B];

    const int row = blockIdx.x;
    const int qb = row % a.n_qb;
    const int bh = row / a.n_qb;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int64_t N = a.N;
    const uint16_t* Qh = a.q + int64_t(bh) * N * D;
    const uint16_t* Kh = a.k + (int64_t(b) * a.Hkv + hk) * N * D;
    const uint16_t* Vh = a.v + (int64_t(b) * a.Hkv + hk) * N * D;
    float* Oh = a.o + int64_t(bh) * N * D;

    const int tid = threadIdx.x;
    const int r = tid / B, c = tid % B;
    const int64_t qrow = int64_t(qb) * B + r;
    const bool valid = qrow < N;
    for (int t = tid; t < B * D; t += 256) {
        const int rr = t / D, dd = t % D;
        const int64_t qq = int64_t(qb) * B + rr;
        Qs[rr][dd] = qq < N ? __uint_as_float(uint32_t(Qh[qq * D + dd]) << 16) : 0.f;
    }
    float m = -INFINITY, l = 0.f;
    float O[D / B];
#pragma unroll
    for (int u = 0; u < D / B; ++u) O[u] = 0.f;
    const bool lam_on = a.lambda > -INFINITY;
    int n_exec = 0, n_skip = 0;
    const int e0 = a.row_ptr[row];
    int e1 = a.row_ptr[row + 1];
    if (e1 > a.col_cap) {
        if (tid == 0) *a.dev_status = SA_ERR_CAPACITY;
        e1 = int(a.col_cap);
    }
    for (int e = e0; e < e1; ++e) {
        const int jblk = a.col_idx[e];
        if (jblk < 0 || jblk >= a.n_kb) {
            if (tid == 0) *a.dev_status = SA_ERR_INVALID_ARGUMENT;
            continue;
        }
        const int64_t kb0 = int64_t(jblk) * B;
        __syncthreads();
        for (int t = tid; t < B * D; t += 256) {
            const int rr = t / D, dd = t % D;
            const int64_t key = kb0 + rr;
            Ks[rr][dd] = key < N ? __uint_as_float(uint32_t(Kh[key * D + dd]) << 16) : 0.f;
            Vs[rr][dd] = key < N ? __uint_as_float(uint32_t(Vh[key * D + dd]) << 16) : 0.f;
        }
        __syncthreads();
        const int64_t key = kb0 + c;
        float s = 0.f;
        for (int d = 0; d < D; ++d) s = fmaf(Qs[r][d], Ks[c][d], s);
        const bool ok = key < N && (!a.causal || key <= qrow);
        Ss[r][c] = ok ? s * a.scale : -INFINITY;
        __syncthreads();
        float rmax = -INFINITY;
        for (int kk = 0; kk < B; ++kk) rmax = fmaxf(rmax, Ss[r][kk]);
        const float m_new = fmaxf(m, rmax);
        if (c == 0) gaps[r] = (valid && rmax > -INFINITY) ? rmax - m_new : -INFINITY;
        __syncthreads();
        bool skip = false;
        if (lam_on) {
            float gmax = -INFINITY;
            for (int kk = 0; kk < B; ++kk) gmax = fmaxf(gmax, gaps[kk]);
            skip = gmax < a.lambda;
        }
        const float msafe = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = expf(m - msafe);
        float p[B];
        float ps = 0.f;
        for (int kk = 0; kk < B; ++kk) {
            p[kk] = expf(Ss[r][kk] - msafe);
            ps += p[kk];
        }
        l = l * alpha + ps;
        m = m_new;
        if (!skip) {
#pragma unroll
            for (int u = 0; u < D / B; ++u) {
                float acc = O[u] * alpha;
                for (int kk = 0; kk < B; ++kk) acc = fmaf(p[kk], Vs[kk][c + B * u], acc);
                O[u] = acc;
            }
        }
        if (tid == 0) {
            if (a.pv_skip) a.pv_skip[e] = skip ? 1 : 0;
            n_exec += skip ? 0 : 1;
            n_skip += skip ? 1 : 0;
        }
    }
    if (valid) {
        const float inv = 1.0f / l;
        if (l == 0.f) *a.dev_status = SA_ERR_EMPTY_ROW;
#pragma unroll
        for (int u = 0; u < D / B; ++u) Oh[qrow * D + c + B * u] = O[u] * inv;
    }
    if (a.counters && tid == 0) {
        atomicAdd(&a.counters[0], (unsigned long long)(e1 > e0 ? e1 - e0 : 0));
        atomicAdd(&a.counters[1], (unsigned long long)n_exec);
        atomicAdd(&a.counters[2], (unsigned long long)n_skip);
    }
}

}  // namespace

hipError_t launch_flash(const FlashArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(k_attn_init, dim3(1), dim3(1), 0, stream, a.dev_status, a.counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = int64_t(a.B) * a.Hq * a.n_qb;
    if (rows > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid{unsigned(rows), 1, 1};
    const dim3 block{256, 1, 1};
    if (a.bq == 16 && a.bk == 16) {
        if (a.D == 128) hipLaunchKernelGGL(k_flash_small<128>, grid, block, 0, stream, a);
        else hipLaunchKernelGGL(k_flash_small<64>, grid, block, 0, stream, a);
    } else if (a.bk == 64) {
        if (a.D == 128) hipLaunchKernelGGL((k_flash_mfma<128, 64>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((k_flash_mfma<64, 64>), grid, block, 0, stream, a);
    } else {
        if (a.D == 128) hipLaunchKernelGGL((k_flash_mfma<128, 128>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((k_flash_mfma<64, 128>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace sa
