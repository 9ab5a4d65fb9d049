// Block-mask prediction kernels (SpargeAttn notes, section 2.2, selective
// token compression; MindIE-SD "稀疏" page, rf_v2 block representatives and
// sinks; "44. Local Sliding and Sparse Attention", Step 2 causal window).
//
//   k_block_stats  one streaming pass over Q and K: per block the mean token
//                  and the mean pairwise cosine ||mean_t x_t/||x_t||||^2.
//                  HBM-bound: every byte of Q and K is read exactly once.
//   k_topcdf       per group of 16 query blocks of one head: compressed
//                  scores against every key-block mean on the fp32 matrix
//                  cores, then per query block (one wavefront each) the
//                  guard/sink/window forcing, the softmax over the candidates,
//                  an exact radix selection for TopCdf and the keep floor, the
//                  dense mask row, its kept count and the group's total.
//   k_csr          per group: row offsets from the group totals, then the
//                  ascending column lists from the mask rows (ballot compaction).
#include <cfloat>

#include "sa_internal.h"

namespace sa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
__device__ inline long long wave_sum_ll(long long v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

// DPP lane move; lanes without a source (or in a disabled row) read 0.
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline uint32_t dpp(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, ROW_MASK, 0xf, false));
}
template <int CTRL>
__device__ inline float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of CH (8 or 16) lanes; every lane of a group ends
// with the same value.
template <int CH>
__device__ inline float group_sum(float v) {
    v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dppf<0x141>(v);  // row_half_mirror: the other quad of the 8
    if constexpr (CH == 16) v += dppf<0x140>(v);  // row_mirror: the other 8 of the 16
    return v;
}

// Inclusive prefix sum over the 64 lanes, in lane order.
__device__ inline uint32_t wave_incl_scan(uint32_t v) {
    v += dpp<0x111>(v);       // row_shr:1
    v += dpp<0x112>(v);       // row_shr:2
    v += dpp<0x114>(v);       // row_shr:4
    v += dpp<0x118>(v);       // row_shr:8
    v += dpp<0x142, 0xa>(v);  // row_bcast:15 -> rows 1 and 3
    v += dpp<0x143, 0xc>(v);  // row_bcast:31 -> rows 2 and 3
    return v;
}

// Orders this wavefront's LDS accesses: every lane's earlier LDS operation is
// complete before any lane's later one starts.
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- block stats
// One wavefront per block, four blocks per workgroup, no LDS and no barriers.
// A token row of D bf16 is split in CH = D/8 chunks of 16 bytes held by CH
// consecutive lanes, so a wave covers 64/CH rows per step; eight steps of
// loads are issued before any is consumed.  Squared norms come from the
// bf16 dot-product instruction (exact products, fp32 accumulation) and are
// summed over the CH lanes of a row with DPP; the per-row-slot sums are
// reduced across the wave once at the end.
template <int D>
__global__ __launch_bounds__(256) void k_block_stats(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k, int64_t N,
                                                     int bq, int bk, int64_t q_blocks, int64_t all_blocks,
                                                     int n_qb, int n_kb, float* __restrict__ qbar,
                                                     float* __restrict__ kbar, float* __restrict__ simq,
                                                     float* __restrict__ simk, int32_t* dev_status) {
    constexpr int CH = D / 8;
    constexpr int RPW = 64 / CH;   // rows per wave step
    constexpr int U = 8;           // steps in flight
    if (blockIdx.x == 0 && threadIdx.x == 0) *dev_status = SA_OK;
    const int lane = threadIdx.x & 63;
    const int64_t blk = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (blk >= all_blocks) return;
    const bool is_q = blk < q_blocks;
    const int64_t local = is_q ? blk : blk - q_blocks;
    const int nb = is_q ? n_qb : n_kb;
    const int b = is_q ? bq : bk;
    const int64_t bh = local / nb;
    const int j = int(local - bh * nb);
    const int64_t t0 = int64_t(j) * b;
    const int len = int(min(int64_t(b), N - t0));
    const uint16_t* src = (is_q ? q : k) + (bh * N + t0) * D;
    const int ch = lane % CH;
    const int slot = lane / CH;

    float ax[8], au[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ax[e] = au[e] = 0.f;
    for (int r0 = 0; r0 < len; r0 += U * RPW) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * RPW + slot;
            raw[u] = r < len ? *(reinterpret_cast<const uint4*>(src + int64_t(r) * D) + ch) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bf16x2 h = __builtin_bit_cast(bf16x2, w[c]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(h, h, ss, false);
            }
            ss = group_sum<CH>(ss);
            const float inv = ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;  // zero rows (and padding) add nothing
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float lo = __uint_as_float(w[c] << 16);
                const float hi = __uint_as_float(w[c] & 0xffff0000u);
                ax[2 * c] += lo;
                ax[2 * c + 1] += hi;
                au[2 * c] = fmaf(lo, inv, au[2 * c]);
                au[2 * c + 1] = fmaf(hi, inv, au[2 * c + 1]);
            }
        }
    }
    // sum the RPW row slots: lanes ch, ch+CH, ... hold the same columns
#pragma unroll
    for (int m = CH; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ax[e] += __shfl_xor(ax[e], m);
            au[e] += __shfl_xor(au[e], m);
        }
    const float inv_len = 1.0f / float(len);
    float um2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float um = au[e] * inv_len;
        um2 = fmaf(um, um, um2);
    }
    um2 = group_sum<CH>(um2);
    if (slot == 0) {
        float4* outm = reinterpret_cast<float4*>((is_q ? qbar : kbar) + local * D + ch * 8);
        outm[0] = make_float4(ax[0] * inv_len, ax[1] * inv_len, ax[2] * inv_len, ax[3] * inv_len);
        outm[1] = make_float4(ax[4] * inv_len, ax[5] * inv_len, ax[6] * inv_len, ax[7] * inv_len);
        if (lane == 0) (is_q ? simq : simk)[local] = um2;
    }
}

// ---------------------------------------------------------------- TopCdf
constexpr int kGroupRows = 16;  // query blocks per workgroup: the N side of the score MFMA

// Row stride (floats) of the LDS score tile: a multiple of 64 plus 4, so the
// 16 rows written by one float4 store land on 16 different bank quads.
inline int score_stride(int n_kb) { return (n_kb + 63) / 64 * 64 + 4; }

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

// Probabilities in fixed point: P = floor(p * 2^31).  The candidates'
// probabilities sum to 1 up to fp32 rounding, so every partial sum of P fits
// in 32 bits, sums are exact and the cumulative mass is monotone; the
// truncation moves a prefix sum by less than n_kb * 2^-31.
constexpr float kFix = 2147483648.0f;
constexpr double kFixD = 2147483648.0;

// Radix digits of the selection keys (probability bits + 1 < 2^30):
// bits 29..22, 21..14, 13..6, 5..0.
__device__ inline int digit_shift(int lv) { return lv == 3 ? 0 : 22 - 8 * lv; }
__device__ inline int digit_width(int lv) { return lv == 3 ? 6 : 8; }

// In the histogram scan lane l owns digits 255-4l .. 252-4l (highest first).
// Finds the first digit, in descending order, at which base + the inclusive
// cumulative value reaches `target`; returns false when none does.
// val(x) extracts the scanned quantity from a bin, cnt(x) the bin count.
struct ScanHit {
    uint32_t digit, before, count_before, bin_count;
};

template <typename Val, typename Cnt>
__device__ inline bool scan_digits(const uint32_t (&vb)[4], const uint32_t (&cb)[4], uint32_t base,
                                   uint32_t target, int lane, Val val, Cnt cnt, ScanHit& out) {
    uint32_t lv = 0, lc = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        lv += val(vb[t]);
        lc += cnt(cb[t]);
    }
    const uint32_t iv = wave_incl_scan(lv);
    const uint32_t ic = wave_incl_scan(lc);
    const unsigned long long hit = __ballot(base + iv >= target);
    if (hit == 0ull) return false;
    const int hl = __ffsll(static_cast<long long>(hit)) - 1;
    uint32_t run = iv - lv, runc = ic - lc;
    uint32_t pos = 3, bef = run, befc = runc, bc = 0;
    bool done = false;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if (!done && base + run + val(vb[t]) >= target) {
            pos = t;
            bef = run;
            befc = runc;
            bc = cnt(cb[t]);
            done = true;
        }
        run += val(vb[t]);
        runc += cnt(cb[t]);
    }
    const uint32_t dg = 255u - 4u * uint32_t(lane) - pos;
    out.digit = __builtin_amdgcn_readlane(dg, hl);
    out.before = __builtin_amdgcn_readlane(bef, hl);
    out.count_before = __builtin_amdgcn_readlane(befc, hl);
    out.bin_count = __builtin_amdgcn_readlane(bc, hl);
    return true;
}

// One query block (row i of head bh) on one wavefront.  Element r of lane l is
// key block j = 64 r + l.  Candidates are ordered by probability descending,
// ties by block index ascending; TopCdf keeps the shortest prefix whose mass
// reaches tau, the floor keeps at least `extra` candidates.  Both cut points
// are found exactly with four histogram passes over the radix digits of the
// probability bits (the TopCdf search carries the mass per bin, the floor
// search the count), so no sort is needed.  Returns the row's kept count.
template <int EPL>
__device__ int select_row(const TopCdfArgs& a, int bh, int i, const float* lrow, const float* simk,
                          uint32_t* hCX, uint32_t* hS, int lane) {
    const RowGeom g = row_geom(a, i);
    const int64_t row = int64_t(bh) * a.n_qb + i;
    const bool forced_row = a.theta > 0.f && a.simq[row] < a.theta;

    float e[EPL];
    uint32_t fbits = 0, cbits = 0;
    float cmax = -FLT_MAX;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        e[r] = 0.f;
        if (r * 64 < g.nv) {
            const int j = r * 64 + lane;
            if (j < g.nv) {
                const float l = lrow[j];
                e[r] = l;
                if (forced_block(a, g, j, simk[j])) {
                    fbits |= 1u << r;
                } else {
                    cbits |= 1u << r;
                    cmax = fmaxf(cmax, l);
                }
            }
        }
    }
    cmax = wave_max(cmax);
    const int n_forced = wave_sum_i(__popc(fbits));
    const int n_cand = wave_sum_i(__popc(cbits));
    float esum = 0.f;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        if ((cbits >> r) & 1u) {
            e[r] = expf(e[r] - cmax);
            esum += e[r];
        }
    }
    esum = wave_sum(esum);
    const float inv_sum = 1.0f / esum;
    uint32_t key[EPL], P[EPL];
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const bool c = (cbits >> r) & 1u;
        const float p = c ? e[r] * inv_sum : 0.f;
        key[r] = c ? __float_as_uint(p) + 1u : 0u;
        P[r] = c ? uint32_t(p * kFix) : 0u;
    }

    int k_cdf = 0;
    bool c_on = false, c_all = false;
    uint32_t T = 0;
    if (a.tau_d >= 1.0) {
        k_cdf = n_cand;
    } else if (a.tau_d > 0.0 && n_cand > 0) {
        c_on = true;
        T = max(1u, uint32_t(ceil(a.tau_d * kFixD)));
    }
    int extra = 0;
    if (a.sparsity >= 0.0) extra = max(0, int(ceil((1.0 - a.sparsity) * double(g.nv))) - n_forced);
    bool x_on = extra > 0 && extra < n_cand;
    uint32_t c_pref = 0, c_acc = 0, c_cnt = 0, c_grp = 0;
    uint32_t x_pref = 0, x_rem = uint32_t(extra);

    for (int lv = 0; lv < 4 && (c_on || x_on); ++lv) {
        const int sh = digit_shift(lv), w = digit_width(lv);
        reinterpret_cast<uint4*>(hCX)[lane] = make_uint4(0, 0, 0, 0);
        reinterpret_cast<uint4*>(hS)[lane] = make_uint4(0, 0, 0, 0);
        wave_lds_sync();
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
            if (r * 64 < g.nv) {
                const uint32_t kk = key[r];
                const uint32_t hi = kk >> (sh + w);
                const uint32_t d = (kk >> sh) & ((1u << w) - 1u);
                const bool mc = c_on && kk != 0u && hi == c_pref;
                const bool mx = x_on && kk != 0u && hi == x_pref;
                if (mc || mx) atomicAdd(&hCX[d], (mc ? 1u : 0u) + (mx ? 65536u : 0u));
                if (mc) atomicAdd(&hS[d], P[r]);
            }
        }
        wave_lds_sync();
        const uint4 cx4 = reinterpret_cast<const uint4*>(hCX)[63 - lane];
        const uint4 s4 = reinterpret_cast<const uint4*>(hS)[63 - lane];
        const uint32_t cx[4] = {cx4.w, cx4.z, cx4.y, cx4.x};  // descending digits
        const uint32_t sv[4] = {s4.w, s4.z, s4.y, s4.x};
        if (c_on) {
            ScanHit h;
            const bool found = scan_digits(sv, cx, c_acc, T, lane, [](uint32_t x) { return x; },
                                           [](uint32_t x) { return x & 0xffffu; }, h);
            if (!found) {  // the candidates' whole mass stays below tau (first level only)
                c_on = false;
                c_all = true;
            } else {
                c_acc += h.before;
                c_cnt += h.count_before;
                c_pref = (c_pref << w) | h.digit;
                c_grp = h.bin_count;
            }
        }
        if (x_on) {
            ScanHit h;
            scan_digits(cx, cx, 0u, x_rem, lane, [](uint32_t x) { return x >> 16; },
                        [](uint32_t x) { return x >> 16; }, h);
            x_rem -= h.before;
            x_pref = (x_pref << w) | h.digit;
        }
    }
    if (c_on) {
        // c_pref is the key at which the cumulative mass reaches tau; it is
        // shared by c_grp candidates of equal P, taken in index order
        const uint32_t Pv = uint32_t(__uint_as_float(c_pref - 1u) * kFix);
        const uint32_t need = T - c_acc;
        uint32_t m = Pv ? (need - 1u) / Pv : c_grp - 1u;
        m = min(m, c_grp - 1u);
        k_cdf = int(c_cnt + m + 1u);
    } else if (c_all) {
        k_cdf = n_cand;
    }
    const int keep = min(n_cand, max(k_cdf, extra));

    uint32_t kbits = 0;
    if (!forced_row && keep > 0) {
        if (keep == n_cand) {
            kbits = cbits;
        } else {
            uint32_t v_thr, quota;
            if (keep == k_cdf) {
                v_thr = c_pref;
                quota = uint32_t(k_cdf) - c_cnt;
            } else {
                v_thr = x_pref;
                quota = x_rem;
            }
            const unsigned long long below = (1ull << lane) - 1ull;
            uint32_t run = 0;
#pragma unroll
            for (int r = 0; r < EPL; ++r) {
                if (r * 64 < g.nv) {
                    const bool gt = key[r] > v_thr;
                    const bool eq = key[r] == v_thr;
                    const unsigned long long eqm = __ballot(eq);
                    const uint32_t rank = run + uint32_t(__popcll(eqm & below));
                    if (gt || (eq && rank < quota)) kbits |= 1u << r;
                    run += uint32_t(__popcll(eqm));
                }
            }
        }
    }
    uint8_t* out = a.mask + row * a.n_kb;
    const uint32_t bits = fbits | kbits;
#pragma unroll
    for (int r = 0; r < EPL; ++r) {
        const int j = r * 64 + lane;
        if (r * 64 < a.n_kb && j < a.n_kb) out[j] = forced_row ? uint8_t(j < g.nv) : uint8_t((bits >> r) & 1u);
    }
    const int cnt = forced_row ? g.nv : n_forced + keep;
    if (lane == 0) a.counts[row] = cnt;
    return cnt;
}

// Dynamic LDS: scores[16][ls] f32 | per wave: counts[256] u32 (TopCdf search
// in the low half, floor search in the high half) and masses[256] u32.
template <int D, int EPL>
__global__ __launch_bounds__(256) void k_topcdf(TopCdfArgs a, int ls) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int32_t wave_tot[4];
    float* scores = reinterpret_cast<float*>(smem);
    uint32_t* hist = reinterpret_cast<uint32_t*>(scores + kGroupRows * ls);

    const int groups = (a.n_qb + kGroupRows - 1) / kGroupRows;
    const int bh = blockIdx.x / groups;  // b * Hq + hq
    const int i0 = (blockIdx.x - bh * groups) * kGroupRows;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int64_t kvh = int64_t(b) * a.Hkv + hk;
    const float* kbar = a.kbar + kvh * a.n_kb * D;
    const float* simk = a.simk + kvh * a.n_kb;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i_last = min(i0 + kGroupRows, a.n_qb) - 1;
    const int ncols = row_geom(a, i_last).nv;  // columns any row of the group can see

    // ---- compressed scores on v_mfma_f32_16x16x4_f32: A = 16 key-block means
    // (rows), B = the group's 16 query-block means (columns).  Lane l feeds
    // operand slot l/16 of row/column l%16; head-dim entry 16c + 4(l/16) + e
    // goes to step (c, e), so each lane reads float4s of contiguous entries.
    // The result lands as query row l%16, key blocks 4(l/16)..+3 of the tile.
    {
        constexpr int C = D / 16;
        const int r16 = lane & 15;
        const int sub = lane >> 4;
        f32x4 qv[C];
        const float* qs = a.qbar + (int64_t(bh) * a.n_qb + min(i0 + r16, a.n_qb - 1)) * D + 4 * sub;
#pragma unroll
        for (int c = 0; c < C; ++c) qv[c] = *reinterpret_cast<const f32x4*>(qs + 16 * c);
        const int ntile = (ncols + 15) >> 4;
        f32x4 kv[C];
        auto load_k = [&](int t) {
            const float* ks = kbar + int64_t(min(t * 16 + r16, ncols - 1)) * D + 4 * sub;
#pragma unroll
            for (int c = 0; c < C; ++c) kv[c] = *reinterpret_cast<const f32x4*>(ks + 16 * c);
        };
        if (wave < ntile) load_k(wave);
        for (int t = wave; t < ntile; t += 4) {
            f32x4 kc[C];
#pragma unroll
            for (int c = 0; c < C; ++c) kc[c] = kv[c];
            if (t + 4 < ntile) load_k(t + 4);
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < C; c += 2)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[c][e], qv[c][e], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kc[c + 1][e], qv[c + 1][e], acc1, 0, 0, 0);
                }
            const f32x4 s = (acc0 + acc1) * a.scale;
            *reinterpret_cast<f32x4*>(scores + r16 * ls + t * 16 + 4 * sub) = s;
        }
    }
    __syncthreads();

    uint32_t* hCX = hist + wave * 512;
    uint32_t* hS = hCX + 256;
    int tot = 0;
    for (int rr = wave; rr < kGroupRows; rr += 4) {
        const int i = i0 + rr;
        if (i >= a.n_qb) break;
        tot += select_row<EPL>(a, bh, i, scores + rr * ls, simk, hCX, hS, lane);
    }
    if (lane == 0) wave_tot[wave] = tot;
    __syncthreads();
    if (threadIdx.x == 0) a.group_tot[blockIdx.x] = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
}

// ---------------------------------------------------------------- CSR
// One workgroup per group of 16 query blocks (the TopCdf grouping).  Its
// first row offset is the sum of the totals of all earlier groups; the
// group's own rows are scanned by one wavefront; then each wavefront
// compacts four mask rows into ascending column lists.
constexpr int kMaxWordsPerLane = SA_MAX_KEY_BLOCKS / 256;

__global__ __launch_bounds__(256) void k_csr(const uint8_t* __restrict__ mask, const int32_t* __restrict__ counts,
                                             const int32_t* __restrict__ group_tot, int n_groups,
                                             int groups_per_head, int n_qb, int n_kb, int64_t rows,
                                             int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                             int64_t col_cap, int32_t* dev_status) {
    __shared__ long long red[4];
    __shared__ long long rp[kGroupRows + 1];
    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    long long s = 0;
    for (int t = tid; t < g; t += 256) s += group_tot[t];
    s = wave_sum_ll(s);
    if (lane == 0) red[wave] = s;
    const int bh = g / groups_per_head;
    const int i0 = (g - bh * groups_per_head) * kGroupRows;
    const int nr = min(kGroupRows, n_qb - i0);
    const int64_t r0 = int64_t(bh) * n_qb + i0;
    __syncthreads();
    if (wave == 0) {
        const long long base = red[0] + red[1] + red[2] + red[3];
        const uint32_t c = lane < nr ? uint32_t(counts[r0 + lane]) : 0u;
        const uint32_t incl = wave_incl_scan(c);
        if (lane < nr) rp[lane] = base + (incl - c);
        if (lane == nr - 1) rp[kGroupRows] = base + incl;
    }
    __syncthreads();
    if (tid < nr) row_ptr[r0 + tid] = int32_t(rp[tid]);
    if (g == n_groups - 1 && tid == 0) {
        row_ptr[rows] = int32_t(rp[kGroupRows]);
        if (rp[kGroupRows] > col_cap) *dev_status = SA_ERR_CAPACITY;
    }

    const unsigned long long below = (1ull << lane) - 1ull;
    if ((n_kb & 3) == 0) {
        // 4 columns per lane per word: column 4(64w + lane) + byte
        const int nw = (n_kb + 255) / 256;
        uint32_t wd[4][kMaxWordsPerLane];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = wave + 4 * q;
            const uint32_t* m = reinterpret_cast<const uint32_t*>(mask + (r0 + min(rr, nr - 1)) * n_kb);
#pragma unroll
            for (int w = 0; w < kMaxWordsPerLane; ++w) {
                const int jw = w * 64 + lane;
                wd[q][w] = (rr < nr && w < nw && 4 * jw < n_kb) ? m[jw] : 0u;
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = wave + 4 * q;
            if (rr >= nr) break;
            long long pos = rp[rr];
#pragma unroll
            for (int w = 0; w < kMaxWordsPerLane; ++w) {
                if (w >= nw) break;
                const uint32_t x = wd[q][w];
                const bool f0 = (x & 0xffu) != 0, f1 = (x & 0xff00u) != 0;
                const bool f2 = (x & 0xff0000u) != 0, f3 = (x & 0xff000000u) != 0;
                const unsigned long long b0 = __ballot(f0), b1 = __ballot(f1), b2 = __ballot(f2), b3 = __ballot(f3);
                long long p = pos + __popcll(b0 & below) + __popcll(b1 & below) + __popcll(b2 & below) +
                              __popcll(b3 & below);
                const int j = 4 * (w * 64 + lane);
                if (f0) { if (p < col_cap) col_idx[p] = j; ++p; }
                if (f1) { if (p < col_cap) col_idx[p] = j + 1; ++p; }
                if (f2) { if (p < col_cap) col_idx[p] = j + 2; ++p; }
                if (f3) { if (p < col_cap) col_idx[p] = j + 3; }
                pos += __popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3);
            }
        }
    } else {
        for (int rr = wave; rr < nr; rr += 4) {
            const uint8_t* m = mask + (r0 + rr) * n_kb;
            long long pos = rp[rr];
            for (int j0 = 0; j0 < n_kb; j0 += 64) {
                const int j = j0 + lane;
                const bool on = j < n_kb && m[j];
                const unsigned long long bal = __ballot(on);
                const long long p = pos + __popcll(bal & below);
                if (on && p < col_cap) col_idx[p] = j;
                pos += __popcll(bal);
            }
        }
    }
}

template <int D, int EPL>
hipError_t launch_topcdf_t(const TopCdfArgs& a, unsigned nwg, size_t lds, int ls, hipStream_t stream) {
    hipLaunchKernelGGL((k_topcdf<D, EPL>), dim3(nwg), dim3(256), lds, stream, a, ls);
    return hipGetLastError();
}

template <int D>
hipError_t launch_topcdf_d(const TopCdfArgs& a, unsigned nwg, size_t lds, int ls, hipStream_t stream) {
    if (a.n_kb <= 64) return launch_topcdf_t<D, 1>(a, nwg, lds, ls, stream);
    if (a.n_kb <= 256) return launch_topcdf_t<D, 4>(a, nwg, lds, ls, stream);
    if (a.n_kb <= 512) return launch_topcdf_t<D, 8>(a, nwg, lds, ls, stream);
    if (a.n_kb <= 1024) return launch_topcdf_t<D, 16>(a, nwg, lds, ls, stream);
    return launch_topcdf_t<D, 32>(a, nwg, lds, ls, stream);
}

}  // namespace

int64_t topcdf_groups(int64_t bh, int64_t n_qb) { return bh * ((n_qb + kGroupRows - 1) / kGroupRows); }

hipError_t launch_block_stats(const uint16_t* q, const uint16_t* k, const PredictShape& s, float* qbar,
                              float* kbar, float* simq, float* simk, int32_t* dev_status,
                              hipStream_t stream) {
    const int64_t qb = int64_t(s.B) * s.Hq * s.n_qb;
    const int64_t kb = int64_t(s.B) * s.Hkv * s.n_kb;
    const int64_t wgs = (qb + kb + 3) / 4;
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid{unsigned(wgs), 1, 1};
    if (s.D == 128)
        hipLaunchKernelGGL(k_block_stats<128>, grid, dim3(256), 0, stream, q, k, s.N, s.bq, s.bk, qb, qb + kb,
                           int(s.n_qb), int(s.n_kb), qbar, kbar, simq, simk, dev_status);
    else
        hipLaunchKernelGGL(k_block_stats<64>, grid, dim3(256), 0, stream, q, k, s.N, s.bq, s.bk, qb, qb + kb,
                           int(s.n_qb), int(s.n_kb), qbar, kbar, simq, simk, dev_status);
    return hipGetLastError();
}

hipError_t launch_topcdf(const TopCdfArgs& a, hipStream_t stream) {
    if (a.n_kb > SA_MAX_KEY_BLOCKS) return hipErrorInvalidValue;
    const int ls = score_stride(a.n_kb);
    const size_t lds = size_t(kGroupRows) * ls * 4 + size_t(4) * 512 * 4;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int64_t nwg = topcdf_groups(int64_t(a.B) * a.Hq, a.n_qb);
    if (nwg > INT32_MAX) return hipErrorInvalidValue;
    if (a.D == 128) return launch_topcdf_d<128>(a, unsigned(nwg), lds, ls, stream);
    return launch_topcdf_d<64>(a, unsigned(nwg), lds, ls, stream);
}

hipError_t launch_csr(const uint8_t* mask, const int32_t* counts, const int32_t* group_tot, int64_t bh,
                      int n_qb, int n_kb, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                      int32_t* dev_status, hipStream_t stream) {
    const int64_t n_groups = topcdf_groups(bh, n_qb);
    if (n_groups > INT32_MAX || n_kb > SA_MAX_KEY_BLOCKS) return hipErrorInvalidValue;
    const int gph = (n_qb + kGroupRows - 1) / kGroupRows;
    hipLaunchKernelGGL(k_csr, dim3(unsigned(n_groups)), dim3(256), 0, stream, mask, counts, group_tot,
                       int(n_groups), gph, n_qb, n_kb, bh * n_qb, row_ptr, col_idx, col_cap, dev_status);
    return hipGetLastError();
}

}  // namespace sa
