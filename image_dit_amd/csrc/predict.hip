// Block-mask prediction kernels (SpargeAttn notes, section 2.2, selective
// token compression; MindIE-SD "稀疏" page, rf_v2 block representatives and
// sinks; "44. Local Sliding and Sparse Attention", Step 2 causal window).
//
//   k_block_stats  one streaming pass over Q and K: per block the mean token
//                  and the mean pairwise cosine ||mean_t x_t/||x_t||||^2.
//                  HBM-bound: every byte of Q and K is read exactly once.
//   k_topcdf       per group of 8..16 query blocks of one head: compressed
//                  scores against every key-block mean on the fp32 matrix
//                  cores, then per query block (a wavefront takes two) the
//                  guard/sink/window forcing, the softmax over the candidates,
//                  an exact radix selection for TopCdf and the keep floor, the
//                  dense mask row, its kept count and the group's total.
//                  Each group's total is also added (a relaxed atomic) to
//                  the total of its super-group of kSuperGroups groups.
//   k_csr          per group: the first row offset from the super-group totals
//                  before it and the group totals before it in its own
//                  super-group (at most G/256 + 255 reads), the group's row
//                  offsets, then the ascending column lists from the mask rows
//                  (ballot compaction).
#include <cfloat>
#include <type_traits>

#include <climits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave-wide reductions without LDS traffic: DPP within each row of 16 lanes
// (quad swaps, then the other quad of 8, then the other 8 of 16), then the
// four row totals through read-lane.  The result is wave-uniform.
template <int CTRL>
__device__ inline uint32_t dpp_all(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xf, 0xf, false));
}
template <class T, class F>
__device__ inline T wave_reduce(T v, F op) {
    auto mv = [](T x, auto ctrl) {
        return __builtin_bit_cast(T, dpp_all<decltype(ctrl)::value>(__builtin_bit_cast(uint32_t, x)));
    };
    v = op(v, mv(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
    v = op(v, mv(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
    v = op(v, mv(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    v = op(v, mv(v, std::integral_constant<int, 0x140>{}));  // row_mirror
    auto rl = [](T x, int l) {
        return __builtin_bit_cast(T, uint32_t(__builtin_amdgcn_readlane(int(__builtin_bit_cast(uint32_t, x)), l)));
    };
    return op(op(rl(v, 0), rl(v, 16)), op(rl(v, 32), rl(v, 48)));
}
__device__ inline float wave_sum(float v) { return wave_reduce(v, [](float x, float y) { return x + y; }); }
__device__ inline float wave_max(float v) { return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); }); }
__device__ inline int wave_sum_i(int v) { return wave_reduce(v, [](int x, int y) { return x + y; }); }
__device__ inline uint32_t wave_max_u(uint32_t v) { return wave_reduce(v, [](uint32_t x, uint32_t y) { return max(x, y); }); }

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
// reduced across the wave once at the end.  GATHER: q and k stay in the
// original token order and row r of the reordered sequence is perm[r]; the
// source rows of the next step are loaded while the current one is consumed.
// QUANT: the same pass also finds each quantization block's largest magnitude
// (a query block; a 64-row half of a key block); then a second pass over the
// block's rows, read again while they are still in the caches, writes their
// E4M3 codes with the rule of k_quant_fp8, so the codes and scales equal that
// kernel's bit for bit.  (Keeping the block in registers instead, 190 VGPRs,
// reads every row once but runs slower at two waves per SIMD.)
template <int D, bool GATHER, bool QUANT>
__global__ __launch_bounds__(256) void k_block_stats(const uint16_t* __restrict__ q,
                                                     const uint16_t* __restrict__ k,
                                                     const int32_t* __restrict__ perm, int64_t N, int64_t Nk,
                                                     int bq, int bk, int64_t q_blocks, int64_t all_blocks,
                                                     int n_qb, int n_kb, float* __restrict__ qbar,
                                                     float* __restrict__ kbar, float* __restrict__ simq,
                                                     float* __restrict__ simk, int32_t* dev_status,
                                                     int32_t* super_tot, int n_super, Quant8 qz) {
    constexpr int CH = D / 8;
    constexpr int RPW = 64 / CH;   // rows per wave step
    constexpr int U = 8;           // steps in flight
    if (blockIdx.x == 0 && threadIdx.x == 0) *dev_status = SA_OK;
    // the super-group totals the TopCdf launch adds to (the grid has more workgroups)
    if (threadIdx.x == 0 && int64_t(blockIdx.x) < n_super) super_tot[blockIdx.x] = 0;
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
    const int64_t Ns = is_q ? N : Nk;  // tokens of this side's sequence
    const int len = int(min(int64_t(b), Ns - t0));
    const uint16_t* src = (is_q ? q : k) + (bh * Ns + (GATHER ? 0 : t0)) * D;
    const int ch = lane % CH;
    const int slot = lane / CH;
    // source rows of one step (rows past the block repeat its last row and are masked)
    auto step_rows = [&](int r0, int (&sr)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = min(r0 + u * RPW + slot, len - 1);
            if constexpr (GATHER) {
                const int32_t p = perm[t0 + r];
                sr[u] = (p >= 0 && p < N) ? p : -1;  // an entry outside 0..N-1 reads row 0
            } else {
                sr[u] = r;
            }
        }
    };
    int sr[U];
    step_rows(0, sr);

    float ax[8], au[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ax[e] = au[e] = 0.f;
    uint32_t amx[2] = {0u, 0u};  // QUANT: largest |x| (bf16 pattern) of rows 0..63 and 64..127
    // one row chunk (row r of the block; zeros past its end) into the sums
    auto consume = [&](const uint4& raw, int r) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        if constexpr (QUANT) {
            uint32_t m = 0u;
#pragma unroll
            for (int c = 0; c < 4; ++c) m = max(m, max(w[c] & 0x7fffu, (w[c] >> 16) & 0x7fffu));
            const int h = r >= 64 ? 1 : 0;  // blocks hold at most 128 rows
            amx[h] = max(amx[h], m);
        }
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
    };
    for (int r0 = 0; r0 < len; r0 += U * RPW) {
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + u * RPW + slot;
            const u32x4* p = reinterpret_cast<const u32x4*>(src + int64_t(max(sr[u], 0)) * D) + ch;
            u32x4 v;
            // streamed once: nontemporal, so the block rows do not displace cached data
            // (QUANT reads them again right after: plain loads keep them cached)
            if constexpr (QUANT) v = *p;
            else v = __builtin_nontemporal_load(p);
            raw[u] = r < len ? make_uint4(v.x, v.y, v.z, v.w) : make_uint4(0, 0, 0, 0);
        }
        if (r0 + U * RPW < len) step_rows(r0 + U * RPW, sr);
#pragma unroll
        for (int u = 0; u < U; ++u) consume(raw[u], r0 + u * RPW + slot);
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
    if constexpr (QUANT) {
        // one quantization block per query block; a key block is one or two 64-row blocks
        const int nh = is_q ? 1 : (len + kKeyQuantRows - 1) / kKeyQuantRows;
        float inv[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t mb = is_q ? max(wave_max_u(amx[0]), wave_max_u(amx[1])) : wave_max_u(amx[h]);
            const float amax = __uint_as_float(mb << 16);
            inv[h] = amax > 0.f ? 448.0f / amax : 0.f;
            if (lane == 0 && h < nh) {
                const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
                if (is_q) qz.q_scale[local] = sc;
                else qz.k_scale[bh * qz.n_kt + int64_t(j) * (bk / kKeyQuantRows) + h] = sc;
            }
        }
        uint8_t* dst = (is_q ? qz.q8 : qz.k8) + (bh * Ns + (GATHER ? 0 : t0)) * D;
        step_rows(0, sr);
        for (int r0 = 0; r0 < len; r0 += U * RPW) {
            uint4 raw[U];
            int rows[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 v = *(reinterpret_cast<const u32x4*>(src + int64_t(max(sr[u], 0)) * D) + ch);
                raw[u] = make_uint4(v.x, v.y, v.z, v.w);
                rows[u] = sr[u];
            }
            if (r0 + U * RPW < len) step_rows(r0 + U * RPW, sr);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = r0 + u * RPW + slot;
                if (r >= len) continue;
                const float iv = inv[is_q ? 0 : (r >= 64 ? 1 : 0)];
                const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
                float y[8];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    y[2 * c] = __uint_as_float(w[c] << 16) * iv;
                    y[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u) * iv;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(y[e], -448.0f), 448.0f);
                int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
                lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
                int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
                hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
                if (rows[u] >= 0)
                    *reinterpret_cast<uint2*>(dst + int64_t(rows[u]) * D + ch * 8) = make_uint2(uint32_t(lo), uint32_t(hi));
            }
        }
    }
}

// ---------------------------------------------------------------- TopCdf
constexpr int kGroupRows = 16;  // most query blocks per workgroup: the N side of the score MFMA

// Row stride (floats) of the LDS score tile: room for every key block plus a
// pad, an odd number of 16-byte quads, so the 16 rows written by one float4
// store land on 16 different bank quads.
inline int score_stride(int n_kb) {
    int ls = (n_kb + 3) / 4 * 4 + 4;
    if ((ls / 4) % 2 == 0) ls += 4;
    return ls;
}

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

// Forcing that does not depend on the query block: the similarity guard on
// the key block and the sink ranges.
__device__ inline bool column_forced(const TopCdfArgs& a, int j, float sk) {
    const int64_t k_first = int64_t(j) * a.bk;
    const int64_t k_end = min(k_first + a.bk, a.Nk);
    bool f = (a.theta > 0.f) && (sk < a.theta);
    f |= (a.sink_front > 0) && (k_first < a.sink_front);
    f |= (a.sink_back > 0) && (k_end > a.Nk - a.sink_back);
    return f;
}

// Causal forcing of key block j for a query block: its sliding window and
// the diagonal block(s) it overlaps.
__device__ inline bool causal_forced(const TopCdfArgs& a, const RowGeom& g, int j) {
    const int64_t k_first = int64_t(j) * a.bk;
    const int64_t k_end = min(k_first + a.bk, a.N);
    return ((a.window > 0) && (k_end - 1 >= g.q_first - a.window + 1)) ||
           ((k_first < g.q_end) && (k_end > g.q_first));
}

// Probabilities in fixed point: P = floor(p * 2^31).  The candidates'
// probabilities sum to 1 up to fp32 rounding, so every partial sum of P fits
// in 32 bits, sums are exact and the cumulative mass is monotone; the
// truncation moves a prefix sum by less than n_kb * 2^-31.
constexpr float kFix = 2147483648.0f;
constexpr float kLog2eF = 1.4426950408889634f;
constexpr double kFixD = 2147483648.0;

// Selection key of a candidate: its probability bits + 1 (so 0 < key < 2^30,
// ordered like the probability); 0 marks a block that is not a candidate and
// kForcedKey a forced one.  P is a function of the key.
constexpr uint32_t kForcedKey = 0x80000000u;
__device__ inline uint32_t key_mass(uint32_t key) { return uint32_t(__uint_as_float(key - 1u) * kFix); }
__device__ inline bool is_candidate(uint32_t key) { return key != 0u && key < kForcedKey; }

// Radix digits of the keys: bits 29..23, 22..16, 15..9, 8..2, 1..0 (128-bin
// histograms, so the histograms of a workgroup fit beside a long score row).
constexpr int kLevels = 5;
constexpr int kBins = 128;
__device__ inline int digit_shift(int lv) { return lv == kLevels - 1 ? 0 : 23 - 7 * lv; }
__device__ inline int digit_width(int lv) { return lv == kLevels - 1 ? 2 : 7; }

// Histogram bins hold a count and a fixed-point mass together: count in the
// high word, mass in the low word.  A bin's mass is a sum of candidate masses,
// below 2^32 (see kFix), so one 64-bit add updates both without a carry
// between them.
struct BinHit {
    uint32_t digit;        // the bin where the target is reached
    uint32_t cnt_before;   // candidates in the bins above it
    uint32_t mass_before;  // their mass
    uint32_t bin_cnt;      // candidates in the bin
    uint32_t bin_mass;     // their mass
};

// In the histogram scan lane l owns digits 127-2l and 126-2l (highest first).
// Finds the first digit, in descending order, at which base + the inclusive
// cumulative mass (BY_MASS) or count reaches `target`; returns false when none
// does.
template <bool BY_MASS>
__device__ inline bool scan_bins(const unsigned long long* hist, uint32_t base, uint32_t target, int lane,
                                 BinHit& h) {
    const uint4 h2 = *reinterpret_cast<const uint4*>(hist + kBins - 2 - 2 * lane);  // digits 126-2l, 127-2l
    const uint32_t m[2] = {h2.z, h2.x};  // descending digits
    const uint32_t c[2] = {h2.w, h2.y};
    const uint32_t lm = m[0] + m[1];
    const uint32_t lc = c[0] + c[1];
    const uint32_t im = wave_incl_scan(lm);
    const uint32_t ic = wave_incl_scan(lc);
    const unsigned long long hit = __ballot(base + (BY_MASS ? im : ic) >= target);
    if (hit == 0ull) return false;
    const int hl = __ffsll(static_cast<long long>(hit)) - 1;
    uint32_t rm = im - lm, rc = ic - lc;
    uint32_t pos = 1, bm = rm, bc = rc, hm = m[1], hc = c[1];
    bool done = false;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (!done && base + (BY_MASS ? rm + m[t] : rc + c[t]) >= target) {
            pos = t;
            bm = rm;
            bc = rc;
            hm = m[t];
            hc = c[t];
            done = true;
        }
        rm += m[t];
        rc += c[t];
    }
    h.digit = __builtin_amdgcn_readlane(uint32_t(kBins - 1) - 2u * uint32_t(lane) - pos, hl);
    h.cnt_before = __builtin_amdgcn_readlane(bc, hl);
    h.mass_before = __builtin_amdgcn_readlane(bm, hl);
    h.bin_cnt = __builtin_amdgcn_readlane(hc, hl);
    h.bin_mass = __builtin_amdgcn_readlane(hm, hl);
    return true;
}

// Histogram (count and mass per bin) of digit `lv` over the candidate keys
// that carry prefix `pref` above it, in this wavefront's kBins-bin LDS array.
__device__ inline void digit_hist(const uint4* row4, int nv, int lv, uint32_t pref, unsigned long long* hist,
                                  int lane) {
    const int sh = digit_shift(lv), w = digit_width(lv);
    uint4* h4 = reinterpret_cast<uint4*>(hist);
    h4[lane] = make_uint4(0, 0, 0, 0);  // kBins / 2 uint4
    wave_lds_sync();
    for (int q = lane; 4 * q < nv; q += 64) {
        const uint4 x = row4[q];
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t kk = 4 * q + t < nv ? xs[t] : 0u;
            // forced keys never match a prefix
            if (kk != 0u && (kk >> (sh + w)) == pref) {
                const uint32_t d = (kk >> sh) & ((1u << w) - 1u);
                atomicAdd(&hist[d], (1ull << 32) | key_mass(kk));
            }
        }
    }
    wave_lds_sync();
}

// Lowest key whose digits down to level lv are `pref`, minus one: keeping the
// candidates above it keeps that whole bin and everything above it (candidate
// keys are at least 1, so a bin starting at 0 keeps every candidate).
__device__ inline uint32_t bin_floor(uint32_t pref, int lv) {
    const uint32_t lb = pref << digit_shift(lv);
    return lb == 0u ? 0u : lb - 1u;
}

// One query block (row i of head bh) on one wavefront, its compressed scores
// in `row` (LDS, 16-byte aligned; overwritten with the selection keys).  Each
// lane takes four consecutive key blocks per step.  Candidates are ordered by
// probability descending, ties by block index ascending; TopCdf keeps the
// shortest prefix whose mass reaches tau, the floor keeps at least `extra`
// candidates.  Both cut points are found exactly with at most five histogram
// passes each over the radix digits of the keys, so no sort is needed.
// Returns the row's kept count.
__device__ int select_row(const TopCdfArgs& a, int bh, int i, float simq_i, uint32_t* row, const uint32_t* colf,
                          unsigned long long* hS, int lane) {
    const RowGeom g = row_geom(a, i);
    const int64_t grow = int64_t(bh) * a.n_qb + i;
    // low-similarity query blocks and sink rows keep their whole valid row
    const bool forced_row = (a.theta > 0.f && simq_i < a.theta) || g.q_first < a.sink_rows;
    const int nv = g.nv;
    uint4* row4 = reinterpret_cast<uint4*>(row);

    // forcing and the candidates' maximum score
    const uint8_t* fpat = a.forced ? a.forced + int64_t(i) * a.n_kb : nullptr;  // this row of the pattern
    float cmax = -FLT_MAX;
    int nf = 0, nc = 0;
    for (int q = lane; 4 * q < nv; q += 64) {
        uint4 x = row4[q];
        uint32_t* xs = reinterpret_cast<uint32_t*>(&x);
        const uint32_t cf = (colf[q >> 3] >> ((4 * q) & 31)) & 0xfu;  // blocks 4q .. 4q+3
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int j = 4 * q + t;
            if (j < nv) {
                const bool f = ((cf >> t) & 1u) || (a.causal && causal_forced(a, g, j)) || (fpat && fpat[j]);
                if (f) {
                    xs[t] = kForcedKey;
                    ++nf;
                } else {
                    cmax = fmaxf(cmax, __uint_as_float(xs[t]));
                    ++nc;
                }
            }
        }
        row4[q] = x;
    }
    cmax = wave_max(cmax);
    const int n_forced = wave_sum_i(nf);
    const int n_cand = wave_sum_i(nc);
    // softmax over the candidates, then the keys
    float esum = 0.f;
    for (int q = lane; 4 * q < nv; q += 64) {
        uint4 x = row4[q];
        uint32_t* xs = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (4 * q + t < nv && xs[t] != kForcedKey) {
                // base-2 exponential of the scaled logit (its rounding moves p by a few
                // 1e-6 relative, far inside the band where ties and the tau cut count as
                // borderline); the compiler keeps results below 2^-126 as denormals
                const float ev = exp2f((__uint_as_float(xs[t]) - cmax) * kLog2eF);
                xs[t] = __float_as_uint(ev);
                esum += ev;
            }
        }
        row4[q] = x;
    }
    esum = wave_sum(esum);
    const float inv_sum = 1.0f / esum;
    for (int q = lane; 4 * q < nv; q += 64) {
        uint4 x = row4[q];
        uint32_t* xs = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (4 * q + t < nv && xs[t] != kForcedKey) xs[t] = __float_as_uint(__uint_as_float(xs[t]) * inv_sum) + 1u;
        row4[q] = x;
    }

    int extra = 0;
    if (a.sparsity >= 0.0) extra = max(0, int(ceil((1.0 - a.sparsity) * double(nv))) - n_forced);
    int k_cdf = 0;
    bool c_on = false;
    uint32_t T = 0;
    if (a.tau_d >= 1.0) {
        k_cdf = n_cand;
    } else if (a.tau_d > 0.0 && n_cand > 0 && extra < n_cand) {
        c_on = true;
        T = max(1u, uint32_t(ceil(a.tau_d * kFixD)));
    }
    // Both cut points are found by descending the radix digits of the keys,
    // one count+mass histogram per level.  The floor search (the extra-th
    // candidate in order) stops at the first bin all of whose candidates it
    // needs; the TopCdf search (the candidate at which the cumulative mass
    // reaches T) stops at the first bin that holds one candidate.  Each ends as
    // a threshold: every candidate above `thr` is kept, plus the first `quota`
    // (lowest indices) of those equal to it, which only a search that reaches
    // the last digit with ties left needs.  While the two searches follow the
    // same digits they share the histogram.
    const bool x_on = extra > 0 && extra < n_cand;
    uint32_t f_pref = 0, f_rem = uint32_t(extra), f_mass = 0, f_thr = 0, f_quota = 0;
    uint32_t c_pref = 0, c_acc = 0, c_cnt = 0, c_thr = 0, c_quota = 0;
    int c_lv = 0;
    bool c_done = !c_on, c_found = true;
    // one TopCdf level on the histogram of prefix c_pref at level c_lv
    auto c_step = [&]() {
        BinHit h;
        if (!scan_bins<true>(hS, c_acc, T, lane, h)) {  // the candidates' whole mass stays below tau
            c_found = false;
            c_done = true;
            return;
        }
        c_acc += h.mass_before;
        c_cnt += h.cnt_before;
        c_pref = (c_pref << digit_width(c_lv)) | h.digit;
        if (h.bin_cnt == 1u) {
            c_thr = bin_floor(c_pref, c_lv);
            c_quota = 0;
            k_cdf = int(c_cnt + 1u);
            c_done = true;
        } else if (c_lv == kLevels - 1) {
            // the key is shared by bin_cnt candidates of equal mass, taken in index order
            const uint32_t Pv = key_mass(c_pref);
            const uint32_t need = T - c_acc;
            uint32_t m = Pv ? (need - 1u) / Pv : h.bin_cnt - 1u;
            m = min(m, h.bin_cnt - 1u);
            c_thr = c_pref;
            c_quota = m + 1u;
            k_cdf = int(c_cnt + m + 1u);
            c_done = true;
        }
        ++c_lv;
    };
    if (x_on) {
        bool f_done = false;
        for (int lv = 0; lv < kLevels && !f_done; ++lv) {
            digit_hist(row4, nv, lv, f_pref, hS, lane);
            if (!c_done && c_lv == lv && c_pref == f_pref) c_step();
            BinHit h;
            scan_bins<false>(hS, 0u, f_rem, lane, h);
            f_rem -= h.cnt_before;
            f_mass += h.mass_before;
            f_pref = (f_pref << digit_width(lv)) | h.digit;
            if (h.bin_cnt == f_rem) {  // every candidate of the bin is needed
                f_thr = bin_floor(f_pref, lv);
                f_quota = 0;
                f_mass += h.bin_mass;
                f_done = true;
            }
        }
        if (!f_done) {  // f_pref is the extra-th key; f_rem of its ties are needed
            f_thr = f_pref;
            f_quota = f_rem;
            f_mass += f_rem * key_mass(f_pref);
        }
        // when the floor's candidates already hold tau of the mass, the TopCdf
        // prefix is no longer than the floor
        if (c_on && f_mass >= T) c_on = false;
    }
    if (c_on) {
        while (!c_done) {
            digit_hist(row4, nv, c_lv, c_pref, hS, lane);
            c_step();
        }
        if (!c_found) k_cdf = n_cand;
    } else if (T != 0u) {
        k_cdf = 0;  // the floor already holds tau of the mass
    }
    const int keep = min(n_cand, max(k_cdf, extra));

    // threshold key and how many of its ties (lowest indices first) are kept
    uint32_t v_thr = 0xffffffffu, quota = 0;
    if (forced_row || keep == 0) {
        v_thr = 0xffffffffu;  // no candidate passes
    } else if (keep == n_cand) {
        v_thr = 0u;  // every candidate passes
    } else if (keep == k_cdf) {
        v_thr = c_thr;
        quota = c_quota;
    } else {
        v_thr = f_thr;
        quota = f_quota;
    }
    uint8_t* out = a.mask + grow * a.n_kb;
    const bool aligned4 = (a.n_kb & 3) == 0;
    const unsigned long long below = (1ull << lane) - 1ull;
    uint32_t run = 0;
    for (int q0 = 0; 4 * q0 < a.n_kb; q0 += 64) {
        const int q = q0 + lane;
        const uint4 x = 4 * q < nv ? row4[q] : make_uint4(0, 0, 0, 0);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
        bool cand[4], eq[4];
        unsigned long long em[4];
        uint32_t before = run;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t kk = 4 * q + t < nv ? xs[t] : 0u;
            cand[t] = is_candidate(kk);
            eq[t] = cand[t] && kk == v_thr;
            em[t] = __ballot(eq[t]);
            before += uint32_t(__popcll(em[t] & below));
        }
        uint32_t rank = before;
        uint32_t word = 0;  // the mask bytes of blocks 4q .. 4q+3
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int j = 4 * q + t;
            const uint32_t kk = j < nv ? xs[t] : 0u;
            const bool kept = cand[t] && (kk > v_thr || (eq[t] && rank < quota));
            if (eq[t]) ++rank;
            const uint32_t bit = forced_row ? uint32_t(j < nv) : uint32_t(kk == kForcedKey || kept);
            word |= bit << (8 * t);
            run += uint32_t(__popcll(em[t]));
        }
        // one 4-byte store per lane when the row starts 4-byte aligned (n_kb % 4 == 0)
        if (aligned4) {
            if (4 * q < a.n_kb) reinterpret_cast<uint32_t*>(out)[q] = word;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (4 * q + t < a.n_kb) out[4 * q + t] = uint8_t(word >> (8 * t));
        }
    }
    const int cnt = forced_row ? nv : n_forced + keep;
    if (lane == 0) a.counts[grow] = cnt;
    return cnt;
}

// Eight wavefronts per group of gr <= 16 query blocks; wavefront w selects query
// blocks 2w and 2w+1.  Dynamic LDS: scores[gr][ls] f32 | query-block
// means[16][D + 4] f32 while the scores are computed, then per selecting
// wavefront a histogram[kBins] u64 | column forcing bits[ceil(n_kb/32)] u32.
constexpr int kTopcdfWaves = 8;
// wavefronts that select rows (two each) and so hold a histogram
__host__ __device__ constexpr int topcdf_sel_waves(int gr) { return (gr + 1) / 2; }
// row stride (floats) of the query-block means in LDS: padded so that eight
// consecutive rows start in different banks
__host__ __device__ constexpr int topcdf_qrow(int d) { return d + 4; }
// LDS bytes that hold the group's query-block means during the score products
// and the selecting wavefronts' histograms after them
__host__ __device__ constexpr int topcdf_union_bytes(int gr, int d) {
    return topcdf_sel_waves(gr) * kBins * 8 > kGroupRows * topcdf_qrow(d) * 4 ? topcdf_sel_waves(gr) * kBins * 8
                                                                             : kGroupRows * topcdf_qrow(d) * 4;
}

template <int D>
__global__ __launch_bounds__(64 * kTopcdfWaves) void k_topcdf(TopCdfArgs a, int ls, int gr) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int32_t wave_tot[kTopcdfWaves];
    __shared__ float simq_g[kGroupRows];
    float* scores = reinterpret_cast<float*>(smem);
    unsigned long long* hist = reinterpret_cast<unsigned long long*>(scores + gr * ls);
    float* qlds = reinterpret_cast<float*>(hist);  // the same bytes, dead once the score products are done
    uint32_t* colf = reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(hist) + topcdf_union_bytes(gr, D));

    const int groups = (a.n_qb + gr - 1) / gr;
    const int g = blockIdx.x;
    const int bh = g / groups;  // b * Hq + hq
    const int i0 = (g - bh * groups) * gr;
    const int hq = bh % a.Hq;
    const int b = bh / a.Hq;
    const int hk = hq / (a.Hq / a.Hkv);
    const int64_t kvh = int64_t(b) * a.Hkv + hk;
    const float* kbar = a.kbar + kvh * a.n_kb * D;
    const float* simk = a.simk + kvh * a.n_kb;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int i_last = min(i0 + gr, a.n_qb) - 1;
    const int ncols = row_geom(a, i_last).nv;  // columns any row of the group can see

    // Loads first, so their latencies overlap: the group's query-block means
    // (one float4 per thread; rows past the group are zero), the key-block
    // similarities for the column forcing, the group's query-block similarities.
    constexpr int QROW = topcdf_qrow(D);
    constexpr int QV4 = kGroupRows * D / 4;
    static_assert(QV4 <= 64 * kTopcdfWaves, "one float4 of query means per thread");
    const int qr = int(threadIdx.x) / (D / 4), qc4 = int(threadIdx.x) % (D / 4);
    f32x4 qv = {0.f, 0.f, 0.f, 0.f};
    if (int(threadIdx.x) < QV4 && qr < gr && i0 + qr < a.n_qb)
        qv = *reinterpret_cast<const f32x4*>(a.qbar + (int64_t(bh) * a.n_qb + i0 + qr) * D + 4 * qc4);
    // this wavefront's first tile of key-block means (see the score loop below)
    constexpr int C = D / 16;
    const int r16 = lane & 15;
    const int sub = lane >> 4;
    const int ntile = (ncols + 15) >> 4;
    f32x4 kv[C];
    auto load_tile = [&](int t) {
        const float* ks = kbar + int64_t(min(t * 16 + r16, ncols - 1)) * D + 4 * sub;
#pragma unroll
        for (int c = 0; c < C; ++c) kv[c] = *reinterpret_cast<const f32x4*>(ks + 16 * c);
    };
    if (wave < ntile) load_tile(wave);
    constexpr int kColSteps = (SA_MAX_KEY_BLOCKS + 64 * kTopcdfWaves - 1) / (64 * kTopcdfWaves);
    float sk[kColSteps];
#pragma unroll
    for (int u = 0; u < kColSteps; ++u) {
        const int j = 64 * (wave + kTopcdfWaves * u) + lane;
        sk[u] = j < ncols ? simk[j] : 0.f;
    }
    if (threadIdx.x < kGroupRows)
        simq_g[threadIdx.x] = a.simq[int64_t(bh) * a.n_qb + min(i0 + int(threadIdx.x), a.n_qb - 1)];
    if (int(threadIdx.x) < QV4) *reinterpret_cast<f32x4*>(qlds + qr * QROW + 4 * qc4) = qv;
    // column forcing as bits: word j/32 of the mask, one ballot per 64 blocks
#pragma unroll
    for (int u = 0; u < kColSteps; ++u) {
        const int j0 = 64 * (wave + kTopcdfWaves * u);
        if (j0 >= ncols) break;
        const int j = j0 + lane;
        const unsigned long long f = __ballot(j < ncols && column_forced(a, j, sk[u]));
        if (lane == 0) {
            colf[j0 >> 5] = uint32_t(f);
            colf[(j0 >> 5) + 1] = uint32_t(f >> 32);
        }
    }
    __syncthreads();

    // ---- compressed scores on v_mfma_f32_16x16x4_f32: A = 16 key-block means
    // (rows), B = the group's 16 query-block means (columns).  Lane l feeds
    // operand slot l/16 of row/column l%16; head-dim entry 16c + 4(l/16) + e
    // goes to step (c, e), so each lane reads float4s of contiguous entries.
    // The result lands as query row l%16, key blocks 4(l/16)..+3 of the tile.
    // A wavefront takes every eighth tile.  The query operand is read from LDS
    // at each step, which leaves the registers for all of a tile's key loads
    // to be in flight at once.
    for (int t = wave; t < ntile; t += kTopcdfWaves) {
        // an opaque offset, so the query reads stay inside the loop
        int qo = r16 * QROW + 4 * sub;
        asm volatile("" : "+v"(qo));
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C; c += 2) {
            const f32x4 q0 = *reinterpret_cast<const f32x4*>(qlds + qo + 16 * c);
            const f32x4 q1 = *reinterpret_cast<const f32x4*>(qlds + qo + 16 * (c + 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[c][e], q0[e], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[c + 1][e], q1[e], acc1, 0, 0, 0);
            }
        }
        if (t + kTopcdfWaves < ntile) load_tile(t + kTopcdfWaves);
        const f32x4 sc = (acc0 + acc1) * a.scale;
        // rows past the group and blocks past the row's room (the last tile's tail) are not stored
        if (r16 < gr && t * 16 + 4 * sub < ls)
            *reinterpret_cast<f32x4*>(scores + r16 * ls + t * 16 + 4 * sub) = sc;
    }
    __syncthreads();

    unsigned long long* hS = hist + wave * kBins;
    int tot = 0;
    for (int rr = 2 * wave; rr < 2 * wave + 2; ++rr) {
        const int i = i0 + rr;
        if (rr >= gr || i >= a.n_qb) break;
        tot += select_row(a, bh, i, simq_g[rr], reinterpret_cast<uint32_t*>(scores + rr * ls), colf, hS, lane);
    }
    if (lane == 0) wave_tot[wave] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
        int sum = 0;
#pragma unroll
        for (int w = 0; w < kTopcdfWaves; ++w) sum += wave_tot[w];
        a.group_tot[g] = sum;
        // read only by the next launch: no ordering needed here
        __hip_atomic_fetch_add(&a.super_tot[g / kSuperGroups], sum, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ---------------------------------------------------------------- CSR
// One workgroup per group of gr query blocks (the TopCdf grouping).  Its
// first row offset is the sum of the super-group totals before its own
// super-group and of the group totals before it inside that one; the group's
// own rows are scanned by one wavefront; then each wavefront compacts four
// mask rows into ascending column lists.
constexpr int kMaxWordsPerLane = SA_MAX_KEY_BLOCKS / 256;

__global__ __launch_bounds__(256) void k_csr(const uint8_t* __restrict__ mask, const int32_t* __restrict__ counts,
                                             const int32_t* __restrict__ group_tot,
                                             const int32_t* __restrict__ super_tot, int n_groups,
                                             int groups_per_head, int gr, int n_qb, int n_kb, int64_t rows,
                                             int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                             int64_t col_cap, int32_t* dev_status) {
    __shared__ long long red[4];
    __shared__ long long rp[kGroupRows + 1];
    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // rows before this group: whole super-groups, then the groups before it in its own
    const int sg = g / kSuperGroups;
    long long s = 0;
    for (int t = tid; t < sg; t += 256) s += super_tot[t];
    if (sg * kSuperGroups + tid < g) s += group_tot[sg * kSuperGroups + tid];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m);
    if (lane == 0) red[wave] = s;

    const int bh = g / groups_per_head;
    const int i0 = (g - bh * groups_per_head) * gr;
    const int nr = min(gr, n_qb - i0);
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

}  // namespace

// Query blocks per TopCdf workgroup.  The kernel runs as one round of long
// workgroups, so its time is that of the CU given the most rows: with
// kDeviceCUs compute units taking workgroups in turn, that is
// ceil(groups / kDeviceCUs) * rows per group, minimised here over 8..16 rows
// (fewer would leave most of the score product's 16 columns unused; ties: the
// larger group, whose rows share one pass over the key-block means).
constexpr int64_t kDeviceCUs = 256;
int topcdf_group_rows(int64_t bh, int64_t n_qb) {
    int best = kGroupRows;
    int64_t best_cost = INT64_MAX;
    for (int g = kGroupRows; g >= kGroupRows / 2; --g) {
        const int64_t groups = bh * ((n_qb + g - 1) / g);
        const int64_t cost = (groups + kDeviceCUs - 1) / kDeviceCUs * g;
        if (cost < best_cost) {
            best_cost = cost;
            best = g;
        }
    }
    return best;
}

int64_t topcdf_groups(int64_t bh, int64_t n_qb) {
    const int g = topcdf_group_rows(bh, n_qb);
    return bh * ((n_qb + g - 1) / g);
}

hipError_t launch_block_stats(const uint16_t* q, const uint16_t* k, const int32_t* perm, const PredictShape& s,
                              float* qbar, float* kbar, float* simq, float* simk, int32_t* dev_status,
                              int32_t* super_tot, int n_super, const Quant8* qz, hipStream_t stream) {
    const int64_t qb = int64_t(s.B) * s.Hq * s.n_qb;
    const int64_t kb = int64_t(s.B) * s.Hkv * s.n_kb;
    const int64_t wgs = (qb + kb + 3) / 4;
    if (wgs > INT32_MAX || n_super > wgs) return hipErrorInvalidValue;
    const dim3 grid{unsigned(wgs), 1, 1};
    const Quant8 z = qz ? *qz : Quant8{};
    if (qz && (s.bq > kQuantMaxBlock || s.bk % kKeyQuantRows != 0 || s.bk > 2 * kKeyQuantRows))
        return hipErrorInvalidValue;
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, q, k, perm, s.N, s.Nk, s.bq, s.bk, qb, qb + kb,
                           int(s.n_qb), int(s.n_kb), qbar, kbar, simq, simk, dev_status, super_tot, n_super, z);
    };
    auto go = [&](auto gather, auto quant) {
        constexpr bool G = decltype(gather)::value;
        constexpr bool Z = decltype(quant)::value;
        if (s.D == 128) launch(k_block_stats<128, G, Z>);
        else launch(k_block_stats<64, G, Z>);
    };
    if (perm && qz) go(std::true_type{}, std::true_type{});
    else if (perm) go(std::true_type{}, std::false_type{});
    else if (qz) go(std::false_type{}, std::true_type{});
    else go(std::false_type{}, std::false_type{});
    return hipGetLastError();
}

hipError_t launch_topcdf(const TopCdfArgs& a, hipStream_t stream) {
    if (a.n_kb > SA_MAX_KEY_BLOCKS) return hipErrorInvalidValue;
    const int ls = score_stride(a.n_kb);
    // column bits: whole 64-block ballots
    const int gr = topcdf_group_rows(int64_t(a.B) * a.Hq, a.n_qb);
    const size_t lds = size_t(gr) * ls * 4 + topcdf_union_bytes(gr, a.D) + size_t(a.n_kb + 63) / 64 * 8;
    if (lds > 160 * 1024) return hipErrorInvalidValue;
    const int64_t nwg = topcdf_groups(int64_t(a.B) * a.Hq, a.n_qb);
    if (nwg > INT32_MAX) return hipErrorInvalidValue;
    const dim3 block{64 * kTopcdfWaves, 1, 1};
    if (a.D == 128)
        hipLaunchKernelGGL(k_topcdf<128>, dim3(unsigned(nwg)), block, lds, stream, a, ls, gr);
    else
        hipLaunchKernelGGL(k_topcdf<64>, dim3(unsigned(nwg)), block, lds, stream, a, ls, gr);
    return hipGetLastError();
}

hipError_t launch_csr(const uint8_t* mask, const int32_t* counts, const int32_t* group_tot, int64_t bh,
                      int n_qb, int n_kb, int32_t* row_ptr, int32_t* col_idx, int64_t col_cap,
                      int32_t* dev_status, hipStream_t stream) {
    const int64_t n_groups = topcdf_groups(bh, n_qb);
    if (n_groups > INT32_MAX || n_kb > SA_MAX_KEY_BLOCKS) return hipErrorInvalidValue;
    const int gr = topcdf_group_rows(bh, n_qb);
    const int gph = (n_qb + gr - 1) / gr;
    hipLaunchKernelGGL(k_csr, dim3(unsigned(n_groups)), dim3(256), 0, stream, mask, counts, group_tot,
                       group_tot + n_groups, int(n_groups), gph, gr, n_qb, n_kb, bh * n_qb, row_ptr, col_idx, col_cap, dev_status);
    return hipGetLastError();
}

}  // namespace sa
