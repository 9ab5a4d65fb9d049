// Host-side token reorder planner: identity, [t,h,w]-window and Hilbert orders.
//
// Window reorder with the first frame kept in front as a sink and text moved
// last: MindIE-SD "稀疏" page, rf_v2 (space-time aware token reorder, first-frame
// sink).  Hilbert order of the visual tokens: SpargeAttn notes, section 2.5; the
// curve variant is J. Skilling, "Programming the Hilbert curve", AIP Conf.
// Proc. 707 (2004), on the enclosing 2^k cube, axis 0 (t) most significant.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstdint>
#include <numeric>
#include <vector>

#include "sparse_attn.h"

namespace {

// Skilling's axes-to-transpose map for 3 axes of `bits` bits, then the
// transposed bits read out most-significant first with axis 0 leading.
uint64_t hilbert3(uint32_t t, uint32_t h, uint32_t w, int bits) {
    uint32_t x[3] = {t, h, w};
    const uint32_t top = 1u << (bits - 1);
    for (uint32_t q = top; q > 1; q >>= 1) {
        const uint32_t low = q - 1;
        for (int i = 0; i < 3; ++i) {
            if (x[i] & q) {
                x[0] ^= low;  // invert the low bits of axis 0
            } else {
                const uint32_t s = (x[0] ^ x[i]) & low;  // exchange low bits of axes 0 and i
                x[0] ^= s;
                x[i] ^= s;
            }
        }
    }
    x[1] ^= x[0];  // Gray encode
    x[2] ^= x[1];
    uint32_t flip = 0;
    for (uint32_t q = top; q > 1; q >>= 1)
        if (x[2] & q) flip ^= q - 1;
    for (uint32_t& v : x) v ^= flip;
    uint64_t idx = 0;
    for (int b = bits - 1; b >= 0; --b)
        for (int i = 0; i < 3; ++i) idx = (idx << 1) | ((x[i] >> b) & 1u);
    return idx;
}

int ceil_log2(int64_t v) {
    int k = 1;
    while ((int64_t(1) << k) < v) ++k;
    return k;
}

}  // namespace

extern "C" int sa_plan_permutation(const sa_layout* L, int32_t* perm, int64_t n) {
    if (!L || !perm || n <= 0 || n != L->n_tokens || n > INT32_MAX) return SA_ERR_INVALID_ARGUMENT;
    if (L->order == SA_ORDER_IDENTITY) {
        for (int64_t i = 0; i < n; ++i) perm[i] = int32_t(i);
        return SA_OK;
    }
    if (L->order != SA_ORDER_WINDOW && L->order != SA_ORDER_HILBERT) return SA_ERR_INVALID_ARGUMENT;
    const int64_t T = L->t, H = L->h, W = L->w, txt = L->txt_len;
    if (T <= 0 || H <= 0 || W <= 0 || txt < 0 || txt + T * H * W != n) return SA_ERR_INVALID_ARGUMENT;
    if (L->first_frame_sink != 0 && L->first_frame_sink != 1) return SA_ERR_INVALID_ARGUMENT;
    if (L->order == SA_ORDER_WINDOW && (L->win_t <= 0 || L->win_h <= 0 || L->win_w <= 0))
        return SA_ERR_INVALID_ARGUMENT;
    if (L->order == SA_ORDER_HILBERT && std::max({T, H, W}) > (int64_t(1) << 20))
        return SA_ERR_INVALID_ARGUMENT;

    int64_t pos = 0;
    const int64_t t0 = L->first_frame_sink ? 1 : 0;
    for (int64_t k = 0; k < t0 * H * W; ++k) perm[pos++] = int32_t(txt + k);  // frame 0, raster

    const int64_t tr = T - t0;  // frames taking part in the reorder
    const int64_t nv = tr * H * W;
    std::vector<uint64_t> key(nv);
    std::vector<int64_t> orig(nv);
    if (L->order == SA_ORDER_WINDOW) {
        const int64_t wt = L->win_t, wh = L->win_h, ww = L->win_w;
        const int64_t nwh = (H + wh - 1) / wh, nww = (W + ww - 1) / ww;
        // window id (raster over windows), then position inside the window (raster t,h,w)
        for (int64_t t = 0; t < tr; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t w = 0; w < W; ++w) {
                    const int64_t e = (t * H + h) * W + w;
                    const uint64_t win = uint64_t(((t / wt) * nwh + h / wh) * nww + w / ww);
                    const uint64_t in = uint64_t(((t % wt) * wh + h % wh) * ww + w % ww);
                    key[e] = (win << 32) | in;
                    orig[e] = txt + ((t + t0) * H + h) * W + w;
                }
    } else {
        const int bits = ceil_log2(std::max({tr, H, W, int64_t(2)}));
        for (int64_t t = 0; t < tr; ++t)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t w = 0; w < W; ++w) {
                    const int64_t e = (t * H + h) * W + w;
                    key[e] = hilbert3(uint32_t(t), uint32_t(h), uint32_t(w), bits);
                    orig[e] = txt + ((t + t0) * H + h) * W + w;
                }
    }
    std::vector<int64_t> sel(nv);
    std::iota(sel.begin(), sel.end(), 0);
    std::stable_sort(sel.begin(), sel.end(), [&](int64_t a, int64_t b) { return key[a] < key[b]; });
    for (int64_t e = 0; e < nv; ++e) perm[pos++] = int32_t(orig[sel[e]]);
    for (int64_t k = 0; k < txt; ++k) perm[pos++] = int32_t(k);
    return SA_OK;
}

// 3-D tile windows as a block pattern: the sliding-tile idea the SparseAttn
// article discusses (Sliding Tile Attention: a query tile shares one set of
// key tiles).  Tiles live on the latent grid of the video tokens that take
// part in the reorder; query block i and key block j are paired when some of
// their tokens lie in tiles within the radius along every axis.
extern "C" int sa_plan_tile_window(const sa_layout* L, int32_t tile_t, int32_t tile_h, int32_t tile_w,
                                   int32_t radius_t, int32_t radius_h, int32_t radius_w, int32_t block_q,
                                   int32_t block_k, uint8_t* pattern, int64_t n_qb, int64_t n_kb) {
    if (!L || !pattern || tile_t <= 0 || tile_h <= 0 || tile_w <= 0 || radius_t < 0 || radius_h < 0 ||
        radius_w < 0 || block_q <= 0 || block_k <= 0)
        return SA_ERR_INVALID_ARGUMENT;
    const int64_t n = L->n_tokens;
    const int64_t T = L->t, H = L->h, W = L->w, txt = L->txt_len;
    if (n <= 0 || n > INT32_MAX || T <= 0 || H <= 0 || W <= 0 || txt < 0 || txt + T * H * W != n)
        return SA_ERR_INVALID_ARGUMENT;
    if (n_qb != (n + block_q - 1) / block_q || n_kb != (n + block_k - 1) / block_k) return SA_ERR_INVALID_ARGUMENT;
    std::vector<int32_t> perm(static_cast<size_t>(n));
    const int st = sa_plan_permutation(L, perm.data(), n);
    if (st != SA_OK) return st;
    const int64_t t0 = L->first_frame_sink ? 1 : 0;
    // tile of the token at each permuted position, packed into one integer (-1: untiled)
    const int64_t nth = (H + tile_h - 1) / tile_h, ntw = (W + tile_w - 1) / tile_w;
    auto tile_of = [&](int64_t x) -> int64_t {
        if (x < txt) return -1;
        const int64_t e = x - txt, t = e / (H * W), h = (e / W) % H, w = e % W;
        if (t < t0) return -1;
        return (((t - t0) / tile_t) * nth + h / tile_h) * ntw + w / tile_w;
    };
    // distinct tiles of each block, with their bounding box
    struct BlockTiles {
        std::vector<int64_t> ids;
        int64_t lo[3] = {INT64_MAX, INT64_MAX, INT64_MAX}, hi[3] = {-1, -1, -1};
    };
    auto collect = [&](int32_t b, int64_t nb) {
        std::vector<BlockTiles> out(static_cast<size_t>(nb));
        for (int64_t i = 0; i < nb; ++i) {
            BlockTiles& bt = out[size_t(i)];
            for (int64_t p = i * b; p < std::min(n, (i + 1) * b); ++p) {
                const int64_t id = tile_of(perm[size_t(p)]);
                if (id < 0) continue;
                bt.ids.push_back(id);
                const int64_t c[3] = {id / (nth * ntw), (id / ntw) % nth, id % ntw};
                for (int a = 0; a < 3; ++a) {
                    bt.lo[a] = std::min(bt.lo[a], c[a]);
                    bt.hi[a] = std::max(bt.hi[a], c[a]);
                }
            }
            std::sort(bt.ids.begin(), bt.ids.end());
            bt.ids.erase(std::unique(bt.ids.begin(), bt.ids.end()), bt.ids.end());
        }
        return out;
    };
    const std::vector<BlockTiles> qt = collect(block_q, n_qb), kt = collect(block_k, n_kb);
    const int64_t rad[3] = {radius_t, radius_h, radius_w};
    for (int64_t i = 0; i < n_qb; ++i) {
        const BlockTiles& a = qt[size_t(i)];
        for (int64_t j = 0; j < n_kb; ++j) {
            const BlockTiles& b = kt[size_t(j)];
            bool on = false;
            if (!a.ids.empty() && !b.ids.empty()) {
                bool boxes = true;  // bounding boxes within the radius: a pair may exist
                for (int d = 0; d < 3; ++d)
                    boxes = boxes && a.lo[d] - rad[d] <= b.hi[d] && b.lo[d] - rad[d] <= a.hi[d];
                for (size_t x = 0; boxes && !on && x < a.ids.size(); ++x) {
                    const int64_t ca[3] = {a.ids[x] / (nth * ntw), (a.ids[x] / ntw) % nth, a.ids[x] % ntw};
                    for (size_t y = 0; !on && y < b.ids.size(); ++y) {
                        const int64_t cb[3] = {b.ids[y] / (nth * ntw), (b.ids[y] / ntw) % nth, b.ids[y] % ntw};
                        on = std::llabs(ca[0] - cb[0]) <= rad[0] && std::llabs(ca[1] - cb[1]) <= rad[1] &&
                             std::llabs(ca[2] - cb[2]) <= rad[2];
                    }
                }
            }
            pattern[i * n_kb + j] = on ? 1 : 0;
        }
    }
    return SA_OK;
}
