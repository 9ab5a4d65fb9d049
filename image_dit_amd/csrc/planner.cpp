// Host-side token reorder planner: identity, [t,h,w]-window and Hilbert orders.
//
// Window reorder with the first frame kept in front as a sink and text moved
// last: MindIE-SD "稀疏" page, rf_v2 (space-time aware token reorder, first-frame
// sink).  Hilbert order of the visual tokens: SpargeAttn notes, section 2.5; the
// curve variant is J. Skilling, "Programming the Hilbert curve", AIP Conf.
// Proc. 707 (2004), on the enclosing 2^k cube, axis 0 (t) most significant.
#include <algorithm>
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
