"""Token reorders and the permute / unpermute pair (fp64 oracle, test infrastructure only).

* Permuting Q, K, V together with both axes of the mask leaves attention
  unchanged up to the same permutation of the output rows; applying the
  inverse permutation restores the original order (SparseAttn article,
  section 3.4; SpargeAttn notes, section 2.5).  Positions must already be
  encoded: the reorder never touches positional information.
* [t,h,w]-window reorder: tokens are grouped by 3-D windows so that a block of
  consecutive tokens covers a compact space-time region; the first frame is
  kept in full attention as a sink (MindIE-SD "sparse" page, rf_v2).  Reading
  used here: frame 0 stays first in raster order, frames 1..t-1 are ordered by
  (window t, window h, window w, t, h, w), text tokens go last in their
  original order.
* Hilbert reorder of the visual tokens only (SpargeAttn notes, section 2.5).
  The pages name no curve variant; this follows J. Skilling, "Programming the
  Hilbert curve", AIP Conf. Proc. 707 (2004): coordinates (t, h, w) on the
  enclosing 2^k cube, k = ceil(log2(max extent)), axis 0 = t most significant,
  the transposed index bits interleaved most-significant first.
"""

import numpy as np

ORDER_IDENTITY, ORDER_WINDOW, ORDER_HILBERT = 0, 1, 2


def hilbert_index(coords: np.ndarray, bits: int) -> np.ndarray:
    """Hilbert index of integer points; coords has shape (npoints, ndim).

    Skilling's axes -> transpose map (undo the excess work, then Gray-encode),
    followed by interleaving the transposed bits, most significant first, with
    axis 0 in front.
    """
    X = [np.array(coords[:, i], dtype=np.int64) for i in range(coords.shape[1])]
    n = len(X)
    top = 1 << (bits - 1)
    q = top
    while q > 1:
        low = q - 1
        for i in range(n):
            on = (X[i] & q) != 0
            # bit set: invert the low bits of axis 0; clear: swap low bits of axis 0 and axis i
            swap = (X[0] ^ X[i]) & low
            x0_on = X[0] ^ low
            x0_off = X[0] ^ swap
            xi_off = X[i] ^ swap
            if i == 0:
                X[0] = np.where(on, x0_on, X[0])
            else:
                X[i] = np.where(on, X[i], xi_off)
                X[0] = np.where(on, x0_on, x0_off)
        q >>= 1
    for i in range(1, n):
        X[i] = X[i] ^ X[i - 1]
    flip = np.zeros_like(X[0])
    q = top
    while q > 1:
        flip = np.where((X[n - 1] & q) != 0, flip ^ (q - 1), flip)
        q >>= 1
    X = [x ^ flip for x in X]
    index = np.zeros_like(X[0])
    for bit in range(bits - 1, -1, -1):
        for i in range(n):
            index = (index << 1) | ((X[i] >> bit) & 1)
    return index


def _bits_for(extent: int) -> int:
    k = 1
    while (1 << k) < extent:
        k += 1
    return k


def plan_permutation(n_tokens: int, order: int, latent=(1, 1, 1), window=(1, 1, 1),
                     txt_len: int = 0, first_frame_sink: bool = False) -> np.ndarray:
    """perm[i] = original index of the token placed at permuted position i."""
    if n_tokens <= 0:
        raise ValueError("n_tokens must be positive")
    if order == ORDER_IDENTITY:
        return np.arange(n_tokens, dtype=np.int64)
    t, h, w = latent
    if min(t, h, w) <= 0 or txt_len < 0 or n_tokens != txt_len + t * h * w:
        raise ValueError("n_tokens must equal txt_len + t*h*w")
    if order not in (ORDER_WINDOW, ORDER_HILBERT):
        raise ValueError("unknown order")
    t0 = 1 if first_frame_sink else 0
    parts = []
    if first_frame_sink:
        parts.append(txt_len + np.arange(h * w, dtype=np.int64))
    tr = t - t0
    if tr > 0:
        tt, hh, ww = np.meshgrid(np.arange(tr), np.arange(h), np.arange(w), indexing="ij")
        tt, hh, ww = tt.ravel(), hh.ravel(), ww.ravel()
        orig = txt_len + ((tt + t0) * h + hh) * w + ww
        if order == ORDER_WINDOW:
            wt, wh, wwin = window
            if min(wt, wh, wwin) <= 0:
                raise ValueError("window extents must be positive")
            keys = (ww, hh, tt, ww // wwin, hh // wh, tt // wt)  # lexsort: last key is primary
            sel = np.lexsort(keys)
        else:
            bits = _bits_for(max(tr, h, w))
            idx = hilbert_index(np.stack([tt, hh, ww], axis=1), bits)
            sel = np.argsort(idx, kind="stable")
        parts.append(orig[sel])
    if txt_len:
        parts.append(np.arange(txt_len, dtype=np.int64))
    perm = np.concatenate(parts)
    return perm


def token_tiles(n_tokens: int, latent, txt_len: int, first_frame_sink: bool, tile) -> np.ndarray:
    """3-D tile of every token in the ORIGINAL order, shape (n_tokens, 3); -1 rows for
    tokens outside the tiling (text, and frame 0 when it is the first-frame sink).

    A video token at latent (t, h, w) lies in tile ((t - t0) // tile_t, h // tile_h,
    w // tile_w), t0 = 1 with the first-frame sink (the frames that take part in the
    reorder are tiled from their own first frame), else 0.
    """
    t, h, w = latent
    if min(t, h, w) <= 0 or txt_len < 0 or n_tokens != txt_len + t * h * w:
        raise ValueError("n_tokens must equal txt_len + t*h*w")
    if min(tile) <= 0:
        raise ValueError("tile extents must be positive")
    t0 = 1 if first_frame_sink else 0
    out = np.full((n_tokens, 3), -1, dtype=np.int64)
    for x in range(txt_len, n_tokens):
        e = x - txt_len
        tt, rem = divmod(e, h * w)
        hh, ww = divmod(rem, w)
        if tt < t0:
            continue
        out[x] = ((tt - t0) // tile[0], hh // tile[1], ww // tile[2])
    return out


def plan_tile_window(n_tokens: int, order: int, latent, window, txt_len: int, first_frame_sink: bool,
                     tile, radius, block_q: int, block_k: int) -> np.ndarray:
    """3-D tile-window pattern of blocks in the permuted order (bool [n_qb, n_kb]).

    The sliding-tile idea of the SparseAttn article (its discussion of Sliding Tile
    Attention: one query tile shares one set of key tiles): query block i and key block
    j are paired when some query token of i and some key token of j lie in tiles that
    differ by at most radius[a] along every axis a.  Untiled tokens pair with nothing.
    """
    if min(radius) < 0:
        raise ValueError("radii must be non-negative")
    perm = plan_permutation(n_tokens, order, latent, window, txt_len, first_frame_sink)
    tiles = token_tiles(n_tokens, latent, txt_len, first_frame_sink, tile)[perm]
    n_qb = -(-n_tokens // block_q)
    n_kb = -(-n_tokens // block_k)

    def block_tiles(b, i):
        rows = tiles[i * b:min((i + 1) * b, n_tokens)]
        return {tuple(r) for r in rows.tolist() if r[0] >= 0}

    qt = [block_tiles(block_q, i) for i in range(n_qb)]
    kt = [block_tiles(block_k, j) for j in range(n_kb)]
    out = np.zeros((n_qb, n_kb), dtype=bool)
    for i in range(n_qb):
        for j in range(n_kb):
            out[i, j] = any(all(abs(a[d] - c[d]) <= radius[d] for d in range(3)) for a in qt[i] for c in kt[j])
    return out


def permute_rows(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """y[..., i, :] = x[..., perm[i], :]"""
    return np.take(x, perm, axis=-2)


def unpermute_rows(y: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x[..., perm[i], :] = y[..., i, :]"""
    x = np.empty_like(y)
    x[..., perm, :] = y
    return x
