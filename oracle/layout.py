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


def permute_rows(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """y[..., i, :] = x[..., perm[i], :]"""
    return np.take(x, perm, axis=-2)


def unpermute_rows(y: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x[..., perm[i], :] = y[..., i, :]"""
    x = np.empty_like(y)
    x[..., perm, :] = y
    return x
