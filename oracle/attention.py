"""Plain-definition attention, restricted softmax and mask ledgers (fp64, test infrastructure only).

Sources (cited by page title and section):

* SparseAttn article ("AIGC 基本功|视频稀疏注意力的误差与布局-SparseAttn"),
  section 3.1: scores s_ij = q_i.k_j / sqrt(d), row softmax p_ij, y_i = sum p_ij v_j;
  restricting row i to a kept set S_i gives weights p_ij / z_i with
  z_i = sum_{j in S_i} p_ij, i.e. a softmax over the kept keys only; an empty S_i
  has no meaning and must be rejected, never padded with an epsilon.
* same article, section 3.2: removed mass alpha_i = 1 - z_i; with r_i the kept
  average and u_i the removed average (original weights renormalised),
  y_i = (1-alpha_i) r_i + alpha_i u_i, so  ytilde_i - y_i = alpha_i (r_i - u_i)  and
  ||ytilde_i - y_i|| <= 2 alpha_i max_j ||v_j||.
* same article, section 3.3: frame-major teaching masks (same frame / same
  position / union) with pair counts T^2P^2, TP^2, PT^2 and union density
  (P+T-1)/(TP); the block-cost ledger of section 04.
* "44. Local Sliding and Sparse Attention", Steps 2 and 4: the local causal
  window (key <= query and query-key < w), its pair count, block-pair masks
  with a causal filter, and the visible/total/density ledger.
* "78. Attention Access Pattern Benchmark", Steps 2 and 4: causal global /
  sliding-window / block-sparse / selective patterns and their ledger.
"""

import numpy as np


def scaled_scores(q: np.ndarray, k: np.ndarray, scale=None) -> np.ndarray:
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    return (q @ k.T) * scale


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax; entries at -inf get weight 0.  Rows must hold a finite entry."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def dense_attention(q, k, v, scale=None):
    """Full attention: returns (y, p)."""
    p = softmax_rows(scaled_scores(q, k, scale))
    return p @ np.asarray(v, dtype=np.float64), p


def restricted_attention(q, k, v, mask, scale=None):
    """Softmax restricted to mask[i, j] == True; returns (ytilde, ptilde).

    Raises ValueError when a row keeps no key (the restricted softmax is
    undefined there).
    """
    mask = np.asarray(mask, dtype=bool)
    if not np.all(mask.any(axis=-1)):
        raise ValueError("a query row keeps no key: restricted softmax undefined")
    s = np.where(mask, scaled_scores(q, k, scale), -np.inf)
    p = softmax_rows(s)
    return p @ np.asarray(v, dtype=np.float64), p


def retained_mass(p: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """z_i: probability mass of the dense row that falls on the kept keys."""
    return np.sum(np.where(mask, p, 0.0), axis=-1)


def removed_mass_parts(p: np.ndarray, mask: np.ndarray, v: np.ndarray):
    """(alpha, r, u): removed mass, kept average, removed average.

    u_i is defined only where alpha_i > 0; it is NaN elsewhere.
    """
    v = np.asarray(v, dtype=np.float64)
    kept = np.where(mask, p, 0.0)
    dropped = np.where(mask, 0.0, p)
    z = kept.sum(axis=-1)
    alpha = dropped.sum(axis=-1)
    r = (kept @ v) / z[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        u = (dropped @ v) / alpha[:, None]
    u[alpha == 0] = np.nan
    return alpha, r, u


def removed_mass_bound(alpha: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Row-wise bound 2 * alpha_i * max_j ||v_j||_2."""
    M = np.max(np.linalg.norm(np.asarray(v, dtype=np.float64), axis=-1))
    return 2.0 * alpha * M


# ---------------------------------------------------------------- teaching masks

def frame_major_coords(T: int, P: int):
    """(frame, position) of each token when frames are flattened one after another."""
    idx = np.arange(T * P)
    return idx // P, idx % P


def spatiotemporal_masks(T: int, P: int):
    """Same-frame, same-position and union masks on the frame-major order."""
    frame, pos = frame_major_coords(T, P)
    spatial = frame[:, None] == frame[None, :]
    temporal = pos[:, None] == pos[None, :]
    return {"full": np.ones((T * P, T * P), dtype=bool), "spatial": spatial,
            "temporal": temporal, "union": spatial | temporal}


def spatiotemporal_pair_counts(T: int, P: int):
    """Closed forms of the allowed-pair counts for the teaching masks."""
    return {"full": T * T * P * P, "spatial": T * P * P, "temporal": P * T * T,
            "union": T * P * (P + T - 1)}


def block_cost(mask: np.ndarray, block: int):
    """Tiles with any allowed pair must be computed whole: useful vs computed pairs."""
    n = mask.shape[0]
    if n % block:
        raise ValueError("block must divide the mask size")
    nb = n // block
    active = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        for j in range(nb):
            active[i, j] = mask[i * block:(i + 1) * block, j * block:(j + 1) * block].any()
    useful = int(mask.sum())
    computed = int(active.sum()) * block * block
    return {"useful_pairs": useful, "active_tiles": int(active.sum()),
            "computed_pairs": computed, "utilization": useful / computed}


# ---------------------------------------------------------------- causal windows

def local_causal_mask(L: int, w: int) -> np.ndarray:
    """key <= query and query - key < w."""
    if not (isinstance(L, int) and isinstance(w, int)) or L <= 0 or w <= 0:
        raise ValueError("sequence length and window must be positive integers")
    qi = np.arange(L)[:, None]
    ki = np.arange(L)[None, :]
    return (ki <= qi) & (qi - ki < w)


def causal_pair_count(L: int) -> int:
    return L * (L + 1) // 2


def window_pair_count(L: int, w: int) -> int:
    """Closed form w*L - w*(w-1)/2 for L >= w (each of the first w-1 rows sees fewer)."""
    if L < w:
        return causal_pair_count(L)
    return w * L - w * (w - 1) // 2


def block_pairs_mask(L: int, b: int, pairs, causal: bool = True) -> np.ndarray:
    """Token mask from active (query_block, key_block) pairs, then the causal filter."""
    if L <= 0 or b <= 0:
        raise ValueError("sequence length and block size must be positive")
    nb = -(-L // b)
    mask = np.zeros((L, L), dtype=bool)
    for qb, kb in pairs:
        if not (0 <= qb < nb and 0 <= kb < nb):
            raise ValueError("block pair out of range")
        if causal and kb > qb:
            raise ValueError("a causal block mask cannot activate a future block")
        mask[qb * b:min((qb + 1) * b, L), kb * b:min((kb + 1) * b, L)] = True
    if causal:
        mask &= np.tril(np.ones((L, L), dtype=bool))
    return mask


def access_summary(mask: np.ndarray):
    if mask.ndim != 2 or mask.shape[0] != mask.shape[1] or mask.dtype != bool:
        raise ValueError("mask must be a square bool array")
    visible = int(mask.sum())
    total = int(mask.size)
    return {"visible_pairs": visible, "total_pairs": total, "density": visible / total}


def min_propagation_layers(distance: int, w: int):
    """Layers of a causal window w needed to carry information over `distance` tokens."""
    if not (isinstance(distance, int) and isinstance(w, int)) or distance < 0 or w <= 0:
        raise ValueError("distance must be >= 0 and window > 0")
    if distance == 0:
        return 0
    if w == 1:
        return float("inf")
    return -(-distance // (w - 1))


PATTERNS = ("global", "sliding_window", "block_sparse", "selective_sparse")


def validate_access_spec(pattern: str, L: int, window: int = 0, block: int = 0, anchors=()):
    issues = []
    if pattern not in PATTERNS:
        issues.append("unknown pattern")
    if L <= 0:
        issues.append("sequence length must be positive")
    if pattern in ("sliding_window", "selective_sparse") and window <= 0:
        issues.append("window must be positive")
    if pattern == "block_sparse" and block <= 0:
        issues.append("block must be positive")
    if any((not isinstance(a, (int, np.integer))) or a < 0 or a >= L for a in anchors):
        issues.append("anchor outside the sequence")
    return issues


def access_mask(pattern: str, L: int, window: int = 0, block: int = 0, anchors=()):
    """Causal access patterns: global, sliding window, same block + anchors, window + anchors."""
    issues = validate_access_spec(pattern, L, window, block, anchors)
    if issues:
        raise ValueError("; ".join(issues))
    qi = np.arange(L)[:, None]
    ki = np.arange(L)[None, :]
    causal = ki <= qi
    anchor = np.zeros((1, L), dtype=bool)
    anchor[0, list(anchors)] = True
    if pattern == "global":
        vis = np.ones((L, L), dtype=bool)
    elif pattern == "sliding_window":
        vis = (qi - ki) < window
    elif pattern == "block_sparse":
        vis = (qi // block == ki // block) | anchor
    else:
        vis = ((qi - ki) < window) | anchor
    return causal & vis


def access_ledger(mask: np.ndarray, local_window: int):
    """Visible keys per query, allowed score count, long-range coverage, density vs causal-global."""
    L = mask.shape[0]
    qi = np.arange(L)[:, None]
    ki = np.arange(L)[None, :]
    long_range = (ki <= qi) & (ki < qi - local_window + 1)
    total_long = int(long_range.sum())
    kept_long = int((mask & long_range).sum())
    score = int(mask.sum())
    return {"visible_keys_mean": float(mask.sum(axis=1).mean()),
            "score_count": score,
            "long_range_coverage": kept_long / total_long if total_long else 1.0,
            "density": score / causal_pair_count(L)}
