"""Block statistics, block-mask prediction and CSR (fp64 oracle, test infrastructure only).

The predictor is a heuristic, so it is written step by step in the order the
SpargeAttn notes give it (section 2.2, "selective token compression"), with
the sink of the MindIE-SD page (rf_v2 first-frame sink), the keep floor of its
``sparsity`` argument, and the causal local window of the "Local Sliding and
Sparse Attention" page (Step 2 table).  Readings taken where the pages are
silent or garbled:

* similarity: the mean pairwise cosine of the block's tokens, diagonal
  included, = ||mean_t x_t/||x_t||||^2 (a zero token contributes a zero unit
  vector).  The printed CosSim formula is also computed, for diagnostics only.
* TopCdf: keep blocks in descending compressed probability while the mass
  accumulated *before* a block is still below tau ("reach tau"), so at least
  one block is kept; tau >= 1 keeps every candidate.
* the compressed scores carry the same 1/sqrt(d) scale as the attention.
* ties in compressed probability: lower block index first.
* low-similarity key blocks leave the compressed softmax and are kept anyway;
  a low-similarity query block keeps its whole valid row.
* sparsity s: a per-row floor of ceil((1-s)*|valid|) kept blocks, forced
  blocks included; TopCdf may keep more.
* sinks: key blocks touching the first ``sink_front`` or the last
  ``sink_back`` tokens are kept by every query block.
* a forced block pattern (e.g. the 3-D tile windows of ``layout.plan_tile_window``)
  adds its blocks of row i to the forced blocks (within the valid set).
* sink rows (the other reading of the first-frame sink, where the first frame
  takes part in full attention as queries too): a query block touching the
  first ``sink_rows`` tokens keeps its whole valid row, as a low-similarity
  query block does.
* keys of another length: with N_k set, the key blocks cover N_k keys (the
  MindIE-SD arguments latent_shape_q and latent_shape_k may differ); the back
  sink counts from the end of the keys.  Causal masks need N_k = N.
* causal: a key block is valid if its first token is not after the query
  block's last token; the window W keeps every valid block holding a key within
  W-1 tokens before the query block's first token; the query block's own
  diagonal blocks are always kept.
"""

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

TAU_BORDER = 1e-5     # |S_excl - tau| within this -> the TopCdf cut may move
THETA_BORDER = 1e-5   # |sim - theta| within this -> the guard decision may flip
LOGIT_TIE = 1e-4      # |s_a - s_b| within this at the cut -> the order may swap


@dataclass
class MaskParams:
    N: int
    block_q: int
    block_k: int
    causal: bool = False
    window: int = 0
    sink_front: int = 0
    sink_back: int = 0
    tau: Optional[float] = None
    theta: Optional[float] = None
    sparsity: Optional[float] = None
    scale: Optional[float] = None
    sink_rows: int = 0
    forced: Optional[np.ndarray] = None  # bool [n_qb, n_kb]: blocks every head keeps
    N_k: Optional[int] = None  # keys per sequence (None: N)

    @property
    def nk(self):
        return self.N if self.N_k is None else self.N_k

    @property
    def n_qb(self):
        return -(-self.N // self.block_q)

    @property
    def n_kb(self):
        return -(-self.nk // self.block_k)


def block_stats(x: np.ndarray, b: int):
    """Per block of b consecutive tokens (last block partial): mean, similarity, printed CosSim.

    x: [N, d] float64.  Returns (means [nb, d], sim [nb], sim_printed [nb]).
    """
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape
    nb = -(-N // b)
    means = np.empty((nb, d))
    sim = np.empty(nb)
    printed = np.empty(nb)
    norms = np.linalg.norm(x, axis=1)
    unit = np.zeros_like(x)
    nz = norms > 0
    unit[nz] = x[nz] / norms[nz, None]
    for j in range(nb):
        blk = slice(j * b, min((j + 1) * b, N))
        means[j] = x[blk].mean(axis=0)
        um = unit[blk].mean(axis=0)
        sim[j] = float(um @ um)
        gram = x[blk] @ x[blk].T
        top = np.abs(gram.max())
        printed[j] = float((gram / top).mean()) if top > 0 else 0.0
    return means, sim, printed


def _valid_blocks(i: int, p: MaskParams) -> np.ndarray:
    j = np.arange(p.n_kb)
    if not p.causal:
        return np.ones(p.n_kb, dtype=bool)
    last_query = min((i + 1) * p.block_q, p.N) - 1
    return j * p.block_k <= last_query


def _forced_blocks(i: int, p: MaskParams, simk: np.ndarray, valid: np.ndarray) -> np.ndarray:
    j = np.arange(p.n_kb)
    k_first = j * p.block_k
    k_end = np.minimum((j + 1) * p.block_k, p.nk)  # one past the block's last token
    forced = np.zeros(p.n_kb, dtype=bool)
    if p.theta is not None and p.theta > 0:
        forced |= simk < p.theta
    if p.sink_front > 0:
        forced |= k_first < p.sink_front
    if p.sink_back > 0:
        forced |= k_end > p.nk - p.sink_back
    if p.causal:
        q_first = i * p.block_q
        q_end = min((i + 1) * p.block_q, p.N)
        if p.window > 0:
            forced |= (k_end - 1) >= q_first - p.window + 1
        forced |= (k_first < q_end) & (k_end > q_first)
    if p.forced is not None:
        forced |= np.asarray(p.forced[i], dtype=bool)
    return forced & valid


def predict_row(i: int, logits_row: np.ndarray, simq_i: float, simk: np.ndarray, p: MaskParams):
    """One query block's kept key blocks.  Returns (row_mask, info)."""
    valid = _valid_blocks(i, p)
    forced = _forced_blocks(i, p, simk, valid)
    info = {"forced_row": False, "k_cdf": 0, "extra": 0, "keep": 0,
            "n_valid": int(valid.sum()), "n_forced": int(forced.sum()),
            "border": set()}
    # guard decisions close to theta may flip under rounding of the statistics
    if p.theta is not None and p.theta > 0:
        if abs(simq_i - p.theta) <= THETA_BORDER or \
                np.any(np.abs(simk[valid] - p.theta) <= THETA_BORDER):
            info["border"].add("theta")
    # a low-similarity query block computes its whole valid row, and so does
    # a query block touching the first sink_rows tokens
    if (p.theta is not None and p.theta > 0 and simq_i < p.theta) or i * p.block_q < p.sink_rows:
        info["forced_row"] = True
        return valid.copy(), info
    cand = valid & ~forced
    idx = np.nonzero(cand)[0]
    if idx.size == 0:  # every candidate left: only the forced blocks remain
        return forced.copy(), info
    # compressed softmax over the candidates, fp64
    s = logits_row[idx]
    e = np.exp(s - s.max())
    prob = e / e.sum()
    # descending probability, ties by lower block index
    order = np.lexsort((idx, -prob))
    prob_sorted = prob[order]
    s_sorted = s[order]
    excl = np.concatenate(([0.0], np.cumsum(prob_sorted)[:-1]))
    if p.tau is None:
        k_cdf = 0
    elif p.tau >= 1.0:
        k_cdf = idx.size
    else:
        k_cdf = int(np.count_nonzero(excl < p.tau))
        for r in (k_cdf - 1, k_cdf):
            if 0 <= r < idx.size and abs(excl[r] - p.tau) <= TAU_BORDER:
                info["border"].add("tau")
    if p.sparsity is not None:
        floor = math.ceil((1.0 - p.sparsity) * float(info["n_valid"]))
        extra = max(0, floor - info["n_forced"])
    else:
        extra = 0
    keep = min(idx.size, max(k_cdf, extra))
    if 0 < keep < idx.size and abs(s_sorted[keep - 1] - s_sorted[keep]) <= LOGIT_TIE:
        info["border"].add("tie")
    info.update(k_cdf=k_cdf, extra=extra, keep=keep)
    row = forced.copy()
    row[idx[order[:keep]]] = True
    return row, info


def compressed_logits(qbar: np.ndarray, kbar: np.ndarray, p: MaskParams, d: int) -> np.ndarray:
    scale = p.scale if p.scale else 1.0 / math.sqrt(d)
    return (qbar @ kbar.T) * scale


def predict_head(q: np.ndarray, k: np.ndarray, p: MaskParams, rows=None):
    """Mask of one (batch, query head) from its permuted Q [N,d] and KV head's K [N,d].

    Returns dict(mask [n_qb, n_kb] bool, info list per row, simq, simk, qbar, kbar).
    ``rows`` restricts the work to some query blocks (others stay False).
    """
    if k.shape[0] != p.nk or q.shape[0] != p.N:
        raise ValueError("q must hold N tokens and k N_k tokens")
    if p.causal and p.nk != p.N:
        raise ValueError("causal masks need as many keys as queries")
    qbar, simq, simq_p = block_stats(q, p.block_q)
    kbar, simk, simk_p = block_stats(k, p.block_k)
    logits = compressed_logits(qbar, kbar, p, q.shape[1])
    mask = np.zeros((p.n_qb, p.n_kb), dtype=bool)
    infos = [None] * p.n_qb
    for i in (range(p.n_qb) if rows is None else rows):
        mask[i], infos[i] = predict_row(i, logits[i], simq[i], simk, p)
    return {"mask": mask, "info": infos, "simq": simq, "simk": simk,
            "simq_printed": simq_p, "simk_printed": simk_p, "qbar": qbar, "kbar": kbar,
            "logits": logits}


def mask_to_csr(masks: np.ndarray):
    """masks [R, n_kb] bool (rows in (batch, head, q-block) order) -> (row_ptr, col_idx) int64."""
    counts = masks.sum(axis=1)
    row_ptr = np.zeros(masks.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(masks)[1].astype(np.int64)
    return row_ptr, col_idx


def csr_to_mask(row_ptr: np.ndarray, col_idx: np.ndarray, n_kb: int) -> np.ndarray:
    R = len(row_ptr) - 1
    m = np.zeros((R, n_kb), dtype=bool)
    for r in range(R):
        m[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return m
