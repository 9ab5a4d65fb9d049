"""Attention restricted to a block CSR, with the PV-skip emulation (fp64 oracle, test infrastructure only).

* Block selection: a query block reads the tokens of its kept key blocks only
  (the block mask M_g of the SpargeAttn notes, section 2.1); in causal mode a
  query additionally reads only keys at or before it.  Without PV skipping the
  result is exactly the restricted softmax of the SparseAttn article, section
  3.1, over that token set, computed here in two passes from its definition.
* PV skip (SpargeAttn notes, sections 2.1 and 2.3): the key blocks are walked
  in ascending order with the online-softmax state (running max m, running
  sum l, unnormalised output O).  For a group of query rows, if the largest
  gap rowmax(S_ij) - m_ij over the group is below lambda (< 0), the P V product
  of that block is skipped for the group while m and l are still updated; the
  output is O / l at the end.  Reading: the group is 32 consecutive query rows
  of the query block (the rows one wavefront owns in the kernel), the skip test
  is strict (gap < lambda), rows whose keys in the block are all masked do not
  take part in the gap (if no row takes part the block is skipped), and rows
  past the end of the sequence do not exist.
"""

import math

import numpy as np

from .attention import restricted_attention

PV_GROUP_ROWS = 32


def _block_tokens(cols, bk, N):
    if len(cols) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([np.arange(j * bk, min((j + 1) * bk, N)) for j in cols])


def attend_qblock(q, k, v, i, cols, bq, bk, causal=False, scale=None, lam=None, replay=None):
    """Output rows of query block i given its kept key blocks ``cols`` (ascending).

    q: [N, d], k: [Nk, d], v: [Nk, dv] float64 in the permuted order (key blocks cover
    the Nk keys; Nk = N for self-attention, and must be for causal).
    lam: PV-skip threshold or None.  replay: optional bool array [len(cols), groups]
    forcing the skip decisions (used to compare against another implementation's
    decisions).  Returns (y [rows, dv], record).
    """
    N, d = q.shape
    Nk = k.shape[0]
    if causal and Nk != N:
        raise ValueError("causal attention needs as many keys as queries")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r0, r1 = i * bq, min((i + 1) * bq, N)
    rows = np.arange(r0, r1)
    cols = np.asarray(cols, dtype=np.int64)
    ngroups = -(-(r1 - r0) // PV_GROUP_ROWS)
    record = {"qk_blocks": int(len(cols)), "pv_exec": 0, "pv_skip": 0,
              "skip": np.zeros((len(cols), ngroups), dtype=bool),
              "gap": np.full((len(cols), ngroups), -np.inf)}
    if lam is None and replay is None:
        keys = _block_tokens(cols, bk, Nk)
        mask = np.ones((len(rows), len(keys)), dtype=bool)
        if causal:
            mask = keys[None, :] <= rows[:, None]
        y, _ = restricted_attention(q[rows], k[keys], v[keys], mask, scale)
        record["pv_exec"] = len(cols) * ngroups
        return y, record
    dv = v.shape[1]
    y = np.empty((len(rows), dv))
    for g in range(ngroups):
        gr = rows[g * PV_GROUP_ROWS:(g + 1) * PV_GROUP_ROWS]
        m = np.full(len(gr), -np.inf)
        l = np.zeros(len(gr))
        O = np.zeros((len(gr), dv))
        for e, j in enumerate(cols):
            kt = np.arange(j * bk, min((j + 1) * bk, Nk))
            S = (q[gr] @ k[kt].T) * scale
            if causal:
                S = np.where(kt[None, :] <= gr[:, None], S, -np.inf)
            rowmax = S.max(axis=1)
            m_new = np.maximum(m, rowmax)
            live = np.isfinite(rowmax)
            gap = np.max(rowmax[live] - m_new[live]) if live.any() else -np.inf
            record["gap"][e, g] = gap
            if replay is not None:
                skip = bool(replay[e, g])
            else:
                skip = bool(gap < lam)
            record["skip"][e, g] = skip
            fin = np.isfinite(m_new)
            alpha = np.where(fin, np.exp(np.where(fin, m - m_new, 0.0)), 1.0)
            Pt = np.where(fin[:, None], np.exp(S - np.where(fin, m_new, 0.0)[:, None]), 0.0)
            l = alpha * l + Pt.sum(axis=1)
            if skip:
                record["pv_skip"] += 1
            else:
                record["pv_exec"] += 1
                O = alpha[:, None] * O + Pt @ v[kt]
            m = m_new
        if np.any(l == 0):
            raise ValueError("a query row keeps no key: restricted softmax undefined")
        y[g * PV_GROUP_ROWS:g * PV_GROUP_ROWS + len(gr)] = O / l[:, None]
    return y, record


def attend_head(q, k, v, row_ptr, col_idx, row_base, bq, bk, causal=False, scale=None,
                lam=None, qblocks=None, replay=None):
    """Apply attend_qblock to the query blocks of one (batch, head).

    row_ptr/col_idx: the global CSR; row_base: CSR row of query block 0 of this
    head.  Returns (y [N, dv] with NaN in blocks not computed, records by block).
    replay: optional dict {block i: bool array} of forced skip decisions.
    """
    N = q.shape[0]
    nqb = -(-N // bq)
    y = np.full((N, v.shape[1]), np.nan)
    recs = {}
    for i in (range(nqb) if qblocks is None else qblocks):
        r = row_base + i
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        rp = None if replay is None else replay.get(i)
        yi, rec = attend_qblock(q, k, v, i, cols, bq, bk, causal, scale, lam, rp)
        y[i * bq:min((i + 1) * bq, N)] = yi
        recs[i] = rec
    return y, recs
