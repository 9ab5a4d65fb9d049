"""Mask rows the block-mask predictor admits (fp64 oracle, test infrastructure only).

The predictor's decisions at its thresholds are comparisons of rounded
quantities: the self-similarity guard against theta, the cumulative mass at the
TopCdf cut against tau (SpargeAttn notes, section 2.2, TopCdf) and the order of
candidates whose compressed logits tie at the cut.  Another implementation that
computes the same statistics with a different rounding may take such a decision
the other way.  A row is admissible when it equals the oracle row or the oracle
row with one combination of its flagged near-boundary decisions taken the other
way; every other block, the forced blocks included, must agree.  Used by the
parity tests and by the benchmark's report of borderline rows.
"""

import dataclasses

import numpy as np

from . import predict as OP


def _tie_equivalent(got, row, logits, cand):
    """True when ``got`` keeps the same forced blocks and as many candidates as ``row`` and
    every candidate on which they differ has a compressed logit within LOGIT_TIE of the
    cut between the kept and the dropped candidates of ``row`` (an order the rounding of
    the statistics may swap)."""
    if np.any((got != row) & ~cand) or got.sum() != row.sum():
        return False
    diff = np.nonzero(got != row)[0]
    if diff.size == 0:
        return True
    kept, dropped = cand & row, cand & ~row
    if not kept.any() or not dropped.any():
        return False
    lo, hi = logits[kept].min(), logits[dropped].max()
    if lo - hi > OP.LOGIT_TIE:
        return False
    return bool(np.all(np.abs(logits[diff] - 0.5 * (lo + hi)) <= OP.LOGIT_TIE))


def admissible_row(got: np.ndarray, i: int, ref: dict, p: OP.MaskParams):
    """Whether a mask row the library predicted for query block i is one the oracle allows.

    The oracle row always is.  A row the oracle flags as borderline may instead equal the
    oracle's row with its flagged decisions taken the other way, one combination at a
    time: a query-block similarity within THETA_BORDER of theta on either side, each
    subset of the valid key blocks whose similarity lies within THETA_BORDER of theta
    (at most four), tau moved by TAU_BORDER either way (the cumulative mass at the cut
    within that band), and a swap among candidates whose logits tie within LOGIT_TIE at
    the cut.  Everything else, the forced blocks included, must agree.
    Returns (ok, kinds) with kinds the set of flags of the row ("" when it equals the
    oracle row)."""
    row = ref["mask"][i]
    info = ref["info"][i]
    if np.array_equal(got, row):
        return True, set()
    border = set(info["border"])
    if not border:
        return False, border
    logits, simq, simk = ref["logits"][i], ref["simq"][i], ref["simk"]
    valid = OP._valid_blocks(i, p)
    th = p.theta if (p.theta is not None and p.theta > 0) else None
    q_opts = [simq]
    k_sets = [simk]
    if th is not None:
        if abs(simq - th) <= OP.THETA_BORDER:
            q_opts = [th - 2 * OP.THETA_BORDER, th + 2 * OP.THETA_BORDER]
        near = np.nonzero(valid & (np.abs(simk - th) <= OP.THETA_BORDER))[0]
        if near.size > 4:
            return False, border
        k_sets = []
        for bits in range(1 << near.size):
            s = simk.copy()
            for n, j in enumerate(near):
                s[j] = th - 2 * OP.THETA_BORDER if (bits >> n) & 1 else th + 2 * OP.THETA_BORDER
            k_sets.append(s)
    t_opts = [p.tau]
    if p.tau is not None and 0 < p.tau < 1:
        t_opts = [p.tau, p.tau - OP.TAU_BORDER, min(1.0, p.tau + OP.TAU_BORDER)]
    for sq in q_opts:
        for sk in k_sets:
            for tau in t_opts:
                pp = p if tau == p.tau else dataclasses.replace(p, tau=tau)
                alt, _ = OP.predict_row(i, logits, sq, sk, pp)
                if np.array_equal(got, alt):
                    return True, border
                cand = valid & ~OP._forced_blocks(i, pp, sk, valid)
                if (th is None or sq >= th) and i * p.block_q >= p.sink_rows and \
                        _tie_equivalent(got, alt, logits, cand):
                    return True, border
    return False, border


def compare_head_mask(gpu_rows: np.ndarray, ref: dict, p: OP.MaskParams, rows=None):
    """gpu_rows [n_qb, n_kb] bool vs an oracle predict_head result.

    Returns (rows not admissible, rows that differ from the oracle row but are admissible,
    rows checked, count of admissible differing rows by flag kind).  See admissible_row.
    """
    bad, border, checked = [], [], 0
    kinds = {"tau": 0, "theta": 0, "tie": 0}
    for i in (range(gpu_rows.shape[0]) if rows is None else rows):
        checked += 1
        ok, flags = admissible_row(gpu_rows[i], i, ref, p)
        if not ok:
            bad.append(i)
        elif flags:
            border.append(i)
            for f in flags:
                kinds[f] += 1
    return bad, border, checked, kinds


def borderline_counts(ref: dict, rows=None):
    """Oracle rows flagged near a decision boundary, by kind (whether or not the library differs)."""
    kinds = {"tau": 0, "theta": 0, "tie": 0}
    for i in (range(len(ref["info"])) if rows is None else rows):
        for f in ref["info"][i]["border"]:
            kinds[f] += 1
    return kinds
