"""Oracle-side composition used by the GPU parity tests (test infrastructure).

Builds the oracle's view of a workload (its own planner, exact bf16 upcast)
and compares the library's outputs with it.  Nothing here calls the HIP path.
"""

import dataclasses

import numpy as np

from oracle import flash as OF
from oracle import layout as OL
from oracle import numerics as ON
from oracle import predict as OP

# Output tolerance against fp64 on the same mask (bf16 inputs).
MAX_ABS = 1e-2
MEAN_ABS = 1e-3
LAMBDA_BORDER = 1e-3


def to_f64(x: np.ndarray) -> np.ndarray:
    """Generator output (uint16 bf16 bits or float32) -> the float64 values the kernels read."""
    if x.dtype == np.uint16:
        return ON.bf16_to_f64(x)
    return ON.bf16_to_f64(ON.f32_to_bf16(x))


def oracle_perm(w) -> np.ndarray:
    return OL.plan_permutation(w.N, w.order, w.latent, w.window, w.txt_len, w.first_frame_sink)


def oracle_perm_k(w) -> np.ndarray:
    """The keys' reorder: their own grid when the workload gives one."""
    if w.latent_k is None and w.txt_len_k is None:
        return oracle_perm(w)
    return OL.plan_permutation(w.N_k, w.order, w.latent if w.latent_k is None else w.latent_k, w.window,
                               w.txt_len if w.txt_len_k is None else w.txt_len_k, w.first_frame_sink)


def permuted(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    return OL.permute_rows(to_f64(x), perm)


def tile_pattern(w):
    """The oracle's tile-window block pattern of the workload, or None."""
    if w.tile is None:
        return None
    return OL.plan_tile_window(w.N, w.order, w.latent, w.window, w.txt_len, w.first_frame_sink, w.tile,
                               w.tile_radius, w.block_q, w.block_k)


def mask_params(w, sparsity="default") -> OP.MaskParams:
    s = w.sparsity if sparsity == "default" else sparsity
    return OP.MaskParams(N=w.N, N_k=None if w.N_k == w.N else w.N_k, block_q=w.block_q, block_k=w.block_k,
                         causal=w.causal, forced=tile_pattern(w),
                         window=w.window_tokens, sink_front=w.sink_front, sink_back=w.sink_back,
                         sink_rows=w.sink_rows,
                         tau=w.tau, theta=w.theta, sparsity=s)


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


def attend_rows(qp, kp, vp, w, rp, ci, row_base, qblocks, skip_bits=None, groups=4):
    """Oracle outputs for some query blocks of one (b, h) on the GPU's CSR.

    skip_bits: the GPU's pv_skip array (uint8, entry-major, ``groups`` per entry)
    replayed so the outputs are compared on identical PV decisions.
    Returns (y dict block -> rows, records dict block -> record).
    """
    ys, recs = {}, {}
    for i in qblocks:
        r = row_base + i
        cols = ci[rp[r]:rp[r + 1]]
        replay = None
        if w.lam is not None and skip_bits is not None:
            ng = -(-(min((i + 1) * w.block_q, w.N) - i * w.block_q) // OF.PV_GROUP_ROWS)
            replay = np.zeros((len(cols), ng), dtype=bool)
            for e in range(len(cols)):
                for g in range(ng):
                    replay[e, g] = bool(skip_bits[(rp[r] + e) * groups + g])
        y, rec = OF.attend_qblock(qp, kp, vp, i, cols, w.block_q, w.block_k, causal=w.causal,
                                  lam=w.lam, replay=replay)
        ys[i], recs[i] = y, rec
    return ys, recs


def lambda_disagreements(rec, lam):
    """(e, g) where the replayed decision differs from the oracle's own decision by more than the border."""
    own = rec["gap"] < lam
    diff = own != rec["skip"]
    far = np.abs(rec["gap"] - lam) > LAMBDA_BORDER
    return int(np.count_nonzero(diff & far)), int(np.count_nonzero(diff))
