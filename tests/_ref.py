"""Oracle-side composition used by the GPU parity tests (test infrastructure).

Builds the oracle's view of a workload (its own planner, exact bf16 upcast)
and compares the library's outputs with it.  Nothing here calls the HIP path.
"""

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


from oracle.admissible import (  # noqa: E402,F401
    _tie_equivalent, admissible_row, borderline_counts, compare_head_mask)


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
