"""Calibration of the selection knobs under output-error bounds.

The search follows the hyper-parameter procedure of the SpargeAttn reading
notes (section 2.4, calibration, after the paper's section 3.6): per
attention layer, first choose the TopCdf mass tau and the similarity guard
theta that give the most sparsity while the relative L1 error of the output,
sum|O - O'| / sum|O|, stays below l1; then, with those fixed, choose the
PV-skip threshold lambda that gives the most combined sparsity while the error
stays below l2.  The notes list (l1, l2) per model family (0.05 / 0.06 for the
video models, 0.07 / 0.08 for the image models, ...).

The error can be measured on every row or, as the Sparse-VideoGen profiling
step described in the SparseAttn article (section 05) does, on a sample of
query rows: here a sample of whole query blocks per head, whose dense outputs
cost one attention call over a CSR that holds every valid key block for the
sampled blocks and a single block elsewhere.

Every output, reference or candidate, comes from the library's own entry
points (``sa_predict_mask_gather`` for the candidate masks,
``sa_sparse_attn_fwd_gather`` for both outputs; with keys on a grid of their
own, which the gather forms do not take, the materialising calls on copies
reordered once); only the error sums use torch reductions on the device.  The
selection rules themselves are plain host logic (``select_tau_theta``,
``select_lambda``).
"""

from dataclasses import dataclass, replace
from typing import Iterable, List, Optional, Sequence

import numpy as np

from . import _lib as L
from .pipeline import PathConfig, SparseAttentionPath


@dataclass(frozen=True)
class Trial:
    """One candidate setting and what it measured."""
    tau: Optional[float]
    theta: Optional[float]
    lam: Optional[float]
    l1: float                  # relative L1 error against the dense output (sampled rows or all)
    mask_sparsity: float       # 1 - kept / valid block pairs
    combined_sparsity: float   # QK + PV block products skipped, over twice the valid pairs


def rel_l1(o_ref, o) -> float:
    """sum|O - O'| / sum|O| (SpargeAttn reading notes, section 2.4), accumulated in fp64."""
    ref = o_ref.double()
    den = float(ref.abs().sum())
    if den == 0.0:
        raise ValueError("reference output is all zero")
    return float((ref - o.double()).abs().sum()) / den


def select_tau_theta(trials: Sequence[Trial], l1: float) -> Optional[Trial]:
    """Most mask sparsity among the trials with error < l1 (ties: smaller error, then the
    earlier trial); None when no trial meets the bound."""
    ok = [(i, t) for i, t in enumerate(trials) if t.l1 < l1]
    if not ok:
        return None
    return min(ok, key=lambda it: (-it[1].mask_sparsity, it[1].l1, it[0]))[1]


def select_lambda(trials: Sequence[Trial], l2: float) -> Optional[Trial]:
    """Most combined sparsity among the trials with error < l2 (ties: smaller error, then the
    earlier trial); None when no trial meets the bound."""
    ok = [(i, t) for i, t in enumerate(trials) if t.l1 < l2]
    if not ok:
        return None
    return min(ok, key=lambda it: (-it[1].combined_sparsity, it[1].l1, it[0]))[1]


def valid_blocks_per_row(cfg: PathConfig) -> np.ndarray:
    """Valid key blocks of each query block of one head (all, or the causal prefix)."""
    i = np.arange(cfg.n_qb)
    if not cfg.causal:
        return np.full(cfg.n_qb, cfg.n_kb, dtype=np.int64)
    last_q = np.minimum((i + 1) * cfg.block_q, cfg.N) - 1
    return np.minimum(cfg.n_kb, last_q // cfg.block_k + 1)


def reference_csr(cfg: PathConfig, sampled: Optional[np.ndarray] = None):
    """Host CSR for the dense reference: every valid key block for the query blocks in
    ``sampled`` (bool [B*Hq*n_qb]; None = all rows), key block 0 alone for the others."""
    nv = np.tile(valid_blocks_per_row(cfg), cfg.B * cfg.Hq)
    take = np.ones(cfg.rows, dtype=bool) if sampled is None else np.asarray(sampled, dtype=bool)
    counts = np.where(take, nv, 1)
    row_ptr = np.zeros(cfg.rows + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.concatenate([np.arange(c, dtype=np.int32) for c in counts]) if cfg.rows else \
        np.zeros(0, dtype=np.int32)
    return row_ptr.astype(np.int32), col_idx


def sample_query_blocks(cfg: PathConfig, per_head: int, seed: int = 0) -> np.ndarray:
    """``per_head`` distinct query blocks of every (batch, head), drawn without replacement
    (bool [B*Hq*n_qb])."""
    rng = np.random.default_rng(seed)
    take = np.zeros(cfg.rows, dtype=bool)
    n = min(per_head, cfg.n_qb)
    for bh in range(cfg.B * cfg.Hq):
        take[bh * cfg.n_qb + rng.choice(cfg.n_qb, size=n, replace=False)] = True
    return take


class Calibrator:
    """Runs candidate settings of one layer's q, k, v (bf16, original token order, on the
    device) through the library and measures their error against the dense output."""

    def __init__(self, cfg: PathConfig, q, k, v, sample_blocks_per_head: Optional[int] = None,
                 seed: int = 0):
        import torch

        self.torch = torch
        self.cfg = cfg
        self.q, self.k, self.v = q, k, v
        # the gather form takes one permutation for queries and keys
        self.gather = cfg.N_k == cfg.N and cfg.latent_k is None and cfg.txt_len_k is None
        self.path = SparseAttentionPath(cfg, device=q.device, materialize=not self.gather)
        if not self.gather:
            self.path.permute(q, k, v)
        self.sampled = (None if sample_blocks_per_head is None
                        else sample_query_blocks(cfg, sample_blocks_per_head, seed))
        # token rows of O the error is measured on
        if self.sampled is None:
            self.rows = None
        else:
            qb = np.nonzero(self.sampled)[0]
            bh, i = qb // cfg.n_qb, qb % cfg.n_qb
            tok = [(b_h, t) for b_h, ii in zip(bh, i)
                   for t in range(ii * cfg.block_q, min((ii + 1) * cfg.block_q, cfg.N))]
            bhs = np.array([x[0] for x in tok], dtype=np.int64)
            pos = np.array([x[1] for x in tok], dtype=np.int64)
            orig = self.path.perm_host.astype(np.int64)[pos]  # O is stored at the original rows
            self.rows = (torch.from_numpy(bhs // cfg.Hq).to(q.device), torch.from_numpy(bhs % cfg.Hq).to(q.device),
                         torch.from_numpy(orig).to(q.device))
        self.o_ref = self._dense()

    def _pick(self, o):
        if self.rows is None:
            return o
        b, h, t = self.rows
        return o[b, h, t]

    def _dense(self):
        torch = self.torch
        cfg = self.cfg
        rp, ci = reference_csr(cfg, self.sampled)
        row_ptr = torch.from_numpy(rp).to(self.q.device)
        col_idx = torch.from_numpy(ci).to(self.q.device)
        o = torch.empty((cfg.B, cfg.Hq, cfg.N, cfg.D), dtype=torch.float32, device=self.q.device)
        status = torch.zeros(1, dtype=torch.int32, device=self.q.device)
        ap = replace(cfg, lam=None).attn_params(len(ci))
        p = self.path
        if self.gather:
            L.sa_sparse_attn_fwd_gather(self.q, self.k, self.v, p.perm, o, ap, row_ptr, col_idx, status)
        else:
            o_perm = torch.empty_like(o)
            L.sa_sparse_attn_fwd(p.qp, p.kp, p.vp, o_perm, ap, row_ptr, col_idx, status)
            L.sa_unpermute(o_perm, o, p.perm)
        torch.cuda.synchronize()
        if int(status.item()) != L.SA_OK:
            raise L.SparseAttnError(int(status.item()), "dense reference")
        return self._pick(o).clone()

    def trial(self, tau=None, theta=None, lam=None, sparsity=None) -> Trial:
        """Predict with (tau, theta, sparsity), attend with lam; measure the error."""
        torch = self.torch
        cfg = replace(self.cfg, tau=tau, theta=theta, lam=lam, sparsity=sparsity)
        p = self.path
        p.cfg = cfg
        p.mp = cfg.mask_params()
        p.ap = cfg.attn_params(p.col_cap)
        if self.gather:
            p.predict_gather(self.q, self.k)
            p.attend_gather(self.q, self.k, self.v)
        else:
            p.predict()
            p.attend()
            p.unpermute()
        torch.cuda.synchronize()
        st = p.statuses()
        if st != (L.SA_OK, L.SA_OK):
            raise L.SparseAttnError(st[0] if st[0] != L.SA_OK else st[1], "trial")
        rp = p.row_ptr.cpu().numpy().astype(np.int64)
        valid = float(np.tile(valid_blocks_per_row(cfg), cfg.B * cfg.Hq).sum())
        kept = float(rp[-1])
        cnt = p.counters.cpu().numpy()
        if lam is None:
            combined = 1.0 - kept / valid
        else:
            # a kept pair always runs QK; its PV runs for the fraction of row groups not skipped
            pv_frac = float(cnt[1]) / max(1.0, float(cnt[1] + cnt[2]))
            combined = 1.0 - (kept + kept * pv_frac) / (2.0 * valid)
        return Trial(tau, theta, lam, rel_l1(self.o_ref, self._pick(p.o)), 1.0 - kept / valid, combined)

    def search(self, taus: Iterable[float], thetas: Iterable[Optional[float]], lams: Iterable[float],
               l1: float, l2: float, sparsity: Optional[float] = None):
        """Stage 1 over tau x theta (lambda off), stage 2 over lambda at the chosen pair.
        Returns (chosen Trial or None, stage-1 trials, stage-2 trials)."""
        stage1: List[Trial] = [self.trial(tau=t, theta=th, sparsity=sparsity) for t in taus for th in thetas]
        best = select_tau_theta(stage1, l1)
        if best is None:
            return None, stage1, []
        stage2 = [best] + [self.trial(tau=best.tau, theta=best.theta, lam=lm, sparsity=sparsity) for lm in lams]
        return select_lambda(stage2, l2), stage1, stage2
