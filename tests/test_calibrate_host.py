"""Host logic of the calibration search (no GPU): the selection rules of the
SpargeAttn reading notes, section 2.4 (most sparsity under the l1 bound, then
most combined sparsity under l2), the dense-reference CSR and the row sample."""

import numpy as np
import pytest

from image_dit_amd import PathConfig
from image_dit_amd import calibrate as C

torch = pytest.importorskip("torch")


def T(l1, ms, cs=None, tau=0.9, theta=None, lam=None):
    return C.Trial(tau, theta, lam, l1, ms, ms if cs is None else cs)


def test_stage1_takes_the_sparsest_setting_under_the_bound():
    trials = [T(0.01, 0.30, tau=0.99), T(0.04, 0.55, tau=0.95), T(0.049, 0.55, tau=0.9),
              T(0.06, 0.80, tau=0.5)]
    best = C.select_tau_theta(trials, 0.05)
    assert best.tau == 0.95            # 0.80 is over the bound; tie at 0.55 -> smaller error
    assert C.select_tau_theta(trials, 0.005) is None
    assert C.select_tau_theta(trials, 0.07).tau == 0.5
    # the bound is strict, as the notes' "L1 < l1"
    assert C.select_tau_theta([T(0.05, 0.9)], 0.05) is None


def test_stage2_compares_combined_sparsity():
    base = T(0.04, 0.55, 0.55)
    trials = [base, T(0.045, 0.55, 0.70, lam=-12.0), T(0.058, 0.55, 0.78, lam=-8.0),
              T(0.07, 0.55, 0.85, lam=-4.0)]
    assert C.select_lambda(trials, 0.06).lam == -8.0
    assert C.select_lambda(trials, 0.05).lam == -12.0
    assert C.select_lambda(trials, 0.041) is base


def test_rel_l1_definition():
    o = torch.tensor([[1.0, -2.0], [3.0, 0.0]])
    o2 = torch.tensor([[1.5, -2.0], [2.0, 0.5]])
    assert C.rel_l1(o, o2) == pytest.approx((0.5 + 1.0 + 0.5) / 6.0)
    assert C.rel_l1(o, o) == 0.0
    with pytest.raises(ValueError):
        C.rel_l1(torch.zeros(3), torch.ones(3))


def cfg(**kw):
    base = dict(B=2, Hq=3, Hkv=1, N=1000, D=128, block_q=128, block_k=64)
    base.update(kw)
    return PathConfig(**base)


def test_reference_csr_dense_and_sampled():
    c = cfg()
    rp, ci = C.reference_csr(c)
    assert rp[-1] == c.rows * c.n_kb and np.all(np.diff(rp) == c.n_kb)
    assert np.array_equal(ci[:c.n_kb], np.arange(c.n_kb))
    take = np.zeros(c.rows, dtype=bool)
    take[[0, 9, 20]] = True
    rp, ci = C.reference_csr(c, take)
    counts = np.diff(rp)
    assert np.all(counts[take] == c.n_kb) and np.all(counts[~take] == 1)
    assert np.all(ci[rp[1]:rp[2]] == 0)


def test_reference_csr_causal_prefix():
    c = cfg(causal=True, N=700)
    nv = C.valid_blocks_per_row(c)
    # query block i ends at token min(128(i+1), N) - 1; key block j is valid if 64 j <= that
    for i in range(c.n_qb):
        last = min(128 * (i + 1), c.N) - 1
        assert nv[i] == sum(1 for j in range(c.n_kb) if 64 * j <= last)
    rp, ci = C.reference_csr(c)
    for r in range(c.rows):
        assert np.array_equal(ci[rp[r]:rp[r + 1]], np.arange(nv[r % c.n_qb]))


def test_sample_query_blocks_per_head():
    c = cfg()
    take = C.sample_query_blocks(c, 3, seed=5)
    per_head = take.reshape(c.B * c.Hq, c.n_qb).sum(axis=1)
    assert np.all(per_head == 3)
    assert np.array_equal(take, C.sample_query_blocks(c, 3, seed=5))
    assert C.sample_query_blocks(c, 99).all()   # more than n_qb: every block
