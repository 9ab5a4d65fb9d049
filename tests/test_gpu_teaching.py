"""The tiny teaching video on the GPU (MI355X only): sparse block covers and a sparse
predicted mask through the 16x16-block attention kernel, against the fp64 oracle.

Four frames of a 4x4 grid (N = 64, d = 64, fp32 inputs rounded to bf16 by the permute
step).  The SparseAttn article (section 3.3) defines three token masks on it: same
frame (spatial), same position (temporal) and their union; section 04 ledgers their
block covers.  Here each cover at b = 16 is handed to the attention call as a CSR, in
the frame-major order and in the pixel-major reorder (window [4,1,1], the page's
argsort by pixel), with PV skip off and on.  Where a cover equals its token mask (same
frame in frame-major order: the four diagonal blocks, 75% of the blocks skipped) the
output is also checked against the restricted softmax of the token mask itself; the
same-position cover in pixel-major order is the same four blocks, of which the mask
uses the sixteen diagonal 4x4 tiles.  The predicted-mask case uses the article's
frame/position construction widened to d = 64: the frame head predicts exactly the
four diagonal blocks, the position head's blocks fall under the similarity guard.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import image_dit_amd as sa  # noqa: E402
from oracle import attention as OA  # noqa: E402
from oracle import predict as OP  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402
from workloads.configs import ORDER_WINDOW  # noqa: E402

import _ref as R  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

T, P, B16 = 4, 16, 16
TINY = CONFIGS["tiny"]
ORDERS = {
    "frame_major": TINY,
    # window [T,1,1] on the 4x4x4 grid is the page's stable argsort by pixel
    "pixel_major": dataclasses.replace(TINY, order=ORDER_WINDOW, window=(T, 1, 1)),
}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def block_cover(mask, b):
    nb = mask.shape[0] // b
    return mask.reshape(nb, b, nb, b).any(axis=(1, 3))


def attend_on_csr(w, q, k, v, cover):
    """Permute q, k, v, run the attention call on the CSR of `cover`, un-permute."""
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg)
    path.permute(dev(q), dev(k), dev(v))
    rp, ci = OP.mask_to_csr(np.tile(cover, (w.B * w.Hq, 1)) if cover.shape[0] != cfg.rows else cover)
    path.row_ptr.copy_(torch.from_numpy(rp.astype(np.int32)))
    path.col_idx[:len(ci)].copy_(torch.from_numpy(ci.astype(np.int32)))
    path.attend()
    path.unpermute()
    torch.cuda.synchronize()
    return path, rp, ci


def check_outputs(w, path, q, k, v, rp, ci, perm, token_masks=None):
    """Every query block of every head against attend_qblock on the same CSR (PV decisions
    replayed), counters exact, un-permute exact; with token_masks {head: mask} also against
    the restricted softmax of the token mask.  Returns (max error, skipped PV groups)."""
    skip = path.pv_skip.cpu().numpy()
    o_perm = path.o_perm.cpu().numpy()
    cfg = path.cfg
    worst, total, n = 0.0, 0.0, 0
    for h in range(w.Hq):
        qp, kp, vp = (R.permuted(x[0, h], perm) for x in (q, k, v))
        r0 = h * cfg.n_qb
        ys, recs = R.attend_rows(qp, kp, vp, w, rp, ci, r0, range(cfg.n_qb), skip, path.groups)
        for i, y in ys.items():
            d = np.abs(o_perm[0, h, i * B16:(i + 1) * B16] - y)
            worst = max(worst, float(d.max()))
            total += float(d.sum())
            n += d.size
            if w.lam is not None:
                far, _ = R.lambda_disagreements(recs[i], w.lam)
                assert far == 0
        if token_masks is not None and h in token_masks and w.lam is None:
            y, _ = OA.restricted_attention(qp, kp, vp, token_masks[h])
            d = np.abs(o_perm[0, h] - y)
            assert d.max() <= R.MAX_ABS and d.mean() <= R.MEAN_ABS
    assert worst <= R.MAX_ABS and total / n <= R.MEAN_ABS
    cnt = path.counters.cpu().numpy()
    nnz = int(rp[-1])
    assert cnt[0] == nnz and cnt[1] + cnt[2] == nnz  # one 16-row group per entry
    assert cnt[2] == int(skip[:nnz].sum())
    if w.lam is None:
        assert cnt[2] == 0
    from oracle import layout as OL
    assert np.array_equal(path.o.cpu().numpy(), OL.unpermute_rows(o_perm, perm))
    return worst, int(cnt[2])


@pytest.mark.parametrize("lam", [None, -8.0])
@pytest.mark.parametrize("mask_name", ["spatial", "temporal", "union"])
@pytest.mark.parametrize("order", list(ORDERS))
def test_teaching_mask_block_cover(order, mask_name, lam):
    w = dataclasses.replace(ORDERS[order], lam=lam)
    q, k, v = generate(w)
    perm = R.oracle_perm(w)
    tm = OA.spatiotemporal_masks(T, P)[mask_name][np.ix_(perm, perm)]
    cover = block_cover(tm, B16)
    exact = np.array_equal(np.kron(cover, np.ones((B16, B16), dtype=bool)), tm)
    path, rp, ci = attend_on_csr(w, q, k, v, cover)
    assert path.statuses()[1] == sa.SA_OK
    assert np.array_equal(path.perm_host.astype(np.int64), perm)
    worst, skipped = check_outputs(w, path, q, k, v, rp, ci, perm, {0: tm} if exact else None)
    kept = int(cover.sum())
    log(f"[teaching] {order} {mask_name} lam={lam}: kept blocks {kept}/16 exact_cover={exact} "
        f"out_max={worst:.3e} pv_skipped={skipped}")
    # the same-frame cover in frame-major order is the four diagonal blocks and equals its
    # token mask; the same-position cover in pixel-major order is the four diagonal blocks
    # too (each holds four 4x4 same-position tiles: a quarter of its pairs are allowed);
    # the others cover every block
    if (order, mask_name) == ("frame_major", "spatial"):
        assert exact and np.array_equal(cover, np.eye(4, dtype=bool))
    elif (order, mask_name) == ("pixel_major", "temporal"):
        assert not exact and np.array_equal(cover, np.eye(4, dtype=bool))
        assert int(tm.sum()) == 256 and np.array_equal(tm, np.kron(np.eye(16, dtype=bool), np.ones((4, 4), bool)))
    else:
        assert cover.all()


@pytest.mark.parametrize("lam", [None, -2.0])
def test_teaching_predicted_mask_is_sparse(lam):
    """Frame/position heads at b = 16, tau = 0.9, theta = 0.5 through the whole path: the
    frame head's predicted mask is exactly the same-frame cover (4 of 16 blocks), the
    position head's rows are forced whole by the guard; outputs against fp64 on the GPU's
    CSR (PV decisions replayed when lambda is set) and, for the frame head, against the
    restricted softmax of the same-frame mask."""
    w = dataclasses.replace(TINY, Hq=2, Hkv=2, seed=7, lam=lam)
    q, k, v = generate(w, "frame_position")
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg)
    mask = torch.zeros((cfg.rows, cfg.n_kb), dtype=torch.uint8, device="cuda")
    path.permute(dev(q), dev(k), dev(v))
    path.predict(mask_out=mask)
    path.attend()
    path.unpermute()
    torch.cuda.synchronize()
    assert path.statuses() == (sa.SA_OK, sa.SA_OK)
    perm = R.oracle_perm(w)
    gmask = mask.cpu().numpy().astype(bool)
    mp = R.mask_params(w)
    for h in range(w.Hq):
        ref = OP.predict_head(R.permuted(q[0, h], perm), R.permuted(k[0, h], perm), mp)
        bad, _, _, _ = R.compare_head_mask(gmask[h * cfg.n_qb:(h + 1) * cfg.n_qb], ref, mp)
        assert not bad
    assert np.array_equal(gmask[:4], np.eye(4, dtype=bool))
    assert gmask[4:].all()
    rp, ci = path.csr_host()
    rp_m, ci_m = OP.mask_to_csr(gmask)
    assert np.array_equal(rp, rp_m) and np.array_equal(ci, ci_m)
    spatial = OA.spatiotemporal_masks(T, P)["spatial"]
    worst, skipped = check_outputs(w, path, q, k, v, rp, ci, perm, {0: spatial})
    log(f"[teaching] predicted lam={lam}: nnz={int(rp[-1])} out_max={worst:.3e} pv_skipped={skipped}")


def test_teaching_pv_skip_on_full_cover():
    """PV skip in the 16x16-block kernel: the frame head over every block, lambda = -2.
    A query block meets its own frame's keys (scores 4.5 in natural units) at its diagonal
    block; the later blocks hold only other frames' keys (scores near 0), so their gap to
    the running maximum is about -4.5 and their PV products are skipped, which the
    outputs, replayed against fp64, and the counters must show."""
    w = dataclasses.replace(TINY, Hq=2, Hkv=2, seed=7, lam=-2.0)
    q, k, v = generate(w, "frame_position")
    perm = R.oracle_perm(w)
    path, rp, ci = attend_on_csr(w, q, k, v, np.ones((4, 4), dtype=bool))
    assert path.statuses()[1] == sa.SA_OK
    worst, skipped = check_outputs(w, path, q, k, v, rp, ci, perm)
    skip = path.pv_skip.cpu().numpy()[:int(rp[-1])].reshape(2, 4, 4).astype(bool)
    log(f"[teaching] full cover lam=-2: out_max={worst:.3e} pv_skipped={skipped}")
    # frame head: block j of query block i is skipped exactly when j > i
    assert np.array_equal(skip[0], np.triu(np.ones((4, 4), dtype=bool), 1))
    assert skipped >= 6
