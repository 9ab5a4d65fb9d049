"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the pin it covers and its source (page title + section).  The
oracle is never compared to itself: the expected values are printed on the
pages, closed forms, brute force over tiny inputs, or library routines.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import flash as F
from oracle import layout as Lay
from oracle import numerics as Num
from oracle import predict as P
from workloads import p1_demo_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf8") as f:
        return json.load(f)


# ------------------------------------------------------------------ P1: p1 demo printed values

def test_p1_demo_printed_values():
    """SparseAttn article, section 04 + appendix: MSE, row error vs bound, densities."""
    g = _golden("p1_demo.json")
    tol = g["printed_digits_rel_tol"]
    q, k, v, frame, pixel = p1_demo_inputs()
    masks = A.spatiotemporal_masks(4, 16)
    assert masks["union"].mean() == g["union_density"]
    for head, key in ((0, "union_mse_head0"), (1, "union_mse_head1")):
        y_full, _ = A.dense_attention(q[head], k[head], v)
        y_u, _ = A.restricted_attention(q[head], k[head], v, masks["union"])
        mse = float(np.mean((y_u - y_full) ** 2))
        assert mse == pytest.approx(g[key], rel=tol)
    y_full, p = A.dense_attention(q[0], k[0], v)
    y_s, _ = A.restricted_attention(q[0], k[0], v, masks["spatial"])
    err = np.linalg.norm(y_s - y_full, axis=1)
    alpha = 1.0 - A.retained_mass(p, masks["spatial"])
    bound = A.removed_mass_bound(np.maximum(alpha, 0.0), v)
    assert float(err.max()) == pytest.approx(g["spatial_head0_max_row_error"], rel=1e-7)
    assert float(bound.max()) == pytest.approx(g["spatial_head0_max_bound"], rel=1e-7)
    assert np.all(err <= bound + 1e-12)


def test_p1_block_ledger_and_reorder():
    """SparseAttn article, section 04: temporal mask tiles before/after the pixel-major reorder."""
    g = _golden("p1_demo.json")
    masks = A.spatiotemporal_masks(4, 16)
    before = A.block_cost(masks["temporal"], 4)
    _, pixel = A.frame_major_coords(4, 16)
    perm = Lay.plan_permutation(64, Lay.ORDER_WINDOW, latent=(4, 4, 4), window=(4, 1, 1))
    after = A.block_cost(masks["temporal"][np.ix_(perm, perm)], 4)
    for key in ("useful_pairs", "active_tiles", "computed_pairs", "utilization"):
        assert before[key] == g["temporal_blocks_before"][key]
        assert after[key] == g["temporal_blocks_after"][key]
    # permute -> attend -> unpermute restores the output (section 3.4; printed error ~2.2e-16)
    q, k, v, _, _ = p1_demo_inputs()
    old, _ = A.restricted_attention(q[1], k[1], v, masks["temporal"])
    new, _ = A.restricted_attention(Lay.permute_rows(q[1], perm), Lay.permute_rows(k[1], perm),
                                    Lay.permute_rows(v, perm), masks["temporal"][np.ix_(perm, perm)])
    assert np.max(np.abs(Lay.unpermute_rows(new, perm) - old)) <= 4 * g["permutation_max_error_about"]


# ------------------------------------------------------------------ P2: pair counts

def test_pair_counts_closed_forms():
    """SparseAttn article, section 3.3: T^2P^2, TP^2, PT^2, union TP(P+T-1)."""
    g = _golden("p1_demo.json")
    for T, Pn in ((4, 16), (3, 5), (2, 7)):
        masks = A.spatiotemporal_masks(T, Pn)
        closed = A.spatiotemporal_pair_counts(T, Pn)
        for name in ("full", "spatial", "temporal", "union"):
            assert int(masks[name].sum()) == closed[name]
        assert masks["union"].mean() == pytest.approx((Pn + T - 1) / (T * Pn), abs=0)
    c = A.spatiotemporal_pair_counts(4, 16)
    assert {k: c[k] for k in g["pair_counts"]} == g["pair_counts"]


def test_window_pair_counts():
    """Local Sliding and Sparse Attention, Step 2 table and Step 5.4 (L=2048, w=256)."""
    g = _golden("access_ledgers.json")["window_ladder"]
    for L, w in ((7, 3), (16, 5), (33, 33), (40, 1)):
        assert int(A.local_causal_mask(L, w).sum()) == A.window_pair_count(L, w)
        assert int(A.local_causal_mask(L, L).sum()) == A.causal_pair_count(L)
    L, w = g["L"], g["w"]
    assert A.window_pair_count(L, w) == g["window_pairs"]
    red = 100.0 * (1.0 - A.window_pair_count(L, w) / A.causal_pair_count(L))
    assert round(red, 2) == g["reduction_percent_2dp"]


def test_local_sparse_page_tests():
    """Local Sliding and Sparse Attention, Step 4: visibility, block pairs, causal filter, ledger."""
    g = _golden("access_ledgers.json")
    m = A.local_causal_mask(5, 2)
    assert m[3, 3] and m[3, 2] and not m[3, 1] and not m[2, 3]
    b = A.block_pairs_mask(4, 2, {(0, 0), (1, 0)})
    assert b[1, 0] and b[3, 0] and not b[0, 1] and not b[0, 3]
    assert not A.block_pairs_mask(4, 2, set()).any()
    with pytest.raises(ValueError):
        A.block_pairs_mask(4, 2, {(2, 0)})
    with pytest.raises(ValueError):
        A.block_pairs_mask(4, 2, {(0, 1)})
    assert A.block_pairs_mask(4, 2, {(0, 1)}, causal=False)[0, 2]
    s = A.access_summary(A.local_causal_mask(4, 2))
    assert s == {"visible_pairs": g["local_causal_4_2"]["visible_pairs"],
                 "total_pairs": g["local_causal_4_2"]["total_pairs"], "density": 7 / 16}
    for dist, w, want in g["propagation_layers"]:
        want = float("inf") if want == "inf" else want
        assert A.min_propagation_layers(dist, w) == want
    with pytest.raises(ValueError):
        A.min_propagation_layers(-1, 2)


def test_access_pattern_page_tests():
    """Attention Access Pattern Benchmark, Step 4: spec contract, causal masks, ledger."""
    assert A.validate_access_spec("sliding_window", 8, window=3) == []
    assert A.validate_access_spec("sliding_window", 8, window=0)
    assert A.validate_access_spec("sliding_window", 8, window=3, anchors=[9])
    glob = A.access_mask("global", 8, window=3)
    win = A.access_mask("sliding_window", 8, window=3)
    sel = A.access_mask("selective_sparse", 8, window=2, anchors=[0])
    assert not np.triu(glob, k=1).any()
    assert win[7, 5] and not win[7, 4]
    assert sel[7, 0] and sel[7, 6]
    gs, ws = A.access_ledger(glob, 3), A.access_ledger(win, 3)
    assert gs["score_count"] > ws["score_count"]
    assert gs["long_range_coverage"] > ws["long_range_coverage"]
    assert 0 < ws["density"] < 1
    # the selective pattern is the causal window plus anchor columns
    ref = A.local_causal_mask(8, 2)
    ref[:, 0] = True
    assert np.array_equal(sel, ref & np.tril(np.ones((8, 8), dtype=bool)))


# ------------------------------------------------------------------ P3, P4, P5, P6

def _rand(seed, n=12, m=9, d=5, dv=3):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(n, d)), rng.normal(size=(m, d)), rng.normal(size=(m, dv)), rng


def test_restricted_weights_are_renormalised_dense_weights():
    """SparseAttn article, section 3.1: ptilde = p / z on kept keys, rows sum to 1."""
    q, k, v, rng = _rand(0)
    mask = rng.random((12, 9)) < 0.4
    mask[np.arange(12), rng.integers(0, 9, 12)] = True
    _, p = A.dense_attention(q, k, v)
    _, pt = A.restricted_attention(q, k, v, mask)
    z = A.retained_mass(p, mask)
    assert np.allclose(pt, np.where(mask, p / z[:, None], 0.0), rtol=1e-13, atol=1e-16)
    assert np.allclose(pt.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_removed_mass_identity_and_bound():
    """SparseAttn article, section 3.2: ytilde - y = alpha (r - u), ||.|| <= 2 alpha M per row."""
    for seed in range(4):
        q, k, v, rng = _rand(seed, n=20, m=15, d=6, dv=4)
        q *= 3.0
        mask = rng.random((20, 15)) < 0.5
        mask[:, 0] = True
        mask[3] = True  # one full row: alpha = 0, error 0
        y, p = A.dense_attention(q, k, v)
        yt, _ = A.restricted_attention(q, k, v, mask)
        alpha, r, u = A.removed_mass_parts(p, mask, v)
        assert np.allclose(yt, r, rtol=0, atol=1e-13)
        full = alpha == 0
        assert np.allclose(yt[~full] - y[~full], alpha[~full, None] * (r[~full] - u[~full]),
                           rtol=0, atol=1e-13)
        assert np.allclose(yt[full], y[full], rtol=0, atol=1e-13)
        err = np.linalg.norm(yt - y, axis=1)
        assert np.all(err <= A.removed_mass_bound(alpha, v) + 1e-12)


def test_counterexample_and_empty_row():
    """SparseAttn article, section 3.2 counterexample and section 09 empty-row check."""
    g = _golden("p1_demo.json")["counterexample"]
    q = np.array([[1.0]])
    k = np.array([[math.log(99.0)], [0.0]])
    v = np.array([[0.0], [100.0]])
    y, p = A.dense_attention(q, k, v)
    yp, _ = A.restricted_attention(q, k, v, np.array([[True, False]]))
    assert p[0, 0] == pytest.approx(g["retained_mass"], abs=1e-15)
    assert y[0, 0] == pytest.approx(g["dense_output"], abs=1e-12)
    assert yp[0, 0] == g["pruned_output"]
    with pytest.raises(ValueError):
        A.restricted_attention(q, k, v, np.array([[False, False]]))


def test_all_ones_mask_is_brute_force_dense():
    """SparseAttn article, section 04 (full mask gives the dense output): brute-force loops."""
    q, k, v, _ = _rand(5, n=5, m=6, d=3, dv=2)
    y, _ = A.restricted_attention(q, k, v, np.ones((5, 6), dtype=bool))
    for i in range(5):
        s = [sum(q[i, c] * k[j, c] for c in range(3)) / math.sqrt(3) for j in range(6)]
        e = [math.exp(x) for x in s]
        tot = sum(e)
        for c in range(2):
            assert y[i, c] == pytest.approx(sum(e[j] * v[j, c] for j in range(6)) / tot, abs=1e-14)


# ------------------------------------------------------------------ P13 equivariance

def test_permutation_equivariance():
    """SparseAttn article, section 3.4: Attn(PQ,PK,PV,PAP^T) = P Attn(Q,K,V,A)."""
    q, k, v, rng = _rand(9, n=24, m=24, d=8, dv=5)
    mask = rng.random((24, 24)) < 0.3
    mask[np.arange(24), np.arange(24)] = True
    perm = rng.permutation(24)
    y, _ = A.restricted_attention(q, k, v, mask)
    yp, _ = A.restricted_attention(Lay.permute_rows(q, perm), Lay.permute_rows(k, perm),
                                   Lay.permute_rows(v, perm), mask[np.ix_(perm, perm)])
    assert np.allclose(Lay.unpermute_rows(yp, perm), y, rtol=0, atol=1e-14)
    assert np.array_equal(Lay.unpermute_rows(Lay.permute_rows(q, perm), perm), q)


# ------------------------------------------------------------------ numerics

def test_bf16_rounding_matches_torch():
    """float32 -> bf16 RNE against torch's conversion (a library routine), incl. exact ties."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = rng.normal(size=20000).astype(np.float32) * np.float32(1e3)
    base = rng.integers(0, 2 ** 16, size=4000).astype(np.uint32) << np.uint32(16)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    near = (base | np.uint32(0x7FFF)).view(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 3.4e38], dtype=np.float32)
    allx = np.concatenate([x, ties, near, specials])
    allx = allx[np.isfinite(allx) | np.isinf(allx)]
    ref = torch.from_numpy(allx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(Num.f32_to_bf16(allx), ref)
    nan = Num.f32_to_bf16(np.array([np.nan], dtype=np.float32))
    assert np.isnan(Num.bf16_to_f64(nan))[0]
    back = Num.bf16_to_f64(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float64).numpy())


# ------------------------------------------------------------------ P8 similarity

def test_similarity_is_mean_pairwise_cosine():
    """SpargeAttn notes, section 2.2 (block self-similarity; the printed CosSim form)."""
    rng = np.random.default_rng(11)
    x = rng.normal(size=(7, 4)) + 0.5
    x[2] = 0.0  # a zero token contributes a zero unit vector
    means, sim, printed = P.block_stats(x, 7)
    brute = 0.0
    for a in range(7):
        for b in range(7):
            na, nb = np.linalg.norm(x[a]), np.linalg.norm(x[b])
            brute += 0.0 if na == 0 or nb == 0 else x[a] @ x[b] / (na * nb)
    assert sim[0] == pytest.approx(brute / 49, abs=1e-14)
    assert np.allclose(means[0], x.mean(axis=0), rtol=0, atol=1e-15)
    gram = x @ x.T
    assert printed[0] == pytest.approx(float(np.mean(gram / abs(gram.max()))), abs=1e-14)
    xbar = x.mean(axis=0)
    assert printed[0] == pytest.approx(float(xbar @ xbar / np.max(np.sum(x * x, axis=1))), abs=1e-14)
    # partial last block: statistics over its real tokens only
    means2, sim2, _ = P.block_stats(x, 3)
    assert np.allclose(means2[2], x[6], atol=0) and sim2[2] == pytest.approx(1.0, abs=1e-15)
    # identical tokens -> similarity 1; opposite pair -> 0
    assert P.block_stats(np.tile(x[:1], (5, 1)), 5)[1][0] == pytest.approx(1.0, abs=1e-14)
    assert P.block_stats(np.stack([x[0], -x[0]]), 2)[1][0] == pytest.approx(0.0, abs=1e-15)


# ------------------------------------------------------------------ P9, TopCdf through the predictor

def test_topcdf_reach_reading_teaching_example():
    """SpargeAttn notes, section 2.2 item 2: [0.6,0.3,0.1], tau=0.8 -> reach keeps 2.

    Built as 3 one-token key blocks whose compressed softmax is exactly
    [0.3, 0.6, 0.1] once the 1/sqrt(d) scale is applied (d=4, scale 1/2).
    tau=0.65 separates the readings: reach keeps 2; the printed
    cumsum<=tau rule, or dropping the scale, would keep 1.
    """
    probs = np.array([0.3, 0.6, 0.1])
    k = np.zeros((3, 4))
    k[:, 0] = np.log(probs)
    q = np.zeros((3, 4))
    q[0, 0] = 2.0
    for tau, want in ((0.8, {0, 1}), (0.65, {0, 1}), (0.5, {1}), (0.95, {0, 1, 2}), (1.0, {0, 1, 2})):
        p = P.MaskParams(N=3, block_q=1, block_k=1, tau=tau)
        out = P.predict_head(q, k, p, rows=[0])
        assert set(np.nonzero(out["mask"][0])[0]) == want, tau
    # sparsity floor: ceil((1-s)*3) blocks at least
    p = P.MaskParams(N=3, block_q=1, block_k=1, tau=0.5, sparsity=0.5)
    assert set(np.nonzero(P.predict_head(q, k, p, rows=[0])["mask"][0])[0]) == {0, 1}
    p = P.MaskParams(N=3, block_q=1, block_k=1, sparsity=0.0)
    assert P.predict_head(q, k, p, rows=[0])["mask"][0].all()
    # ties in probability: lower block index first
    k2 = np.zeros((3, 4))
    p = P.MaskParams(N=3, block_q=1, block_k=1, sparsity=0.5)  # ceil(1.5) = 2 blocks
    assert set(np.nonzero(P.predict_head(q, k2, p, rows=[0])["mask"][0])[0]) == {0, 1}


def _brute_forced(i, p, simk):
    """Forced key blocks from token-level definitions (sinks, causal window, diagonal)."""
    qs = range(i * p.block_q, min((i + 1) * p.block_q, p.N))
    out = np.zeros(p.n_kb, dtype=bool)
    for j in range(p.n_kb):
        ks = range(j * p.block_k, min((j + 1) * p.block_k, p.N))
        valid = (not p.causal) or any(kk <= qq for kk in ks for qq in qs)
        if not valid:
            continue
        f = p.theta is not None and p.theta > 0 and simk[j] < p.theta
        f |= any(kk < p.sink_front or kk >= p.N - p.sink_back for kk in ks)
        if p.causal:
            f |= p.window > 0 and any(kk <= qq and qq - kk < p.window for kk in ks for qq in qs)
            f |= any(kk == qq for kk in ks for qq in qs)
        out[j] = f
    return out


@pytest.mark.parametrize("N,bq,bk,W,sf,sb", [(100, 16, 8, 20, 3, 0), (77, 8, 16, 9, 0, 5),
                                              (64, 16, 16, 0, 1, 1), (50, 10, 10, 35, 0, 0),
                                              (64, 16, 16, 0, 16, 16), (80, 16, 16, 16, 17, 15)])
def test_forced_blocks_match_token_definitions(N, bq, bk, W, sf, sb):
    """Sinks (MindIE-SD rf_v2 first-frame sink), causal window (Local Sliding page), diagonal."""
    rng = np.random.default_rng(N)
    simk = rng.random(-(-N // bk))
    for theta in (0.3, None):
        _check_forced(P.MaskParams(N=N, block_q=bq, block_k=bk, causal=True, window=W,
                                   sink_front=sf, sink_back=sb, theta=theta), simk)


def _check_forced(p, simk):
    N, bq, bk = p.N, p.block_q, p.block_k
    for i in range(p.n_qb):
        valid = P._valid_blocks(i, p)
        got = P._forced_blocks(i, p, simk, valid)
        assert np.array_equal(got, _brute_forced(i, p, simk)), i
        # valid blocks: a key at or before the block's last query exists
        qs_last = min((i + 1) * bq, N) - 1
        assert np.array_equal(valid, np.arange(p.n_kb) * bk <= qs_last)


def test_keep_floor_counts_forced_blocks():
    """MindIE-SD sparsity argument: the floor ceil((1-s)|valid|) includes forced (sink) blocks."""
    d = 4
    q = np.zeros((6, d))
    q[0, 0] = 1.0
    k = np.zeros((6, d))
    k[:, 0] = [0.0, 5.0, 4.0, 3.0, 2.0, 1.0]  # block 0 is the sink; candidates 1..5 descending
    for s, want in ((0.5, {0, 1, 2}), (0.2, {0, 1, 2, 3, 4}), (0.99, {0, 1})):
        p = P.MaskParams(N=6, block_q=1, block_k=1, sink_front=1, tau=1e-9, sparsity=s)
        got = set(np.nonzero(P.predict_head(q, k, p, rows=[0])["mask"][0])[0])
        assert got == want, s


def test_predicted_mask_guard_and_floor():
    """SpargeAttn notes, section 2.2: low-sim rows full, low-sim columns kept; keep floor."""
    rng = np.random.default_rng(4)
    d, b = 8, 4
    base = rng.normal(size=(6, d)) * 3
    q = np.repeat(base, b, axis=0) + 0.01 * rng.normal(size=(24, d))
    k = q.copy()
    k[8:12] = rng.normal(size=(4, d))  # key block 2 incoherent
    q[16:20] = rng.normal(size=(4, d))  # query block 4 incoherent
    p = P.MaskParams(N=24, block_q=b, block_k=b, tau=0.5, theta=0.6)
    out = P.predict_head(q, k, p)
    assert out["simk"][2] < 0.6 and out["simq"][4] < 0.6
    assert out["mask"][:, 2].all()            # forced column
    assert out["mask"][4].all()               # forced row
    for i in (0, 1, 3, 5):
        assert out["mask"][i, i]              # coherent diagonal blocks dominate
    p2 = P.MaskParams(N=24, block_q=b, block_k=b, tau=0.5, theta=0.6, sparsity=0.5)
    out2 = P.predict_head(q, k, p2)
    for i in range(6):
        assert out2["mask"][i].sum() >= math.ceil(0.5 * 6)


# ------------------------------------------------------------------ P7 predicted-mask special cases

def test_predicted_mask_p1_head0_is_spatial():
    """p1 demo head 0, frame-major, b=16, tau=0.9, theta=0.5 -> the 4 diagonal blocks."""
    q, k, v, _, _ = p1_demo_inputs()
    p = P.MaskParams(N=64, block_q=16, block_k=16, tau=0.9, theta=0.5)
    out = P.predict_head(q[0], k[0], p)
    assert np.array_equal(out["mask"], np.eye(4, dtype=bool))
    tok = A.block_pairs_mask(64, 16, set(zip(*np.nonzero(out["mask"]))), causal=False)
    assert np.array_equal(tok, A.spatiotemporal_masks(4, 16)["spatial"])
    assert int(tok.sum()) == 1024


def test_sink_rows_make_full_rows_of_the_first_frame():
    """MindIE-SD first-frame sink read as full rows: query blocks touching the first
    sink_rows tokens keep their whole valid row; the other rows stay the spatial mask."""
    q, k, v, _, _ = p1_demo_inputs()
    eye = np.eye(4, dtype=bool)
    for sink_rows, full in ((0, []), (16, [0]), (17, [0, 1]), (64, [0, 1, 2, 3])):
        p = P.MaskParams(N=64, block_q=16, block_k=16, tau=0.9, theta=0.5, sink_rows=sink_rows)
        out = P.predict_head(q[0], k[0], p)
        want = eye.copy()
        want[full] = True
        assert np.array_equal(out["mask"], want), sink_rows
        assert [i for i in range(4) if out["info"][i]["forced_row"]] == full
    # causal: the whole valid row of query block 0 is block 0 alone
    p = P.MaskParams(N=64, block_q=16, block_k=16, causal=True, tau=0.9, theta=0.5, sink_rows=16)
    out = P.predict_head(q[0], k[0], p)
    assert np.array_equal(out["mask"][0], [True, False, False, False])
    # query block 1 is no sink row: its diagonal block is forced and block 0, its only
    # candidate, holds all the compressed mass
    assert np.array_equal(out["mask"][1], [True, True, False, False])
    assert not out["info"][1]["forced_row"]


def test_forced_pattern_blocks_are_kept_and_counted():
    """A forced block pattern joins the forced blocks: always kept, counted by the floor."""
    q, k, v, _, _ = p1_demo_inputs()
    forced = np.zeros((4, 4), dtype=bool)
    forced[0, 3] = forced[2, 1] = True
    p = P.MaskParams(N=64, block_q=16, block_k=16, tau=0.9, theta=0.5, forced=forced)
    out = P.predict_head(q[0], k[0], p)
    assert np.array_equal(out["mask"], np.eye(4, dtype=bool) | forced)
    assert out["info"][0]["n_forced"] == 1 and out["info"][1]["n_forced"] == 0
    # the floor ceil((1-s)|valid|) = 2 is met by the forced block plus the top candidate
    p = P.MaskParams(N=64, block_q=16, block_k=16, tau=1e-9, theta=0.5, sparsity=0.5, forced=forced)
    out = P.predict_head(q[0], k[0], p)
    assert out["mask"][0].sum() == 2 and out["mask"][0][3] and out["mask"][0][0]


def test_tile_window_pattern_hand_examples():
    """Sliding tiles on a 1-D latent of 16 tokens, tiles of 4 = blocks: radius 1 pairs each
    block with its neighbours (tridiagonal); radius 0 with itself; blocks of 8 tokens hold
    two tiles each."""
    tri = np.eye(4, dtype=bool) | np.eye(4, k=1, dtype=bool) | np.eye(4, k=-1, dtype=bool)
    got = Lay.plan_tile_window(16, Lay.ORDER_IDENTITY, (1, 1, 16), (1, 1, 1), 0, False, (1, 1, 4), (0, 0, 1), 4, 4)
    assert np.array_equal(got, tri)
    got = Lay.plan_tile_window(16, Lay.ORDER_IDENTITY, (1, 1, 16), (1, 1, 1), 0, False, (1, 1, 4), (0, 0, 0), 4, 4)
    assert np.array_equal(got, np.eye(4, dtype=bool))
    got = Lay.plan_tile_window(16, Lay.ORDER_IDENTITY, (1, 1, 16), (1, 1, 1), 0, False, (1, 1, 4), (0, 0, 0), 8, 4)
    assert np.array_equal(got, np.array([[1, 1, 0, 0], [0, 0, 1, 1]], dtype=bool))
    # text (2 tokens, first in the original order) and the first-frame sink are untiled:
    # with the window order they sit first (frame 0) and last (text); 2 frames of 2x4
    n = 2 + 3 * 2 * 4
    tiles = Lay.token_tiles(n, (3, 2, 4), 2, True, (1, 2, 2))
    assert np.all(tiles[:2] == -1) and np.all(tiles[2:10] == -1)      # text, frame 0
    assert tuple(tiles[10]) == (0, 0, 0) and tuple(tiles[10 + 8 + 3]) == (1, 0, 1)
    got = Lay.plan_tile_window(n, Lay.ORDER_WINDOW, (3, 2, 4), (1, 2, 2), 2, True, (1, 2, 2), (0, 0, 0), 4, 4)
    # permuted order: frame 0 (8 tokens, blocks 0-1), then 4 windows of 4 tokens (blocks 2-5,
    # one tile each), then text (block 6): only the tiled blocks pair, each with itself
    want = np.zeros((7, 7), dtype=bool)
    want[2:6, 2:6] = np.eye(4, dtype=bool)
    assert np.array_equal(got, want)
    # a radius covering the whole grid pairs every tiled block with every tiled block
    got = Lay.plan_tile_window(n, Lay.ORDER_WINDOW, (3, 2, 4), (1, 2, 2), 2, True, (1, 2, 2), (5, 5, 5), 4, 4)
    assert np.array_equal(got, np.outer(want.any(1), want.any(1)))


def test_keys_of_another_length_duplicated_keys():
    """Keys of another length (MindIE-SD latent_shape_k != latent_shape_q): repeating every
    key and value twice leaves dense attention unchanged (each weight halves), and on the
    p1 demo the predicted row of query block i becomes {i, i+4}: the diagonal block and its
    copy share its mass (~0.4995 each), so reaching tau = 0.9 takes both, lower index first."""
    q, k, v, _, _ = p1_demo_inputs()
    q0, k0, v0 = q[0], k[0], v
    k2, v2 = np.concatenate([k0, k0]), np.concatenate([v0, v0])
    for bk in (16, 24):  # 24: a partial last key block
        n_kb = -(-128 // bk)
        y2, _ = F.attend_qblock(q0, k2, v2, 1, range(n_kb), 16, bk)
        y1, _ = F.attend_qblock(q0, k0, v0, 1, range(-(-64 // bk)), 16, bk)
        assert np.allclose(y2, y1, rtol=1e-12, atol=1e-12)
    p = P.MaskParams(N=64, N_k=128, block_q=16, block_k=16, tau=0.9, theta=0.5)
    out = P.predict_head(q0, k2, p)
    want = np.zeros((4, 8), dtype=bool)
    for i in range(4):
        want[i, i] = want[i, i + 4] = True
    assert np.array_equal(out["mask"], want)
    # the back sink counts from the end of the keys
    p = P.MaskParams(N=64, N_k=128, block_q=16, block_k=16, tau=0.9, theta=0.5, sink_back=1)
    out = P.predict_head(q0, k2, p)
    assert out["mask"][:, 7].all() and out["info"][0]["n_forced"] == 1
    with pytest.raises(ValueError):
        P.predict_head(q0, k2, P.MaskParams(N=64, N_k=128, block_q=16, block_k=16, causal=True, tau=0.9))


def test_predicted_mask_p1_head1_pixel_major_is_temporal():
    """p1 demo head 1 after the pixel-major reorder, b=4 -> the 16 diagonal tiles (256 pairs)."""
    q, k, v, _, pixel = p1_demo_inputs()
    perm = np.argsort(pixel, kind="stable")
    p = P.MaskParams(N=64, block_q=4, block_k=4, tau=0.9, theta=0.5)
    out = P.predict_head(q[1][perm], k[1][perm], p)
    assert np.array_equal(out["mask"], np.eye(16, dtype=bool))
    tok = A.block_pairs_mask(64, 4, set(zip(*np.nonzero(out["mask"]))), causal=False)
    assert np.array_equal(tok, A.spatiotemporal_masks(4, 16)["temporal"][np.ix_(perm, perm)])


def test_predicted_mask_iid_blocks_all_forced():
    """iid N(0,1) blocks (tiny workload, d=64, b=16): sim ~ 1/b < 0.5 -> every row full."""
    from workloads import generate, get_config

    cfg = get_config("tiny")
    q, k, _ = generate(cfg)
    qb = Num.bf16_to_f64(Num.f32_to_bf16(q[0, 0]))
    kb = Num.bf16_to_f64(Num.f32_to_bf16(k[0, 0]))
    p = P.MaskParams(N=64, block_q=16, block_k=16, tau=0.9, theta=0.5)
    out = P.predict_head(qb, kb, p)
    assert np.all(out["simq"] < 0.5) and np.all(out["simk"] < 0.5)
    assert out["mask"].all()


# ------------------------------------------------------------------ CSR

def test_csr_roundtrip_bruteforce():
    rng = np.random.default_rng(2)
    m = rng.random((13, 9)) < 0.3
    rp, ci = P.mask_to_csr(m)
    pos = 0
    for r in range(13):
        cols = [j for j in range(9) if m[r, j]]
        assert rp[r] == pos and list(ci[pos:pos + len(cols)]) == cols
        pos += len(cols)
    assert rp[-1] == pos
    assert np.array_equal(P.csr_to_mask(rp, ci, 9), m)


# ------------------------------------------------------------------ P10 lambda emulation

def _block_case(seed, N=100, d=16, causal=False):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(N, d)) * 2
    k = rng.normal(size=(N, d)) * 2
    v = rng.normal(size=(N, d))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_lambda_off_equals_restricted_softmax(causal):
    """SpargeAttn notes, section 2.1: the online recurrence equals the two-pass softmax."""
    q, k, v = _block_case(1)
    bq, bk = 40, 16
    for i in range(3):
        cols = [0, 2, 3, 6] if not causal else [j for j in range(7) if j * bk <= min((i + 1) * bq, 100) - 1]
        y2, _ = F.attend_qblock(q, k, v, i, cols, bq, bk, causal=causal)
        yo, rec = F.attend_qblock(q, k, v, i, cols, bq, bk, causal=causal, lam=-np.inf)
        assert np.allclose(yo, y2, rtol=0, atol=1e-14)
        assert rec["pv_skip"] == 0
        # definition check: token mask from the kept blocks
        rows = np.arange(i * bq, min((i + 1) * bq, 100))
        keys = np.concatenate([np.arange(j * bk, min((j + 1) * bk, 100)) for j in cols])
        tm = np.zeros((len(rows), 100), dtype=bool)
        tm[:, keys] = True
        if causal:
            tm &= np.arange(100)[None, :] <= rows[:, None]
        yr, _ = A.restricted_attention(q[rows], k, v, tm)
        assert np.allclose(y2, yr, rtol=0, atol=1e-14)


def test_lambda_skip_drops_only_small_weights():
    """SpargeAttn notes, section 2.3: skipped groups only lose weights below e^lambda."""
    rng = np.random.default_rng(7)
    N, d, bq, bk = 96, 16, 64, 16
    u = np.zeros(d)
    u[0] = 1.0
    q = 8.0 * u + rng.normal(size=(N, d))
    k = 0.5 * rng.normal(size=(N, d))
    k[:16] = 8.0 * u + rng.normal(size=(16, d))  # a dominant first block: later gaps are negative
    v = rng.normal(size=(N, d))
    cols = list(range(6))
    for lam in (-2.0, -4.0, -8.0):
        y_full, _ = F.attend_qblock(q, k, v, 0, cols, bq, bk, lam=-np.inf)
        y_s, rec = F.attend_qblock(q, k, v, 0, cols, bq, bk, lam=lam)
        assert np.array_equal(rec["skip"], rec["gap"] < lam)
        dropped = 0
        for e, j in enumerate(cols):
            for g in range(rec["skip"].shape[1]):
                if rec["skip"][e, g]:
                    dropped += PV_rows(g, bq, N) * min(bk, N - j * bk)
        bound = dropped * math.exp(lam) * np.abs(v).max()
        assert np.max(np.abs(y_s - y_full)) <= bound + 1e-15
        assert rec["pv_exec"] + rec["pv_skip"] == len(cols) * rec["skip"].shape[1]
    assert rec["pv_skip"] > 0  # the case really exercises skipping


def PV_rows(g, bq, N):
    return min(F.PV_GROUP_ROWS, bq - g * F.PV_GROUP_ROWS)


# ------------------------------------------------------------------ P11, P12 layout

def test_window_reorder_pixel_major_special_case():
    """Window [T,1,1] on the 4x4x4 grid equals argsort(pixel, stable) (SparseAttn article, section 04)."""
    _, pixel = A.frame_major_coords(4, 16)
    perm = Lay.plan_permutation(64, Lay.ORDER_WINDOW, latent=(4, 4, 4), window=(4, 1, 1))
    assert np.array_equal(perm, np.argsort(pixel, kind="stable"))


def test_window_reorder_single_window_is_raster():
    """One window covering the whole grid: raster (t, h, w) order inside it."""
    perm = Lay.plan_permutation(8, Lay.ORDER_WINDOW, latent=(2, 2, 2), window=(2, 2, 2))
    assert list(perm) == list(range(8))
    perm = Lay.plan_permutation(12, Lay.ORDER_WINDOW, latent=(2, 3, 2), window=(2, 2, 1))
    # windows (h//2, w): (0,0),(0,1),(1,0),(1,1); inside each: t, then h
    assert list(perm) == [0, 2, 6, 8, 1, 3, 7, 9, 4, 10, 5, 11]


def test_window_reorder_sink_and_text_hand_example():
    """MindIE-SD rf_v2: first frame first, [t,h,w] windows, text last (hand-worked 3x2x2 case)."""
    perm = Lay.plan_permutation(14, Lay.ORDER_WINDOW, latent=(3, 2, 2), window=(2, 1, 2),
                                txt_len=2, first_frame_sink=True)
    assert list(perm) == [2, 3, 4, 5, 6, 7, 10, 11, 8, 9, 12, 13, 0, 1]


def _hilbert_order(dims, bits):
    grids = np.meshgrid(*[np.arange(n) for n in dims], indexing="ij")
    pts = np.stack([g.ravel() for g in grids], axis=1)
    idx = Lay.hilbert_index(pts, bits)
    return pts, idx


@pytest.mark.parametrize("ndim,bits", [(2, 1), (2, 2), (2, 3), (2, 5), (3, 1), (3, 2), (3, 3), (3, 4)])
def test_hilbert_curve_properties(ndim, bits):
    """Skilling (2004) Hilbert index: bijection on the 2^k cube, starts at the origin,
    consecutive points are unit neighbours."""
    n = 1 << bits
    pts, idx = _hilbert_order((n,) * ndim, bits)
    assert np.array_equal(np.sort(idx), np.arange(n ** ndim))
    path = pts[np.argsort(idx)]
    assert np.all(path[0] == 0)
    steps = np.abs(np.diff(path, axis=0)).sum(axis=1)
    assert np.all(steps == 1)


def test_hilbert_plan_is_permutation_on_ragged_grid():
    perm = Lay.plan_permutation(28 * 30 * 53, Lay.ORDER_HILBERT, latent=(28, 30, 53))
    assert np.array_equal(np.sort(perm), np.arange(28 * 30 * 53))
    # locality: the average step between consecutive tokens stays small
    t, rem = np.divmod(perm, 30 * 53)
    h, w = np.divmod(rem, 53)
    steps = np.abs(np.diff(t)) + np.abs(np.diff(h)) + np.abs(np.diff(w))
    assert steps.mean() < 1.5


def test_attend_head_over_a_csr_equals_the_restricted_softmax():
    """The per-head driver of the block attention over a global CSR (row_base offset,
    query blocks picked or all) gives, row for row, the restricted softmax of the
    token mask that the CSR's blocks define; blocks it is not asked for stay NaN."""
    rng = np.random.default_rng(17)
    N, d, bq, bk = 70, 8, 16, 16
    q, k, v = rng.normal(size=(N, d)), rng.normal(size=(N, d)), rng.normal(size=(N, 3))
    nqb, nkb = -(-N // bq), -(-N // bk)
    blocks = rng.random((nqb, nkb)) < 0.5
    blocks[np.arange(nqb), np.arange(nqb) % nkb] = True  # every row keeps a block
    # a CSR that starts with two rows of another head, so row_base matters
    rp, ci = [0, 1, 2], [0, 1]
    for i in range(nqb):
        cols = np.nonzero(blocks[i])[0]
        ci += cols.tolist()
        rp.append(rp[-1] + len(cols))
    rp, ci = np.array(rp), np.array(ci)
    tok = np.repeat(np.repeat(blocks, bq, axis=0), bk, axis=1)[:N, :N]
    want, _ = A.restricted_attention(q, k, v, tok)
    y, recs = F.attend_head(q, k, v, rp, ci, 2, bq, bk)
    assert set(recs) == set(range(nqb))
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
    y2, _ = F.attend_head(q, k, v, rp, ci, 2, bq, bk, qblocks=[1, 3])
    rows = np.zeros(N, dtype=bool)
    rows[1 * bq:2 * bq] = rows[3 * bq:4 * bq] = True
    assert np.allclose(y2[rows], want[rows], rtol=1e-12, atol=1e-12)
    assert np.isnan(y2[~rows]).all()
