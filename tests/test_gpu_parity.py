"""GPU parity: the HIP path through the C ABI against the fp64 oracle (MI355X only).

Reduced-size versions of the five workloads (several tiles, ragged tails),
checked step by step: permutation (bit-exact), block statistics, predicted
mask (exact except oracle-flagged borderline rows), CSR (bit-exact against
the GPU's own mask), attention outputs on the GPU's CSR (max-abs 1e-2,
mean-abs 1e-3 against fp64), PV-skip decisions and counters.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import image_dit_amd as sa  # noqa: E402
from oracle import attention as OA  # noqa: E402
from oracle import layout as OL  # noqa: E402
from oracle import numerics as ON  # noqa: E402
from oracle import predict as OP  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402

import _ref as R  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

rep = dataclasses.replace
SMALL = {
    "tiny": CONFIGS["tiny"],
    "image_s": rep(CONFIGS["image"], Hq=3, Hkv=3, latent=(1, 20, 37)),
    "video_s": rep(CONFIGS["video"], Hq=2, Hkv=2, latent=(9, 16, 24), txt_len=20,
                   sink_front=16 * 24, sink_back=20),
    "long_video_s": rep(CONFIGS["long_video"], Hq=2, Hkv=2, latent=(6, 10, 21)),
    "long_video_d64": rep(CONFIGS["long_video"], Hq=2, Hkv=2, latent=(5, 9, 23), D=64, seed=41),
    "causal_s": rep(CONFIGS["causal_long"], Hq=4, Hkv=2, latent=(1, 1, 2000), window_tokens=512),
    "causal_s64": rep(CONFIGS["causal_long"], Hq=2, Hkv=1, latent=(1, 1, 777), window_tokens=300,
                      block_k=64, seed=51),
    # PV skip on 128-key blocks, and on causal 64-key tiles (the diagonal masking path)
    "image_s_lam": rep(CONFIGS["image"], Hq=3, Hkv=3, latent=(1, 20, 37), lam=-8.0, seed=61),
    "causal_s64_lam": rep(CONFIGS["causal_long"], Hq=2, Hkv=1, latent=(1, 1, 777), window_tokens=300,
                          block_k=64, lam=-8.0, seed=71),
    # the first frame (16x24 tokens, three query blocks) as full rows as well as sink columns
    "video_s_sink_rows": rep(CONFIGS["video"], Hq=2, Hkv=2, latent=(9, 16, 24), txt_len=20,
                             sink_front=16 * 24, sink_back=20, sink_rows=16 * 24, seed=91),
    # 3-D tile windows ([4,8,4] tiles, one tile of reach) forced on top of the prediction
    "video_s_tiles": rep(CONFIGS["video"], Hq=2, Hkv=2, latent=(9, 16, 24), txt_len=20,
                         sink_front=16 * 24, sink_back=20, tile=(4, 8, 4), tile_radius=(1, 1, 1), seed=93),
    # keys and values on a grid of their own (half the width; the first key frame and the key
    # text are the sinks), one case per attention kernel: 16-blocks, 128-key blocks with and
    # without PV skip, 64-key blocks with PV skip, and d = 64
    "tiny_kv": rep(CONFIGS["tiny"], latent_k=(2, 4, 4), seed=101),
    "video_s_kv": rep(CONFIGS["video"], Hq=2, Hkv=2, latent=(9, 16, 24), txt_len=20, latent_k=(9, 16, 12),
                      sink_front=16 * 12, sink_back=20, seed=103),
    "image_s_lam_kv": rep(CONFIGS["image"], Hq=3, Hkv=3, latent=(1, 20, 37), latent_k=(1, 10, 19), lam=-8.0,
                          seed=105),
    # (theta off: at this size every block falls under the 0.6 guard and the rows would be full)
    "long_video_s_kv": rep(CONFIGS["long_video"], Hq=2, Hkv=2, latent=(6, 10, 21), latent_k=(3, 10, 21),
                           theta=None, seed=107),
    "long_video_d64_kv": rep(CONFIGS["long_video"], Hq=2, Hkv=2, latent=(5, 9, 23), latent_k=(5, 9, 12), D=64,
                             theta=None, lam=None, seed=109),
}

# Degenerate and ragged sizes: a single token, one partial query block, a last block of
# one row or one key, on every attention kernel (16-blocks, 128/64 and 128/128 with and
# without PV skip, causal, d = 64)
_im = CONFIGS["image"]
_ca = CONFIGS["causal_long"]
_ti = CONFIGS["tiny"]
EDGE = {
    "edge_n1_128x64_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 1), block_k=64, lam=-8.0, seed=201),
    "edge_n1_128x128": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 1), seed=202),
    "edge_n1_16x16": rep(_ti, latent=(1, 1, 1), seed=203),
    "edge_n65_128x64_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 65), block_k=64, lam=-8.0, seed=204),
    "edge_n129_128x128_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 129), lam=-8.0, seed=205),
    "edge_n129_128x64": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 129), block_k=64, seed=206),
    "edge_n17_16x16_lam": rep(_ti, latent=(1, 1, 17), lam=-8.0, seed=207),
    "edge_causal_n1": rep(_ca, Hq=2, Hkv=1, latent=(1, 1, 1), window_tokens=64, sink_front=1, block_k=64,
                          seed=208),
    "edge_causal_n130_lam": rep(_ca, Hq=2, Hkv=1, latent=(1, 1, 130), window_tokens=64, block_k=64, lam=-8.0,
                                seed=209),
    "edge_causal_n129_128x128": rep(_ca, Hq=2, Hkv=1, latent=(1, 1, 129), window_tokens=64, seed=210),
    "edge_d64_n65_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 65), D=64, block_k=64, lam=-8.0, seed=211),
    # PV skip on 128-key blocks (one decision per block over its two 64-key tiles): causal
    # with a window, d = 64, and a last block whose second tile lies past the end
    "causal_s_lam": rep(_ca, Hq=4, Hkv=2, latent=(1, 1, 2000), window_tokens=512, lam=-8.0, seed=212),
    "image_s_d64_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 20, 37), D=64, lam=-8.0, seed=213),
    "edge_n193_128x128_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 193), lam=-8.0, seed=214),
}
SMALL.update(EDGE)


def library_tile_pattern(w):
    """The library's tile-window pattern of the workload (host), or None."""
    if w.tile is None:
        return None
    lay = sa.make_layout(w.N, w.order, w.latent, w.window, w.txt_len, w.first_frame_sink)
    return sa.sa_plan_tile_window(lay, w.tile, w.tile_radius, w.block_q, w.block_k)


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_path(w, sparsity="default", inputs=None):
    cfg = sa.config_from_workload(w, sparsity)
    path = sa.SparseAttentionPath(cfg, forced=library_tile_pattern(w))
    q, k, v = generate(w) if inputs is None else inputs
    mask = torch.zeros((cfg.rows, cfg.n_kb), dtype=torch.uint8, device="cuda")
    simq = torch.zeros(cfg.rows, dtype=torch.float32, device="cuda")
    simk = torch.zeros(cfg.B * cfg.Hkv * cfg.n_kb, dtype=torch.float32, device="cuda")
    qd, kd, vd = dev(q), dev(k), dev(v)
    path.permute(qd, kd, vd)
    path.predict(mask_out=mask, sim_q=simq, sim_k=simk)
    path.attend()
    path.unpermute()
    torch.cuda.synchronize()
    return path, (q, k, v), mask.cpu().numpy().astype(bool), simq.cpu().numpy(), simk.cpu().numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_path_parity(name):
    check_path_parity(name, SMALL[name])


def random_workload(seed):
    """A seeded random configuration: reorder and generator of one of the four bf16
    workloads, its shape, head dim, block pair, GQA ratio (causal generator), sinks,
    causal window, tau / theta / sparsity / lambda, all within the compiled limits."""
    rng = np.random.default_rng(seed)
    base = ["image", "video", "long_video", "causal_long"][seed % 4]
    w = CONFIGS[base]
    D = int(rng.choice([64, 128]))
    bk = int(rng.choice([64, 128]))
    lam = [None, -8.0, -4.0][int(rng.integers(3))]
    tau = None if rng.random() < 0.3 else float(rng.uniform(0.5, 0.99))
    spars = float(rng.uniform(0.3, 0.9)) if (tau is None or rng.random() < 0.5) else None
    theta = None if rng.random() < 0.5 else float(rng.uniform(0.2, 0.8))
    kw = dict(D=D, block_k=bk, lam=lam, tau=tau, sparsity=spars, theta=theta, seed=1000 + seed)
    if base == "causal_long":
        hkv = int(rng.integers(1, 3))
        N = int(rng.integers(100, 1500))
        kw.update(Hkv=hkv, Hq=hkv * int(rng.choice([1, 2, 4])), latent=(1, 1, N),
                  window_tokens=int(rng.choice([0, 64, 300])), sink_front=int(rng.integers(0, 8)))
    else:
        t, h, ww = int(rng.integers(1, 6)), int(rng.integers(2, 13)), int(rng.integers(3, 18))
        txt = int(rng.choice([0, 8, 20])) if base == "video" else 0
        kw.update(Hq=2, Hkv=2, B=int(rng.integers(1, 3)), latent=(t, h, ww), txt_len=txt)
        # keys on a grid of half the width, or (video) tile windows; first-frame sink rows
        ww_k = ww
        extra = rng.random()
        if extra < 0.25:
            ww_k = max(3, ww // 2)
            kw.update(latent_k=(t, h, ww_k))
        elif extra < 0.5 and base == "video":
            kw.update(tile=(2, 4, 4), tile_radius=(1, 1, 1))
        if base == "video":
            kw.update(window=(2, 4, 4), sink_front=h * ww_k if w.first_frame_sink else 0, sink_back=txt)
            if rng.random() < 0.25:
                kw.update(sink_rows=h * ww)
    return rep(w, **kw)


RANDOM = {f"random_{s}": random_workload(s) for s in range(64)}


@pytest.mark.parametrize("name", list(RANDOM))
def test_random_config_parity(name):
    w = RANDOM[name]
    log(f"[random] {name}: {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} D={w.D} bk={w.block_k} "
        f"tau={w.tau} theta={w.theta} s={w.sparsity} lam={w.lam} causal={w.causal} W={w.window_tokens}")
    check_path_parity(name, w)


def check_path_parity(name, w):
    log(f"[parity] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} N_k={w.N_k} D={w.D} bq={w.block_q} bk={w.block_k}")
    path, (q, k, v), gmask, gsimq, gsimk = run_path(w)
    cfg = path.cfg
    st_pred, st_attn = path.statuses()
    assert st_pred == sa.SA_OK and st_attn == sa.SA_OK

    # (a1) permutation: planner and gathered rows, bit-exact (keys on their own grid have
    # their own reorder)
    perm = R.oracle_perm(w)
    perm_k = R.oracle_perm_k(w)
    assert np.array_equal(path.perm_host.astype(np.int64), perm)
    assert np.array_equal(path.perm_k_host.astype(np.int64), perm_k)
    want_q = ON.f32_to_bf16(q) if q.dtype == np.float32 else q
    assert np.array_equal(host_bits(path.qp), np.take(want_q, perm, axis=2))
    want_k = ON.f32_to_bf16(k) if k.dtype == np.float32 else k
    assert np.array_equal(host_bits(path.kp), np.take(want_k, perm_k, axis=2))
    want_v = ON.f32_to_bf16(v) if v.dtype == np.float32 else v
    assert np.array_equal(host_bits(path.vp), np.take(want_v, perm_k, axis=2))

    qp = R.permuted(q, perm)
    kp = R.permuted(k, perm_k)
    vp = R.permuted(v, perm_k)
    G = w.Hq // w.Hkv
    mp = R.mask_params(w)
    qbar_g = path.workspace_view(0, torch.float32, (cfg.B, cfg.Hq, cfg.n_qb, cfg.D)).cpu().numpy()
    kbar_g = path.workspace_view(1, torch.float32, (cfg.B, cfg.Hkv, cfg.n_kb, cfg.D)).cpu().numpy()
    rp, ci = path.csr_host()
    o_perm = path.o_perm.cpu().numpy()
    skip = path.pv_skip.cpu().numpy() if path.pv_skip is not None else None
    groups = path.groups

    n_bad = n_border = n_rows = 0
    errs_max, errs_sum, errs_n = 0.0, 0.0, 0
    lam_far = lam_diff = 0
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // G
            ref = OP.predict_head(qp[b, h], kp[b, hk], mp)
            # (a2) block statistics
            r0 = (b * w.Hq + h) * cfg.n_qb
            assert np.allclose(qbar_g[b, h], ref["qbar"], rtol=1e-5, atol=1e-5)
            assert np.allclose(kbar_g[b, hk], ref["kbar"], rtol=1e-5, atol=1e-5)
            assert np.allclose(gsimq[r0:r0 + cfg.n_qb], ref["simq"], rtol=1e-5, atol=1e-5)
            kb0 = (b * w.Hkv + hk) * cfg.n_kb
            assert np.allclose(gsimk[kb0:kb0 + cfg.n_kb], ref["simk"], rtol=1e-5, atol=1e-5)
            # (a3) predicted mask; sink rows are whole valid rows on the GPU too, and
            # every block of a forced pattern is kept
            for i in range(cfg.n_qb):
                if i * w.block_q < w.sink_rows:
                    assert np.array_equal(gmask[r0 + i], OP._valid_blocks(i, mp)), i
                if mp.forced is not None:
                    assert np.all(gmask[r0 + i][mp.forced[i] & OP._valid_blocks(i, mp)]), i
            # every row equals the oracle row, or one the oracle allows by taking a flagged
            # near-boundary decision the other way (forced blocks always agree)
            bad, border, checked, _ = R.compare_head_mask(gmask[r0:r0 + cfg.n_qb], ref, mp)
            n_bad += len(bad)
            n_border += len(border)
            n_rows += checked
            # (a5) attention on the GPU's CSR, PV decisions replayed
            ys, recs = R.attend_rows(qp[b, h], kp[b, hk], vp[b, hk], w, rp, ci, r0, range(cfg.n_qb),
                                     skip, groups)
            for i, y in ys.items():
                got = o_perm[b, h, i * w.block_q:i * w.block_q + y.shape[0]]
                d = np.abs(got - y)
                errs_max = max(errs_max, float(d.max()))
                errs_sum += float(d.sum())
                errs_n += d.size
                if w.lam is not None:
                    f, dd = R.lambda_disagreements(recs[i], w.lam)
                    lam_far += f
                    lam_diff += dd
    log(f"[parity] {name}: rows={n_rows} mask_mismatch={n_bad} borderline={n_border} "
        f"out_max={errs_max:.3e} out_mean={errs_sum / errs_n:.3e} lam_diff={lam_diff} lam_far={lam_far}")
    assert n_bad == 0
    assert errs_max <= R.MAX_ABS and errs_sum / errs_n <= R.MEAN_ABS
    assert lam_far == 0

    # (a4) CSR is exactly the GPU mask, rows ascending
    rp_m, ci_m = OP.mask_to_csr(gmask)
    assert np.array_equal(rp, rp_m) and np.array_equal(ci, ci_m)

    # counters: QK blocks = nnz; PV decisions of real groups add up; skips = bits set
    cnt = path.counters.cpu().numpy()
    nnz = int(rp[-1])
    assert cnt[0] == nnz
    real_groups = 0
    skipped = 0
    for r in range(cfg.rows):
        i = r % cfg.n_qb
        ng = -(-(min((i + 1) * w.block_q, w.N) - i * w.block_q) // 32)
        real_groups += ng * (rp[r + 1] - rp[r])
        if skip is not None:
            for e in range(rp[r], rp[r + 1]):
                skipped += int(skip[e * groups:e * groups + ng].sum())
    assert cnt[1] + cnt[2] == real_groups
    if skip is not None:
        assert cnt[2] == skipped
    if w.lam is None:
        assert cnt[2] == 0

    # (a6) unpermute is the exact inverse scatter
    o = path.o.cpu().numpy()
    assert np.array_equal(o, OL.unpermute_rows(o_perm, perm))


def test_dense_when_sparsity_zero():
    """Sparsity 0 keeps every block: the output is dense attention (all-ones mask)."""
    w = rep(SMALL["image_s"], tau=None, sparsity=0.0, Hq=2, Hkv=2)
    path, (q, k, v), gmask, _, _ = run_path(w)
    assert gmask.all()
    perm = R.oracle_perm(w)
    o = path.o.cpu().numpy()
    for b in range(w.B):
        for h in range(w.Hq):
            y, _ = OA.dense_attention(R.to_f64(q[b, h]), R.to_f64(k[b, h]), R.to_f64(v[b, h]))
            d = np.abs(o[b, h] - y)
            assert d.max() <= R.MAX_ABS and d.mean() <= R.MEAN_ABS


@pytest.mark.parametrize("sparsity,tau", [(0.3, None), (0.7, None), (None, 0.5), (0.5, 0.9)])
def test_exact_ties_rank_by_block_index(sparsity, tau):
    """Key blocks that are bit-exact copies of one another tie exactly in probability, and
    the selection ranks equal candidates by block index: among the candidate copies of one
    block a row keeps the lowest indices first.  Every row must also be one the oracle
    allows.  With five distinct blocks repeated across the row, the floor and TopCdf cuts
    fall inside groups of copies."""
    w = rep(SMALL["video_s"], theta=None, tau=tau, sparsity=sparsity)
    q, k, v = generate(w)
    perm, perm_k = R.oracle_perm(w), R.oracle_perm_k(w)
    kp = np.take(k, perm_k, axis=2)
    bk, Nk = w.block_k, kp.shape[2]
    n_kb = -(-Nk // bk)
    src = np.arange(n_kb) % 5
    full = [j for j in range(n_kb) if (j + 1) * bk <= Nk]
    for j in full:
        if src[j] != j:
            kp[:, :, j * bk:(j + 1) * bk] = kp[:, :, src[j] * bk:(src[j] + 1) * bk]
    k2 = np.empty_like(k)
    k2[:, :, perm_k] = kp
    path, _, gmask, _, _ = run_path(w, inputs=(q, k2, v))
    cfg = path.cfg
    assert path.statuses()[0] == sa.SA_OK
    mp = R.mask_params(w)
    qp, kpf = R.permuted(q, perm), R.permuted(k2, perm_k)
    split_groups = 0
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // (w.Hq // w.Hkv)
            ref = OP.predict_head(qp[b, h], kpf[b, hk], mp)
            r0 = (b * w.Hq + h) * cfg.n_qb
            bad, _, _, _ = R.compare_head_mask(gmask[r0:r0 + cfg.n_qb], ref, mp)
            assert not bad, f"rows not admissible: {bad[:8]}"
            for i in range(cfg.n_qb):
                if ref["info"][i]["forced_row"]:
                    continue
                valid = OP._valid_blocks(i, mp)
                cand = valid & ~OP._forced_blocks(i, mp, ref["simk"], valid)
                row = gmask[r0 + i]
                for g in range(5):
                    members = [j for j in full if src[j] == g and cand[j]]
                    kept = row[members]
                    # kept copies come first in index order
                    assert not np.any(~kept[:-1] & kept[1:]), (b, h, i, g, kept)
                    split_groups += int(kept.any() and not kept.all())
    assert split_groups > 0  # a cut fell inside a group of exact ties


def test_permute_fp32_round_to_nearest_even():
    rng = np.random.default_rng(3)
    N, D = 333, 64
    x = (rng.normal(size=(2, 3, N, D)) * 50).astype(np.float32)
    bits = x.view(np.uint32)
    bits[0, 0, :, :8] = (bits[0, 0, :, :8] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)  # exact ties
    perm = rng.permutation(N).astype(np.int32)
    y = torch.empty((2, 3, N, D), dtype=torch.bfloat16, device="cuda")
    sa.sa_permute(dev(x), y, torch.from_numpy(perm).cuda())
    torch.cuda.synchronize()
    want = np.take(ON.f32_to_bf16(x), perm, axis=2)
    assert np.array_equal(host_bits(y), want)
    back = torch.empty((2, 3, N, D), dtype=torch.float32, device="cuda")
    yf = dev(ON.bf16_to_f64(want).astype(np.float32))
    sa.sa_unpermute(yf, back, torch.from_numpy(perm).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), OL.unpermute_rows(ON.bf16_to_f64(want).astype(np.float32), perm))


def test_permute_entries_outside_the_sequence():
    """Entries outside 0..N-1 are caught by the kernels' own bounds checks: the gather
    writes a zero row, the scatter stores nothing."""
    rng = np.random.default_rng(5)
    N, D = 100, 16
    x = rng.normal(size=(1, 2, N, D)).astype(np.float32)
    perm = np.arange(N, dtype=np.int32)
    perm[5], perm[7] = N, -1
    y = torch.empty((1, 2, N, D), dtype=torch.bfloat16, device="cuda")
    sa.sa_permute(dev(x), y, torch.from_numpy(perm).cuda())
    torch.cuda.synchronize()
    got = host_bits(y)
    want = ON.f32_to_bf16(x)
    ok = np.ones(N, dtype=bool)
    ok[[5, 7]] = False
    assert np.array_equal(got[:, :, ok], want[:, :, ok])
    assert not got[:, :, ~ok].any()
    yf = dev(x)
    back = torch.full((1, 2, N, D), 7.0, dtype=torch.float32, device="cuda")
    sa.sa_unpermute(yf, back, torch.from_numpy(perm).cuda())
    torch.cuda.synchronize()
    b = back.cpu().numpy()
    assert np.array_equal(b[:, :, ok], x[:, :, ok])
    assert np.all(b[:, :, ~ok] == 7.0)  # rows 5 and 7 are nobody's target


def test_empty_row_gives_nan_and_status():
    w = rep(SMALL["long_video_s"], lam=None)
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg)
    q, k, v = generate(w)
    path.permute(dev(q), dev(k), dev(v))
    rows, n_kb = cfg.rows, cfg.n_kb
    rp = np.zeros(rows + 1, dtype=np.int32)
    cols = []
    for r in range(rows):
        c = [] if r == 3 else [0, r % n_kb] if r % n_kb else [0]
        cols += c
        rp[r + 1] = len(cols)
    path.row_ptr.copy_(torch.from_numpy(rp))
    path.col_idx[:len(cols)].copy_(torch.from_numpy(np.array(cols, dtype=np.int32)))
    path.attend()
    torch.cuda.synchronize()
    assert path.statuses()[1] == sa.SA_ERR_EMPTY_ROW
    o = path.o_perm.cpu().numpy()
    i = 3 % cfg.n_qb
    blk = o[0, 3 // cfg.n_qb, i * 128:(i + 1) * 128]
    assert np.isnan(blk).all()
    assert np.isfinite(o[0, 0, :128]).all()


@pytest.mark.parametrize("name,lam", [("tiny", None), ("image_s", None), ("image_s_lam", -8.0),
                                      ("long_video_s", None), ("long_video_s", -8.0)])
def test_malformed_csr_is_contained(name, lam):
    """A column outside [0, n_kb) and a negative row_ptr entry, on every attention kernel:
    the bad column is skipped (its row equals the row without it), the two rows the
    negative entry bounds come out NaN, the status word reports it, and every other row is
    unchanged."""
    w = rep(SMALL[name], lam=lam)
    cfg = sa.config_from_workload(w)
    rows, n_kb, n_qb = cfg.rows, cfg.n_kb, cfg.n_qb
    log(f"[csr] {name}: lam={lam} bq={w.block_q} bk={w.block_k} rows={rows} n_kb={n_kb}")
    assert rows >= 3
    bad_col_row, neg = 0, rows - 1  # rp[rows - 1] < 0 bounds rows rows-2 and rows-1
    q, k, v = generate(w)
    outs = []
    for bad in (False, True):
        path = sa.SparseAttentionPath(cfg)
        path.permute(dev(q), dev(k), dev(v))
        cols, rp = [], np.zeros(rows + 1, dtype=np.int32)
        for r in range(rows):
            c = [0] if r % n_kb == 0 else [0, r % n_kb]
            if r == bad_col_row:
                c = [0, n_kb + 5] if bad else [0]
            cols += c
            rp[r + 1] = len(cols)
        if bad:
            rp[neg] = -1
        path.row_ptr.copy_(torch.from_numpy(rp))
        path.col_idx[:len(cols)].copy_(torch.from_numpy(np.array(cols, dtype=np.int32)))
        path.attend()
        torch.cuda.synchronize()
        outs.append((path.statuses()[1], path.o_perm.cpu().numpy()))
    (st_ok, o_ok), (st_bad, o_bad) = outs
    assert st_ok == sa.SA_OK
    assert st_bad in (sa.SA_ERR_INVALID_ARGUMENT, sa.SA_ERR_EMPTY_ROW)
    for r in range(rows):
        bh, i = divmod(r, n_qb)
        b, h = divmod(bh, w.Hq)
        t0, t1 = i * w.block_q, min((i + 1) * w.block_q, w.N)
        if r in (neg - 1, neg):
            assert np.isnan(o_bad[b, h, t0:t1]).all(), r
        else:
            assert np.array_equal(o_bad[b, h, t0:t1], o_ok[b, h, t0:t1]), r


def test_capacity_overflow_sets_status():
    w = SMALL["image_s"]
    cfg = sa.config_from_workload(w)
    full = sa.SparseAttentionPath(cfg)
    q, k, v = generate(w)
    full.permute(dev(q), dev(k), dev(v))
    full.predict()
    torch.cuda.synchronize()
    rp, ci = full.csr_host()
    cap = int(rp[-1]) // 2
    small = sa.SparseAttentionPath(cfg, col_cap=cap)
    small.permute(dev(q), dev(k), dev(v))
    small.predict()
    torch.cuda.synchronize()
    assert small.statuses()[0] == sa.SA_ERR_CAPACITY
    rp2, ci2 = small.csr_host()
    assert np.array_equal(rp2, rp) and np.array_equal(ci2, ci[:cap])


def test_rerun_is_bitwise_deterministic():
    w = SMALL["long_video_s"]
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg)
    q, k, v = (dev(x) for x in generate(w))
    outs = []
    for _ in range(2):
        path.run(q, k, v)
        torch.cuda.synchronize()
        rp, ci = path.csr_host()
        outs.append((rp, ci, path.o.cpu().numpy().copy(), path.pv_skip.cpu().numpy().copy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][2].view(np.uint32), outs[1][2].view(np.uint32))
    assert np.array_equal(outs[0][3], outs[1][3])


def _bf16_inputs(w):
    out = []
    for x in generate(w):
        out.append(dev(x) if x.dtype == np.uint16 else torch.from_numpy(x).cuda().to(torch.bfloat16))
    return out


def run_both_forms(cfg, qd, kd, vd, forced=None):
    """The materialising form (permute, predict, attend, unpermute) and the gather
    form (predict_gather, attend_gather) on the same bf16 inputs; host copies of
    everything each writes."""
    res = []
    for fused in (False, True):
        path = sa.SparseAttentionPath(cfg, materialize=not fused, forced=forced)
        mask = torch.zeros((cfg.rows, cfg.n_kb), dtype=torch.uint8, device="cuda")
        simq = torch.zeros(cfg.rows, dtype=torch.float32, device="cuda")
        simk = torch.zeros(cfg.B * cfg.Hkv * cfg.n_kb, dtype=torch.float32, device="cuda")
        if fused:
            path.predict_gather(qd, kd, mask_out=mask, sim_q=simq, sim_k=simk)
            path.attend_gather(qd, kd, vd)
        else:
            path.permute(qd, kd, vd)
            path.predict(mask_out=mask, sim_q=simq, sim_k=simk)
            path.attend()
            path.unpermute()
        torch.cuda.synchronize()
        rp, ci = path.csr_host()
        nnz = int(rp[-1])
        res.append(dict(
            status=path.statuses(), rp=rp, ci=ci, mask=mask.cpu().numpy(),
            simq=simq.cpu().numpy().view(np.uint32), simk=simk.cpu().numpy().view(np.uint32),
            qbar=path.workspace_view(0, torch.float32, (cfg.B, cfg.Hq, cfg.n_qb, cfg.D)).cpu().numpy().view(np.uint32),
            kbar=path.workspace_view(1, torch.float32, (cfg.B, cfg.Hkv, cfg.n_kb, cfg.D)).cpu().numpy().view(np.uint32),
            skip=path.pv_skip[:min(nnz, path.col_cap) * path.groups].cpu().numpy(),
            counters=path.counters.cpu().numpy(), o=path.o.cpu().numpy().view(np.uint32)))
        del path
    return res


def assert_forms_identical(a, b):
    for key in a:
        x, y = np.asarray(a[key]), np.asarray(b[key])
        if not np.array_equal(x, y):
            if x.shape == y.shape and x.ndim == 4:  # o: [B, H, N, D] as uint32 bits
                neq = x != y
                rows = neq.any(axis=3)
                log(f"  {key}: {int(np.count_nonzero(neq))} elements differ in {int(rows.sum())} rows, "
                    f"first rows {np.argwhere(rows)[:6].tolist()}")
            assert False, key


@pytest.mark.parametrize("name", list(SMALL) + [n for n, w in RANDOM.items() if w.N_k == w.N])
def test_gather_form_bit_identical(name):
    """Reading q, k, v through the permutation inside the kernels gives the
    materialised path's CSR, mask, block statistics, skip flags, counters and
    outputs bit for bit."""
    w = SMALL[name] if name in SMALL else RANDOM[name]
    cfg = sa.config_from_workload(w)
    log(f"[gather] {name}: N={w.N} D={w.D} bq={w.block_q} bk={w.block_k} lam={w.lam} causal={w.causal}")
    if w.N_k != w.N:
        # one permutation serves queries and keys in the gather form: keys on another grid
        # are refused before anything runs
        with pytest.raises(ValueError):
            sa.SparseAttentionPath(cfg, materialize=False)
        return
    qd, kd, vd = _bf16_inputs(w)
    a, b = run_both_forms(cfg, qd, kd, vd, forced=library_tile_pattern(w))
    assert a["status"] == (sa.SA_OK, sa.SA_OK)
    assert_forms_identical(a, b)
