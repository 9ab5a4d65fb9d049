"""GPU parity at the workloads' full sizes (MI355X only), on sampled outputs.

The whole path runs exactly as the benchmark runs it.  The oracle then checks
what it can afford one by one: the full permutation and sampled permuted
rows (bit-exact), the block statistics and the predicted mask rows of the
first head in full and of the last head on a sample (each row the oracle's, or
one it allows at a flagged near-boundary decision), the full CSR against the GPU's own
mask (bit-exact), the counters against the CSR and skip flags, and the
outputs of sampled query blocks against fp64 on the GPU's CSR.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import image_dit_amd as sa  # noqa: E402
from oracle import layout as OL  # noqa: E402
from oracle import predict as OP  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402

import _ref as R  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

# the four workloads at full size, plus one head at the largest supported
# key-block count (n_kb = SA_MAX_KEY_BLOCKS = 2048, 64-key blocks over 131072
# tokens): with PV skip on the Hilbert-ordered field, and causal without it
FULL_W = {name: CONFIGS[name] for name in ["image", "video", "long_video", "causal_long"]}
FULL_W["max_blocks_lam"] = dataclasses.replace(CONFIGS["long_video"], Hq=1, Hkv=1, latent=(2, 256, 256), seed=81)
FULL_W["max_blocks_causal"] = dataclasses.replace(CONFIGS["causal_long"], Hq=2, Hkv=1, block_k=64, seed=82)
# the video workload with keys and values on a grid of half its width (12514 keys for 24802
# queries; the first key frame and the key text are the sinks); materialising form only
FULL_W["video_kv"] = dataclasses.replace(CONFIGS["video"], latent_k=(16, 32, 24), sink_front=32 * 24, seed=83)
# the image workload with PV skip on its 128-key blocks (a whole-block decision per 32-row group)
FULL_W["image_lam"] = dataclasses.replace(CONFIGS["image"], lam=-8.0, seed=84)
FULL = list(FULL_W)
FULL_GATHER = [name for name in FULL if FULL_W[name].N_k == FULL_W[name].N]


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    w = FULL_W[name]
    log(f"[full] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} N_k={w.N_k} D={w.D} bq={w.block_q} bk={w.block_k}")
    q, k, v = generate(w)
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg)
    mask = torch.zeros((cfg.rows, cfg.n_kb), dtype=torch.uint8, device="cuda")
    qd, kd, vd = dev(q), dev(k), dev(v)
    path.permute(qd, kd, vd)
    path.predict(mask_out=mask)
    path.attend()
    path.unpermute()
    torch.cuda.synchronize()
    assert path.statuses() == (sa.SA_OK, sa.SA_OK)
    del qd, kd, vd

    rng = np.random.default_rng(12345)
    perm = R.oracle_perm(w)
    perm_k = R.oracle_perm_k(w)
    assert np.array_equal(path.perm_host.astype(np.int64), perm)
    assert np.array_equal(path.perm_k_host.astype(np.int64), perm_k)
    # sampled permuted rows, bit-exact
    for src, dst, H, pm in ((q, path.qp, w.Hq, perm), (k, path.kp, w.Hkv, perm_k), (v, path.vp, w.Hkv, perm_k)):
        bs, hs, ts = rng.integers(0, w.B, 64), rng.integers(0, H, 64), rng.integers(0, len(pm), 64)
        got = dst[torch.from_numpy(bs).cuda(), torch.from_numpy(hs).cuda(), torch.from_numpy(ts).cuda()]
        got = got.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, src[bs, hs, pm[ts]])

    gmask = mask.cpu().numpy().astype(bool)
    rp, ci = path.csr_host()
    rp_m, ci_m = OP.mask_to_csr(gmask)
    assert np.array_equal(rp, rp_m) and np.array_equal(ci, ci_m)
    skip = path.pv_skip.cpu().numpy()[:int(rp[-1]) * path.groups]
    cnt = path.counters.cpu().numpy()
    assert cnt[0] == int(rp[-1])
    i_of_row = np.arange(cfg.rows) % cfg.n_qb
    qrows = np.minimum((i_of_row + 1) * w.block_q, w.N) - i_of_row * w.block_q
    ngr = -(-qrows // 32)
    real = int(np.sum(ngr * np.diff(rp)))
    assert cnt[1] + cnt[2] == real
    ent_row = np.repeat(np.arange(cfg.rows), np.diff(rp))
    flags = skip.reshape(-1, path.groups)
    live = np.arange(path.groups)[None, :] < ngr[ent_row][:, None]
    assert cnt[2] == int(flags[live].sum())

    mp = R.mask_params(w)
    G = w.Hq // w.Hkv
    o = path.o.cpu().numpy() if w.B * w.Hq * w.N * w.D < 2e8 else None
    # the first head row by row in full, the last head on 24 sampled query blocks
    heads = [(0, 0), (w.B - 1, w.Hq - 1)]
    n_bad = n_border = n_rows = 0
    flagged = {"tau": 0, "theta": 0, "tie": 0}
    worst_max, sum_abs, n_el = 0.0, 0.0, 0
    for hi, (b, h) in enumerate(heads):
        hk = h // G
        qp = R.permuted(q[b, h], perm)
        kp = R.permuted(k[b, hk], perm_k)
        vp = R.permuted(v[b, hk], perm_k)
        rows = list(range(cfg.n_qb)) if hi == 0 else \
            sorted(set(np.linspace(0, cfg.n_qb - 1, 24).astype(int).tolist()))
        ref = OP.predict_head(qp, kp, mp, rows=rows)
        r0 = (b * w.Hq + h) * cfg.n_qb
        gm = gmask[r0:r0 + cfg.n_qb]
        bad, border, checked, _ = R.compare_head_mask(gm, ref, mp, rows)
        for kk, c in R.borderline_counts(ref, rows).items():
            flagged[kk] += c
        n_bad += len(bad)
        n_border += len(border)
        n_rows += checked
        rows = sorted(set(np.linspace(0, cfg.n_qb - 1, 24).astype(int).tolist()))
        qbar = path.workspace_view(0, torch.float32, (cfg.B, cfg.Hq, cfg.n_qb, cfg.D))[b, h].cpu().numpy()
        assert np.allclose(qbar, ref["qbar"], rtol=1e-5, atol=1e-5)
        qblocks = rows[:: max(1, len(rows) // 6)]
        ys, recs = R.attend_rows(qp, kp, vp, w, rp, ci, r0, qblocks, skip, path.groups)
        for i, y in ys.items():
            toks = perm[i * w.block_q:i * w.block_q + y.shape[0]]
            got = o[b, h, toks] if o is not None else \
                path.o[b, h, torch.from_numpy(toks).cuda()].cpu().numpy()
            d = np.abs(got - y)
            worst_max = max(worst_max, float(d.max()))
            sum_abs += float(d.sum())
            n_el += d.size
            if w.lam is not None:
                far, _ = R.lambda_disagreements(recs[i], w.lam)
                assert far == 0
    if name.startswith("max_blocks"):
        assert cfg.n_kb == sa.SA_MAX_KEY_BLOCKS
    log(f"[full] {name}: nnz={int(rp[-1])} checked_rows={n_rows} mismatch={n_bad} differing_borderline={n_border} "
        f"flagged={flagged} "
        f"out_max={worst_max:.3e} out_mean={sum_abs / n_el:.3e} pv_exec={cnt[1]} pv_skip={cnt[2]}")
    assert n_bad == 0
    assert worst_max <= R.MAX_ABS and sum_abs / n_el <= R.MEAN_ABS


@pytest.mark.parametrize("name", FULL_GATHER)
def test_full_size_gather_form_bit_identical(name):
    """At full size, the gather form (the one the benchmark times) equals the
    materialising form bit for bit: CSR, mask, statistics, skip flags,
    counters and every output element."""
    from test_gpu_parity import assert_forms_identical, run_both_forms
    w = FULL_W[name]
    log(f"[full-gather] {name}: B={w.B} Hq={w.Hq} N={w.N} D={w.D} bq={w.block_q} bk={w.block_k} lam={w.lam}")
    cfg = sa.config_from_workload(w)
    q, k, v = generate(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    del q, k, v
    a, b = run_both_forms(cfg, qd, kd, vd)
    assert a["status"] == (sa.SA_OK, sa.SA_OK)
    assert_forms_identical(a, b)
    log(f"[full-gather] {name}: nnz={int(a['rp'][-1])} identical")
