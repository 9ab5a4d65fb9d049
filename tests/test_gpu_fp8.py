"""GPU parity of the FP8 QK path (SpargeAttn notes, section 2.4) against the fp64 oracle (MI355X only).

1. sa_quantize_fp8 equals oracle.quant.quantize_blocks bit for bit: every E4M3
   code and every block scale, through the permutation or without it, on
   ragged sizes, an all-zero block, signed zeros and exact rounding ties.
2. sa_sparse_attn_fwd_qk8 on the GPU's CSR equals the oracle's attention over
   the dequantized operands (value(code) * scale, V in bf16) at the bf16
   path's tolerance (max-abs 1e-2, mean-abs 1e-3), PV decisions replayed and
   checked, counters exact.
3. Against the attention over the unquantized operands (lambda off), each
   output row stays within (exp(2 Delta) - 1) * max|v| + 1e-2, Delta being the
   row's largest score error caused by the quantization (computed exactly by
   the oracle): the softmax weights move by a factor within exp(+-2 Delta).
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import image_dit_amd as sa  # noqa: E402
from oracle import layout as OL  # noqa: E402
from oracle import predict as OP  # noqa: E402
from oracle import quant as OQ  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402

import _ref as R  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

rep = dataclasses.replace
_im, _lv, _vi = CONFIGS["image"], CONFIGS["long_video"], CONFIGS["video"]
CASES = {
    # 64-key tiles with PV skip (the lambda kernel), gather form
    "long_video_s": rep(_lv, Hq=2, Hkv=2, latent=(6, 10, 21)),
    # 64-key tiles without PV skip
    "long_video_s_nolam": rep(_lv, Hq=2, Hkv=2, latent=(6, 10, 21), lam=None, seed=301),
    # 128-key blocks (two tiles per block, one scale each)
    "image_s": rep(_im, Hq=3, Hkv=3, latent=(1, 20, 37)),
    "video_s": rep(_vi, Hq=2, Hkv=2, latent=(9, 16, 24), txt_len=20, sink_front=16 * 24, sink_back=20),
    # grouped heads (two query heads per key head), causal with a sliding window, with and
    # without PV skip
    "causal_s64_gqa_lam": rep(CONFIGS["causal_long"], Hq=4, Hkv=2, latent=(1, 1, 1000), window_tokens=300,
                              block_k=64, lam=-8.0, seed=303),
    "causal_s_gqa": rep(CONFIGS["causal_long"], Hq=4, Hkv=2, latent=(1, 1, 1000), window_tokens=300, seed=307),
    # ragged ends: one partial query block; a 128-key block whose second tile lies past the end
    "edge_n65_128x64_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 65), block_k=64, lam=-8.0, seed=304),
    "edge_n129_128x128": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 129), seed=305),
    "edge_n1_128x64_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 1), block_k=64, lam=-8.0, seed=306),
    # PV skip on 128-key blocks (one decision per block)
    "image_s_lam": rep(_im, Hq=3, Hkv=3, latent=(1, 20, 37), lam=-8.0, seed=308),
    "edge_n193_128x128_lam": rep(_im, Hq=2, Hkv=2, latent=(1, 1, 193), lam=-8.0, seed=309),
}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def bf16_dev_from_f32(x: np.ndarray):
    """float32 values that are exact bf16 -> device bf16."""
    bits = (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), x)
    return dev(bits)


# ------------------------------------------------------------------ 1. the quantizer

def _quant_gpu(xd, perm_d, block):
    B, H, N, D = xd.shape
    codes = torch.empty((B, H, N, D), dtype=torch.uint8, device="cuda")
    scales = torch.empty(B * H * -(-N // block), dtype=torch.float32, device="cuda")
    sa.sa_quantize_fp8(xd, perm_d, block, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy().reshape(B, H, -1)


def _check_quant(x_f64, xd, perm, block, what):
    """x_f64: [B, H, N, D] values in the original order; perm: numpy or None."""
    B, H, N, D = x_f64.shape
    perm_d = None if perm is None else torch.from_numpy(perm.astype(np.int32)).cuda()
    codes, scales = _quant_gpu(xd, perm_d, block)
    order = np.arange(N) if perm is None else perm
    bad_codes = bad_scales = 0
    for b in range(B):
        for h in range(H):
            want_c, want_s = OQ.quantize_blocks(x_f64[b, h][order], block)
            got_c = codes[b, h][order]
            bad_codes += int(np.count_nonzero(got_c != want_c))
            bad_scales += int(np.count_nonzero(scales[b, h].view(np.uint32) != want_s.view(np.uint32)))
    log(f"[fp8] quantize {what}: B={B} H={H} N={N} D={D} block={block} "
        f"code_mismatch={bad_codes} scale_mismatch={bad_scales}")
    assert bad_codes == 0 and bad_scales == 0


@pytest.mark.parametrize("name", ["long_video_s", "image_s", "video_s"])
def test_quantize_matches_oracle_on_workloads(name):
    w = CASES[name]
    q, k, _ = generate(w)
    perm = R.oracle_perm(w)
    for x, block, what in ((q, w.block_q, "q"), (k, OQ.KEY_QUANT_ROWS, "k")):
        _check_quant(R.to_f64(x), dev(x), perm, block, f"{name}.{what} gather")
        _check_quant(R.to_f64(x), dev(x), None, block, f"{name}.{what} identity")


@pytest.mark.parametrize("D,N,block", [(64, 1000, 64), (64, 1000, 128), (128, 77, 37), (128, 1, 128),
                                       (64, 300, 1)])
def test_quantize_ragged_sizes(D, N, block):
    rng = np.random.default_rng(N * 7 + D + block)
    x = (rng.standard_normal((2, 3, N, D)) * rng.uniform(0.01, 50, (2, 3, 1, 1))).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    perm = rng.permutation(N)
    _check_quant(x.astype(np.float64), bf16_dev_from_f32(x), perm, block, "random gather")
    _check_quant(x.astype(np.float64), bf16_dev_from_f32(x), None, block, "random identity")


def test_quantize_zero_block_signed_zeros_and_ties():
    """Block 0 all zeros (some negative zeros): scale 1, zero codes with their signs.
    Block 1 has amax exactly 448, so x * (448 / amax) is x itself and every listed value
    is an exact rounding tie of E4M3 (or a value just off one); block 2 is tiny values
    that fall into the subnormal codes."""
    D = 128
    x = np.zeros((1, 1, 192, D), dtype=np.float32)
    x[0, 0, 3, :64] = -0.0
    ties = np.array([1.0625, 1.1875, -1.0625, -1.1875, 3 * 2.0 ** -10, 2.0 ** -10, -(2.0 ** -11),
                     15 * 2.0 ** -10, 432.0, -432.0, 1.0625 + 2.0 ** -7, 2.5, 3.25, 0.0, -0.0, 448.0],
                    dtype=np.float32)
    blk1 = np.resize(ties, (64, D)).astype(np.float32)
    blk1[0, 0] = 448.0
    x[0, 0, 64:128] = blk1
    rng = np.random.default_rng(5)
    x[0, 0, 128:192] = (rng.standard_normal((64, D)) * 1e-3).astype(np.float32)
    x[0, 0, 130, 7] = 0.25
    x = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    _check_quant(x.astype(np.float64), bf16_dev_from_f32(x), None, 64, "zeros/ties/subnormals")
    codes, scales = _quant_gpu(bf16_dev_from_f32(x), None, 64)
    assert scales[0, 0, 0] == 1.0 and np.all(codes[0, 0, :64] & 0x7F == 0)
    assert np.all(codes[0, 0, 3, :64] == 0x80) and np.all(codes[0, 0, 3, 64:] == 0x00)


# ------------------------------------------------------------------ 2./3. attention

def run_fp8(w, fused=True):
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg, materialize=not fused, qk_fp8=True)
    q, k, v = generate(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    if fused:
        path.predict_gather(qd, kd)
        path.attend_gather(qd, kd, vd)
    else:
        path.permute(qd, kd, vd)
        path.predict()
        path.attend()
        path.unpermute()
    torch.cuda.synchronize()
    return path, (q, k, v)


def _oracle_operands(w, q, k, v, perm):
    """Reordered fp64 operands: exact (bf16 values) and dequantized (oracle codes)."""
    qp, kp, vp = R.permuted(q, perm), R.permuted(k, perm), R.permuted(v, perm)
    qh = np.empty_like(qp)
    kh = np.empty_like(kp)
    for b in range(w.B):
        for h in range(w.Hq):
            c, s = OQ.quantize_blocks(qp[b, h], w.block_q)
            qh[b, h] = OQ.dequantize_blocks(c, s, w.block_q)
        for h in range(w.Hkv):
            c, s = OQ.quantize_blocks(kp[b, h], OQ.KEY_QUANT_ROWS)
            kh[b, h] = OQ.dequantize_blocks(c, s, OQ.KEY_QUANT_ROWS)
    return qp, kp, vp, qh, kh


def check_fp8_parity(name, w, fused=True):
    log(f"[fp8] {name}: fused={fused} B={w.B} Hq={w.Hq} Hkv={w.Hkv} N={w.N} bq={w.block_q} bk={w.block_k} "
        f"lam={w.lam}")
    path, (q, k, v) = run_fp8(w, fused)
    cfg = path.cfg
    st_pred, st_attn = path.statuses()
    assert st_pred == sa.SA_OK and st_attn == sa.SA_OK
    perm = R.oracle_perm(w)
    assert np.array_equal(path.perm_host.astype(np.int64), perm)
    qp, kp, vp, qh, kh = _oracle_operands(w, q, k, v, perm)
    rp, ci = path.csr_host()
    o = path.o.cpu().numpy()
    o_perm = OL.permute_rows(o, perm)
    skip = path.pv_skip.cpu().numpy()
    G = w.Hq // w.Hkv
    scale = 1.0 / np.sqrt(w.D)
    err_max = err_sum = 0.0
    err_n = 0
    lam_far = lam_diff = 0
    bound_worst = 0.0  # largest |o - exact| / bound over rows (lambda off)
    rel_num = rel_den = 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // G
            r0 = (b * w.Hq + h) * cfg.n_qb
            ys, recs = R.attend_rows(qh[b, h], kh[b, hk], vp[b, hk], w, rp, ci, r0, range(cfg.n_qb), skip,
                                     path.groups)
            for i, y in ys.items():
                got = o_perm[b, h, i * w.block_q:i * w.block_q + y.shape[0]]
                d = np.abs(got - y)
                err_max = max(err_max, float(d.max()))
                err_sum += float(d.sum())
                err_n += d.size
                if w.lam is not None:
                    f, dd = R.lambda_disagreements(recs[i], w.lam)
                    lam_far += f
                    lam_diff += dd
            if w.lam is None and not w.causal:
                # 3. distance to the attention over the unquantized operands, per row
                ye, _ = R.attend_rows(qp[b, h], kp[b, hk], vp[b, hk], w, rp, ci, r0, range(cfg.n_qb))
                for i, y in ye.items():
                    rows = np.arange(i * w.block_q, i * w.block_q + y.shape[0])
                    cols = ci[rp[r0 + i]:rp[r0 + i + 1]]
                    keys = np.concatenate([np.arange(j * w.block_k, min((j + 1) * w.block_k, w.N)) for j in cols])
                    ds = np.abs(qh[b, h][rows] @ kh[b, hk][keys].T - qp[b, h][rows] @ kp[b, hk][keys].T) * scale
                    delta = ds.max(axis=1)
                    vmax = np.abs(vp[b, hk][keys]).max()
                    bound = (np.exp(2 * delta) - 1) * vmax + R.MAX_ABS
                    got = o_perm[b, h, rows]
                    dev_row = np.abs(got - y).max(axis=1)
                    bound_worst = max(bound_worst, float((dev_row / bound).max()))
                    rel_num += float(np.abs(got - y).sum())
                    rel_den += float(np.abs(y).sum())
    msg = (f"[fp8] {name}: out_max={err_max:.3e} out_mean={err_sum / err_n:.3e} lam_diff={lam_diff} "
           f"lam_far={lam_far}")
    if w.lam is None and not w.causal:
        msg += f" vs_unquantized: rel_l1={rel_num / rel_den:.3e} worst_row/bound={bound_worst:.3f}"
    log(msg)
    assert err_max <= R.MAX_ABS and err_sum / err_n <= R.MEAN_ABS
    assert lam_far == 0
    if w.lam is None and not w.causal:
        assert bound_worst <= 1.0

    # counters: QK blocks = nnz; executed + skipped = real groups x entries; skips = bits set
    cnt = path.counters.cpu().numpy()
    assert cnt[0] == int(rp[-1])
    real = skipped = 0
    for r in range(cfg.rows):
        i = r % cfg.n_qb
        ng = -(-(min((i + 1) * w.block_q, w.N) - i * w.block_q) // 32)
        real += ng * (rp[r + 1] - rp[r])
        for e in range(rp[r], rp[r + 1]):
            skipped += int(skip[e * path.groups:e * path.groups + ng].sum())
    assert cnt[1] + cnt[2] == real and cnt[2] == skipped
    if w.lam is None:
        assert cnt[2] == 0
    return path


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_attention_parity(name):
    check_fp8_parity(name, CASES[name])


@pytest.mark.parametrize("name", ["long_video_s", "image_s"])
def test_fp8_materialized_form(name):
    """The same path on reordered copies (no permutation inside the kernels)."""
    check_fp8_parity(name, CASES[name], fused=False)


def test_fp8_mask_unchanged():
    """The FP8 option changes the attention only: prediction runs on bf16 and gives the same CSR."""
    w = CASES["long_video_s"]
    cfg = sa.config_from_workload(w)
    q, k, _ = generate(w)
    a = sa.SparseAttentionPath(cfg, materialize=False, qk_fp8=True)
    b = sa.SparseAttentionPath(cfg, materialize=False)
    for p in (a, b):
        p.predict_gather(dev(q), dev(k))
    torch.cuda.synchronize()
    ra, ca = a.csr_host()
    rb, cb = b.csr_host()
    assert np.array_equal(ra, rb) and np.array_equal(ca, cb)


# ------------------------------------------------------------------ full size

@pytest.mark.parametrize("name", ["long_video", "video"])
def test_fp8_full_size_sampled(name):
    """The FP8 step as `bench.py --qk fp8` runs it (gather form, full size): the codes and
    scales of sampled blocks bit-exact, and the outputs of sampled query blocks of two heads
    against fp64 over the dequantized operands on the GPU's CSR (PV decisions replayed)."""
    w = CONFIGS[name]
    log(f"[fp8 full] {name}: B={w.B} Hq={w.Hq} N={w.N} bq={w.block_q} bk={w.block_k} lam={w.lam}")
    q, k, v = generate(w)
    cfg = sa.config_from_workload(w)
    path = sa.SparseAttentionPath(cfg, materialize=False, qk_fp8=True)
    qd, kd, vd = dev(q), dev(k), dev(v)
    path.predict_gather(qd, kd)
    path.attend_gather(qd, kd, vd)
    torch.cuda.synchronize()
    assert path.statuses() == (sa.SA_OK, sa.SA_OK)
    del qd, kd, vd
    perm = R.oracle_perm(w)
    rp, ci = path.csr_host()
    skip = path.pv_skip.cpu().numpy()
    q8 = path.q8.cpu().numpy()
    k8 = path.k8.cpu().numpy()
    qs = path.q_scale.cpu().numpy().reshape(w.B, w.Hq, -1)
    ks = path.k_scale.cpu().numpy().reshape(w.B, w.Hkv, -1)
    rng = np.random.default_rng(7)
    G = w.Hq // w.Hkv
    err_max = err_sum = 0.0
    err_n = lam_far = 0
    for h in (0, w.Hq - 1):
        hk = h // G
        # the oracle's codes of this head, in the reordered order
        qp, kp = R.permuted(q[:, h:h + 1], perm)[0, 0], R.permuted(k[:, hk:hk + 1], perm)[0, 0]
        cq, sq = OQ.quantize_blocks(qp, w.block_q)
        ck, sk = OQ.quantize_blocks(kp, OQ.KEY_QUANT_ROWS)
        assert np.array_equal(q8[0, h][perm], cq) and np.array_equal(qs[0, h].view(np.uint32), sq.view(np.uint32))
        assert np.array_equal(k8[0, hk][perm], ck) and np.array_equal(ks[0, hk].view(np.uint32), sk.view(np.uint32))
        qh = OQ.dequantize_blocks(cq, sq, w.block_q)
        kh = OQ.dequantize_blocks(ck, sk, OQ.KEY_QUANT_ROWS)
        vp = R.permuted(v[:, hk:hk + 1], perm)[0, 0]
        r0 = h * cfg.n_qb
        blocks = sorted(set(rng.integers(0, cfg.n_qb, 6).tolist()) | {cfg.n_qb - 1})
        ys, recs = R.attend_rows(qh, kh, vp, w, rp, ci, r0, blocks, skip, path.groups)
        o = path.o[0, h][torch.from_numpy(perm.astype(np.int64)).cuda()].cpu().numpy()
        for i, y in ys.items():
            d = np.abs(o[i * w.block_q:i * w.block_q + y.shape[0]] - y)
            err_max = max(err_max, float(d.max()))
            err_sum += float(d.sum())
            err_n += d.size
            if w.lam is not None:
                lam_far += R.lambda_disagreements(recs[i], w.lam)[0]
    log(f"[fp8 full] {name}: out_max={err_max:.3e} out_mean={err_sum / err_n:.3e} lam_far={lam_far}")
    assert err_max <= R.MAX_ABS and err_sum / err_n <= R.MEAN_ABS
    assert lam_far == 0


# ------------------------------------------------------------------ quantization inside the prediction

@pytest.mark.parametrize("name,fused", [("long_video_s", True), ("image_s", True), ("video_s", True),
                                        ("causal_s_gqa", True), ("causal_s64_gqa_lam", True),
                                        ("edge_n65_128x64_lam", True), ("edge_n129_128x128", True),
                                        ("long_video_s", False), ("image_s", False)])
def test_predict_mask_qk8_equals_separate_quantizer(name, fused):
    """sa_predict_mask_qk8 writes the CSR of the plain prediction and, in the same pass, the
    codes and scales sa_quantize_fp8 writes (which equal the oracle's), bit for bit; through
    the permutation (fused) or on reordered copies (perm None)."""
    w = CASES[name]
    cfg = sa.config_from_workload(w)
    q, k, _ = generate(w)
    qd, kd = dev(q), dev(k)
    path = sa.SparseAttentionPath(cfg, materialize=not fused, qk_fp8=True)
    ref = sa.SparseAttentionPath(cfg, materialize=not fused, qk_fp8=True)
    if fused:
        perm = path.perm
        qi, ki = qd, kd
    else:
        perm = None
        path.permute(qd, kd, kd)
        qi, ki = path.qp, path.kp
    sa.sa_predict_mask_qk8(qi, ki, perm, path.mp, path.ws, path.row_ptr, path._cols(), path.q8, path.q_scale,
                           path.k8, path.k_scale, path.status[0:1])
    if fused:
        sa.sa_predict_mask_gather(qd, kd, ref.perm, ref.mp, ref.ws, ref.row_ptr, ref._cols(), ref.status[0:1])
    else:
        sa.sa_predict_mask(qi, ki, ref.mp, ref.ws, ref.row_ptr, ref._cols(), ref.status[0:1])
    ref.quantize(qi, ki, perm, perm)
    torch.cuda.synchronize()
    assert path.statuses()[0] == sa.SA_OK and ref.statuses()[0] == sa.SA_OK
    ra, ca = path.csr_host()
    rb, cb = ref.csr_host()
    assert np.array_equal(ra, rb) and np.array_equal(ca, cb)
    for a, b in ((path.q8, ref.q8), (path.k8, ref.k8)):
        assert torch.equal(a, b)
    for a, b in ((path.q_scale, ref.q_scale), (path.k_scale, ref.k_scale)):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    log(f"[fp8] predict+quantize {name} fused={fused}: codes and scales equal, nnz={int(ra[-1])}")
