"""Benchmark of the block-sparse attention forward path on one MI355X.

A step is one pass of the whole path over one batch: reorder Q, K, V,
predict the block mask, sparse attention, inverse reorder of the output.  By
default (bf16 inputs) the reorder is the gather form: the mask prediction and
the attention read Q, K, V through the token permutation and the attention
writes O back in the original order (two launches of work per step,
bit-identical to the materialising form, which ``--form materialize`` times:
three permute copies, prediction, attention, un-permute).
Default workload: the long-video shape (B=1, 24 heads, latent [28,30,53] ->
N=44520, d=128, Hilbert order, b_q=128 / b_k=64, tau=0.95, theta=0.6,
lambda=-8) at sparsity 0.8.  Inputs are synthetic, seeded, and resident in
HBM before timing starts.

Prints ONE JSON line.  ``value`` is executed TFLOP/s of the whole step
(executed QK + PV flops of the sparse attention over the step time);
``roofline`` covers the sparse attention kernel (bf16 MFMA bound);
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload (rank 0, N=1 only).

``--qk fp8`` times the FP8 QK variant instead (Q and K quantized to per-block
E4M3 codes inside each step -- in the gather form by the mask prediction's
own pass over them --, QK products on the fp8 matrix cores, P V in bf16);
its roofline peak is the time-weighted mix of the fp8 and bf16 peaks over
its QK and PV flops, and it has no oracle leg.

Extra modes (not the benchmark line):
  --mode attn      only the sparse attention launch, repeated (for rocprofv3 counters)
  --mode predict   only the mask prediction launch, repeated (for rocprofv3 counters)
  --mode reorder   only the reorder copies of the materialising form (three permutes and
                   the un-permute), repeated (for rocprofv3 counters)
  --mode copy      a plain device copy of known size (HBM counter calibration)
  --mode ceilings  what the box reaches outside this library: a bf16 GEMM through torch
                   (hipBLASLt) and torch's dense flash attention at the workload's shape
"""

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "block-sparse attn fwd: ms/call + executed TFLOP/s (MFMA %) at sparsity 0.8"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "flash_traffic_long_video.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the attention kernel needs about ten dispatches before its clock settles
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_video")
    ap.add_argument("--sparsity", type=float, default=None, help="override the workload's sparsity")
    ap.add_argument("--mode", default="path", choices=["path", "attn", "predict", "reorder", "copy", "ceilings"])
    ap.add_argument("--no-lambda", action="store_true", help="turn the workload's PV skip off")
    ap.add_argument("--lam", type=float, default=None, help="override the workload's PV-skip threshold")
    ap.add_argument("--form", default="gather", choices=["gather", "materialize"],
                    help="reorder inside the kernels' loads (bf16 inputs) or as separate copies")
    ap.add_argument("--qk", default="bf16", choices=["bf16", "fp8"],
                    help="QK products on bf16 operands, or on per-block E4M3 codes (quantized inside the step)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget")
    ap.add_argument("--no-cpu", action="store_true")
    return ap.parse_args()


def flash_source_hash():
    """Hash of the attention kernels' source: flash.hip and the argument block they take."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "image_dit_amd", "csrc")
    with open(os.path.join(csrc, "flash.hip"), "rb") as fh:
        h.update(fh.read())
    with open(os.path.join(csrc, "sa_internal.h"), encoding="utf8") as fh:
        text = fh.read()
    i = text.index("struct FlashArgs {")
    h.update(text[i:text.index("};", i)].encode())
    return h.hexdigest()[:16]


def attn_kernel_name(cfg, gather, fp8=False):
    """The attention kernel the attention entry point launches for this configuration."""
    if cfg.block_q == 16 and cfg.block_k == 16:
        return "k_flash_small"
    g = "true" if gather else "false"
    f = "true" if fp8 else "false"
    sub = 1 if cfg.block_k == 64 else 2
    return f"k_flash_{'lam' if cfg.lam is not None else 'dma'}<{cfg.D}, {sub}, {g}, {f}>"


def executed_flops(cfg, rp, ci, skip, groups):
    """Executed QK and PV flops at real token counts, from the CSR and the PV-skip flags."""
    import numpy as np

    N, bq, bk, d = cfg.N, cfg.block_q, cfg.block_k, cfg.D
    rows = len(rp) - 1
    i = np.arange(rows) % cfg.n_qb
    qrows = np.minimum((i + 1) * bq, N) - i * bq
    cnt = np.diff(rp)
    kcols = np.minimum((ci + 1) * bk, N) - ci * bk          # tokens per kept key block
    row_of = np.repeat(np.arange(rows), cnt)
    qk = 2.0 * float(np.sum(qrows[row_of] * kcols)) * d
    pv = 0.0
    for g in range(groups):
        grow = np.clip(qrows - g * 32, 0, 32)[row_of]          # rows of group g in each entry's q-block
        done = grow * kcols
        if skip is not None and cfg.lam is not None:
            done = done * (1 - skip[np.arange(len(ci)) * groups + g])
        pv += 2.0 * float(np.sum(done)) * d
    return qk, pv


def cpu_model():
    try:
        with open("/proc/cpuinfo", encoding="utf8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, path, q, k, v, budget_s, gmask0=None):
    """Oracle on a bounded sample: prediction of one head + attention of the first query blocks.
    With gmask0 (the library's mask rows of head 0) the oracle's rows of that head are also
    compared with it (admissible rows, borderline counts)."""
    import numpy as np

    from oracle import flash as OF
    from oracle import layout as OL
    from oracle import numerics as ON
    from oracle import predict as OP
    from oracle.admissible import borderline_counts, compare_head_mask

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = path.cfg
    h = 0
    perm = OL.plan_permutation(w.N, w.order, w.latent, w.window, w.txt_len, w.first_frame_sink)
    qp = OL.permute_rows(ON.bf16_to_f64(q[0, h]), perm)
    kp = OL.permute_rows(ON.bf16_to_f64(k[0, h]), perm)
    vp = OL.permute_rows(ON.bf16_to_f64(v[0, h]), perm)
    mp = OP.MaskParams(N=w.N, block_q=w.block_q, block_k=w.block_k, causal=w.causal, window=w.window_tokens,
                       sink_front=w.sink_front, sink_back=w.sink_back, tau=w.tau, theta=w.theta,
                       sparsity=cfg.sparsity, sink_rows=w.sink_rows)
    t0 = time.perf_counter()
    ref = OP.predict_head(qp, kp, mp)
    t_pred = time.perf_counter() - t0
    mask_check = None
    if gmask0 is not None:
        bad, differ, checked, kinds = compare_head_mask(gmask0, ref, mp)
        mask_check = {"head": 0, "rows": checked, "not_admissible": len(bad), "differing_borderline": len(differ),
                      "differing_by_kind": kinds, "flagged_borderline": borderline_counts(ref)}
    rp, ci = path.csr_host()
    skip_gpu = path.pv_skip.cpu().numpy() if (path.pv_skip is not None and w.lam is not None) else None
    lam_stats = {"decisions": 0, "near_border": 0, "differ": 0, "differ_outside_border": 0}
    t0 = time.perf_counter()
    flops = 0.0
    nblk = 0
    while nblk < cfg.n_qb and (time.perf_counter() - t0) < budget_s:
        cols = ci[rp[nblk]:rp[nblk + 1]]
        _, rec = OF.attend_qblock(qp, kp, vp, nblk, cols, w.block_q, w.block_k, causal=w.causal,
                                  lam=w.lam if w.lam is not None else None)
        if skip_gpu is not None:
            ng = rec["skip"].shape[1]
            gpu = np.array([[bool(skip_gpu[(rp[nblk] + e) * path.groups + g]) for g in range(ng)]
                            for e in range(len(cols))], dtype=bool).reshape(len(cols), ng)
            near = np.abs(rec["gap"] - w.lam) <= 1e-3
            diff = gpu != rec["skip"]
            lam_stats["decisions"] += int(gpu.size)
            lam_stats["near_border"] += int(near.sum())
            lam_stats["differ"] += int(diff.sum())
            lam_stats["differ_outside_border"] += int((diff & ~near).sum())
        rows = min((nblk + 1) * w.block_q, w.N) - nblk * w.block_q
        kts = np.array([min((j + 1) * w.block_k, w.N) - j * w.block_k for j in cols], dtype=np.float64)
        flops += 2.0 * rows * kts.sum() * w.D  # QK
        for g in range(rec["skip"].shape[1]):
            grows = min(OF.PV_GROUP_ROWS, rows - g * OF.PV_GROUP_ROWS)
            flops += 2.0 * grows * float(kts[~rec["skip"][:, g]].sum()) * w.D  # PV of executed groups
        nblk += 1
    t_attn = time.perf_counter() - t0
    # per-head prediction cost is shared by the head's n_qb query blocks
    t_pred_share = t_pred * nblk / cfg.n_qb
    value = flops / (t_attn + t_pred_share) / 1e12
    out = {"value": value, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": (f"head 0: block stats + mask prediction of all {cfg.n_qb} query blocks "
                      f"({t_pred:.2f} s, charged pro rata) and fp64 attention with PV-skip emulation "
                      f"on the first {nblk} query blocks over the GPU's CSR ({t_attn:.2f} s)"),
           "threads": int(threads), "host_cpus": os.cpu_count(), "model": cpu_model(),
           "thread_setting": f"NumPy BLAS threads as the environment sets them (OMP_NUM_THREADS="
                             f"{os.environ.get('OMP_NUM_THREADS', 'unset')})"}
    if mask_check is not None:
        out["mask_check"] = mask_check
    if skip_gpu is not None:
        out["mask_check"] = dict(out.get("mask_check", {}), lambda_decisions=lam_stats)
    return out


def _event_ms(torch, f, reps):
    f()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        f()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def ceilings(torch, w):
    """Reference points outside the library on the same box: a square bf16 GEMM and torch's
    dense flash attention (flash backend only, so no fallback runs) at the workload's shape."""
    out = {"mode": "ceilings", "workload": w.name}
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    ms = _event_ms(torch, lambda: torch.matmul(a, b), 20)
    out["gemm_bf16"] = {"m=n=k": n, "ms": round(ms, 4), "tflops": round(2.0 * n ** 3 / ms / 1e9, 1)}
    del a, b
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel

        q = torch.randn(w.B, w.Hq, w.N, w.D, device="cuda", dtype=torch.bfloat16)
        k = torch.randn(w.B, w.Hq, w.N, w.D, device="cuda", dtype=torch.bfloat16)
        v = torch.randn(w.B, w.Hq, w.N, w.D, device="cuda", dtype=torch.bfloat16)

        def run():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=w.causal)

        ms = _event_ms(torch, run, 5)
        dense = 4.0 * w.B * w.Hq * w.D * (w.N * (w.N + 1) / 2 if w.causal else float(w.N) ** 2)
        out["sdpa_flash"] = {"shape": [w.B, w.Hq, w.N, w.D], "causal": w.causal, "ms": round(ms, 3),
                             "tflops": round(dense / ms / 1e9, 1)}
    except Exception as e:  # the flash backend is not available for this device or shape
        out["sdpa_flash"] = {"error": str(e).splitlines()[0][:200] if str(e) else type(e).__name__}
    out["peak_bf16_tflops"] = PEAK_BF16_TFLOPS
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}); the path would shard over "
              "(batch, head) with no communication between GPUs", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import image_dit_amd as sa
    from workloads import CONFIGS, generate

    torch.cuda.set_device(0)
    if args.mode == "copy":
        nbytes = 1 << 30
        a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "launches": 3}))
        return

    w = CONFIGS[args.workload]
    if args.sparsity is not None:
        w = w.with_sparsity(args.sparsity)
    if args.no_lambda:
        w = dataclasses.replace(w, lam=None)
    if args.lam is not None:
        w = dataclasses.replace(w, lam=args.lam)
    if args.mode == "ceilings":
        print(json.dumps(ceilings(torch, w)))
        return
    cfg = sa.config_from_workload(w)
    gather = args.form == "gather" and w.dtype == "bf16"
    fp8 = args.qk == "fp8"
    path = sa.SparseAttentionPath(cfg, materialize=not gather, qk_fp8=fp8)
    t_gen = time.perf_counter()
    q, k, v = generate(w)
    t_gen = time.perf_counter() - t_gen

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(x).cuda()

    qd, kd, vd = dev(q), dev(k), dev(v)
    torch.cuda.synchronize()

    # the step's stages; the gather form has no separate reorder copies; with FP8 QK
    # operands the gather form's prediction writes the codes in its pass over Q and K,
    # and the materialising form quantizes the reordered copies (its own stage)
    if gather:
        stages = [("permute", lambda: None), ("predict", lambda: path.predict_gather(qd, kd))]
        if fp8:
            stages += [("attn", lambda: path.attend_qk8_gather(vd))]
        else:
            stages += [("attn", lambda: path.attend_gather(qd, kd, vd))]
        stages += [("unpermute", lambda: None)]
    else:
        stages = [("permute", lambda: path.permute(qd, kd, vd)), ("predict", path.predict)]
        if fp8:
            stages += [("quantize", lambda: path.quantize(path.qp, path.kp)),
                       ("attn", path.attend_qk8)]
        else:
            stages += [("attn", path.attend)]
        stages += [("unpermute", path.unpermute)]
    idx = {name: j for j, (name, _) in enumerate(stages)}

    def run_step():
        for _, f in stages:
            f()

    if args.mode in ("attn", "predict"):
        run_step()
        for _ in range(max(1, args.steps)):
            stages[idx[args.mode]][1]()
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "form": "gather" if gather else "materialize",
                          "launches": max(1, args.steps) + 1}))
        return
    if args.mode == "reorder":
        if gather:
            path = sa.SparseAttentionPath(cfg, materialize=True)
        for _ in range(max(1, args.steps)):
            path.permute(qd, kd, vd)
            path.unpermute()
        torch.cuda.synchronize()
        print(json.dumps({"mode": "reorder", "launches": max(1, args.steps)}))
        return

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # One event before each stage that launches work, nothing else: a stage
    # ends where the next recorded one starts (the last stage of a step at the
    # next step's first event, or at `end`).  Every recorded event is a queue
    # marker that leaves the GPU idle for a few microseconds, so the gather
    # form records two per step (before the prediction, before the attention).
    K = args.steps
    real = [j for j, (name, _) in enumerate(stages) if not (gather and name in ("permute", "unpermute"))]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in real] for _ in range(K)]
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(K):
        for x, j in enumerate(real):
            ev[s][x].record(stream)
            stages[j][1]()
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = ev[0][0].elapsed_time(end)
    stage = np.zeros(len(stages))
    for s in range(K):
        for x, j in enumerate(real):
            nxt = ev[s][x + 1] if x + 1 < len(real) else (ev[s + 1][0] if s + 1 < K else end)
            stage[j] += ev[s][x].elapsed_time(nxt)
    stage /= K
    ms_step = total_ms / K

    st = path.statuses()
    if st != (sa.SA_OK, sa.SA_OK):
        raise RuntimeError(f"device status {st}")
    rp, ci = path.csr_host()
    skip = path.pv_skip.cpu().numpy() if path.pv_skip is not None else None
    qk, pv = executed_flops(cfg, rp, ci, skip, path.groups)
    exec_flops = qk + pv
    N, d, B, Hq, Hkv = cfg.N, cfg.D, cfg.B, cfg.Hq, cfg.Hkv
    dense_flops = 4.0 * B * Hq * N * N * d if not cfg.causal else 4.0 * B * Hq * d * N * (N + 1) / 2
    # combined QK+PV skipped fraction (block products), SpargeAttn notes section 3.2 "Sparsity"
    cnt = path.counters.cpu().numpy()
    nnz = int(rp[-1])
    ib = np.arange(cfg.rows) % cfg.n_qb
    if cfg.causal:
        valid_blocks = np.minimum(cfg.n_kb, (np.minimum((ib + 1) * cfg.block_q, N) - 1) // cfg.block_k + 1)
    else:
        valid_blocks = np.full(cfg.rows, cfg.n_kb)
    mask_sparsity = 1.0 - nnz / float(valid_blocks.sum())
    pv_groups_total = cnt[1] + cnt[2]
    combined = 1.0 - (nnz + cnt[1] * (nnz / max(1, pv_groups_total))) / (2.0 * valid_blocks.sum())

    attn_ms = stage[idx["attn"]]
    attn_tflops = exec_flops / (attn_ms * 1e-3) / 1e12
    # the attention kernel's MFMA peak: bf16, or (FP8 QK) the time-weighted mix of the
    # fp8 QK and bf16 PV peaks
    peak = PEAK_BF16_TFLOPS if not fp8 else exec_flops / (qk / PEAK_FP8_TFLOPS + pv / PEAK_BF16_TFLOPS)
    n_qb, n_kb = cfg.n_qb, cfg.n_kb
    pred_bytes = (2 * (B * Hq * N * d + B * Hkv * N * d) + 4 * (B * Hq * n_qb + B * Hkv * n_kb) * d
                  + 4 * (B * Hq * n_qb + B * Hkv * n_kb) + 2 * B * Hq * n_qb * n_kb
                  + 4 * (B * Hq * n_qb + 1) + 4 * nnz + (4 * N if gather else 0)
                  # FP8, gather form: the codes of Q and K are written in the same pass
                  + ((B * Hq * N * d + B * Hkv * N * d) if (fp8 and gather) else 0))
    perm_bytes = (B * Hq * N * d + 2 * B * Hkv * N * d) * ((4 if w.dtype == "f32" else 2) + 2)
    unperm_bytes = 2 * 4 * B * Hq * N * d
    # quantize: Q and K read (bf16) and written (one byte per element), plus the scales
    quant_bytes = 3 * (B * Hq * N * d + B * Hkv * N * d) + 4 * (B * Hq * n_qb + B * Hkv * -(-N // 64))

    # HBM bytes per attention launch measured with rocprofv3 counters on this kernel source
    # (null when no record matches the source, workload, sparsity, form and QK type)
    traffic = None
    try:
        with open(TRAFFIC_FILE, encoding="utf8") as f:
            records = json.load(f)["records"]
        sha = flash_source_hash()
        for tr in records:
            if tr["source_sha"] == sha and tr["workload"] == args.workload \
                    and abs(tr["sparsity"] - (cfg.sparsity or 0)) < 1e-9 \
                    and tr["form"] == ("gather" if gather else "materialize") and tr["qk"] == args.qk:
                traffic = tr["hbm_bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None

    out = {
        "metric": METRIC,
        "value": round(exec_flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 e4m3 (QK) + bf16 (PV)" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: B{B} Hq{Hq} Hkv{Hkv} latent{list(w.latent)} txt{w.txt_len} N{N} d{d} "
                         f"order{w.order} bq{cfg.block_q} bk{cfg.block_k} tau{w.tau} theta{w.theta} "
                         f"lambda{w.lam} sparsity{cfg.sparsity}"),
            "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "block_q": cfg.block_q, "block_k": cfg.block_k,
            "sparsity_target": cfg.sparsity,
            "reorder": "gather (inside the kernels' loads)" if gather else "materialized copies",
            "qk": "fp8 e4m3, one scale per 128-row query block and per 64-key tile" if fp8 else "bf16",
        },
        "ms": {name: round(stage[j], 4) for name, j in idx.items()
               if not (gather and name in ("permute", "unpermute"))},
        "attn_executed_tflops": round(attn_tflops, 2),
        "attn_mfma_frac": round(attn_tflops / peak, 4),
        "dense_equiv_tflops_step": round(dense_flops / (ms_step * 1e-3) / 1e12, 2),
        "dense_equiv_tflops_attn_plus_predict": round(
            dense_flops / ((attn_ms + stage[idx["predict"]] + (stage[idx["quantize"]] if "quantize" in idx else 0.0))
                           * 1e-3) / 1e12, 2),
        "executed_tflop": round(exec_flops / 1e12, 4),
        "dense_tflop": round(dense_flops / 1e12, 4),
        "mask_sparsity": round(mask_sparsity, 4),
        "combined_qk_pv_sparsity": round(float(combined), 4),
        "pv_group_blocks": {"executed": int(cnt[1]), "skipped": int(cnt[2])},
        "predict_gbs": round(pred_bytes / (stage[idx["predict"]] * 1e-3) / 1e9, 1),
        "predict_hbm_frac": round(pred_bytes / (stage[idx["predict"]] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        **({} if gather else {"permute_gbs": round(perm_bytes / (stage[idx["permute"]] * 1e-3) / 1e9, 1),
                              "unpermute_gbs": round(unperm_bytes / (stage[idx["unpermute"]] * 1e-3) / 1e9, 1)}),
        **({} if "quantize" not in idx else
           {"quantize_gbs": round(quant_bytes / (stage[idx["quantize"]] * 1e-3) / 1e9, 1)}),
        "roofline": {
            "bound": "mfma",
            "kernel": attn_kernel_name(cfg, gather, fp8) + " (+ k_attn_init), per "
                      + ("sa_sparse_attn_fwd_qk8" if fp8 else
                         "sa_sparse_attn_fwd_gather" if gather else "sa_sparse_attn_fwd") + " call",
            "achieved": round(attn_tflops, 2),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / peak, 4),
            "traffic": traffic,
        },
        "wall_s_timed": round(t_wall, 3),
        "gen_s": round(t_gen, 1),
    }
    if not args.no_cpu and not fp8:  # (the oracle sample follows the bf16 path)
        # the library's mask rows of head 0, for the oracle's row-by-row check (after timing)
        mask = torch.zeros((cfg.rows, cfg.n_kb), dtype=torch.uint8, device="cuda")
        if gather:
            path.predict_gather(qd, kd, mask_out=mask)
        else:
            path.permute(qd, kd, vd)
            path.predict(mask_out=mask)
        torch.cuda.synchronize()
        gmask0 = mask[:cfg.n_qb].cpu().numpy().astype(bool)
        out["cpu_baseline"] = cpu_baseline(w, path, q, k, v, args.cpu_seconds, gmask0)
        out["borderline"] = out["cpu_baseline"].pop("mask_check", None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
