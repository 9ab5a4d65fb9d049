"""Seeded synthetic Q/K/V generators (NumPy PCG64), in BNSD layout.

Only random draws and layout live here.  Rounding to bf16 is done by torch's
own float32 -> bfloat16 conversion (round to nearest even), so this module
carries no arithmetic of the attention method.

Recipes (the same ones the design doc lists):

* smooth field (image / video / long_video): per (batch, head, channel) a sum
  of 8 sinusoids over the normalised latent coordinates,
  F = sum_m sin(2*pi*(f_t t/T + f_h h/H + f_w w/W) + phi_m), f ~ U(0,1)^3,
  phi ~ U(0, 2*pi), amplitude 1 each.  Q = F + 0.3*N(0,1), K = F + 0.3*N(0,1)
  (shared field, independent noise); 1% of tokens (Bernoulli per token,
  independent for Q and K) are scaled by 8.  Text tokens, when present, are
  iid N(0,1) and are prepended.  V ~ N(0,1).  Keys on a grid of their own
  (``latent_k``) sample the same field (same draws) at that grid's normalised
  coordinates, with ``txt_len_k`` text tokens; V then has the keys' length.
* causal_long: per KV head an orthonormal U (128x16, QR of a Gaussian) and a
  drift z_r(t) = 2 sin(2*pi*f_r*t/N + phi_r), f_r ~ U(0.5, 4); Q and K of every
  head in the group are N(0,1) + U z(t); the keys at positions 0..3 are
  scaled by 10.  V ~ N(0,1).
* tiny: Q, K, V iid N(0,1) in float32.
"""

import numpy as np

from .configs import Workload

_NSIN = 8          # sinusoids per channel
_NOISE = 0.3       # noise standard deviation on the smooth field
_OUTLIER_P = 0.01  # fraction of outlier tokens
_OUTLIER_X = 8.0   # outlier scale
_DRIFT_RANK = 16
_DRIFT_AMP = 2.0
_SINK_KEYS = 4
_SINK_X = 10.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, via torch's RNE conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _field_draws(rng: np.random.Generator, C: int):
    """Frequencies U(0,1)^3 and phases U(0, 2*pi) of the _NSIN sinusoids of each channel."""
    freq = rng.uniform(0.0, 1.0, size=(C, _NSIN, 3))
    phase = rng.uniform(0.0, 2.0 * np.pi, size=(C, _NSIN))
    return freq, phase


def _eval_field(freq: np.ndarray, phase: np.ndarray, latent) -> np.ndarray:
    """Sum of the sinusoids over a (T,H,W) grid -> float32 [T*H*W, C].

    Coordinates are normalised (t/T, h/H, w/W), so one set of draws evaluated
    on two grids gives the same field sampled at two resolutions.
    sin(a+b+c) is expanded into four products so the whole grid is one batched
    matrix product per channel instead of T*H*W*_NSIN sine evaluations.
    """
    T, H, W = latent
    C = freq.shape[0]
    two_pi = 2.0 * np.pi
    a = two_pi * freq[:, :, 0:1] * (np.arange(T) / T)[None, None, :] + phase[:, :, None]
    b = two_pi * freq[:, :, 1:2] * (np.arange(H) / H)[None, None, :]
    c = two_pi * freq[:, :, 2:3] * (np.arange(W) / W)[None, None, :]
    sa, ca = np.sin(a), np.cos(a)
    sb, cb = np.sin(b), np.cos(b)
    sc, cc = np.sin(c), np.cos(c)
    # U: (C, T, 4M), Wm: (C, 4M, H*W)
    U = np.concatenate([sa, ca, ca, -sa], axis=1).transpose(0, 2, 1)
    hw = lambda x, y: (x[:, :, :, None] * y[:, :, None, :]).reshape(C, _NSIN, H * W)
    Wm = np.concatenate([hw(cb, cc), hw(sb, cc), hw(cb, sc), hw(sb, sc)], axis=1)
    F = np.matmul(U, Wm)  # (C, T, H*W)
    return np.ascontiguousarray(F.reshape(C, T * H * W).T, dtype=np.float32)


def _outliers(rng: np.random.Generator, x: np.ndarray) -> None:
    hit = rng.random(x.shape[0]) < _OUTLIER_P
    x[hit] *= _OUTLIER_X


def _gen_field(cfg: Workload):
    rng = np.random.default_rng(cfg.seed)
    B, H, D, N, Nk = cfg.B, cfg.Hq, cfg.D, cfg.N, cfg.N_k
    assert cfg.Hq == cfg.Hkv
    txt_k = cfg.txt_len if cfg.txt_len_k is None else cfg.txt_len_k
    q = np.empty((B, H, N, D), dtype=np.uint16)
    k = np.empty((B, H, Nk, D), dtype=np.uint16)
    for b in range(B):
        for h in range(H):
            freq, phase = _field_draws(rng, D)
            F = _eval_field(freq, phase, cfg.latent)
            Fk = F if cfg.latent_k is None else _eval_field(freq, phase, cfg.latent_k)
            for dst, field, txt in ((q, F, cfg.txt_len), (k, Fk, txt_k)):
                n = txt + field.shape[0]
                x = np.empty((n, D), dtype=np.float32)
                x[txt:] = field + _NOISE * rng.standard_normal((n - txt, D), dtype=np.float32)
                if txt:
                    x[:txt] = rng.standard_normal((txt, D), dtype=np.float32)
                _outliers(rng, x)
                dst[b, h] = bf16_bits(x)
    v = bf16_bits(rng.standard_normal((B, H, Nk, D), dtype=np.float32))
    return q, k, v


def _gen_causal(cfg: Workload):
    rng = np.random.default_rng(cfg.seed)
    B, Hq, Hkv, D, N = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.N
    G = Hq // Hkv
    q = np.empty((B, Hq, N, D), dtype=np.uint16)
    k = np.empty((B, Hkv, N, D), dtype=np.uint16)
    t = np.arange(N, dtype=np.float64)
    for b in range(B):
        for hk in range(Hkv):
            U, _ = np.linalg.qr(rng.standard_normal((D, _DRIFT_RANK)))
            f = rng.uniform(0.5, 4.0, size=_DRIFT_RANK)
            phi = rng.uniform(0.0, 2.0 * np.pi, size=_DRIFT_RANK)
            z = _DRIFT_AMP * np.sin(2.0 * np.pi * f[None, :] * t[:, None] / N + phi[None, :])
            drift = (z @ U.T).astype(np.float32)  # (N, D)
            for g in range(G):
                x = rng.standard_normal((N, D), dtype=np.float32)
                x += drift
                q[b, hk * G + g] = bf16_bits(x)
            x = rng.standard_normal((N, D), dtype=np.float32)
            x += drift
            x[:_SINK_KEYS] *= _SINK_X
            k[b, hk] = bf16_bits(x)
    v = bf16_bits(rng.standard_normal((B, Hkv, N, D), dtype=np.float32))
    return q, k, v


def _gen_iid_f32(cfg: Workload):
    rng = np.random.default_rng(cfg.seed)
    shape_q = (cfg.B, cfg.Hq, cfg.N, cfg.D)
    shape_kv = (cfg.B, cfg.Hkv, cfg.N_k, cfg.D)
    q = rng.standard_normal(shape_q).astype(np.float32)
    k = rng.standard_normal(shape_kv).astype(np.float32)
    v = rng.standard_normal(shape_kv).astype(np.float32)
    return q, k, v


def _gen_iid_bf16(cfg: Workload):
    q, k, v = _gen_iid_f32(cfg)
    return bf16_bits(q), bf16_bits(k), bf16_bits(v)


def _gen_frame_position(cfg: Workload):
    """The teaching video of the SparseAttn article (section 04) widened to head dim D:
    4 frames of 4x4 positions in frame-major order; query head h carries amplitude 6 on
    the one-hot of the token's frame (h even, dims 0..t-1) or of its position (h odd,
    dims t..t+h*w-1); every dim gets N(0, 0.15^2) noise; K equals Q; V ~ N(0, 1).
    float32, like the tiny workload."""
    t, hh, ww = cfg.latent
    P = hh * ww
    N = t * P
    if cfg.txt_len or cfg.N != N or cfg.D < t + P or cfg.Hq != cfg.Hkv:
        raise ValueError("the frame/position construction needs a bare video grid, D >= t + h*w, Hq == Hkv")
    rng = np.random.default_rng(cfg.seed)
    frame = np.arange(N) // P
    pos = np.arange(N) % P
    q = np.zeros((cfg.B, cfg.Hq, N, cfg.D), dtype=np.float64)
    for h in range(cfg.Hq):
        if h % 2 == 0:
            q[:, h, np.arange(N), frame] = 6.0
        else:
            q[:, h, np.arange(N), t + pos] = 6.0
    q = (q + rng.normal(0.0, 0.15, size=q.shape)).astype(np.float32)
    v = rng.standard_normal((cfg.B, cfg.Hkv, N, cfg.D)).astype(np.float32)
    return q, q.copy(), v


def generate(cfg: Workload, kind: str = "auto"):
    """Return (q, k, v) numpy arrays in BNSD, in the ORIGINAL token order.

    bf16 workloads return uint16 bit patterns; the tiny workload returns float32.
    ``kind`` overrides the recipe: "iid" draws iid N(0,1) (bf16 unless the
    workload is fp32), used for shape sweeps in tests; "frame_position" is the
    structured teaching input (fp32, see _gen_frame_position).
    """
    if kind == "iid":
        return _gen_iid_f32(cfg) if cfg.dtype == "f32" else _gen_iid_bf16(cfg)
    if kind == "frame_position":
        return _gen_frame_position(cfg)
    if cfg.name == "tiny" or cfg.dtype == "f32":
        return _gen_iid_f32(cfg)
    if cfg.name == "causal_long":
        return _gen_causal(cfg)
    return _gen_field(cfg)


def p1_demo_inputs():
    """The two-head teaching video of the SparseAttn article (section 04 and its appendix).

    4 frames of 4x4 positions (N=64), d = 4 frame dims + 16 position dims = 20.
    Head 0 carries amplitude 6 on the one-hot of its frame, head 1 on the
    one-hot of its position; N(0, 0.15^2) noise from default_rng(7); K equals Q;
    one V of shape (64, 3) drawn after the noise, shared by both heads.
    Returns (q[2,64,20], k[2,64,20], v[64,3], frame[64], pixel[64]) in float64.
    """
    T, P = 4, 16
    n, d = T * P, T + P
    rng = np.random.default_rng(7)
    frame = np.arange(n) // P
    pixel = np.arange(n) % P
    q = np.zeros((2, n, d))
    rows = np.arange(n)
    q[0, rows, frame] = 6.0
    q[1, rows, T + pixel] = 6.0
    q = q + rng.normal(0.0, 0.15, size=(2, n, d))
    v = rng.normal(size=(n, 3))
    return q, q.copy(), v, frame, pixel
