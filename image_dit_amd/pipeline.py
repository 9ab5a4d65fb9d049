"""One call of the whole path: reorder -> predict mask -> sparse attention -> inverse reorder.

Two equivalent forms: ``run`` materialises the reordered q, k, v (three
permute calls), predicts, attends and undoes the reorder on O; ``run_fused``
passes the permutation to the gather entry points instead, which read q, k, v
in the original order and write O there, with bit-identical results.
Torch only allocates device memory and supplies the stream; every step runs
in the HIP library through the C ABI (``_lib``).
"""

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

from . import _lib as L


@dataclass
class PathConfig:
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    block_q: int
    block_k: int
    order: int = L.SA_ORDER_IDENTITY
    latent: Tuple[int, int, int] = (1, 1, 1)
    window: Tuple[int, int, int] = (1, 1, 1)
    txt_len: int = 0
    first_frame_sink: bool = False
    causal: bool = False
    window_tokens: int = 0
    sink_front: int = 0
    sink_rows: int = 0
    sink_back: int = 0
    tau: Optional[float] = None
    theta: Optional[float] = None
    sparsity: Optional[float] = None
    lam: Optional[float] = None
    scale: float = 0.0
    # keys and values on their own latent grid (MindIE-SD latent_shape_k); None = the queries'
    latent_k: Optional[Tuple[int, int, int]] = None
    txt_len_k: Optional[int] = None

    @property
    def N_k(self):
        if self.latent_k is None and self.txt_len_k is None:
            return self.N
        t, h, w = self.latent if self.latent_k is None else self.latent_k
        return (self.txt_len if self.txt_len_k is None else self.txt_len_k) + t * h * w

    @property
    def n_qb(self):
        return -(-self.N // self.block_q)

    @property
    def n_kb(self):
        return -(-self.N_k // self.block_k)

    @property
    def rows(self):
        return self.B * self.Hq * self.n_qb

    def mask_params(self):
        return L.make_mask_params(self.B, self.Hq, self.Hkv, self.N, self.D, self.block_q, self.block_k,
                                  self.causal, self.window_tokens, self.sink_front, self.sink_back,
                                  self.tau, self.theta, self.sparsity, self.scale, self.sink_rows,
                                  0 if self.N_k == self.N else self.N_k)

    def attn_params(self, col_cap=0):
        return L.make_attn_params(self.B, self.Hq, self.Hkv, self.N, self.D, self.block_q, self.block_k,
                                  self.causal, self.lam, self.scale, col_cap, 0 if self.N_k == self.N else self.N_k)

    def layout(self):
        return L.make_layout(self.N, self.order, self.latent, self.window, self.txt_len, self.first_frame_sink)

    def layout_k(self):
        """Token layout of the keys and values (the queries' unless latent_k / txt_len_k are set)."""
        if self.N_k == self.N and self.latent_k is None and self.txt_len_k is None:
            return self.layout()
        return L.make_layout(self.N_k, self.order, self.latent if self.latent_k is None else self.latent_k,
                             self.window, self.txt_len if self.txt_len_k is None else self.txt_len_k,
                             self.first_frame_sink)


def config_from_workload(w, sparsity="default") -> PathConfig:
    """PathConfig from a workloads.Workload (duck-typed: no import of the oracle side)."""
    return PathConfig(B=w.B, Hq=w.Hq, Hkv=w.Hkv, N=w.N, D=w.D, block_q=w.block_q, block_k=w.block_k,
                      order=w.order, latent=w.latent, window=w.window, txt_len=w.txt_len,
                      first_frame_sink=w.first_frame_sink, causal=w.causal, window_tokens=w.window_tokens,
                      sink_front=w.sink_front, sink_back=w.sink_back, sink_rows=getattr(w, "sink_rows", 0),
                      tau=w.tau, theta=w.theta,
                      sparsity=w.sparsity if sparsity == "default" else sparsity, lam=w.lam,
                      latent_k=getattr(w, "latent_k", None), txt_len_k=getattr(w, "txt_len_k", None))


class SparseAttentionPath:
    """Owns the device buffers of one workload shape and runs the four entry points."""

    def __init__(self, cfg: PathConfig, device="cuda", col_cap: Optional[int] = None, want_skip=True,
                 materialize=True, forced: Optional[np.ndarray] = None, qk_fp8=False):
        """forced: optional host block pattern [n_qb, n_kb] (nonzero = key block always kept by
        that query block, in every head), e.g. from ``sa_plan_tile_window``.
        qk_fp8: take the QK products on per-block E4M3 codes instead of bf16: the gather form
        writes them during the mask prediction (sa_predict_mask_qk8) and the attention reads
        them (sa_sparse_attn_fwd_qk8); the materialising form quantizes the reordered copies
        (sa_quantize_fp8) before the attention."""
        import torch

        self.cfg = cfg
        self.device = device
        self.perm_host = L.sa_plan_permutation(cfg.layout())
        self.perm = torch.from_numpy(self.perm_host).to(device)
        # keys on their own grid get their own reorder (materialising form only: the gather
        # entry points take one permutation)
        self.keys_differ = cfg.N_k != cfg.N or cfg.latent_k is not None or cfg.txt_len_k is not None
        if self.keys_differ and not materialize:
            raise ValueError("keys on another latent grid need the materialising form")
        self.perm_k_host = L.sa_plan_permutation(cfg.layout_k()) if self.keys_differ else self.perm_host
        self.perm_k = torch.from_numpy(self.perm_k_host).to(device) if self.keys_differ else self.perm
        bf = torch.bfloat16
        B, Hq, Hkv, N, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.D
        Nk = cfg.N_k
        # reordered copies (only for the materialising form)
        self.qp = torch.empty((B, Hq, N, D), dtype=bf, device=device) if materialize else None
        self.kp = torch.empty((B, Hkv, Nk, D), dtype=bf, device=device) if materialize else None
        self.vp = torch.empty((B, Hkv, Nk, D), dtype=bf, device=device) if materialize else None
        self.mp = cfg.mask_params()
        ws_bytes = L.sa_predict_workspace_bytes(self.mp)
        if ws_bytes == 0:
            raise L.SparseAttnError(L.SA_ERR_INVALID_ARGUMENT, "sa_predict_workspace_bytes")
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        self.ws_off = L.sa_predict_workspace_offsets(self.mp)
        self.col_cap = cfg.rows * cfg.n_kb if col_cap is None else col_cap
        self.ap = cfg.attn_params(self.col_cap)
        self.row_ptr = torch.empty(cfg.rows + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(max(self.col_cap, 1), dtype=torch.int32, device=device)
        self.status = torch.zeros(2, dtype=torch.int32, device=device)
        self.groups = -(-cfg.block_q // L.SA_PV_GROUP_ROWS)
        self.pv_skip = (torch.empty(max(self.col_cap, 1) * self.groups, dtype=torch.uint8, device=device)
                        if want_skip else None)
        self.counters = torch.zeros(3, dtype=torch.int64, device=device)
        self.o_perm = torch.empty((B, Hq, N, D), dtype=torch.float32, device=device) if materialize else None
        self.o = torch.empty((B, Hq, N, D), dtype=torch.float32, device=device)
        self.qk_fp8 = qk_fp8
        self._quantized = False  # the codes of the last predict_gather are in place
        if qk_fp8:
            u8 = torch.uint8
            self.q8 = torch.empty((B, Hq, N, D), dtype=u8, device=device)
            self.k8 = torch.empty((B, Hkv, Nk, D), dtype=u8, device=device)
            self.q_scale = torch.empty(B * Hq * cfg.n_qb, dtype=torch.float32, device=device)
            self.k_scale = torch.empty(B * Hkv * -(-Nk // L.SA_FP8_KEY_ROWS), dtype=torch.float32, device=device)
        self.forced = None
        if forced is not None:
            forced = np.asarray(forced)
            if forced.shape != (cfg.n_qb, cfg.n_kb):
                raise ValueError(f"forced pattern must be [{cfg.n_qb}, {cfg.n_kb}]")
            self.forced = torch.from_numpy(np.ascontiguousarray(forced != 0).astype(np.uint8)).to(device)

    # --- the four steps (each one C-ABI call, or three for the permute) ---
    def permute(self, q, k, v, stream=None):
        L.sa_permute(q, self.qp, self.perm, stream)
        L.sa_permute(k, self.kp, self.perm_k, stream)
        L.sa_permute(v, self.vp, self.perm_k, stream)

    def _cols(self):
        return self.col_idx[:self.col_cap] if self.col_cap > 0 else self.col_idx[:0]

    def predict(self, mask_out=None, sim_q=None, sim_k=None, stream=None):
        if self.forced is not None:
            L.sa_predict_mask_ex(self.qp, self.kp, None, self.forced, self.mp, self.ws, self.row_ptr, self._cols(),
                                 self.status[0:1], mask_out, sim_q, sim_k, stream)
            return
        L.sa_predict_mask(self.qp, self.kp, self.mp, self.ws, self.row_ptr, self._cols(), self.status[0:1],
                          mask_out, sim_q, sim_k, stream)

    def quantize(self, q, k, perm=None, perm_k=None, stream=None):
        """E4M3 codes and block scales of q (blocks of block_q rows) and k (64-row blocks)."""
        L.sa_quantize_fp8(q, perm, self.cfg.block_q, self.q8, self.q_scale, stream)
        L.sa_quantize_fp8(k, perm_k, L.SA_FP8_KEY_ROWS, self.k8, self.k_scale, stream)

    def attend(self, stream=None):
        if self.qk_fp8:
            self.quantize(self.qp, self.kp, stream=stream)
            self.attend_qk8(stream)
            return
        L.sa_sparse_attn_fwd(self.qp, self.kp, self.vp, self.o_perm, self.ap, self.row_ptr, self.col_idx,
                             self.status[1:2], self.pv_skip, self.counters, stream)

    def attend_qk8(self, stream=None):
        """The attention of attend on the codes of the last quantize call (FP8 QK path)."""
        L.sa_sparse_attn_fwd_qk8(self.q8, self.q_scale, self.k8, self.k_scale, self.vp, None, self.o_perm,
                                 self.ap, self.row_ptr, self.col_idx, self.status[1:2], self.pv_skip,
                                 self.counters, stream)

    def unpermute(self, stream=None):
        L.sa_unpermute(self.o_perm, self.o, self.perm, stream)

    def run(self, q, k, v, stream=None):
        self.permute(q, k, v, stream)
        self.predict(stream=stream)
        self.attend(stream)
        self.unpermute(stream)
        return self.o

    # --- the fused form: the reorder is an index map inside the two kernels' loads ---
    def predict_gather(self, q, k, mask_out=None, sim_q=None, sim_k=None, stream=None):
        if self.qk_fp8 and self.forced is None and mask_out is None and sim_q is None and sim_k is None:
            # the prediction's pass over q and k also writes their E4M3 codes
            L.sa_predict_mask_qk8(q, k, self.perm, self.mp, self.ws, self.row_ptr, self._cols(), self.q8,
                                  self.q_scale, self.k8, self.k_scale, self.status[0:1], stream)
            self._quantized = True
            return
        if self.forced is not None:
            L.sa_predict_mask_ex(q, k, self.perm, self.forced, self.mp, self.ws, self.row_ptr, self._cols(),
                                 self.status[0:1], mask_out, sim_q, sim_k, stream)
            return
        L.sa_predict_mask_gather(q, k, self.perm, self.mp, self.ws, self.row_ptr, self._cols(),
                                 self.status[0:1], mask_out, sim_q, sim_k, stream)

    def attend_gather(self, q, k, v, stream=None):
        if self.qk_fp8:
            if not self._quantized:  # codes not written by the last predict_gather
                self.quantize(q, k, self.perm, self.perm, stream)
            self._quantized = False
            self.attend_qk8_gather(v, stream)
            return
        L.sa_sparse_attn_fwd_gather(q, k, v, self.perm, self.o, self.ap, self.row_ptr, self.col_idx,
                                    self.status[1:2], self.pv_skip, self.counters, stream)

    def attend_qk8_gather(self, v, stream=None):
        """The attention of attend_gather on the codes of the last quantize call (FP8 QK path)."""
        L.sa_sparse_attn_fwd_qk8(self.q8, self.q_scale, self.k8, self.k_scale, v, self.perm, self.o, self.ap,
                                 self.row_ptr, self.col_idx, self.status[1:2], self.pv_skip, self.counters, stream)

    def run_fused(self, q, k, v, stream=None):
        """q, k, v: bf16 in the original token order; returns O (fp32) in the original order."""
        self.predict_gather(q, k, stream=stream)
        self.attend_gather(q, k, v, stream)
        return self.o

    # --- inspection helpers (host copies, for tests and reports) ---
    def workspace_view(self, idx, dtype, shape):
        import torch
        start = self.ws_off[idx]
        nbytes = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
        return self.ws[start:start + nbytes].view(dtype).view(*shape)

    def csr_host(self):
        rp = self.row_ptr.cpu().numpy().astype(np.int64)
        nnz = int(rp[-1])
        ci = self.col_idx[:min(nnz, self.col_cap)].cpu().numpy().astype(np.int64)
        return rp, ci

    def statuses(self):
        s = self.status.cpu().numpy()
        return int(s[0]), int(s[1])
