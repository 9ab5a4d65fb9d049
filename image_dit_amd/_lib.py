"""ctypes binding of libsparse_attn.so: same names as the C ABI, argument marshalling only.

Every computation happens in the HIP library.  If the library is missing the
functions raise; there is no fallback path.
"""

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint8, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsparse_attn.so")

SA_OK = 0
SA_ERR_INVALID_ARGUMENT = -1
SA_ERR_UNSUPPORTED = -2
SA_ERR_CAPACITY = -3
SA_ERR_EMPTY_ROW = -4
SA_ERR_HIP = -5
SA_BF16 = 0
SA_F32 = 1
SA_ORDER_IDENTITY = 0
SA_ORDER_WINDOW = 1
SA_ORDER_HILBERT = 2
SA_PV_GROUP_ROWS = 32
SA_MAX_KEY_BLOCKS = 2048
SA_NOALLOC_SCRATCH_BYTES = 64 << 20
SA_FP8_KEY_ROWS = 64

EXPORTS = ("sa_status_string", "sa_plan_permutation", "sa_permute", "sa_unpermute",
           "sa_predict_workspace_bytes", "sa_predict_workspace_offsets", "sa_predict_mask",
           "sa_sparse_attn_fwd", "sa_predict_mask_gather", "sa_sparse_attn_fwd_gather",
           "sa_plan_tile_window", "sa_predict_mask_ex", "sa_predict_mask_gather_noalloc",
           "sa_quantize_fp8", "sa_sparse_attn_fwd_qk8", "sa_predict_mask_qk8")


class SaLayout(ctypes.Structure):
    _fields_ = [("n_tokens", c_int64), ("order", c_int32), ("t", c_int32), ("h", c_int32),
                ("w", c_int32), ("win_t", c_int32), ("win_h", c_int32), ("win_w", c_int32),
                ("txt_len", c_int32), ("first_frame_sink", c_int32)]


class SaMaskParams(ctypes.Structure):
    _fields_ = [("B", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("D", c_int32), ("N", c_int64),
                ("block_q", c_int32), ("block_k", c_int32), ("causal", c_int32),
                ("sink_rows", c_int32), ("window", c_int64), ("sink_front", c_int64),
                ("sink_back", c_int64), ("tau", c_double), ("theta", c_double),
                ("sparsity", c_double), ("scale", c_float), ("n_keys", c_int32)]


class SaAttnParams(ctypes.Structure):
    _fields_ = [("B", c_int32), ("Hq", c_int32), ("Hkv", c_int32), ("D", c_int32), ("Dv", c_int32),
                ("block_q", c_int32), ("block_k", c_int32), ("causal", c_int32), ("N", c_int64),
                ("lam", c_float), ("scale", c_float), ("col_cap", c_int64), ("n_keys", c_int64)]


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {sa_status_string(code)} ({code})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m image_dit_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    L.sa_status_string.argtypes = [c_int]
    L.sa_status_string.restype = c_char_p
    L.sa_plan_permutation.argtypes = [POINTER(SaLayout), POINTER(c_int32), c_int64]
    L.sa_plan_permutation.restype = c_int
    L.sa_permute.argtypes = [c_void_p, c_int, c_void_p, c_void_p, c_int32, c_int32, c_int64, c_int32, c_void_p]
    L.sa_permute.restype = c_int
    L.sa_unpermute.argtypes = [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int64, c_int32, c_void_p]
    L.sa_unpermute.restype = c_int
    L.sa_predict_workspace_bytes.argtypes = [POINTER(SaMaskParams)]
    L.sa_predict_workspace_bytes.restype = c_size_t
    L.sa_predict_workspace_offsets.argtypes = [POINTER(SaMaskParams), POINTER(c_int64)]
    L.sa_predict_workspace_offsets.restype = c_int
    L.sa_predict_mask.argtypes = [c_void_p, c_void_p, POINTER(SaMaskParams), c_void_p, c_size_t, c_void_p,
                                  c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.sa_predict_mask.restype = c_int
    L.sa_sparse_attn_fwd.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(SaAttnParams),
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    L.sa_sparse_attn_fwd.restype = c_int
    L.sa_predict_mask_gather.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(SaMaskParams), c_void_p, c_size_t,
                                         c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p]
    L.sa_predict_mask_gather.restype = c_int
    L.sa_sparse_attn_fwd_gather.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                            POINTER(SaAttnParams), c_void_p, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p]
    L.sa_sparse_attn_fwd_gather.restype = c_int
    L.sa_plan_tile_window.argtypes = [POINTER(SaLayout)] + [c_int32] * 8 + [POINTER(c_uint8), c_int64, c_int64]
    L.sa_plan_tile_window.restype = c_int
    L.sa_predict_mask_ex.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, POINTER(SaMaskParams), c_void_p,
                                     c_size_t, c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p]
    L.sa_predict_mask_ex.restype = c_int
    L.sa_predict_mask_gather_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(SaMaskParams), c_void_p,
                                                 c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                                 c_void_p]
    L.sa_predict_mask_gather_noalloc.restype = c_int
    L.sa_quantize_fp8.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_int64, c_int32, c_int32, c_void_p,
                                  c_void_p, c_void_p]
    L.sa_quantize_fp8.restype = c_int
    L.sa_sparse_attn_fwd_qk8.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                         POINTER(SaAttnParams), c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]
    L.sa_sparse_attn_fwd_qk8.restype = c_int
    L.sa_predict_mask_qk8.argtypes = [c_void_p, c_void_p, c_void_p, POINTER(SaMaskParams), c_void_p, c_size_t,
                                      c_void_p, c_void_p, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p]
    L.sa_predict_mask_qk8.restype = c_int
    _lib = L
    return L


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _need(*specs):
    """Refuse tensors the C ABI would misread.  Each spec is (tensor, name, dtype names,
    optional): every element type is checked first, then that every tensor is
    contiguous and in device memory."""
    import torch
    for t, name, dts, optional in specs:
        if t is None:
            if not optional:
                raise ValueError(f"{name} is required")
            continue
        want = tuple(getattr(torch, d) for d in dts)
        if t.dtype not in want:
            raise TypeError(f"{name}: dtype {t.dtype} not accepted (expected {' or '.join(dts)})")
    for t, name, _, _ in specs:
        if t is None:
            continue
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _a(t, name, *dts, optional=False):
    return (t, name, dts, optional)


def _stream(stream):
    if stream is None:
        import torch
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def _check(code: int, where: str):
    if code != SA_OK:
        raise SparseAttnError(code, where)


def sa_status_string(code: int) -> str:
    return lib().sa_status_string(code).decode()


def make_layout(n_tokens, order=SA_ORDER_IDENTITY, latent=(1, 1, 1), window=(1, 1, 1), txt_len=0,
                first_frame_sink=False) -> SaLayout:
    t, h, w = latent
    wt, wh, ww = window
    return SaLayout(n_tokens, order, t, h, w, wt, wh, ww, txt_len, int(first_frame_sink))


def sa_plan_permutation(layout: SaLayout) -> np.ndarray:
    """Host-only planner: returns perm (int32 [N]) with perm[i] = original index at position i."""
    perm = np.empty(layout.n_tokens, dtype=np.int32)
    code = lib().sa_plan_permutation(ctypes.byref(layout), perm.ctypes.data_as(POINTER(c_int32)),
                                     c_int64(layout.n_tokens))
    _check(code, "sa_plan_permutation")
    return perm


def sa_plan_tile_window(layout: SaLayout, tile, radius, block_q: int, block_k: int) -> np.ndarray:
    """Host-only: the 3-D tile-window block pattern (uint8 [n_qb, n_kb]) in the order
    sa_plan_permutation gives for the layout."""
    n = int(layout.n_tokens)
    n_qb, n_kb = -(-n // block_q), -(-n // block_k)
    out = np.zeros((n_qb, n_kb), dtype=np.uint8)
    code = lib().sa_plan_tile_window(ctypes.byref(layout), *(int(x) for x in tile), *(int(x) for x in radius),
                                     block_q, block_k, out.ctypes.data_as(POINTER(c_uint8)), n_qb, n_kb)
    _check(code, "sa_plan_tile_window")
    return out


def sa_permute(x, y, perm, stream=None):
    """y[b,h,i,:] = bf16(x[b,h,perm[i],:]); x bf16 or fp32 [B,H,N,D]; y bf16 [B,H,N,D]."""
    import torch
    _need(_a(x, "x", "float32", "bfloat16"), _a(y, "y", "bfloat16"), _a(perm, "perm", "int32"))
    if tuple(y.shape) != tuple(x.shape) or perm.numel() != x.shape[2]:
        raise ValueError("sa_permute: y must have x's shape and perm N entries")
    B, H, N, D = x.shape
    dt = SA_F32 if x.dtype == torch.float32 else SA_BF16
    code = lib().sa_permute(_ptr(x), dt, _ptr(y), _ptr(perm), B, H, N, D, _stream(stream))
    _check(code, "sa_permute")


def sa_unpermute(y, x, perm, stream=None):
    """x[b,h,perm[i],:] = y[b,h,i,:]; fp32 [B,H,N,Dv]."""
    _need(_a(y, "y", "float32"), _a(x, "x", "float32"), _a(perm, "perm", "int32"))
    if tuple(y.shape) != tuple(x.shape) or perm.numel() != y.shape[2]:
        raise ValueError("sa_unpermute: x must have y's shape and perm N entries")
    B, H, N, Dv = y.shape
    code = lib().sa_unpermute(_ptr(y), _ptr(x), _ptr(perm), B, H, N, Dv, _stream(stream))
    _check(code, "sa_unpermute")


def make_mask_params(B, Hq, Hkv, N, D, block_q, block_k, causal=False, window=0, sink_front=0,
                     sink_back=0, tau=None, theta=None, sparsity=None, scale=0.0,
                     sink_rows=0, n_keys=0) -> SaMaskParams:
    return SaMaskParams(B, Hq, Hkv, D, N, block_q, block_k, int(causal), sink_rows, window, sink_front,
                        sink_back, -1.0 if tau is None else tau, 0.0 if theta is None else theta,
                        -1.0 if sparsity is None else sparsity, scale, n_keys)


def make_attn_params(B, Hq, Hkv, N, D, block_q, block_k, causal=False, lam=None, scale=0.0,
                     col_cap=0, n_keys=0) -> SaAttnParams:
    return SaAttnParams(B, Hq, Hkv, D, D, block_q, block_k, int(causal), N,
                        float("-inf") if lam is None else lam, scale, col_cap, n_keys)


def sa_predict_workspace_bytes(p: SaMaskParams) -> int:
    return int(lib().sa_predict_workspace_bytes(ctypes.byref(p)))


def sa_predict_workspace_offsets(p: SaMaskParams):
    off = (c_int64 * 6)()
    _check(lib().sa_predict_workspace_offsets(ctypes.byref(p), off), "sa_predict_workspace_offsets")
    return list(off)


def sa_predict_mask(q, k, p: SaMaskParams, ws, row_ptr, col_idx, dev_status, mask_out=None, sim_q=None,
                    sim_k=None, stream=None):
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(ws, "ws", "uint8"),
          _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"), _a(dev_status, "dev_status", "int32"),
          _a(mask_out, "mask_out", "uint8", optional=True), _a(sim_q, "sim_q", "float32", optional=True),
          _a(sim_k, "sim_k", "float32", optional=True))
    code = lib().sa_predict_mask(_ptr(q), _ptr(k), ctypes.byref(p), _ptr(ws), ws.numel() * ws.element_size(),
                                 _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(mask_out), _ptr(sim_q),
                                 _ptr(sim_k), _ptr(dev_status), _stream(stream))
    _check(code, "sa_predict_mask")


def sa_sparse_attn_fwd(q, k, v, o, p: SaAttnParams, row_ptr, col_idx, dev_status, pv_skip=None,
                       counters=None, stream=None):
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(v, "v", "bfloat16"), _a(o, "o", "float32"),
          _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"), _a(dev_status, "dev_status", "int32"),
          _a(pv_skip, "pv_skip", "uint8", optional=True), _a(counters, "counters", "int64", optional=True))
    code = lib().sa_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), ctypes.byref(p), _ptr(row_ptr),
                                    _ptr(col_idx), _ptr(pv_skip), _ptr(counters), _ptr(dev_status),
                                    _stream(stream))
    _check(code, "sa_sparse_attn_fwd")


def sa_predict_mask_gather(q, k, perm, p: SaMaskParams, ws, row_ptr, col_idx, dev_status, mask_out=None,
                           sim_q=None, sim_k=None, stream=None):
    """sa_predict_mask on q[:, :, perm], k[:, :, perm] without materialising them (q, k bf16, original order)."""
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(perm, "perm", "int32"), _a(ws, "ws", "uint8"),
          _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"), _a(dev_status, "dev_status", "int32"),
          _a(mask_out, "mask_out", "uint8", optional=True), _a(sim_q, "sim_q", "float32", optional=True),
          _a(sim_k, "sim_k", "float32", optional=True))
    code = lib().sa_predict_mask_gather(_ptr(q), _ptr(k), _ptr(perm), ctypes.byref(p), _ptr(ws),
                                        ws.numel() * ws.element_size(), _ptr(row_ptr), _ptr(col_idx),
                                        col_idx.numel(), _ptr(mask_out), _ptr(sim_q), _ptr(sim_k),
                                        _ptr(dev_status), _stream(stream))
    _check(code, "sa_predict_mask_gather")


def sa_predict_mask_ex(q, k, perm, forced, p: SaMaskParams, ws, row_ptr, col_idx, dev_status, mask_out=None,
                       sim_q=None, sim_k=None, stream=None):
    """sa_predict_mask with an optional permutation (None: q, k already reordered) and an
    optional forced block pattern (device uint8 [n_qb, n_kb], shared by all heads)."""
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(perm, "perm", "int32", optional=True), _a(ws, "ws", "uint8"),
          _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"), _a(dev_status, "dev_status", "int32"),
          _a(mask_out, "mask_out", "uint8", optional=True), _a(sim_q, "sim_q", "float32", optional=True),
          _a(sim_k, "sim_k", "float32", optional=True), _a(forced, "forced", "uint8", optional=True))
    code = lib().sa_predict_mask_ex(_ptr(q), _ptr(k), _ptr(perm), _ptr(forced), ctypes.byref(p), _ptr(ws),
                                    ws.numel() * ws.element_size(), _ptr(row_ptr), _ptr(col_idx),
                                    col_idx.numel(), _ptr(mask_out), _ptr(sim_q), _ptr(sim_k),
                                    _ptr(dev_status), _stream(stream))
    _check(code, "sa_predict_mask_ex")


def sa_sparse_attn_fwd_gather(q, k, v, perm, o, p: SaAttnParams, row_ptr, col_idx, dev_status, pv_skip=None,
                              counters=None, stream=None):
    """sa_sparse_attn_fwd on the reordered q, k, v, with o written back in the original order."""
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(v, "v", "bfloat16"), _a(perm, "perm", "int32"), _a(o, "o", "float32"),
          _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"), _a(dev_status, "dev_status", "int32"),
          _a(pv_skip, "pv_skip", "uint8", optional=True), _a(counters, "counters", "int64", optional=True))
    code = lib().sa_sparse_attn_fwd_gather(_ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(o), ctypes.byref(p),
                                           _ptr(row_ptr), _ptr(col_idx), _ptr(pv_skip), _ptr(counters),
                                           _ptr(dev_status), _stream(stream))
    _check(code, "sa_sparse_attn_fwd_gather")


def sa_predict_mask_gather_noalloc(q, k, perm, p: SaMaskParams, row_ptr, col_idx, dev_status, mask_out=None,
                                   sim_q=None, sim_k=None, stream=None):
    """sa_predict_mask_gather with the library's fixed per-GPU workspace (allocates nothing)."""
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(perm, "perm", "int32"),
          _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"), _a(dev_status, "dev_status", "int32"),
          _a(mask_out, "mask_out", "uint8", optional=True), _a(sim_q, "sim_q", "float32", optional=True),
          _a(sim_k, "sim_k", "float32", optional=True))
    code = lib().sa_predict_mask_gather_noalloc(_ptr(q), _ptr(k), _ptr(perm), ctypes.byref(p), _ptr(row_ptr),
                                                _ptr(col_idx), col_idx.numel(), _ptr(mask_out), _ptr(sim_q),
                                                _ptr(sim_k), _ptr(dev_status), _stream(stream))
    _check(code, "sa_predict_mask_gather_noalloc")


def sa_quantize_fp8(x, perm, block, codes, scales, stream=None):
    """Per-block E4M3 codes and scales of x (bf16 [B, H, N, D], original order); blocks of
    `block` rows of the order perm gives (None: identity)."""
    _need(_a(x, "x", "bfloat16"), _a(perm, "perm", "int32", optional=True), _a(codes, "codes", "uint8"),
          _a(scales, "scales", "float32"))
    if x.dim() != 4 or tuple(codes.shape) != tuple(x.shape):
        raise ValueError("x must be [B, H, N, D] and codes of the same shape")
    B, H, N, D = x.shape
    nb = -(-N // block)
    if scales.numel() != B * H * nb:
        raise ValueError(f"scales must hold B*H*ceil(N/block) = {B * H * nb} entries")
    code = lib().sa_quantize_fp8(_ptr(x), _ptr(perm), B, H, N, D, block, _ptr(codes), _ptr(scales),
                                 _stream(stream))
    _check(code, "sa_quantize_fp8")


def sa_sparse_attn_fwd_qk8(q8, q_scale, k8, k_scale, v, perm, o, p: SaAttnParams, row_ptr, col_idx, dev_status,
                           pv_skip=None, counters=None, stream=None):
    """sparse attention with FP8 QK operands (codes and scales from sa_quantize_fp8); perm None:
    everything in the reordered order, else as sa_sparse_attn_fwd_gather."""
    _need(_a(q8, "q8", "uint8"), _a(q_scale, "q_scale", "float32"), _a(k8, "k8", "uint8"),
          _a(k_scale, "k_scale", "float32"), _a(v, "v", "bfloat16"), _a(perm, "perm", "int32", optional=True),
          _a(o, "o", "float32"), _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"),
          _a(dev_status, "dev_status", "int32"), _a(pv_skip, "pv_skip", "uint8", optional=True),
          _a(counters, "counters", "int64", optional=True))
    code = lib().sa_sparse_attn_fwd_qk8(_ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(v), _ptr(perm),
                                        _ptr(o), ctypes.byref(p), _ptr(row_ptr), _ptr(col_idx), _ptr(pv_skip),
                                        _ptr(counters), _ptr(dev_status), _stream(stream))
    _check(code, "sa_sparse_attn_fwd_qk8")


def sa_predict_mask_qk8(q, k, perm, p: SaMaskParams, ws, row_ptr, col_idx, q8, q_scale, k8, k_scale, dev_status,
                        stream=None):
    """sa_predict_mask_ex (perm None: q, k already reordered) that also writes the E4M3 codes and
    block scales sa_quantize_fp8 would write for q and k."""
    _need(_a(q, "q", "bfloat16"), _a(k, "k", "bfloat16"), _a(perm, "perm", "int32", optional=True),
          _a(ws, "ws", "uint8"), _a(row_ptr, "row_ptr", "int32"), _a(col_idx, "col_idx", "int32"),
          _a(q8, "q8", "uint8"), _a(q_scale, "q_scale", "float32"), _a(k8, "k8", "uint8"),
          _a(k_scale, "k_scale", "float32"), _a(dev_status, "dev_status", "int32"))
    if tuple(q8.shape) != tuple(q.shape) or tuple(k8.shape) != tuple(k.shape):
        raise ValueError("q8 and k8 must have the shapes of q and k")
    code = lib().sa_predict_mask_qk8(_ptr(q), _ptr(k), _ptr(perm), ctypes.byref(p), _ptr(ws),
                                     ws.numel() * ws.element_size(), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(),
                                     _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale), _ptr(dev_status),
                                     _stream(stream))
    _check(code, "sa_predict_mask_qk8")
