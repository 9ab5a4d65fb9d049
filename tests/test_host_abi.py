"""Host-side checks of the C-ABI library (no GPU needed).

* the library loads and exports every function include/sparse_attn.h declares;
* the C++ planner (sa_plan_permutation) matches the oracle's independent
  planner bit for bit;
* invalid arguments are rejected synchronously, before any HIP call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import image_dit_amd as sa
from oracle import layout as Lay
from workloads import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sa.LIB_PATH), reason="library not built")


def _declared_functions():
    text = open(HEADER, encoding="utf8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(declared) == set(sa.EXPORTS)
    L = sa.lib()
    for name in declared:
        assert hasattr(L, name), name
    nm = os.popen(f"nm -D --defined-only {sa.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert sa.sa_status_string(code) and sa.sa_status_string(code) != "unknown status"
    assert sa.sa_status_string(17) == "unknown status"


def _layouts():
    out = []
    for w in CONFIGS.values():
        out.append((w.N, w.order, w.latent, w.window, w.txt_len, w.first_frame_sink))
    rng = np.random.default_rng(0)
    for _ in range(40):
        t, h, w = (int(x) for x in rng.integers(1, 9, size=3))
        txt = int(rng.integers(0, 5))
        win = tuple(int(x) for x in rng.integers(1, 5, size=3))
        sink = bool(rng.integers(0, 2))
        order = int(rng.integers(1, 3))
        out.append((txt + t * h * w, order, (t, h, w), win, txt, sink))
    out.append((4 * 4 * 4, Lay.ORDER_WINDOW, (4, 4, 4), (4, 1, 1), 0, False))
    out.append((1 * 1 * 1, Lay.ORDER_HILBERT, (1, 1, 1), (1, 1, 1), 0, False))
    out.append((17 * 1 * 40 + 3, Lay.ORDER_HILBERT, (17, 1, 40), (1, 1, 1), 3, True))
    return out


@pytest.mark.parametrize("case", range(len(_layouts())))
def test_planner_matches_oracle(case):
    N, order, latent, window, txt, sink = _layouts()[case]
    got = sa.sa_plan_permutation(sa.make_layout(N, order, latent, window, txt, sink))
    want = Lay.plan_permutation(N, order, latent, window, txt, sink)
    assert got.dtype == np.int32
    assert np.array_equal(got.astype(np.int64), want)


def test_planner_rejects_bad_layouts():
    bad = [sa.make_layout(10, sa.SA_ORDER_WINDOW, (2, 2, 2), (1, 1, 1), 1),   # 1 + 8 != 10
           sa.make_layout(8, sa.SA_ORDER_WINDOW, (2, 2, 2), (0, 1, 1)),        # zero window
           sa.make_layout(8, 7, (2, 2, 2)),                                    # unknown order
           sa.make_layout(0, sa.SA_ORDER_IDENTITY)]
    for lay in bad:
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sa_plan_permutation(lay)
        assert e.value.code == sa.SA_ERR_INVALID_ARGUMENT
    perm = np.empty(8, dtype=np.int32)
    lay = sa.make_layout(8, sa.SA_ORDER_IDENTITY)
    code = sa.lib().sa_plan_permutation(ctypes.byref(lay), perm.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 7)
    assert code == sa.SA_ERR_INVALID_ARGUMENT


TILE_CASES = [
    # (N, order, latent, window, txt, sink), tile, radius, block_q, block_k
    ((16, sa.SA_ORDER_IDENTITY, (1, 1, 16), (1, 1, 1), 0, False), (1, 1, 4), (0, 0, 1), 4, 4),
    ((2 + 3 * 2 * 4, sa.SA_ORDER_WINDOW, (3, 2, 4), (1, 2, 2), 2, True), (1, 2, 2), (0, 0, 1), 4, 4),
    ((20 + 9 * 16 * 24, sa.SA_ORDER_WINDOW, (9, 16, 24), (4, 8, 4), 20, True), (4, 8, 4), (1, 1, 1), 128, 128),
    ((9 * 16 * 24, sa.SA_ORDER_WINDOW, (9, 16, 24), (4, 8, 4), 0, False), (4, 8, 4), (0, 1, 2), 128, 64),
    ((6 * 10 * 21, sa.SA_ORDER_HILBERT, (6, 10, 21), (1, 1, 1), 0, False), (2, 4, 4), (1, 1, 1), 128, 64),
    ((777, sa.SA_ORDER_IDENTITY, (1, 1, 777), (1, 1, 1), 0, False), (1, 1, 64), (0, 0, 2), 128, 64),
]


@pytest.mark.parametrize("case", range(len(TILE_CASES)))
def test_tile_window_planner_matches_oracle(case):
    (N, order, latent, window, txt, sink), tile, radius, bq, bk = TILE_CASES[case]
    got = sa.sa_plan_tile_window(sa.make_layout(N, order, latent, window, txt, sink), tile, radius, bq, bk)
    want = Lay.plan_tile_window(N, order, latent, window, txt, sink, tile, radius, bq, bk)
    assert got.shape == want.shape
    assert np.array_equal(got.astype(bool), want)


def test_tile_window_planner_rejects_bad_arguments():
    lay = sa.make_layout(16, sa.SA_ORDER_IDENTITY, (1, 1, 16))
    for tile, radius in (((0, 1, 4), (0, 0, 1)), ((1, 1, 4), (0, -1, 1))):
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sa_plan_tile_window(lay, tile, radius, 4, 4)
        assert e.value.code == sa.SA_ERR_INVALID_ARGUMENT
    with pytest.raises(sa.SparseAttnError):  # the latent must hold every token
        sa.sa_plan_tile_window(sa.make_layout(16, sa.SA_ORDER_IDENTITY, (1, 1, 8)), (1, 1, 4), (0, 0, 1), 4, 4)
    out = np.zeros((4, 4), dtype=np.uint8)
    code = sa.lib().sa_plan_tile_window(ctypes.byref(lay), 1, 1, 4, 0, 0, 1, 4, 4,
                                        out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), 4, 3)  # wrong n_kb
    assert code == sa.SA_ERR_INVALID_ARGUMENT


# -------------------------------------------------------------- validation (no device work)

FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every case below fails validation


def _mask_params(**kw):
    base = dict(B=1, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64, tau=0.9)
    base.update(kw)
    return sa.make_mask_params(**base)


def _predict_code(p, ws_bytes=1 << 30, **ptrs):
    args = dict(q=FAKE, k=FAKE, ws=FAKE, row_ptr=FAKE, col_idx=FAKE, status=FAKE)
    args.update(ptrs)
    return sa.lib().sa_predict_mask(args["q"], args["k"], ctypes.byref(p), args["ws"], ws_bytes,
                                    args["row_ptr"], args["col_idx"], 100, None, None, None,
                                    args["status"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(Hq=3, Hkv=2), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(N=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(block_q=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(block_k=300), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(tau=1.5), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(tau=0.0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(tau=None, sparsity=None), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(sparsity=1.0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(window=64), sa.SA_ERR_INVALID_ARGUMENT),           # window needs causal
    (dict(causal=True, window=-1), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(sink_front=1001), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(theta=2.0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(D=96), sa.SA_ERR_UNSUPPORTED),
    (dict(N=4096 * 64 + 1, block_k=64), sa.SA_ERR_UNSUPPORTED),  # more key blocks than supported
    (dict(N=sa.SA_MAX_KEY_BLOCKS * 64 + 1, block_k=64), sa.SA_ERR_UNSUPPORTED),  # one block past the limit
    (dict(sink_rows=-1), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(sink_rows=1001), sa.SA_ERR_INVALID_ARGUMENT),  # more than N tokens
])
def test_predict_rejects_invalid_parameters(kw, code):
    p = _mask_params(**kw)
    assert sa.sa_predict_workspace_bytes(p) == 0
    assert _predict_code(p) == code
    assert _predict_gather_code(p) == code


def test_predict_ex_validates_like_predict():
    """sa_predict_mask_ex takes the same checks; NULL perm and NULL pattern are allowed."""
    bad = _mask_params(B=0)
    good = _mask_params()

    def code(p, q=FAKE, ws=FAKE):
        return sa.lib().sa_predict_mask_ex(q, FAKE, None, None, ctypes.byref(p), ws, 1 << 30, FAKE, FAKE, 100,
                                           None, None, None, FAKE, None)
    assert code(bad) == sa.SA_ERR_INVALID_ARGUMENT
    assert code(good, q=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert code(good, ws=None) == sa.SA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,code", [
    (dict(n_keys=-1), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(n_keys=500, causal=True), sa.SA_ERR_INVALID_ARGUMENT),   # a causal mask needs N_k = N
    (dict(n_keys=300, sink_front=301), sa.SA_ERR_INVALID_ARGUMENT),  # sinks count keys
    (dict(n_keys=300, sink_back=301), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(n_keys=sa.SA_MAX_KEY_BLOCKS * 64 + 1, block_k=64), sa.SA_ERR_UNSUPPORTED),
])
def test_predict_rejects_bad_key_lengths(kw, code):
    p = _mask_params(**kw)
    assert sa.sa_predict_workspace_bytes(p) == 0
    assert _predict_code(p) == code


def test_key_length_sizes_the_key_side_of_the_workspace():
    """kbar and simk follow the keys' block count, everything else the queries'."""
    p = _mask_params(B=2, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64, n_keys=300,
                     sink_front=300, sink_back=300)
    off = sa.sa_predict_workspace_offsets(p)
    n_qb, n_kb = 8, 5
    sizes = [2 * 4 * n_qb * 128 * 4, 2 * 2 * n_kb * 128 * 4, 2 * 4 * n_qb * 4, 2 * 2 * n_kb * 4,
             2 * 4 * n_qb * n_kb, 2 * 4 * n_qb * 4]
    for i in range(6):
        end = off[i] + sizes[i]
        nxt = off[i + 1] if i < 5 else sa.sa_predict_workspace_bytes(p)
        assert end <= nxt
    # n_keys = N is the same call as n_keys = 0
    assert sa.sa_predict_workspace_bytes(_mask_params(n_keys=1000)) == sa.sa_predict_workspace_bytes(_mask_params())


def test_gather_forms_reject_keys_of_another_length():
    """The gather entry points take one permutation for queries and keys."""
    assert _predict_gather_code(_mask_params(n_keys=300)) == sa.SA_ERR_UNSUPPORTED
    assert _attn_gather_code(sa.make_attn_params(1, 4, 2, 1000, 128, 128, 64, n_keys=300)) == sa.SA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(n_keys=-1), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(n_keys=1 << 31), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(n_keys=500, causal=True), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(n_keys=(1 << 30) // 128), sa.SA_ERR_UNSUPPORTED),  # a key head of 2 GiB
])
def test_attn_rejects_bad_key_lengths(kw, code):
    base = dict(B=1, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64)
    base.update(kw)
    assert _attn_code(sa.make_attn_params(**base)) == code


def test_predict_accepts_the_largest_key_block_count():
    p = _mask_params(N=sa.SA_MAX_KEY_BLOCKS * 64, block_k=64)
    assert sa.sa_predict_workspace_bytes(p) > 0


def _predict_gather_code(p, ws_bytes=1 << 30, perm=FAKE, **ptrs):
    args = dict(q=FAKE, k=FAKE, ws=FAKE, row_ptr=FAKE, col_idx=FAKE, status=FAKE)
    args.update(ptrs)
    return sa.lib().sa_predict_mask_gather(args["q"], args["k"], perm, ctypes.byref(p), args["ws"], ws_bytes,
                                           args["row_ptr"], args["col_idx"], 100, None, None, None,
                                           args["status"], None)


def test_predict_gather_rejects_bad_buffers():
    p = _mask_params()
    need = sa.sa_predict_workspace_bytes(p)
    assert _predict_gather_code(p, perm=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _predict_gather_code(p, ws_bytes=need - 1) == sa.SA_ERR_INVALID_ARGUMENT
    assert _predict_gather_code(p, q=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _predict_gather_code(p, k=ctypes.c_void_p((1 << 20) + 2)) == sa.SA_ERR_INVALID_ARGUMENT


def test_predict_rejects_bad_buffers():
    p = _mask_params()
    need = sa.sa_predict_workspace_bytes(p)
    assert need > 0
    assert _predict_code(p, ws_bytes=need - 1) == sa.SA_ERR_INVALID_ARGUMENT
    assert _predict_code(p, q=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _predict_code(p, status=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _predict_code(p, ws=ctypes.c_void_p((1 << 20) + 16)) == sa.SA_ERR_INVALID_ARGUMENT  # not 256-aligned
    assert _predict_code(p, k=ctypes.c_void_p((1 << 20) + 2)) == sa.SA_ERR_INVALID_ARGUMENT    # not 16-aligned


def test_workspace_layout():
    p = _mask_params(B=2, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64)
    off = sa.sa_predict_workspace_offsets(p)
    n_qb, n_kb = 8, 16
    sizes = [2 * 4 * n_qb * 128 * 4, 2 * 2 * n_kb * 128 * 4, 2 * 4 * n_qb * 4, 2 * 2 * n_kb * 4,
             2 * 4 * n_qb * n_kb, 2 * 4 * n_qb * 4]
    for i in range(6):
        assert off[i] % 256 == 0
        end = off[i] + sizes[i]
        nxt = off[i + 1] if i < 5 else sa.sa_predict_workspace_bytes(p)
        assert end <= nxt


def _attn_code(p, **ptrs):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, row_ptr=FAKE, col_idx=FAKE, status=FAKE)
    args.update(ptrs)
    return sa.lib().sa_sparse_attn_fwd(args["q"], args["k"], args["v"], args["o"], ctypes.byref(p),
                                       args["row_ptr"], args["col_idx"], None, None, args["status"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(Hq=5, Hkv=2), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(lam=0.5), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(lam=float("nan")), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(D=32), sa.SA_ERR_UNSUPPORTED),
    (dict(block_q=64, block_k=64), sa.SA_ERR_UNSUPPORTED),
    (dict(block_q=128, block_k=32), sa.SA_ERR_UNSUPPORTED),
])
def test_attn_rejects_invalid_parameters(kw, code):
    base = dict(B=1, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64)
    base.update(kw)
    assert _attn_code(sa.make_attn_params(**base)) == code
    assert _attn_gather_code(sa.make_attn_params(**base)) == code


def _attn_gather_code(p, perm=FAKE, **ptrs):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, row_ptr=FAKE, col_idx=FAKE, status=FAKE)
    args.update(ptrs)
    return sa.lib().sa_sparse_attn_fwd_gather(args["q"], args["k"], args["v"], perm, args["o"], ctypes.byref(p),
                                              args["row_ptr"], args["col_idx"], None, None, args["status"], None)


def test_attn_gather_rejects_bad_buffers():
    p = sa.make_attn_params(1, 4, 2, 1000, 128, 128, 64)
    assert _attn_gather_code(p, perm=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _attn_gather_code(p, v=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _attn_gather_code(p, q=ctypes.c_void_p((1 << 20) + 4)) == sa.SA_ERR_INVALID_ARGUMENT


def test_attn_rejects_heads_of_2gib():
    # a head of k or v is addressed with 32-bit offsets below 2^31 bytes
    assert _attn_code(sa.make_attn_params(1, 1, 1, (1 << 30) // 128, 128, 128, 64)) == sa.SA_ERR_UNSUPPORTED
    assert _attn_gather_code(sa.make_attn_params(1, 1, 1, (1 << 30) // 128, 128, 128, 64)) == sa.SA_ERR_UNSUPPORTED
    assert _attn_code(sa.make_attn_params(1, 1, 1, (1 << 30) // 64, 64, 128, 64)) == sa.SA_ERR_UNSUPPORTED


def test_attn_rejects_more_rows_than_int32():
    # B * Hq * n_qb query-block rows, one workgroup and one row_ptr entry each
    assert _attn_code(sa.make_attn_params(1 << 12, 1 << 12, 1 << 12, 128 * 128, 128, 128, 64)) == \
        sa.SA_ERR_UNSUPPORTED
    assert _attn_code(sa.make_attn_params(1 << 10, 1 << 10, 1 << 10, 128 * 128, 128, 128, 64, col_cap=-1)) == \
        sa.SA_ERR_INVALID_ARGUMENT


def test_predict_rejects_more_rows_than_int32():
    p = _mask_params(B=1 << 12, Hq=1 << 12, Hkv=1 << 12, N=128 * 128, block_q=128, block_k=128)
    assert sa.sa_predict_workspace_bytes(p) == 0
    assert _predict_code(p) == sa.SA_ERR_UNSUPPORTED


def test_attn_rejects_bad_buffers():
    p = sa.make_attn_params(1, 4, 2, 1000, 128, 128, 64)
    assert _attn_code(p, v=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _attn_code(p, o=ctypes.c_void_p((1 << 20) + 4)) == sa.SA_ERR_INVALID_ARGUMENT


def test_permute_rejects_invalid_arguments():
    L = sa.lib()
    assert L.sa_permute(FAKE, sa.SA_BF16, FAKE, FAKE, 1, 1, 10, 12, None) == sa.SA_ERR_INVALID_ARGUMENT  # D % 8
    assert L.sa_permute(FAKE, 7, FAKE, FAKE, 1, 1, 10, 16, None) == sa.SA_ERR_INVALID_ARGUMENT
    assert L.sa_permute(None, sa.SA_BF16, FAKE, FAKE, 1, 1, 10, 16, None) == sa.SA_ERR_INVALID_ARGUMENT
    assert L.sa_unpermute(FAKE, FAKE, FAKE, 1, 0, 10, 16, None) == sa.SA_ERR_INVALID_ARGUMENT
    # one int32 (row, chunk) index per thread
    assert L.sa_permute(FAKE, sa.SA_BF16, FAKE, FAKE, 1, 1, 1 << 26, 256, None) == sa.SA_ERR_UNSUPPORTED
    assert L.sa_unpermute(FAKE, FAKE, FAKE, 1, 1, 1 << 26, 128, None) == sa.SA_ERR_UNSUPPORTED


def test_binding_refuses_tensors_the_abi_would_misread():
    """The Python binding checks element type, contiguity and device before any call:
    an fp16 tensor is not silently read as bf16, an int64 permutation is not read as
    int32, a strided view is refused, and host memory is refused (no GPU needed)."""
    import torch

    x = torch.zeros((1, 2, 8, 16), dtype=torch.float16)
    y = torch.zeros((1, 2, 8, 16), dtype=torch.bfloat16)
    perm = torch.arange(8, dtype=torch.int32)
    with pytest.raises(TypeError):
        sa.sa_permute(x, y, perm)
    with pytest.raises(TypeError):
        sa.sa_permute(x.float(), y, perm.long())
    with pytest.raises(ValueError, match="contiguous"):
        sa.sa_permute(torch.zeros((1, 2, 16, 8), dtype=torch.float32).transpose(2, 3), y, perm)
    with pytest.raises(ValueError, match="device"):
        sa.sa_permute(x.float(), y, perm)
    o = torch.zeros((1, 2, 8, 16), dtype=torch.float32)
    with pytest.raises(TypeError):
        sa.sa_unpermute(o.double(), o, perm)
    p = sa.make_attn_params(1, 2, 2, 8, 16, 128, 64)
    rp = torch.zeros(3, dtype=torch.int32)
    st = torch.zeros(1, dtype=torch.int32)
    with pytest.raises(TypeError):
        sa.sa_sparse_attn_fwd(y.half(), y, y, o, p, rp, rp, st)
    with pytest.raises(TypeError):
        sa.sa_sparse_attn_fwd(y, y, y, o, p, rp.long(), rp, st)


def test_noalloc_prediction_refuses_workspaces_over_its_array():
    """The allocation-free prediction entry refuses, before touching the GPU, parameters
    whose workspace exceeds its fixed per-GPU array, and rejects invalid ones as usual."""
    big = sa.make_mask_params(1, 64, 64, 131072, 128, 128, 64, tau=0.9)
    assert sa.sa_predict_workspace_bytes(big) > sa.SA_NOALLOC_SCRATCH_BYTES
    L = sa.lib()
    fake = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    args = (fake, fake, fake)
    rc = L.sa_predict_mask_gather_noalloc(*args, ctypes.byref(big), fake, fake, 0, None, None, None, fake, None)
    assert rc == sa.SA_ERR_CAPACITY
    bad = sa.make_mask_params(1, 2, 2, 1000, 96, 128, 64, tau=0.9)  # head dim not compiled
    rc = L.sa_predict_mask_gather_noalloc(*args, ctypes.byref(bad), fake, fake, 0, None, None, None, fake, None)
    assert rc == sa.SA_ERR_UNSUPPORTED
    rc = L.sa_predict_mask_gather_noalloc(fake, fake, None, ctypes.byref(big), fake, fake, 0, None, None, None,
                                          fake, None)
    assert rc == sa.SA_ERR_INVALID_ARGUMENT


# ------------------------------------------------------------------ FP8 QK entry points

def _quant_code(x=FAKE, perm=None, B=1, H=2, N=1000, D=128, block=64, codes=FAKE, scales=FAKE):
    return sa.lib().sa_quantize_fp8(x, perm, B, H, N, D, block, codes, scales, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(N=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(block=0), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(block=129), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(D=96), sa.SA_ERR_UNSUPPORTED),
    (dict(x=None), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(codes=None), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(scales=None), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(x=ctypes.c_void_p((1 << 20) + 8)), sa.SA_ERR_INVALID_ARGUMENT),
    (dict(codes=ctypes.c_void_p((1 << 20) + 4)), sa.SA_ERR_INVALID_ARGUMENT),
])
def test_quantize_fp8_rejects_bad_arguments(kw, code):
    assert _quant_code(**kw) == code


def _qk8_code(p, perm=None, **ptrs):
    args = dict(q8=FAKE, qs=FAKE, k8=FAKE, ks=FAKE, v=FAKE, o=FAKE, row_ptr=FAKE, col_idx=FAKE, status=FAKE)
    args.update(ptrs)
    return sa.lib().sa_sparse_attn_fwd_qk8(args["q8"], args["qs"], args["k8"], args["ks"], args["v"], perm,
                                           args["o"], ctypes.byref(p), args["row_ptr"], args["col_idx"], None, None,
                                           args["status"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), sa.SA_ERR_UNSUPPORTED),                          # FP8 QK path: head dim 128 only
    (dict(block_q=16, block_k=16, D=128), sa.SA_ERR_UNSUPPORTED),
    (dict(block_k=32), sa.SA_ERR_UNSUPPORTED),
    (dict(N=4096 * 64), sa.SA_ERR_UNSUPPORTED),                   # key-tile scales must fit the table
    (dict(lam=0.5), sa.SA_ERR_INVALID_ARGUMENT),
])
def test_qk8_rejects_unsupported_shapes(kw, code):
    base = dict(B=1, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64)
    base.update(kw)
    assert _qk8_code(sa.make_attn_params(**base)) == code


def test_qk8_rejects_bad_buffers():
    p = sa.make_attn_params(1, 4, 2, 1000, 128, 128, 64, lam=-8.0)
    assert _qk8_code(p, q8=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _qk8_code(p, k8=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _qk8_code(p, qs=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _qk8_code(p, ks=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _qk8_code(p, v=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _qk8_code(p, q8=ctypes.c_void_p((1 << 20) + 8)) == sa.SA_ERR_INVALID_ARGUMENT
    assert _qk8_code(p, ks=ctypes.c_void_p((1 << 20) + 2)) == sa.SA_ERR_INVALID_ARGUMENT


def _pq8_code(p, **ptrs):
    args = dict(q=FAKE, k=FAKE, perm=None, ws=FAKE, row_ptr=FAKE, col_idx=FAKE, q8=FAKE, qs=FAKE, k8=FAKE, ks=FAKE,
                status=FAKE)
    args.update(ptrs)
    return sa.lib().sa_predict_mask_qk8(args["q"], args["k"], args["perm"], ctypes.byref(p), args["ws"], 1 << 30,
                                        args["row_ptr"], args["col_idx"], 100, args["q8"], args["qs"], args["k8"],
                                        args["ks"], args["status"], None)


def test_predict_mask_qk8_rejects_bad_arguments():
    p = _mask_params(block_q=128, block_k=64)
    assert _pq8_code(p, q8=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _pq8_code(p, ks=None) == sa.SA_ERR_INVALID_ARGUMENT
    assert _pq8_code(p, k8=ctypes.c_void_p((1 << 20) + 4)) == sa.SA_ERR_INVALID_ARGUMENT
    assert _pq8_code(p, qs=ctypes.c_void_p((1 << 20) + 2)) == sa.SA_ERR_INVALID_ARGUMENT
    assert _pq8_code(_mask_params(block_q=128, block_k=32)) == sa.SA_ERR_UNSUPPORTED
    assert _pq8_code(_mask_params(block_q=256, block_k=64)) == sa.SA_ERR_UNSUPPORTED
    assert _pq8_code(_mask_params(B=0)) == sa.SA_ERR_INVALID_ARGUMENT
