"""GPU: the whole path driven from plain C (image_dit_amd/examples/path_demo.c, built
with the library): HIP runtime allocations, the two gather-form calls on the
default stream, no Python or torch in that process.  Its outputs equal the
Python binding's bit for bit on the same inputs."""

import dataclasses
import os
import subprocess
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import image_dit_amd as sa  # noqa: E402
from image_dit_amd.build import DEMO  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

rep = dataclasses.replace
CASES = {
    # PV skip on 64-key tiles over the Hilbert order
    "long_video_lam": rep(CONFIGS["long_video"], Hq=2, Hkv=2, latent=(6, 10, 21), seed=301),
    # 128-key blocks, window order with text and first-frame sinks, lambda off
    "video": rep(CONFIGS["video"], Hq=2, Hkv=2, latent=(5, 16, 24), txt_len=20, sink_front=16 * 24,
                 sink_back=20, seed=302),
    # causal GQA with a sliding window and sink tokens
    "causal": rep(CONFIGS["causal_long"], Hq=4, Hkv=2, latent=(1, 1, 1500), window_tokens=300, seed=303),
}


def _arg(x):
    return "none" if x is None else repr(float(x))


@pytest.mark.parametrize("name", list(CASES))
def test_c_caller_matches_the_binding(name, tmp_path):
    assert os.path.exists(DEMO), f"{DEMO} is missing: build with python -m image_dit_amd.build"
    w = CASES[name]
    cfg = sa.config_from_workload(w)
    q, k, v = generate(w)
    path = sa.SparseAttentionPath(cfg, materialize=False)
    for arr, fn in ((q, "q.bin"), (k, "k.bin"), (v, "v.bin")):
        arr.tofile(tmp_path / fn)
    path.perm_host.astype(np.int32).tofile(tmp_path / "perm.bin")
    args = [DEMO, str(tmp_path), str(w.B), str(w.Hq), str(w.Hkv), str(w.N), str(w.D), str(w.block_q),
            str(w.block_k), str(int(w.causal)), str(w.window_tokens), str(w.sink_front), str(w.sink_back),
            _arg(cfg.tau), _arg(cfg.theta), _arg(cfg.sparsity), _arg(cfg.lam)]
    print(f"[c-path] {name}: N={w.N} bq={w.block_q} bk={w.block_k} lam={w.lam}", flush=True)
    sys.stdout.flush()
    res = subprocess.run(args, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    f = res.stdout.split()
    assert f[:3] == ["status", str(sa.SA_OK), str(sa.SA_OK)], res.stdout
    nnz = int(f[4])

    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    o = path.run_fused(dev(q), dev(k), dev(v))
    torch.cuda.synchronize()
    assert path.statuses() == (sa.SA_OK, sa.SA_OK)
    rp, ci = path.csr_host()
    assert int(rp[-1]) == nnz
    assert np.array_equal(np.fromfile(tmp_path / "row_ptr.bin", dtype=np.int32), rp)
    assert np.array_equal(np.fromfile(tmp_path / "col_idx.bin", dtype=np.int32), ci)
    assert np.array_equal(np.fromfile(tmp_path / "counters.bin", dtype=np.int64), path.counters.cpu().numpy())
    got = np.fromfile(tmp_path / "o.bin", dtype=np.uint32)
    assert np.array_equal(got, o.cpu().numpy().view(np.uint32).ravel())
