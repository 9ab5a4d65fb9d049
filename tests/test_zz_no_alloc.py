"""The allocation-free prediction entry point against the workspace form (MI355X only).

sa_predict_mask_gather_noalloc keeps its workspace in a fixed per-GPU array of the
library.  Two calls in a row, the second on a smaller input (so stale contents of the
array from the first call are present), must each give the CSR, mask and block
similarities of sa_predict_mask_gather with a caller workspace, bit for bit.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import image_dit_amd as sa  # noqa: E402
from workloads import CONFIGS, generate  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def dev(x):
    return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()


def predict_both(w):
    cfg = sa.config_from_workload(w)
    q, k, _ = generate(w)
    qd, kd = dev(q), dev(k)
    outs = []
    for noalloc in (False, True):
        path = sa.SparseAttentionPath(cfg, materialize=False)
        mask = torch.full((cfg.rows, cfg.n_kb), 7, dtype=torch.uint8, device="cuda")
        simq = torch.full((cfg.rows,), -1.0, dtype=torch.float32, device="cuda")
        simk = torch.full((cfg.B * cfg.Hkv * cfg.n_kb,), -1.0, dtype=torch.float32, device="cuda")
        if noalloc:
            sa.sa_predict_mask_gather_noalloc(qd, kd, path.perm, path.mp, path.row_ptr, path._cols(),
                                              path.status[0:1], mask, simq, simk)
        else:
            path.predict_gather(qd, kd, mask_out=mask, sim_q=simq, sim_k=simk)
        torch.cuda.synchronize()
        rp, ci = path.csr_host()
        outs.append(dict(status=path.statuses()[0], rp=rp, ci=ci, mask=mask.cpu().numpy(),
                         simq=simq.cpu().numpy().view(np.uint32), simk=simk.cpu().numpy().view(np.uint32)))
    return outs


def test_noalloc_prediction_equals_workspace_form_twice():
    big = dataclasses.replace(CONFIGS["long_video"], Hq=3, Hkv=3, latent=(6, 10, 21))
    small = dataclasses.replace(CONFIGS["image"], Hq=2, Hkv=2, latent=(1, 20, 37), seed=7)
    for w in (big, small):
        a, b = predict_both(w)
        print(f"[noalloc] {w.name}: N={w.N} nnz={int(a['rp'][-1])}", flush=True)
        sys.stdout.flush()
        assert a["status"] == sa.SA_OK and b["status"] == sa.SA_OK
        for key in ("rp", "ci", "mask", "simq", "simk"):
            assert np.array_equal(a[key], b[key]), key


def test_noalloc_prediction_refuses_a_workspace_over_its_array():
    w = dataclasses.replace(CONFIGS["causal_long"], Hq=64, Hkv=64, latent=(1, 1, 131072), block_k=64)
    cfg = sa.config_from_workload(w)
    mp = cfg.mask_params()
    assert sa.sa_predict_workspace_bytes(mp) > sa.SA_NOALLOC_SCRATCH_BYTES
    t = torch.zeros(8, dtype=torch.bfloat16, device="cuda")
    i = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(sa.SparseAttnError) as e:
        sa.sa_predict_mask_gather_noalloc(t, t, i, mp, i, i, i[:1])
    assert e.value.code == sa.SA_ERR_CAPACITY
