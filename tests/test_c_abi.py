"""The C ABI from plain C (no GPU): a C99 program that includes the public
header, links the library and calls its host-only entry points; its output is
checked against the oracle's planner and the Python binding."""

import os
import shutil
import subprocess

import numpy as np
import pytest

import image_dit_amd as sa
from image_dit_amd import _lib
from oracle import layout as OL

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.fixture(scope="module")
def demo_output(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(_lib.LIB_PATH):
        pytest.skip("needs gcc and the built library")
    out = tmp_path_factory.mktemp("c_abi") / "plan_demo"
    libdir = os.path.dirname(_lib.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi", "plan_demo.c"),
                    "-L", libdir, "-lsparse_attn", f"-Wl,-rpath,{libdir}", "-o", str(out)], check=True)
    res = subprocess.run([str(out)], check=True, capture_output=True, text=True, timeout=60)
    return res.stdout.splitlines()


def test_c_program_sees_the_status_strings(demo_output):
    assert demo_output[0] == f"status {sa.sa_status_string(sa.SA_OK)}|{sa.sa_status_string(sa.SA_ERR_UNSUPPORTED)}"


@pytest.mark.parametrize("line,order,txt,sink", [(1, OL.ORDER_WINDOW, 6, True), (2, OL.ORDER_HILBERT, 0, False)])
def test_c_program_plans_like_the_oracle(demo_output, line, order, txt, sink):
    f = demo_output[line].split()
    assert f[0] == "perm" and int(f[1]) == sa.SA_OK
    n = int(f[2])
    got = np.array([int(x) for x in f[3:]], dtype=np.int64)
    want = OL.plan_permutation(n, order, (3, 5, 7), (2, 4, 4), txt, sink)
    assert len(got) == n and np.array_equal(got, want)


def test_c_program_sizes_the_workspace_like_the_binding(demo_output):
    p = sa.make_mask_params(B=1, Hq=4, Hkv=2, N=1000, D=128, block_q=128, block_k=64, tau=0.9)
    assert demo_output[3] == f"ws {sa.sa_predict_workspace_bytes(p)}"
    assert demo_output[4] == "ws_bad 0"
