"""The C ABI driven from plain C (tests/c_client/dconv1d_client.c, built by
__graft_entry__.build()): eval-mode and training-mode block results against the float64
oracle, and rejected calls returning their status codes."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from normalisation_dilated_conv1d_amd.inputs import prenorm_inputs

from test_gpu_parity import TOL_F32, announce, maxrel

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(__file__), "c_client", "dconv1d_client")


@pytest.mark.skipif(not os.path.exists(CLIENT), reason="C client not built")
@pytest.mark.parametrize("N,C,L,d", [(2, 16, 512, 128), (3, 40, 700, 9)])
def test_c_client_matches_oracle(N, C, L, d, tmp_path):
    announce("C client", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 80_000 + C + d)
    mom = 0.1
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([N, C, L, d], dtype="<i8").tobytes())
        f.write(np.array([p["eps"], mom], dtype="<f4").tobytes())
        for k in ("x", "running_mean", "running_var", "gamma", "beta", "W", "b"):
            f.write(np.ascontiguousarray(p[k].numpy(), dtype="<f4").tobytes())
    res = subprocess.run([CLIENT, str(inp), str(outp)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    got = np.fromfile(outp, dtype="<f4")
    nx = N * C * L
    out, out_t = got[:nx].reshape(N, C, L), got[nx:2 * nx].reshape(N, C, L)
    rm, rv = got[2 * nx:2 * nx + C], got[2 * nx + C:]
    ref = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"], p["beta"],
                               p["eps"], p["W"], p["b"], d)
    ref_t, rm_t, rv_t, _, _ = oracle.prenorm_block_train(p["x"], p["running_mean"],
                                                         p["running_var"], p["gamma"], p["beta"],
                                                         p["eps"], mom, p["W"], p["b"], d)
    errs = [maxrel(out, ref), maxrel(out_t, ref_t), maxrel(rm, rm_t), maxrel(rv, rv_t)]
    assert max(errs) <= TOL_F32, errs
