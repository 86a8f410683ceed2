"""Results must not depend on how many workgroups a launch has: the same samples computed
alone and inside larger batches give bitwise-equal outputs. The batch sizes are chosen so
that the library picks a different tile (and so a different grid and workgroup shape) for
each: for the float32 block's direct kernel at C=256, L=4096 the 64x64 tile below N=4, the
64x128 tile for 4 <= N < 8, the 64x256 tile for 8 <= N < 16 and the 128x256 tile from
N=16 (and the Winograd kernel's grid and channel tile at each N); for the bf16 block at C=512, L=16384 the
256-channel tile at N=1 and the 512-channel tile from N=2; and for Conv1d+GroupNorm the
single-launch kernel at 16 and at 640 workgroups. Every output is a fixed sequence of MFMA
steps over the same K order whatever the tile, so equal bits are the bar. A missing
barrier or a read of another tile's half-written LDS would show up here as a difference
between grid sizes."""
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
from normalisation_dilated_conv1d_amd.inputs import groupnorm_inputs, prenorm_inputs

from test_gpu_parity import announce, to_dev

pytestmark = pytest.mark.gpu


def _block(q, n0, n1, d, bf16=False):
    fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
    x = q["x"][n0:n1].contiguous()
    return fn(x, q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"], q["W"],
              q["b"], d)


@pytest.mark.parametrize("form", ["0", "1"])
def test_f32_block_same_bits_for_every_tile(form, monkeypatch):
    """Each conv form on its own (DCONV1D_WINOGRAD=0: the direct kernel, whose tile changes
    with N; =1: the Winograd kernel, whose grid changes with N). Without the override the
    library picks the form by shape, N included, so a sample's bits may differ between
    batch sizes that fall on either side of that choice."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", form)
    N, C, L, d = 20, 256, 4096, 128
    announce("grid invariance f32", (N, C, L, d), "DCONV1D_WINOGRAD", form)
    q = to_dev(prenorm_inputs(N, C, L, 90_001))
    full = _block(q, 0, N, d)                 # 128 x 256 tiles, 640 workgroups
    mid = _block(q, 2, 12, d)                 # N = 10: 64 x 256 tiles
    five = _block(q, 7, 12, d)                # N = 5: 64 x 128 tiles
    small = _block(q, 3, 6, d)                # N = 3: 64 x 64 tiles
    one = _block(q, 19, 20, d)                # N = 1
    torch.cuda.synchronize()
    assert torch.equal(full[2:12], mid)
    assert torch.equal(full[7:12], five)
    assert torch.equal(full[3:6], small)
    assert torch.equal(full[19:20], one)


def test_bf16_block_same_bits_for_both_tiles():
    N, C, L, d = 3, 512, 16384, 128
    announce("grid invariance bf16", (N, C, L, d))
    q = to_dev(prenorm_inputs(N, C, L, 90_002, bf16=True))
    full = _block(q, 0, N, d, bf16=True)      # 512-channel tile (8 waves)
    one = _block(q, 1, 2, d, bf16=True)       # N = 1: 256-channel tile (4 waves)
    torch.cuda.synchronize()
    assert torch.equal(full[1:2], one)


@pytest.mark.parametrize("form", ["0", "1"])
def test_groupnorm_single_launch_same_bits_at_any_grid(form, monkeypatch):
    """Both conv forms of the single-launch kernel (DCONV1D_WINOGRAD=0: three taps; =1: the
    library's choice, Winograd for this dilation-1 layer)."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", form)
    N, C_in, C_out, T, G = 40, 128, 256, 1024, 32
    announce("grid invariance groupnorm", form, (N, C_in, C_out, T, G))
    q = to_dev(groupnorm_inputs(N, C_in, C_out, T, 90_003, with_bias=True))

    def gn(n0, n1):
        return dc.conv1d_groupnorm_fwd(q["x"][n0:n1].contiguous(), q["W"], q["bias"],
                                       q["gamma"], q["beta"], q["eps"], G, 1, 1)

    full = gn(0, N)       # 640 workgroups, more than one round on 256 CUs
    one = gn(7, 8)        # 16 workgroups
    some = gn(30, 33)
    torch.cuda.synchronize()
    assert torch.equal(full[7:8], one)
    assert torch.equal(full[30:33], some)
