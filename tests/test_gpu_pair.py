"""GPU: two neighbouring leading modes in one launch (k_pair), against the oracle.

Omega and U(n) come from the oracle, so only the step kernels are compared. Each case
runs the fused plan with the pair launch and with one launch per mode. Both must meet
the parity bar of gpu_helpers.weight_check over four steps, with every step's fp32
update checked (gpu_helpers.checked_step), and so must the core moments. The timing records must show which launches ran. The shapes cover:
* a pair after the trailing two-mode launch and after the three-mode projection;
* a pair behind a full-rank leading mode (A > 1);
* 1 to 4 row blocks of the first product, with 16 to 64 values in its k;
* three 16-row blocks of j0 in one workgroup;
* fp32, fp16 and bf16 data."""
import numpy as np
import pytest

import tensor_gradient_compression_amd as tg
from gpu_helpers import CoreSplit, DeltaCapture, checked_step, make_lib, make_oracle, weight_check
from synth import (TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33, BF16_64x64x48x48x25,
                   GradStream, init_weights)
from synth.gen import custom

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tg.load_library()


# (name, workload, pair launches per step in the projection, in the reconstruction)
CASES = [
    # modes 1, 0 after the trailing pair and 0, 1 before it; 32 and 16 values of k
    ("fp32-32x32x16x16", F32_32x32x16x16, 1, 1),
    # a pair behind a full-rank leading mode (A = 3); the reconstruction's I1 = 8 is too
    # narrow, so it runs one launch per mode
    ("f32-5mode-behind-full-rank", custom((3, 32, 16, 16, 8), "f32", (3, 16, 8, 8, 4), 0.05), 1, 0),
    # after the three-mode projection (48 values of k); the reconstruction's first
    # product has three row blocks (J1 = 48)
    ("bf16-after-three-mode", custom((16, 48, 32, 16, 8), "bf16", (8, 16, 16, 8, 4), 0.05), 1, 1),
    # three 16-row blocks of j0 in one workgroup (J0 = 48); the reconstruction (J0 = 64,
    # J1 = 32) would need its rows split, so it runs one launch per mode
    ("f32-rank-48", custom((64, 32, 16, 16), "f32", (48, 16, 8, 8), 0.05), 1, 0),
    # four row blocks of the first product (J1 = 56) over 64 values of k, fp16
    ("f16-four-row-blocks", custom((32, 64, 16, 16), "f16", (16, 56, 8, 8), 0.05), 1, 0),
]


@pytest.mark.parametrize("pairs", [True, False], ids=["pair", "per-mode"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_pair_steps_match_oracle(case, pairs):
    name, wl, npj, nrc = case
    gs = GradStream(wl, seed=21)
    W0 = init_weights(wl, seed=21)
    lib, orc = make_lib(wl, T=10 ** 6), make_oracle(wl, T=10 ** 6)
    assert lib.set_pair_fusion(pairs) == True   # noqa: E712  (applies to every case)
    g1 = gs.next()
    orc.refresh(g1)
    lib.set_omega(orc.omega)
    for n, U in enumerate(orc.factors):
        if U is not None:
            lib.set_factor(n, U)
    lib.mark_refreshed()
    lib.timing_enable(True)
    cap = DeltaCapture(lib, wl)
    split = CoreSplit(orc)
    W = tg.to_device(W0, wl.dtype)
    Wo = W0
    g = g1
    slack = 0.0
    for step in range(4):
        what = f"{name}/{'pair' if pairs else 'per-mode'} step {step + 1}"
        Wo, _ = checked_step(lib, orc, cap, W, Wo, g, wl, what, align=split)
        slack += wl.lr * 1e-5 * np.abs(orc.last["delta"]).max()
        weight_check(tg.to_host(W, wl.dtype), Wo, wl.dtype, what, delta_backed=True, slack=slack)
        g = gs.next()
    rec = lib.timing_read()
    got = (rec.get("modeprod_pair_project", (0,))[0], rec.get("modeprod_pair_reconstruct", (0,))[0])
    assert got == ((4 * npj, 4 * nrc) if pairs else (0, 0)), got
    mc, vc, ms, vs = lib.get_moments()
    scale = np.abs(orc.mC).max() + 1e-30
    assert np.abs(mc - orc.mC).max() <= 1e-4 * scale


def test_pair_reports_where_it_does_not_apply():
    # columns after the pair not a multiple of 16; complex data; a single compressed
    # leading mode; 40 values of k in the projection and, in the reconstruction, 64 x 40
    # output rows that would not fit one workgroup
    for shape, dtype, ranks in (((8, 8, 6, 6), "f32", (4, 4, 3, 3)),
                                ((12, 10, 9), "c64", (5, 4, 3)),
                                ((64, 32, 16, 16), "f32", (64, 16, 8, 8)),
                                ((64, 40, 16, 16), "f32", (32, 16, 8, 8))):
        lib = make_lib(custom(shape, dtype, ranks, 0.05))
        assert not lib.set_pair_fusion(True), shape
        assert lib.set_pair_fusion(False)
