"""GPU: the refresh's one-read Gram launch for the last three modes.

Each case refreshes one handle with that launch and one with a Gram launch per mode,
from the same seeded gradient. The first must match the oracle: Omega bit for bit,
eigenvalues within rtol 1e-4 of the oracle's fp64 Gram spectrum, factor projectors
within 1e-4. The two GPU paths must agree to the fp32 rounding of their partial sums
(rtol 1e-6, and 1e-6 of the largest eigenvalue for the small ones). The shapes cover:
* 16-byte and 16-bit operand reads;
* one to four 16-row blocks per mode, ragged blocks;
* more slabs than workgroups, and a single slab;
* a refresh without a sparse part."""
import numpy as np
import pytest

import tensor_gradient_compression_amd as tg
from gpu_helpers import factor_check, make_lib, make_oracle
from synth import GradStream
from synth.gen import custom

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tg.load_library()


CASES = [
    # (48, 48, 25) slabs as in the full-size workload: 16-byte reads of the slab rows in
    # the first of the three modes, 16-bit reads in the other two
    ("bf16-48x48x25", custom((3, 48, 48, 25), "bf16", (2, 24, 24, 13), 0.05)),
    # ragged 16-row blocks in every mode, fp16
    ("f16-32x40x17", custom((2, 32, 40, 17), "f16", (2, 9, 20, 9), 0.05)),
    # last mode a multiple of 8: 16-byte reads in two modes; more slabs than workgroups
    ("bf16-300x16x16x8", custom((300, 16, 16, 8), "bf16", (300, 8, 8, 4), 0.05)),
    # four 16-row blocks (three block groups) in two modes
    ("bf16-64x64x8", custom((2, 64, 64, 8), "bf16", (1, 32, 32, 4), 0.05)),
    # slab rows of 25 values: 16-bit reads in every mode; a 5-wide last mode
    ("bf16-8x5x5", custom((7, 8, 5, 5), "bf16", (3, 4, 3, 2), 0.05)),
    # a three-mode tensor is a single slab; no sparse part
    ("f16-3mode-k0", custom((40, 24, 20), "f16", (20, 12, 10), 0.0)),
]


@pytest.mark.parametrize("masked", [False, True], ids=["residual-copy", "masked-read"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_one_read_gram_matches_oracle_and_per_mode(case, masked):
    """Both ways of reading the residual: the copy the top-k pass writes, and the
    gradient itself with Omega's entries cleared in the staged tiles through the bitmask
    (every Gram launch, the one-read and the per-mode ones)."""
    name, wl = case
    g = GradStream(wl, seed=11).next()
    G = tg.to_device(g, wl.dtype)
    fused, single = make_lib(wl), make_lib(wl)
    assert fused.set_gram_fusion(True, masked=masked)
    assert single.set_gram_fusion(False, masked=masked)
    fused.timing_enable(True)
    single.timing_enable(True)
    fused.refresh(G)
    single.refresh(G)
    torch.cuda.synchronize()
    d = len(wl.shape)
    lead = sum(1 for n in range(d - 3) if wl.ranks[n] < wl.shape[n])
    rec = fused.timing_read()
    assert rec["gram3_tail"][0] == 1
    assert rec.get("gram", (0, 0.0))[0] == lead
    rec = single.timing_read()
    assert "gram3_tail" not in rec and rec["gram"][0] == lead + 3

    orc = make_oracle(wl)
    orc.refresh(g)
    assert np.array_equal(fused.get_omega(), orc.omega)
    factor_check(fused, orc)
    for n in range(d):
        w = orc.eigvals[n]
        if w is None:
            continue
        got = fused.get_eigvals(n)
        np.testing.assert_allclose(got, w, rtol=1e-4, atol=1e-5 * w[0])
        np.testing.assert_allclose(got, single.get_eigvals(n), rtol=1e-6, atol=1e-6 * w[0])


def test_one_read_gram_reports_where_it_does_not_apply():
    # last mode above 32; only two modes; fp32 data; complex data; a full-rank mode
    # among the last three
    for shape, dtype, ranks in (((33, 17, 60), "bf16", (13, 8, 31)),
                                ((48, 25), "bf16", (24, 13)),
                                ((8, 16, 16, 8), "f32", (4, 8, 8, 4)),
                                ((12, 10, 9), "c64", (5, 4, 3)),
                                ((4, 16, 16, 8), "bf16", (2, 16, 8, 4))):
        lib = make_lib(custom(shape, dtype, ranks, 0.05))
        assert not lib.set_gram_fusion(True), shape
        assert lib.set_gram_fusion(False)
