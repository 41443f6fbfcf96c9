"""GPU: tgrad_refresh_noalloc (the refresh with its scratch in the library's static device
array) against tgrad_refresh, through the C ABI.

Two calls in a row on one GPU share the array: a bf16 tensor whose last three modes take
the one-read Gram, then a smaller fp32 tensor. Each must match the allocating refresh to
the parity bar (Omega bit for bit, factor projectors within 1e-4, Gram eigenvalues to
fp32 rounding of the partial sums) and the oracle, and a step on the refreshed factors
must give the same weights as the handle refreshed the usual way."""
import numpy as np
import pytest

import tensor_gradient_compression_amd as tg
from gpu_helpers import factor_check, make_lib, make_oracle, projector, weight_check
from synth import TINY_F32, GradStream, init_weights
from synth.gen import custom

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _compare(wl, seed):
    print(f"CASE noalloc {wl.name}", flush=True)
    g = GradStream(wl, seed=seed).next()
    G = tg.to_device(g, wl.dtype)
    ref, nal = make_lib(wl), make_lib(wl)
    ref.refresh(G)
    nal.refresh_noalloc(G)
    torch.cuda.synchronize()
    assert np.array_equal(nal.get_omega(), ref.get_omega())
    for n, (I, r) in enumerate(zip(wl.shape, wl.ranks)):
        if r >= I:
            continue
        a, b = nal.get_factor(n), ref.get_factor(n)
        assert np.abs(projector(a) - projector(b)).max() <= 1e-4, n
        ea, eb = nal.get_eigvals(n), ref.get_eigvals(n)
        np.testing.assert_allclose(ea, eb, rtol=1e-6, atol=1e-6 * eb[0])
    orc = make_oracle(wl)
    orc.refresh(g)
    assert np.array_equal(nal.get_omega(), orc.omega)
    factor_check(nal, orc)
    # both handles step from their refresh
    W0 = init_weights(wl, seed=seed)
    Wr, Wn = tg.to_device(W0, wl.dtype), tg.to_device(W0, wl.dtype)
    g2 = GradStream(wl, seed=seed + 1).next()
    ref.step(Wr, tg.to_device(g2, wl.dtype))
    nal.step(Wn, tg.to_device(g2, wl.dtype))
    torch.cuda.synchronize()
    weight_check(tg.to_host(Wn, wl.dtype), tg.to_host(Wr, wl.dtype), wl.dtype, wl.name)
    # a second call on the same handle reuses the array: the same outcome
    om1 = nal.get_omega().copy()
    nal.refresh_noalloc(G)
    torch.cuda.synchronize()
    assert np.array_equal(nal.get_omega(), om1)
    assert nal.get_info().eig_unconverged == 0


def test_noalloc_refresh_two_calls_then_smaller():
    _compare(custom((6, 5, 48, 25), "bf16", (3, 3, 24, 13), 0.05, T=100), seed=3)
    _compare(TINY_F32, seed=4)


def test_noalloc_refresh_refuses_low_rank_first():
    wl = custom((6, 5, 48, 25), "bf16", (3, 3, 24, 13), 0.05)
    lib = make_lib(wl)
    lib.set_options(order="lowrank_first")
    G = tg.to_device(GradStream(wl, seed=1).next(), wl.dtype)
    with pytest.raises(tg.TGradError, match="invalid argument"):
        lib.refresh_noalloc(G)
