"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Omega must match bit for bit; factor subspaces within 1e-4 (projector max-abs); weights
within the bar of gpu_helpers.weight_check; the gradient left untouched by a step. Inputs come from the seeded generator in synth/."""
import numpy as np
import pytest

import oracle as O
import tensor_gradient_compression_amd as tg
from gpu_helpers import (DeltaCapture, CoreSplit, apply_check, checked_step, delta_rel, factor_check,
                         make_lib, make_oracle, omega_properties, weight_check)
from synth import (TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33, BF16_64x64x48x48x25,
                   GradStream, init_weights)
from synth.gen import custom

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    tg.load_library()


def dev(x, dtype):
    return tg.to_device(x, dtype)


def host(t, dtype):
    return tg.to_host(t, dtype)


# --------------------------------------------------------------------------- top-k

def _topk_inputs():
    r = np.random.default_rng(7)
    cases = []
    for dtype in ("f32", "f16", "bf16", "c64"):
        wl = custom((7, 5, 3), dtype, (7, 5, 3), 0.0)
        g = GradStream(wl, seed=3).next()
        N = 105
        for k in (0, 1, 17, 52, 104, 105):
            cases.append((f"{dtype}-tiny-k{k}", wl.shape, dtype, min(1.0, k / N + 1e-12), g))
    q = (np.round(r.standard_normal((33, 17, 5)) * 2) / 2).astype(np.float32)
    cases.append(("f16-quantized-ties", q.shape, "f16", 0.37, O.encode(q, "f16")))
    cases.append(("bf16-quantized-ties", q.shape, "bf16", 0.5, O.encode(q, "bf16")))
    eq = np.full((1000, 3), -1.25, np.float32)
    cases.append(("f32-all-equal", eq.shape, "f32", 0.3, eq))
    z = np.zeros((64, 65), np.float32)
    z[::3, ::2] = -0.0
    z[5, 7] = 1e-42
    z[9, 1] = -1e-42
    z[11, 11] = 3e-39
    cases.append(("f32-signed-zeros-subnormals", z.shape, "f32", 0.01, z))
    wl1 = F32_32x32x16x16
    cases.append(("fp32-32x32x16x16", wl1.shape, "f32", 0.05, GradStream(wl1).next()))
    big = r.standard_normal((4099, 1031)).astype(np.float32)
    cases.append(("f32-ragged-4M", big.shape, "f32", 0.05, big))
    cz = (r.standard_normal((301, 77)) + 1j * r.standard_normal((301, 77))).astype(np.complex64)
    cz[3, 3] = cz[0, 0]
    cz[5, 5] = np.conj(cz[0, 0])
    cases.append(("c64-dup-magnitudes", cz.shape, "c64", 0.2, cz))
    # non-finite values: NaN (several payloads and signs) ranks above +-Inf, which rank
    # above every finite value; ties among them go to the lowest index
    for dtype in ("f32", "f16", "bf16"):
        x = r.standard_normal((13, 11, 7)).astype(np.float32)
        x.reshape(-1)[[5, 77, 300, 811]] = np.inf
        x.reshape(-1)[[9, 500]] = -np.inf
        x.reshape(-1)[[40, 41, 900]] = 1e30 if dtype != "f16" else 6e4
        enc = O.encode(x, dtype).reshape(-1)
        bits = enc.view(np.uint32 if dtype == "f32" else np.uint16)
        if dtype == "f32":
            nan_bits = [0x7FC00000, 0xFFC00001, 0x7F800001, 0x7FFFFFFF]
        elif dtype == "f16":
            nan_bits = [0x7E00, 0xFE01, 0x7C01, 0x7FFF]
        else:
            nan_bits = [0x7FC0, 0xFFC1, 0x7F81, 0x7FFF]
        for pos, nb in zip((3, 150, 151, 1000), nan_bits):
            bits[pos] = nb
        enc = enc.reshape(x.shape)
        for k in (1, 4, 9, 12, 200):
            cases.append((f"{dtype}-nonfinite-k{k}", x.shape, dtype, k / x.size + 1e-12, enc))
    zc = (r.standard_normal((17, 19)) + 1j * r.standard_normal((17, 19))).astype(np.complex64)
    f = zc.reshape(-1)
    f[2] = complex(np.nan, 0.0)
    f[30] = complex(1.0, np.nan)
    f[31] = complex(np.inf, np.nan)
    f[60] = complex(np.inf, 0.0)
    f[61] = complex(0.0, -np.inf)
    f[90] = complex(-np.inf, np.inf)
    f[100] = complex(3e38, 3e38)      # |z|^2 overflows fp32 but not fp64
    for k in (1, 3, 6, 8, 40):
        cases.append((f"c64-nonfinite-k{k}", zc.shape, "c64", k / zc.size + 1e-12, zc))
    return cases


@pytest.mark.parametrize("case", _topk_inputs(), ids=lambda c: c[0])
def test_topk_bit_exact(case):
    name, shape, dtype, rho, g = case
    lib = tg.TGrad(shape, shape, dtype, rho, 1000)
    G = dev(g, dtype)
    before = host(G, dtype).copy()
    lib.refresh(G)
    torch.cuda.synchronize()
    om = lib.get_omega()
    exp = O.select_omega(O.topk_keys(g, dtype), lib.k)
    assert om.dtype == np.uint32 and np.array_equal(om, exp), name
    assert np.array_equal(host(G, dtype).view(np.uint8), before.view(np.uint8)), "refresh modified grad"


def test_topk_fp16_and_complex64_full_sizes():
    for wl in (F16_4x64x64x64x64, C64_64x64x64x33):
        g = GradStream(wl).next()
        lib = tg.TGrad(wl.shape, wl.shape, wl.dtype, wl.sparse_ratio, 1000)
        lib.refresh(dev(g, wl.dtype))
        om = lib.get_omega()
        assert np.array_equal(om, O.select_omega(O.topk_keys(g, wl.dtype), wl.k))


# --------------------------------------------------------------------------- refresh: factors

# Every case keeps r_n <= N / I_n: a larger rank than the mode-n unfolding can have
# leaves core entries that are zero up to rounding, and Adam's m / (sqrt(v) + eps)
# turns that rounding noise into O(1) updates on which no two implementations agree.
FACTOR_CASES = [
    ("tiny-fp32-8x8x6x6", TINY_F32),
    ("fp32-32x32x16x16", F32_32x32x16x16),
    ("odd-5mode", custom((9, 7, 5, 11, 3), "f32", (4, 3, 5, 2, 1), 0.05)),
    ("narrow-lastmode-64", custom((3, 5, 64), "f32", (2, 5, 12), 0.1)),
    ("bf16-odd", custom((33, 17, 60), "bf16", (13, 8, 31), 0.05)),
    # 16-bit tensors whose two trailing modes take the wave-per-slab kernels
    ("bf16-slab-48x25", custom((6, 5, 48, 25), "bf16", (3, 3, 24, 13), 0.05)),
    ("f16-slab-40x17", custom((9, 40, 17), "f16", (5, 20, 9), 0.05)),
    ("bf16-slab-ragged", custom((7, 33, 24), "bf16", (4, 17, 12), 0.05)),
    ("bf16-slab-k0", custom((5, 16, 8), "bf16", (3, 8, 4), 0.0)),
    # ... and whose mode d-3 joins them in the projection's first launch (a workgroup
    # of 16 waves per leading index, in rounds of 16 slabs: three rounds a unit; two
    # rounds with ragged slab blocks; one round a unit without a sparse part; more
    # leading indices than the grid has workgroups)
    ("bf16-slab3-48x48x25", custom((3, 48, 48, 25), "bf16", (2, 24, 24, 13), 0.05)),
    ("f16-slab3-ragged", custom((2, 32, 40, 17), "f16", (2, 9, 20, 9), 0.05)),
    ("bf16-slab3-k0", custom((2, 16, 16, 8), "bf16", (1, 8, 8, 4), 0.0)),
    ("bf16-slab3-300-units", custom((300, 16, 8, 8), "bf16", (300, 8, 4, 4), 0.05)),
    # four output column blocks per wave (R1 R2 = 512); R0 = 32 over four rounds
    ("bf16-slab3-wide-core", custom((2, 16, 40, 17), "bf16", (1, 8, 32, 16), 0.05)),
    ("bf16-slab3-r0-32", custom((2, 64, 16, 8), "bf16", (1, 32, 8, 4), 0.05)),
    # compressed modes wider than 64 (the eigensolver for 64 < I <= 128 keeps A packed in
    # LDS and V in registers): 128 real, an odd width with a bye in every round, and the
    # narrowest; complex ones (the complex Gram has 256 stacked rows, four launches of 64
    # output blocks; each mode product runs as two real ones and a combine pass): a
    # leading 128, a last mode of 100 (its update goes through the dense apply), and two
    # leading 128s with small trailing modes, the shape of a spectral layer's weights
    ("f32-128", custom((128, 20, 6), "f32", (40, 10, 3), 0.05)),
    ("bf16-128x24", custom((128, 24, 8), "bf16", (48, 12, 4), 0.05)),
    ("c64-128", custom((128, 12, 6), "c64", (30, 6, 3), 0.05)),
    ("c64-last-100", custom((10, 6, 100), "c64", (4, 3, 20), 0.05)),
    ("c64-128x128x6x4", custom((128, 128, 6, 4), "c64", (24, 24, 4, 3), 0.05)),
    ("f32-127-odd", custom((127, 16, 5), "f32", (31, 8, 2), 0.05)),
    ("f16-65", custom((65, 30, 4), "f16", (16, 10, 2), 0.05)),
    # ... and whose mode d-2 (I0 a multiple of 12) joins the reconstruction's last launch
    # (12 waves a unit, rounds of 12 slabs): 3 rounds a unit with ragged row and column
    # blocks; one round a unit; k = 0; more units than the grid has workgroups
    ("bf16-rec3-36x40x17", custom((3, 36, 40, 17), "bf16", (2, 18, 20, 9), 0.05)),
    ("f16-rec3-12x24x16", custom((5, 12, 24, 16), "f16", (3, 6, 12, 8), 0.05)),
    ("bf16-rec3-k0", custom((2, 24, 32, 8), "bf16", (1, 12, 16, 4), 0.0)),
    ("bf16-rec3-300-units", custom((300, 12, 24, 8), "bf16", (300, 6, 12, 4), 0.05)),
    ("f16-64", custom((64, 20, 9), "f16", (32, 7, 4), 0.05)),
    ("c64-small", custom((12, 10, 9), "c64", (5, 4, 3), 0.05)),
    ("c64-64", custom((64, 6, 33), "c64", (32, 6, 16), 0.05)),
    ("one-mode", custom((50,), "f32", (1,), 0.1, signal_ranks=(1,))),
]


@pytest.mark.parametrize("masked", [False, True], ids=["residual-copy", "masked-read"])
@pytest.mark.parametrize("case", FACTOR_CASES, ids=lambda c: c[0])
def test_refresh_factors_match_oracle(case, masked):
    """The refresh against the oracle, with the Grams reading the residual copy that the
    top-k pass writes or the gradient with Omega cleared through the bitmask."""
    name, wl = case
    g = GradStream(wl, seed=5).next()
    lib, orc = make_lib(wl), make_oracle(wl)
    if masked:
        lib.set_gram_fusion(lib.set_gram_fusion(True), masked=True)
    G = dev(g, wl.dtype)
    before = host(G, wl.dtype).copy()
    lib.refresh(G)
    orc.refresh(g)
    torch.cuda.synchronize()
    assert np.array_equal(lib.get_omega(), orc.omega)
    factor_check(lib, orc)
    for n, w in enumerate(orc.eigvals):
        if w is not None:
            got = lib.get_eigvals(n)
            np.testing.assert_allclose(got, w, rtol=1e-4, atol=1e-5 * w[0])
    assert np.array_equal(host(G, wl.dtype).view(np.uint8), before.view(np.uint8))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("masked", [False, True], ids=["residual-copy", "masked-read"])
@pytest.mark.parametrize("name,wl", [("c64-64x64x64x33", C64_64x64x64x33),
                                     ("f16-64x64x64x64", F16_4x64x64x64x64)],
                         ids=lambda x: x if isinstance(x, str) else "")
def test_full_size_refresh_factors_match_oracle(name, wl, masked):
    """The complex64 (64,64,64,33) and fp16 (64,64,64,64) workloads at full size: one
    refresh against the oracle's (Omega bit for bit, projectors and eigenvalues), with
    the Grams reading the residual copy (the complex one on the fp32 / complex Gram
    kernel) or the gradient through the bitmask (the general kernel)."""
    g = GradStream(wl, seed=3).next()
    lib, orc = make_lib(wl), make_oracle(wl)
    if masked:
        lib.set_gram_fusion(lib.set_gram_fusion(True), masked=True)
    lib.refresh(dev(g, wl.dtype))
    orc.refresh(g)
    torch.cuda.synchronize()
    assert np.array_equal(lib.get_omega(), orc.omega)
    factor_check(lib, orc)
    for n, w in enumerate(orc.eigvals):
        if w is not None:
            np.testing.assert_allclose(lib.get_eigvals(n), w, rtol=1e-4, atol=1e-5 * w[0])


# --------------------------------------------------------------------------- steps, pinned factors

STEP_CASES = FACTOR_CASES + [
    ("identity-middle", custom((10, 6, 8), "f32", (4, 6, 3), 0.05)),
    ("rank-one", custom((16, 12, 10), "f32", (1, 1, 1), 0.05, signal_ranks=(1, 1, 1))),
    ("k-zero", custom((10, 9, 8), "f32", (5, 4, 4), 0.0)),
]


@pytest.mark.parametrize("fused", [1, 4, 3, 2, 0], ids=["fused", "fused-rec2", "fused-two-mode-slabs",
                                                    "fused-tiles", "one-mode"])
@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: c[0])
def test_steps_with_pinned_omega_and_factors(case, fused):
    """Omega and U(n) injected from the oracle, so only the step kernels are compared;
    every launch plan (trailing modes per launch with the default kernel choice, which is
    one wave per slab for small 16-bit slabs and three-mode first projection and last
    reconstruction launches where they apply; the same with the two-mode reconstruction;
    the two-mode slab kernels only; workgroup tiles only; one mode per launch)."""
    name, wl = case
    gs = GradStream(wl, seed=8)
    W0 = init_weights(wl, seed=8)
    lib, orc = make_lib(wl, T=10 ** 6), make_oracle(wl, T=10 ** 6)
    if not lib.set_fusion(fused):
        pytest.skip("the two trailing modes are not both compressed")
    g1 = gs.next()
    orc.refresh(g1)
    lib.set_omega(orc.omega)
    for n, U in enumerate(orc.factors):
        if U is not None:
            lib.set_factor(n, U)
    lib.mark_refreshed()
    cap = DeltaCapture(lib, wl)
    align = CoreSplit(orc)
    W = dev(W0, wl.dtype)
    Wo = W0
    g = g1
    slack = 0.0
    for step in range(4):
        G = dev(g, wl.dtype)
        what = f"{name}/plan{fused} step {step + 1}"
        Wo, _ = checked_step(lib, orc, cap, W, Wo, g, wl, what, G=G, align=align)
        slack += wl.lr * 1e-5 * np.abs(orc.last["delta"]).max()
        # the gradient is only read
        assert np.array_equal(host(G, wl.dtype).view(np.uint8), np.ascontiguousarray(g).view(np.uint8)), \
            f"{name}: the step wrote to grad at step {step + 1}"
        crit = weight_check(host(W, wl.dtype), Wo, wl.dtype, what, delta_backed=True, slack=slack)
        print(f"WEIGHTS {what}: {crit}")
        g = gs.next()
    mc, vc, ms, vs = lib.get_moments()
    np.testing.assert_allclose(ms, orc.mS, rtol=1e-6, atol=1e-7)      # sparse path: same inputs
    np.testing.assert_allclose(vs, orc.vS, rtol=1e-6, atol=1e-12)
    scale = np.abs(orc.mC).max() + 1e-30
    assert np.abs(mc - orc.mC).max() <= 1e-4 * scale


# Single fp32 mode products on the streaming kernel: every tile of 64 trailing columns
# owned by one wave, loads a tile ahead. Cases: ragged last tiles (B not a multiple of
# 64), R not a multiple of 16, I not a multiple of 4, several leading indices, and more
# tiles than waves in the grid.
STREAM_CASES = [
    ("f32-40x60", custom((4, 40, 60, 12), "f32", (3, 20, 30, 6), 0.05), 0),
    ("bf16-64x30", custom((2, 64, 24, 16), "bf16", (2, 30, 12, 8), 0.05), 0),
    ("f16-tall-ragged", custom((3, 50, 7, 20), "f16", (2, 13, 5, 12), 0.05), 0),
    # 65 and 96 tiles for 8 and for 4 waves: each wave walks 8 to 24 tiles, ending after
    # either of its two register sets
    ("f32-many-tiles-2-wg", custom((24, 40, 52, 16), "f32", (12, 20, 26, 8), 0.02), 2),
    ("f32-many-tiles-1-wg", custom((24, 40, 52, 16), "f32", (12, 20, 26, 8), 0.02), 1),
    # contractions of 64 (16 k-steps) in the projection of a 64-wide mode
    ("f32-proj-64", custom((4, 64, 40, 16), "f32", (3, 32, 20, 8), 0.05), 0),
    # complex: the interleaved tensor as a real one, Re M and Im M in two accumulator
    # sets; rows of 16 complex values (half a tile); 64 output rows (four row blocks in
    # both sets); a 64-long contraction
    ("c64-40x48", custom((4, 40, 48, 6), "c64", (3, 20, 24, 3), 0.05), 0),
    ("c64-64x20-r64", custom((3, 64, 20, 8), "c64", (2, 32, 10, 4), 0.05), 0),
    ("c64-16-rows", custom((5, 24, 16, 1), "c64", (4, 12, 8, 1), 0.05), 0),
]


@pytest.mark.parametrize("fused", [1, 0], ids=["fused", "one-mode"])
@pytest.mark.parametrize("case", STREAM_CASES, ids=lambda c: c[0])
def test_stream_products_match_tiled_and_oracle(case, fused):
    """Two libraries with the oracle's Omega and factors, one with the streaming kernels
    for its single mode products and one with the tiled kernel only, over two steps. For
    real data whose last mode is not streamed as rows, the same fp32 update Delta bit
    for bit (both accumulate the same fp32 MFMA steps in the same k order), and Delta
    against the oracle's at the parity bar. For complex data (the streaming kernel sums
    the Re M and Im M products apart, the tiled one the real-block product) and where the
    last mode's products stream rows (their k order is permuted), each library's Delta
    against its own oracle run at the parity bar (rounding-level differences in the
    core gradient move Adam's first-step update sign(g) on near-zero entries, which the
    oracle comparison aligns and a library-to-library one cannot)."""
    name, wl, wg = case
    gs = GradStream(wl, seed=5)
    W0 = init_weights(wl, seed=5)
    libs = [make_lib(wl, T=10 ** 6), make_lib(wl, T=10 ** 6)]
    if wg:
        libs[0].set_stream_products(True, max_workgroups=wg)
    orcs = [make_oracle(wl, T=10 ** 6), make_oracle(wl, T=10 ** 6)]
    for lib in libs:
        if not lib.set_fusion(fused):
            pytest.skip("the two trailing modes are not both compressed")
        lib.set_pair_fusion(False)
    libs[1].set_stream_products(False)
    g = gs.next()
    for orc in orcs:
        orc.refresh(g)
    caps = []
    for lib in libs:
        lib.set_omega(orcs[0].omega)
        for n, U in enumerate(orcs[0].factors):
            if U is not None:
                lib.set_factor(n, U)
        lib.mark_refreshed()
        caps.append(DeltaCapture(lib, wl))
    aligns = [CoreSplit(orc) for orc in orcs]
    Ws = [dev(W0, wl.dtype), dev(W0, wl.dtype)]
    Wos = [W0, W0]
    for step in range(2):
        what = f"{name}/plan{fused} step {step + 1}"
        libs[0].timing_enable(True)
        Wos[0], _ = checked_step(libs[0], orcs[0], caps[0], Ws[0], Wos[0], g, wl, what,
                                 align=aligns[0])
        rec = libs[0].timing_read()
        assert "streamprod_reconstruct" in rec, (what, sorted(rec))
        if name.endswith("proj-64"):
            assert "streamprod_project" in rec, (what, sorted(rec))
        rows = "rowprod_project" in rec or "rowprod_reconstruct_apply" in rec
        if wl.dtype == "c64" or rows:
            Wos[1], _ = checked_step(libs[1], orcs[1], caps[1], Ws[1], Wos[1], g, wl,
                                     what + " (tiled)", align=aligns[1])
        else:
            libs[1].step(Ws[1], dev(g, wl.dtype))
            orcs[1].step(Wos[1], g)
            assert np.array_equal(caps[0].host(), caps[1].host()), f"{what}: streamed Delta differs"
            assert np.array_equal(host(Ws[0], wl.dtype).view(np.uint8),
                                  host(Ws[1], wl.dtype).view(np.uint8))
        g = gs.next()


# The row stream over the last mode (one-mode plan: the first projection, with the COO
# gather on the gradient's rows, and the weight-updating last reconstruction). Cases:
# a row tail inside the last group of values (K not a multiple of 16 or 32), ragged
# 16-row tiles, 16-bit and complex rows (complex rows of 62 and 80 fp32 values, the
# latter five groups), many Omega entries, no sparse part, and a factor too large for
# registers (the tiled kernel then runs).
ROW_CASES = [
    ("f32-tail-23", custom((37, 5, 23), "f32", (20, 5, 11), 0.05), True),
    ("bf16-tail-46", custom((9, 13, 46), "bf16", (5, 13, 20), 0.05), True),
    ("f16-64-dense-omega", custom((11, 7, 64), "f16", (6, 7, 32), 0.3), True),
    ("c64-31", custom((7, 9, 31), "c64", (4, 9, 12), 0.05), True),
    ("c64-40-five-groups", custom((6, 5, 40), "c64", (3, 5, 8), 0.05), True),
    ("f32-k0", custom((12, 6, 20), "f32", (6, 6, 10), 0.0), True),
    ("f32-factor-too-large", custom((8, 10, 80), "f32", (4, 10, 64), 0.05), False),
]


@pytest.mark.parametrize("case", ROW_CASES, ids=lambda c: c[0])
def test_row_products_match_oracle(case):
    """The one-mode plan with Omega and factors pinned from the oracle, over two steps:
    the last mode's products run on the row kernel where the factor fits in registers
    (else on the tiled kernel), Delta against the oracle's at the parity bar, the
    weight update bit for bit against the rounding of the library's own Delta, the
    sparse moments against the oracle's (S comes from the fused gather), and the
    gradient untouched."""
    name, wl, rows = case
    gs = GradStream(wl, seed=3)
    W0 = init_weights(wl, seed=3)
    lib, orc = make_lib(wl, T=10 ** 6), make_oracle(wl, T=10 ** 6)
    assert lib.set_fusion(0)
    g = gs.next()
    orc.refresh(g)
    lib.set_omega(orc.omega)
    for n, U in enumerate(orc.factors):
        if U is not None:
            lib.set_factor(n, U)
    lib.mark_refreshed()
    cap = DeltaCapture(lib, wl)
    align = CoreSplit(orc)
    W, Wo = dev(W0, wl.dtype), W0
    for step in range(2):
        what = f"{name} step {step + 1}"
        G = dev(g, wl.dtype)
        before = host(G, wl.dtype).copy()
        lib.timing_enable(True)
        Wo, _ = checked_step(lib, orc, cap, W, Wo, g, wl, what, G=G, align=align)
        rec = lib.timing_read()
        got = "rowprod_project" in rec and "rowprod_reconstruct_apply" in rec
        assert got == rows, (what, sorted(rec))
        if rows and wl.k > 0:
            assert "gather_residual" not in rec, (what, sorted(rec))
        if wl.k > 0:
            mS = lib.get_moments()[2]
            np.testing.assert_allclose(mS, orc.mS.reshape(-1), rtol=1e-5,
                                       atol=1e-6 * np.abs(orc.mS).max(), err_msg=what)
        assert np.array_equal(host(G, wl.dtype).view(np.uint8), before.view(np.uint8)), what
        g = gs.next()


# --------------------------------------------------------------------------- independent runs

RUN_CASES = [
    ("tiny-fp32-8x8x6x6", TINY_F32, None),
    ("fp32-32x32x16x16", F32_32x32x16x16, None),
    ("bf16-odd", custom((33, 17, 60), "bf16", (13, 8, 31), 0.05, T=4, steps=9), None),
    ("c64-small", custom((12, 10, 9), "c64", (5, 4, 3), 0.05, T=3, steps=7), None),
    ("fp16-64x64x64x64-one-layer-3-steps", F16_4x64x64x64x64, 3),
    ("c64-64x64x64x33-3-steps", C64_64x64x64x33, 3),
]


@pytest.mark.parametrize("case", RUN_CASES, ids=lambda c: c[0])
def test_independent_runs_match_oracle(case):
    """Each side refreshes on its own schedule; Omega bit-exact at every refresh."""
    name, wl, nsteps = case
    nsteps = nsteps or wl.steps
    gs = GradStream(wl, seed=0)
    W0 = init_weights(wl, seed=0)
    lib, orc = make_lib(wl), make_oracle(wl)
    W = dev(W0, wl.dtype)
    Wo = W0
    for t in range(1, nsteps + 1):
        g = gs.next()
        lib.step(W, dev(g, wl.dtype))
        Wo = orc.step(Wo, g)
        if (t - 1) % wl.T == 0:
            torch.cuda.synchronize()
            assert np.array_equal(lib.get_omega(), orc.omega), f"{name}: Omega differs at t={t}"
            factor_check(lib, orc)
    torch.cuda.synchronize()
    weight_check(host(W, wl.dtype), Wo, wl.dtype, f"{name} after {nsteps} steps")


# --------------------------------------------------------------------------- exact reductions

@pytest.mark.parametrize("dtype", ["f32", "c64", "bf16", "f16"])
def test_full_rank_k0_is_bitwise_oracle(dtype):
    """Full Tucker ranks and k = 0: the step is dense Adam; with identical inputs the fp32
    arithmetic is the same operation sequence on both sides, so W matches bit for bit."""
    shape = (6, 5, 4, 3)
    wl = custom(shape, dtype, shape, 0.0, T=5, steps=10, signal_ranks=(2, 2, 2, 2))
    gs = GradStream(wl, seed=21)
    W0 = init_weights(wl, seed=21)
    lib, orc = make_lib(wl), make_oracle(wl)
    W, Wo = dev(W0, dtype), W0
    for _ in range(10):
        g = gs.next()
        lib.step(W, dev(g, dtype))
        Wo = orc.step(Wo, g)
    torch.cuda.synchronize()
    assert np.array_equal(host(W, dtype).view(np.uint8), np.ascontiguousarray(Wo).view(np.uint8))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rho_one_is_bitwise_oracle(dtype):
    """rho = 1: the sparse part is the whole gradient, the core is zero and its Adam
    update is exactly zero, so W follows dense Adam on S bit for bit."""
    shape = (6, 5, 4, 3)
    wl = custom(shape, dtype, (3, 2, 2, 1), 1.0, T=5, steps=8, signal_ranks=(2, 2, 2, 1))
    gs = GradStream(wl, seed=4)
    W0 = init_weights(wl, seed=4)
    lib, orc = make_lib(wl), make_oracle(wl)
    W, Wo = dev(W0, dtype), W0
    for _ in range(8):
        g = gs.next()
        lib.step(W, dev(g, dtype))
        Wo = orc.step(Wo, g)
    torch.cuda.synchronize()
    assert np.array_equal(host(W, dtype).view(np.uint8), np.ascontiguousarray(Wo).view(np.uint8))


def test_deterministic_rerun():
    wl = F32_32x32x16x16
    outs = []
    for _ in range(2):
        gs = GradStream(wl, seed=2)
        lib = make_lib(wl)
        W = dev(init_weights(wl, seed=2), wl.dtype)
        for _ in range(12):
            lib.step(W, dev(gs.next(), wl.dtype))
        torch.cuda.synchronize()
        outs.append((host(W, wl.dtype), [lib.get_factor(n) for n in range(4)], lib.get_omega()))
    assert np.array_equal(outs[0][0], outs[1][0])
    for a, b in zip(outs[0][1], outs[1][1]):
        assert np.array_equal(a, b)
    assert np.array_equal(outs[0][2], outs[1][2])


def test_misaligned_grad_is_rejected():
    """grad is read in 16-byte pieces: a view 2 bytes off is refused with EINVAL before
    any work, and the handle still steps afterwards."""
    wl = custom((8, 6, 5), "bf16", (4, 3, 5), 0.1, T=2)
    lib = make_lib(wl)
    G = dev(GradStream(wl, seed=1).next(), "bf16")
    W = dev(init_weights(wl, seed=1), "bf16")
    buf = torch.zeros(G.numel() + 8, dtype=torch.bfloat16, device="cuda")
    bad = buf[1:1 + G.numel()]
    assert bad.data_ptr() % 16 != 0
    with pytest.raises(tg.TGradError, match="invalid argument"):
        lib.step(W, bad)
    with pytest.raises(tg.TGradError, match="invalid argument"):
        lib.refresh(bad)
    assert lib.t == 0
    lib.step(W, G)
    torch.cuda.synchronize()
    assert lib.t == 1


@pytest.mark.parametrize("name,wl", [("fp32-32x32x16x16", F32_32x32x16x16),
                                     ("c64-small", custom((12, 10, 9), "c64", (5, 4, 3), 0.05, T=3, steps=7))],
                         ids=lambda x: x if isinstance(x, str) else "")
def test_checkpoint_resume_is_exact(name, wl):
    """Save after n1 steps, restore into a fresh handle, continue across a refresh:
    weights, moments, Omega, factors and the step count match an uninterrupted run bit
    for bit, and the resumed run matches the oracle run through all n1 + n2 steps (Omega
    bit for bit at every refresh, factors within the projector bar, weights within the
    weight bar). A state for another shape is refused."""
    n1, n2 = 4, 5
    gs = GradStream(wl, seed=5)
    grads = [gs.next() for _ in range(n1 + n2)]
    W0 = init_weights(wl, seed=5)
    orc = make_oracle(wl, T=4)
    Wo = W0
    for g in grads[:n1]:
        Wo = orc.step(Wo, g)
    a = make_lib(wl, T=4)
    Wa = dev(W0, wl.dtype)
    for g in grads:
        a.step(Wa, dev(g, wl.dtype))
    b = make_lib(wl, T=4)
    Wb = dev(W0, wl.dtype)
    for g in grads[:n1]:
        b.step(Wb, dev(g, wl.dtype))
    state = b.save_state()
    b.close()
    c = make_lib(wl, T=4)
    c.load_state(state)
    assert c.t == n1
    for i, g in enumerate(grads[n1:]):
        c.step(Wb, dev(g, wl.dtype))
        Wo = orc.step(Wo, g)
        if (n1 + i) % 4 == 0:     # step n1 + i + 1 refreshed
            torch.cuda.synchronize()
            assert np.array_equal(c.get_omega(), orc.omega)
            factor_check(c, orc)
    torch.cuda.synchronize()
    weight_check(host(Wb, wl.dtype), Wo, wl.dtype, f"{name} resumed run")
    assert np.array_equal(host(Wa, wl.dtype).view(np.uint8), host(Wb, wl.dtype).view(np.uint8))
    for x, y in zip(a.get_moments(), c.get_moments()):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(a.get_omega(), c.get_omega())
    for n, (I, r) in enumerate(zip(wl.shape, wl.ranks)):
        if r < I:
            assert np.array_equal(a.get_factor(n).view(np.uint32), c.get_factor(n).view(np.uint32))
    assert a.t == c.t == n1 + n2
    other = tg.TGrad(tuple(x + 1 for x in wl.shape), wl.ranks, wl.dtype, wl.sparse_ratio, 4)
    with pytest.raises(tg.TGradError, match="invalid argument"):
        other.load_state(state)


def test_checkpoint_refuses_other_hyperparameters():
    """A saved state resumes only into a handle with the same refresh period, Adam betas
    and eps, and options; a different learning rate (a schedule) is accepted."""
    wl = F32_32x32x16x16
    a = make_lib(wl, T=4)
    W = dev(init_weights(wl, seed=1), wl.dtype)
    a.step(W, dev(GradStream(wl, seed=1).next(), wl.dtype))
    state = a.save_state()

    def fresh(T=4, lr=wl.lr, betas=wl.betas, eps=wl.eps, **opts):
        h = tg.TGrad(wl.shape, wl.ranks, wl.dtype, wl.sparse_ratio, T, lr, betas, eps)
        if opts:
            h.set_options(**opts)
        return h

    for bad in (dict(T=5), dict(betas=(0.8, 0.999)), dict(betas=(0.9, 0.99)), dict(eps=1e-6),
                dict(selection="randk"), dict(seed=3), dict(weight_decay=1e-4),
                dict(sparse_scale=0.5), dict(remap_moments=True), dict(order="lowrank_first")):
        h = fresh(**bad)
        with pytest.raises(tg.TGradError, match="invalid argument"):
            h.load_state(state)
        assert h.t == 0, bad
    h = fresh(lr=3e-4)
    h.load_state(state)
    assert h.t == 1


def test_timing_records_every_kernel():
    wl = F32_32x32x16x16
    lib = make_lib(wl)
    lib.timing_enable(True)
    gs = GradStream(wl)
    W = dev(init_weights(wl), wl.dtype)
    for _ in range(3):
        lib.step(W, dev(gs.next(), wl.dtype))
    rec = lib.timing_read()
    for name in ("topk_hist", "topk_compact", "modeprod2_project_first",
                 "modeprod_pair_project", "adam_fused", "modeprod_pair_reconstruct",
                 "modeprod2_reconstruct_apply", "gram", "eigensolver"):
        assert name in rec, name
    assert "gather_residual" not in rec        # folded into the fused first projection
    assert "modeprod_project" not in rec       # modes 1 and 0 in one launch
    assert rec["adam_fused"][0] == 3
    assert rec["modeprod2_project_first"][0] == 3
    assert rec["modeprod_pair_project"][0] == 3 and rec["modeprod_pair_reconstruct"][0] == 3
    assert lib.set_pair_fusion(False)
    lib.step(W, dev(gs.next(), wl.dtype))
    rec = lib.timing_read()
    # modes 1 and 0 one by one, on the streaming kernel (trailing parts of 64 and 1024)
    assert rec["streamprod_project"][0] == 2 and rec["streamprod_reconstruct"][0] == 2
    assert "modeprod_pair_project" not in rec
    lib.set_stream_products(False)
    lib.step(W, dev(gs.next(), wl.dtype))
    rec = lib.timing_read()
    assert rec["modeprod_project"][0] == 2 and rec["modeprod_reconstruct"][0] == 2
    assert "streamprod_project" not in rec and "streamprod_reconstruct" not in rec
    assert lib.set_fusion(False)
    lib.step(W, dev(gs.next(), wl.dtype))
    rec = lib.timing_read()
    assert rec["modeprod_project_first"][0] == 1 and rec["modeprod_reconstruct_apply"][0] == 1
    assert rec["gather_residual"][0] == 1


def test_launch_record_matches_the_launches():
    """tgrad_last_launches lists exactly the launches the timing records see, and on the
    one-mode-per-launch plan its algorithmic bytes and flops are the hand count: each
    mode product reads its input once and writes its output once (fp32), the gather reads
    k indices and k values and writes k fp32 values and k zeros, Adam moves 24 B per core
    and sparse value, the last product also reads and writes W and reads the k indices
    and sparse updates. With the sparse values' Adam update on the second stream (the
    default, when the first projection takes the gather) it is its own launch,
    adam_sparse, right after that first projection, and adam_fused covers the core."""
    wl = F32_32x32x16x16
    for overlap in (2, 0):
        lib = make_lib(wl)
        assert lib.set_fusion(False)
        lib.set_adam_overlap(overlap)
        gs = GradStream(wl)
        W = dev(init_weights(wl), wl.dtype)
        lib.step(W, dev(gs.next(), wl.dtype))          # t = 1 refreshes
        names = [n for n, *_ in lib.last_launches()]
        assert names[:3] == ["topk_hist", "topk_count", "topk_compact"] and "eigensolver" in names
        lib.timing_enable(True)
        lib.step(W, dev(gs.next(), wl.dtype))
        rec = lib.timing_read()
        got = lib.last_launches()
        counts = {}
        for n, *_ in got:
            counts[n] = counts.get(n, 0) + 1
        assert counts == {n: c for n, (c, _) in rec.items()}
        _check_launch_record(wl, got, overlap)
        lib.close()


def _check_launch_record(wl, got, overlap):
    N, k, es = wl.numel, wl.k, 4
    shape, ranks = list(wl.shape), list(wl.ranks)

    def streams(cur, n, I, R):
        # the streaming kernel's documented conditions (fp32 in and out, no apply)
        B = int(np.prod(cur[n + 1:], dtype=np.int64))
        return I <= 64 and R <= 64 and B >= 32 and B % 4 == 0

    def rows(I, R):
        # the last mode's row kernel: the factor in registers (fp32 rows: groups of 16)
        nq, ncb = -(-I // 16), -(-R // 16)
        return nq <= 5 and ncb <= 5 and nq * 4 * ncb <= 64

    # the COO gather: its own launch on a copy of G, unless the first projection is the
    # row stream over the last mode, which takes it (k indices read, k values written)
    row_gather = rows(shape[3], ranks[3])
    exp = [] if row_gather else [("gather_residual", k * (4 + es) + k * (4 + es), 0)]
    cur, size = list(shape), N
    for j, n in enumerate([3, 2, 1, 0]):
        out = size // cur[n] * ranks[n]
        name = "modeprod_project_first" if j == 0 else "modeprod_project"
        if streams(cur, n, cur[n], ranks[n]):
            name = "streamprod_project"
        if n == 3 and rows(cur[n], ranks[n]):
            name = "rowprod_project"
        gb = 8 * k if (j == 0 and row_gather) else 0
        exp.append((name, size * 4 + out * 4 + gb, 2 * (size // cur[n]) * cur[n] * ranks[n]))
        if j == 0 and row_gather and overlap == 2:
            exp.append(("adam_sparse", k * 24, 0))
        cur[n] = ranks[n]
        size = out
    ncore = size
    forked = row_gather and overlap == 2
    exp.append(("adam_fused", (ncore + (0 if forked else k)) * 24, 0))
    for j, n in enumerate([0, 1, 2, 3]):
        out = size // cur[n] * shape[n]
        last = j == 3
        b = size * 4 + ((2 * N * es + 8 * k) if last else out * 4)
        name = "modeprod_reconstruct_apply" if last else "modeprod_reconstruct"
        if not last and streams(cur, n, cur[n], shape[n]):
            name = "streamprod_reconstruct"
        if last and rows(cur[n], shape[n]):
            name = "rowprod_reconstruct_apply"
        exp.append((name, b, 2 * (size // cur[n]) * cur[n] * shape[n]))
        cur[n] = shape[n]
        size = out
    assert sum(n.startswith("streamprod") for n, *_ in exp) == 4   # modes 1 and 0 both ways
    assert [(n, br + bw, fl) for n, _m, br, bw, fl in got] == exp


def test_timing_only_one_kernel():
    wl = F32_32x32x16x16
    lib = make_lib(wl)
    gs = GradStream(wl)
    W = dev(init_weights(wl), wl.dtype)
    lib.step(W, dev(gs.next(), wl.dtype))          # the refresh step, untimed
    lib.timing_only("adam_fused")
    lib.timing_enable(True)
    for _ in range(2):
        lib.step(W, dev(gs.next(), wl.dtype))
    rec = lib.timing_read()
    assert list(rec) == ["adam_fused"] and rec["adam_fused"][0] == 2
    assert rec["adam_fused"][1] > 0.0
    lib.timing_only(None)
    lib.step(W, dev(gs.next(), wl.dtype))
    rec = lib.timing_read()
    assert "adam_fused" in rec and "modeprod2_reconstruct_apply" in rec
    with pytest.raises(ValueError):
        lib.timing_only("no_such_kernel")


# --------------------------------------------------------------------------- full size, bf16 (64,64,48,48,25)

@pytest.mark.timeout(900)
def test_bf16_64x64x48x48x25_full_size_two_steps():
    """bf16 (64,64,48,48,25), the full tensor, two steps: the first in the bench's launch
    plan (three-mode reconstruction), the second with the two-mode reconstruction.

    Step 1 refreshes: Omega is checked by its complete characterisation (no sort of 236M
    keys), each factor's projector against the fp64 Gram eigenvectors of the residual.
    Then the oracle steps with the library's Omega and factors (set into it, as they came
    from the refresh), and both steps are compared in full (CoreSplit): the core Adam
    moments (1e-5 of the largest), the fp32 update Delta of every element against the
    oracle's reconstruction of the library's core update plus its own sparse update
    (relative max-norm 1e-5), the weight update as the exact rounding of W - lr Delta,
    all 235.9M weights against the oracle's update of the same W, and the sparse
    moments."""
    wl = BF16_64x64x48x48x25
    gs = GradStream(wl, seed=0)
    g = gs.next()
    W0 = init_weights(wl, seed=0)
    lib = make_lib(wl)
    cap = DeltaCapture(lib, wl)
    G = dev(g, wl.dtype)
    W = dev(W0, wl.dtype)
    print("CASE bf16-(64,64,48,48,25) step 1 (refresh)", flush=True)
    lib.step(W, G)          # t = 1: refresh, then the step
    torch.cuda.synchronize()
    om = lib.get_omega()
    omega_properties(O.topk_keys(g, wl.dtype), om, wl.k)
    assert np.array_equal(host(G, wl.dtype).view(np.uint8), g.view(np.uint8))   # only read
    R32 = O.decode(g, wl.dtype).reshape(-1).copy()
    R32[om] = 0
    R = R32.reshape(wl.shape)
    del R32
    Us = []
    for n in range(5):
        Ug = lib.get_factor(n)
        Uo, w, gap = O.hosvd_factor(R, n, wl.ranks[n])
        err = np.abs(Ug.astype(np.float64) @ Ug.T.astype(np.float64)
                     - Uo.astype(np.float64) @ Uo.T.astype(np.float64)).max()
        assert err <= 1e-4, (n, err, gap)
        Us.append(Ug)
    del R
    assert lib.get_info().eig_unconverged == 0
    # the oracle, stepped with the library's refresh outcome
    orc = make_oracle(wl)
    orc.omega = om.copy()
    orc.factors = Us
    orc.refreshed_for = 1
    align = CoreSplit(orc)
    Wprev, Wo = W0, W0
    for t in (1, 2):
        if t == 2:
            # the second step in the plan with the two-mode reconstruction
            assert lib.set_fusion(4)
            g = gs.next()
            print("CASE bf16-(64,64,48,48,25) step 2 (two-mode reconstruction)", flush=True)
            Wprev = host(W, wl.dtype)
            lib.step(W, dev(g, wl.dtype))
            torch.cuda.synchronize()
        Wo = orc.step(Wo, g)
        dg = cap.host()
        Wg = host(W, wl.dtype)
        apply_check(Wprev, Wg, dg, wl.dtype, wl.lr, what=f"step {t}")
        expected, n_steep, du = align.expected_delta(lib, t)
        rel = delta_rel(dg, expected)
        print(f"DELTA bf16-(64,64,48,48,25) step {t}: rel {rel:.3e} (against the oracle's own "
              f"Delta: {delta_rel(dg, orc.last['delta']):.3e}; steep core entries {n_steep}, "
              f"max |du| {du:.2e})", flush=True)
        assert n_steep <= 1e-4 * orc.mC.size, n_steep
        assert rel <= 1e-5, (t, rel)
        # every weight against the oracle's update of the same W: the rounding of
        # W - lr Delta with the oracle's Delta (reconstructed from the library's core
        # update, as above); at most one bf16 ulp apart where the two fp32 values straddle
        # a rounding boundary
        w32 = O.real_view(O.decode(Wprev, wl.dtype))
        Wexp = O.encode((w32 - np.float32(wl.lr) * expected.astype(np.float32)).reshape(wl.shape),
                        wl.dtype)
        slack = wl.lr * 1e-5 * np.abs(expected).max()
        crit = weight_check(Wg, Wexp, wl.dtype, f"bf16-(64,64,48,48,25) step {t}", delta_backed=True,
                            slack=slack)
        print(f"WEIGHTS bf16-(64,64,48,48,25) step {t}: {crit}", flush=True)
        del expected, w32, Wexp
        _, _, ms, vs = lib.get_moments()
        np.testing.assert_allclose(ms, orc.mS, rtol=1e-6, atol=1e-7)
        np.testing.assert_allclose(vs, orc.vS, rtol=1e-6, atol=1e-12)
        del dg, Wg, ms, vs
