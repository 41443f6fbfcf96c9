"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names the fact it pins: brute-force definitions on tiny inputs, exact
rational arithmetic, torch.optim.Adam, torch's rounding casts, and the identities the
pages state (Tucker/HOSVD, stable rank, the dense-Adam reductions, eq. (10))."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from synth import (TINY_F32, F32_32x32x16x16, F16_4x64x64x64x64, C64_64x64x64x33, BF16_64x64x48x48x25,
                   GradStream, init_weights)
from synth.gen import custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- mode algebra

def _brute_mode_product(X, M, n):
    shp = list(X.shape)
    out_shape = shp.copy()
    out_shape[n] = M.shape[0]
    Y = np.zeros(out_shape, dtype=np.result_type(X, M))
    for idx in itertools.product(*[range(s) for s in out_shape]):
        acc = 0
        for i in range(shp[n]):
            src = list(idx)
            src[n] = i
            acc += M[idx[n], i] * X[tuple(src)]
        Y[idx] = acc
    return Y


@pytest.mark.parametrize("cplx", [False, True])
def test_mode_product_matches_definition(cplx):
    r = rng(1)
    X = r.standard_normal((3, 4, 2, 5))
    if cplx:
        X = X + 1j * r.standard_normal(X.shape)
    for n in range(4):
        M = r.standard_normal((2, X.shape[n]))
        if cplx:
            M = M + 1j * r.standard_normal(M.shape)
        np.testing.assert_allclose(O.mode_product(X, M, n), _brute_mode_product(X, M, n),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("cplx", [False, True])
def test_gram_matches_definition(cplx):
    r = rng(2)
    X = r.standard_normal((3, 4, 2, 3))
    if cplx:
        X = X + 1j * r.standard_normal(X.shape)
    for n in range(4):
        I = X.shape[n]
        ref = np.zeros((I, I), dtype=X.dtype)
        for i in range(I):
            for j in range(I):
                a = np.take(X, i, axis=n)
                b = np.take(X, j, axis=n)
                ref[i, j] = np.sum(a * np.conj(b))
        np.testing.assert_allclose(O.gram(X, n), ref, rtol=1e-12, atol=1e-12)


def test_projection_uses_conjugate_transpose():
    r = rng(3)
    R = (r.standard_normal((4, 3)) + 1j * r.standard_normal((4, 3))).astype(np.complex64)
    U = np.linalg.qr(r.standard_normal((4, 2)) + 1j * r.standard_normal((4, 2)))[0].astype(np.complex64)
    C = O.project(R, [U, None])
    for j in range(2):
        for b in range(3):
            ref = sum(np.conj(complex(U[i, j])) * complex(R[i, b]) for i in range(4))
            assert abs(C[j, b] - ref) < 1e-6
    # a full unitary factor makes project -> reconstruct the identity
    Uf = np.linalg.qr(r.standard_normal((4, 4)) + 1j * r.standard_normal((4, 4)))[0]
    back = O.reconstruct(O.project(R, [Uf, None]), [Uf, None])
    np.testing.assert_allclose(back, R, atol=1e-6)


# --------------------------------------------------------------------------- top-k

def _exact_mag2(v):
    if np.isinf(v).any() if np.iscomplexobj(v) else np.isinf(v):
        return float("inf")
    if isinstance(v, complex) or np.iscomplexobj(v):
        v = complex(v)
        return Fraction(v.real) ** 2 + Fraction(v.imag) ** 2
    return abs(Fraction(float(v)))


def _brute_topk(G32, k):
    flat = np.asarray(G32).reshape(-1)
    order = sorted(range(flat.size), key=lambda i: (-_exact_mag2(flat[i]), i))
    return np.array(sorted(order[:k]), dtype=np.uint32)


def _tiny_cases():
    r = rng(4)
    out = []
    base = r.standard_normal(60).astype(np.float32)
    out.append(("random", base))
    out.append(("quantized-ties", (np.round(base * 2) / 2).astype(np.float32)))
    out.append(("all-equal", np.full(37, -1.5, np.float32)))
    z = np.zeros(24, np.float32)
    z[::3] = -0.0
    z[5] = 1e-42            # subnormal
    z[7] = -1e-42
    z[11] = 2e-42
    out.append(("signed-zeros-subnormals", z))
    inf = base[:20].copy()
    inf[3] = np.inf
    inf[9] = -np.inf
    out.append(("infinities", inf))
    return out


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_topk_matches_brute_force(dtype):
    for name, x in _tiny_cases():
        G = O.encode(x, dtype)
        G32 = O.decode(G, dtype)
        N = G32.size
        for k in sorted({0, 1, N // 3, N // 2, N - 1, N}):
            got = O.select_omega(O.topk_keys(G, dtype), k)
            exp = _brute_topk(G32, k)
            assert np.array_equal(got, exp), (dtype, name, k)


def test_topk_complex_matches_brute_force():
    r = rng(5)
    re = r.standard_normal(50).astype(np.float32)
    im = r.standard_normal(50).astype(np.float32)
    G = (re + 1j * im).astype(np.complex64)
    G[7] = G[3]                      # exact duplicates -> index tie-break
    G[20] = np.conj(G[3])            # same magnitude, different phase
    G[30] = 1j * G[3].real + G[3].imag   # swapped parts: same |z|^2
    for k in (0, 1, 10, 25, 49, 50):
        got = O.select_omega(O.topk_keys(G, "c64"), k)
        assert np.array_equal(got, _brute_topk(G, k)), k


def test_topk_nan_ranks_above_inf():
    x = np.array([1.0, np.inf, np.nan, 3.0, -np.nan], np.float32)
    got = O.select_omega(O.topk_keys(x, "f32"), 3)
    assert set(got.tolist()) == {1, 2, 4}
    z = np.array([1 + 1j, complex(np.nan, 0), complex(np.inf, 0), 2j], np.complex64)
    got = O.select_omega(O.topk_keys(z, "c64"), 2)
    assert set(got.tolist()) == {1, 2}


# --------------------------------------------------------------------------- residual

@pytest.mark.parametrize("dtype", ["f32", "bf16", "c64"])
def test_residual_plus_scatter_is_gradient(dtype):
    wl = custom((6, 5, 4), dtype, (3, 3, 2), 0.1)
    G = GradStream(wl, seed=9).next()
    G32 = O.decode(G, dtype)
    om = O.select_omega(O.topk_keys(G, dtype), wl.k)
    S = O.gather(G32, om)
    R = O.residual(G32, om)
    back = R.copy().reshape(-1)
    back[om.astype(np.int64)] = S
    assert np.array_equal(back.view(np.uint8), np.ascontiguousarray(G32).reshape(-1).view(np.uint8))
    mask = np.zeros(G32.size, bool)
    mask[om] = True
    assert np.all(R.reshape(-1)[mask] == 0)
    assert np.array_equal(R.reshape(-1)[~mask], G32.reshape(-1)[~mask])


# --------------------------------------------------------------------------- factors

@pytest.mark.parametrize("cplx", [False, True])
def test_factors_orthonormal_eigen_canonical(cplx):
    wl = custom((10, 9, 8, 7), "c64" if cplx else "f32", (5, 4, 4, 3), 0.05)
    G = GradStream(wl, seed=11).next()
    o = O.TGradOracle(wl.shape, wl.ranks, wl.dtype, wl.sparse_ratio, wl.T, wl.lr, *wl.betas, wl.eps)
    o.refresh(G)
    R = O.residual(O.decode(G, wl.dtype), o.omega)
    for n, U in enumerate(o.factors):
        Ud = U.astype(np.complex128 if cplx else np.float64)
        np.testing.assert_allclose(Ud.conj().T @ Ud, np.eye(U.shape[1]), atol=2e-6)
        H = O.gram(R, n)
        lam = o.eigvals[n][:U.shape[1]]
        resid = H @ Ud - Ud * lam[None, :]
        assert np.linalg.norm(resid) <= 1e-5 * np.linalg.norm(H)
        assert np.all(np.diff(o.eigvals[n]) <= 1e-9 * o.eigvals[n][0])     # descending
        for c in range(U.shape[1]):
            i = int(np.argmax(np.abs(Ud[:, c])))
            assert abs(Ud[i, c].imag) < 1e-6 and Ud[i, c].real > 0


def _hosvd_full(R, ranks):
    """fp64 factors and spectra (not rounded to fp32), via the oracle's Gram."""
    Us, lams = [], []
    for n, r in enumerate(ranks):
        w, V = np.linalg.eigh(O.gram(R, n))
        Us.append(V[:, ::-1][:, :r])
        lams.append(w[::-1])
    return Us, lams


@pytest.mark.parametrize("cplx", [False, True])
def test_hosvd_truncation_error_identities(cplx):
    """Textbook truncated HOSVD: one truncated mode loses exactly the discarded Gram
    eigenvalues; all modes truncated lose at most their sum, and exactly the telescoped
    sum of the per-mode losses."""
    r = rng(12)
    R = r.standard_normal((8, 7, 6, 5))
    if cplx:
        R = R + 1j * r.standard_normal(R.shape)
    ranks = (3, 4, 2, 3)
    Us, lams = _hosvd_full(R, ranks)
    nrm2 = np.vdot(R, R).real
    for n in range(4):
        P = Us[n] @ Us[n].conj().T
        err = R - O.mode_product(R, P, n)
        np.testing.assert_allclose(np.vdot(err, err).real, lams[n][ranks[n]:].sum(), rtol=1e-10,
                                   atol=1e-12 * nrm2)
    L = O.reconstruct(O.project(R, Us), Us)
    total = np.vdot(R - L, R - L).real
    bound = sum(l[rk:].sum() for l, rk in zip(lams, ranks))
    assert total <= bound * (1 + 1e-10)
    tele, X = 0.0, R.copy()
    for n in range(4):
        P = Us[n] @ Us[n].conj().T
        Xp = O.mode_product(X, P, n)
        tele += np.vdot(X - Xp, X - Xp).real
        X = Xp
    np.testing.assert_allclose(total, tele, rtol=1e-9)


def test_noise_free_tucker_is_lossless():
    r = rng(13)
    shape, sranks = (12, 10, 8, 6), (3, 2, 2, 1)
    core = r.standard_normal(sranks)
    facs = [np.linalg.qr(r.standard_normal((i, s)))[0] for i, s in zip(shape, sranks)]
    X = O.reconstruct(core, facs)
    ranks = (4, 3, 2, 2)
    Us, lams = _hosvd_full(X, ranks)
    for n, s in enumerate(sranks):
        assert np.all(np.abs(lams[n][s:]) <= 1e-13 * lams[n][0])     # Gram rank = signal rank
        assert lams[n][s - 1] > 1e-6 * lams[n][0]
    back = O.reconstruct(O.project(X, Us), Us)
    np.testing.assert_allclose(back, X, atol=1e-12)


def test_stable_rank_properties():
    """Mode-k stable rank sr_k = ||T||_F^2 / ||T_(k)||_2^2: >= 1, <= rank(T_(k)), = 1 for a
    rank-1 tensor, invariant under an orthogonal transform in mode k (App. K)."""
    r = rng(14)

    def sr(T, k):
        H = O.gram(T, k)
        return np.trace(H).real / np.linalg.eigvalsh(H)[-1]

    T = r.standard_normal((6, 5, 4))
    for k in range(3):
        s = sr(T, k)
        assert 1 - 1e-12 <= s <= np.linalg.matrix_rank(O.unfold(T, k)) + 1e-9
        Q = np.linalg.qr(r.standard_normal((T.shape[k], T.shape[k])))[0]
        assert abs(sr(O.mode_product(T, Q, k), k) - s) < 1e-9
    a, b, c = r.standard_normal(6), r.standard_normal(5), r.standard_normal(4)
    rank1 = np.einsum("i,j,k->ijk", a, b, c)
    for k in range(3):
        assert abs(sr(rank1, k) - 1) < 1e-12


def test_eq10_parameter_count():
    with open(os.path.join(GOLDEN, "eq10_param_count.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        N, M, r = case["N"], case["M"], case["r"]
        expected = r ** 4 + 2 * r * N + 2 * r * M
        assert O.lowrank_param_count((N, N, M, M), (r, r, r, r)) == expected


# --------------------------------------------------------------------------- Adam reductions

def _torch_adam_run(W0, grads, wl):
    p = torch.nn.Parameter(torch.from_numpy(O.decode(W0, wl.dtype).copy()))
    opt = torch.optim.Adam([p], lr=wl.lr, betas=wl.betas, eps=wl.eps, foreach=False)
    for g in grads:
        p.grad = torch.from_numpy(O.decode(g, wl.dtype).copy())
        opt.step()
    return p.detach().numpy()


@pytest.mark.parametrize("dtype", ["f32", "c64"])
@pytest.mark.parametrize("mode", ["full-rank-k0", "rho-one"])
def test_reduces_to_dense_adam(dtype, mode):
    """Full Tucker ranks with k = 0, and rho = 1 (the sparse part is the whole gradient),
    both reduce to dense Adam: checked against torch.optim.Adam over 10 steps that
    cross a refresh (T = 5)."""
    shape = (6, 5, 4, 3)
    rho = 0.0 if mode == "full-rank-k0" else 1.0
    wl = custom(shape, dtype, shape, rho, T=5, steps=10, signal_ranks=(2, 2, 2, 2))
    gs = GradStream(wl, seed=21)
    W = init_weights(wl, seed=21)
    grads = [gs.next() for _ in range(10)]
    o = O.TGradOracle(shape, shape if mode == "full-rank-k0" else (3, 2, 2, 1), dtype, rho, 5,
                      wl.lr, *wl.betas, wl.eps)
    Wo = W
    for g in grads:
        Wo = o.step(Wo, g)
    ref = _torch_adam_run(W, grads, wl)
    got = O.decode(Wo, dtype)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel <= 1e-6, rel


def test_full_rank_k0_is_bitwise_dense_adam_order():
    shape = (5, 4, 3)
    wl = custom(shape, "f32", shape, 0.0, T=3, steps=7)
    gs = GradStream(wl, seed=5)
    W = init_weights(wl, seed=5)
    o = O.TGradOracle(shape, shape, "f32", 0.0, 3, wl.lr, *wl.betas, wl.eps)
    Wd, m, v = W.copy(), np.zeros(W.size, np.float32), np.zeros(W.size, np.float32)
    Wo = W
    for t in range(1, 8):
        g = gs.next()
        Wo = o.step(Wo, g)
        Wd, m, v = O.dense_adam_reference(Wd, g, m, v, t, "f32", wl.lr, *wl.betas, wl.eps)
        assert np.array_equal(Wo.view(np.uint32), Wd.view(np.uint32))


def test_adam_matches_torch_single_tensor():
    r = rng(30)
    g_seq = [r.standard_normal(1000).astype(np.float32) * s for s in (1.0, 1e-3, 5.0, 0.1)]
    m = np.zeros(1000, np.float32)
    v = np.zeros(1000, np.float32)
    p = torch.nn.Parameter(torch.zeros(1000))
    opt = torch.optim.Adam([p], lr=1.0, betas=(0.9, 0.999), eps=1e-8, foreach=False)
    for t, g in enumerate(g_seq, 1):
        before = p.detach().clone()
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        u_torch = (before - p.detach()).numpy()
        u, m, v = O.adam(g, m, v, t, 0.9, 0.999, 1e-8)
        np.testing.assert_allclose(u, u_torch, rtol=2e-6, atol=1e-7)


# --------------------------------------------------------------------------- rounding

def _rounding_probe_values():
    r = rng(40)
    vals = [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 1e-40, -3e-39, 65504.0, 65520.0, 70000.0,
            3.4e38, 1e-8, 6e-8, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11]
    vals += list(r.standard_normal(4000) * 10.0 ** r.uniform(-8, 4, 4000))
    x = np.array(vals, np.float32)
    bits = x.view(np.uint32)
    halfway = ((bits & ~np.uint32(0xFFFF)) | np.uint32(0x8000)).view(np.float32)   # bf16 ties
    return np.concatenate([x, halfway[np.isfinite(halfway)]])


def test_bf16_rounding_matches_torch():
    x = _rounding_probe_values()
    mine = O.encode(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    n = np.array([np.nan], np.float32)
    assert np.isnan(O.decode(O.encode(n, "bf16"), "bf16")[0])


def test_f16_rounding_matches_torch():
    x = _rounding_probe_values()
    mine = O.encode(x, "f16").view(np.uint16)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


# --------------------------------------------------------------------------- step-level properties

def test_column_sign_flip_leaves_real_steps_unchanged():
    """Real Adam in a fixed basis is odd in g: flipping a factor column flips the matching
    core slice, m flips, v does not, u flips, and the reconstruction flips it back."""
    wl = custom((8, 7, 6), "f32", (4, 3, 3), 0.05, T=100)
    gs1, gs2 = GradStream(wl, seed=3), GradStream(wl, seed=3)
    W = init_weights(wl, seed=3)
    a = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.05, 100, wl.lr, *wl.betas, wl.eps)
    b = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.05, 100, wl.lr, *wl.betas, wl.eps)
    g1 = gs1.next()
    gs2.next()
    b.refresh(g1)
    b.factors[1] = b.factors[1].copy()
    b.factors[1][:, 2] *= -1
    b.factors[0] = b.factors[0].copy()
    b.factors[0][:, 0] *= -1
    Wa, Wb = a.step(W, g1), b.step(W, g1)
    assert np.array_equal(Wa, Wb)
    for _ in range(4):
        g = gs1.next()
        gs2.next()
        Wa, Wb = a.step(Wa, g), b.step(Wb, g)
        assert np.array_equal(Wa, Wb)


def test_reconstruction_error_falls_with_k_and_r():
    """Diagnostic of the pages' Fig. 3 (gradient reconstruction error): with outliers in
    the gradient, extracting a sparse part first cuts ||G - (L + S)|| / ||G|| far below
    low-rank alone, and at a fixed Omega the error falls as the ranks grow. (It is not
    monotone in rho: zeroing more residual entries makes the residual less low-rank.)"""
    wl = custom((16, 16, 8, 8), "f32", (8, 8, 4, 4), 0.05, signal_ranks=(4, 4, 2, 2))
    G = O.decode(GradStream(wl, seed=8).next(), "f32")

    def err(rho, ranks):
        k = int(math.floor(rho * G.size))
        om = O.select_omega(O.topk_keys(G, "f32"), k)
        R = O.residual(G, om)
        Us = [O.hosvd_factor(R, n, r)[0] for n, r in enumerate(ranks)]
        L = O.reconstruct(O.project(R, Us), Us)
        approx = L.copy().reshape(-1)
        approx[om.astype(np.int64)] += G.reshape(-1)[om.astype(np.int64)]
        return np.linalg.norm(G.reshape(-1) - approx) / np.linalg.norm(G)

    e0, e1 = err(0.0, (8, 8, 4, 4)), err(0.01, (8, 8, 4, 4))
    assert e1 < 0.1 * e0, (e0, e1)
    e = [err(0.05, rk) for rk in ((2, 2, 1, 1), (4, 4, 2, 2), (8, 8, 4, 4), (12, 12, 6, 6))]
    assert all(x > y for x, y in zip(e, e[1:])), e


def test_k_is_floor_of_rho_n():
    with open(os.path.join(GOLDEN, "sparse_budget.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        o = O.TGradOracle(case["shape"], case["shape"], "f32", case["rho"], 1, 1e-3, 0.9, 0.999, 1e-8)
        assert o.k == case["k"]


def test_refresh_schedule_every_T():
    wl = custom((6, 5, 4), "f32", (3, 3, 2), 0.05, T=4)
    o = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.05, 4, wl.lr, *wl.betas, wl.eps)
    calls = []
    orig = o.refresh

    def spy(G, serves=None):
        calls.append(o.t)
        orig(G, serves)
    o.refresh = spy
    gs, W = GradStream(wl), init_weights(wl)
    for _ in range(10):
        W = o.step(W, gs.next())
    assert calls == [1, 5, 9]


def test_moments_persist_across_refresh():
    wl = custom((6, 5, 4), "f32", (3, 3, 2), 0.1, T=2)
    o = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.1, 2, wl.lr, *wl.betas, wl.eps)
    gs, W = GradStream(wl), init_weights(wl)
    W = o.step(W, gs.next())
    W = o.step(W, gs.next())
    m_before = o.mC.copy()
    o.refresh(gs.next())
    assert np.array_equal(o.mC, m_before) and o.t == 2


# --------------------------------------------------------------------------- variants

def test_splitmix64_reference_outputs():
    """The rand-k keys at step counter 0 are the published SplitMix64 stream >> 33."""
    with open(os.path.join(GOLDEN, "splitmix64.json")) as f:
        fx = json.load(f)
    ref = np.array([int(x) for x in fx["outputs"]], np.uint64)
    keys = O.randk_keys(len(ref), fx["seed"], 0)
    assert np.array_equal(keys, ref >> np.uint64(33))


def test_randk_is_a_uniform_subset_independent_of_g():
    """Random-sampling Omega: k distinct ascending indices, the same for any gradient,
    different per refresh step and seed, and every element equally likely (chi-square
    over 400 draws of 100 out of 1000, far inside the 1e-6 tail)."""
    N, k = 1000, 100
    o1 = O.TGradOracle((10, 10, 10), (10, 10, 10), "f32", k / N, 1, 1e-3, 0.9, 0.999, 1e-8,
                       selection="randk", seed=7)
    o2 = O.TGradOracle((10, 10, 10), (10, 10, 10), "f32", k / N, 1, 1e-3, 0.9, 0.999, 1e-8,
                       selection="randk", seed=7)
    r = rng(50)
    o1.refresh(r.standard_normal((10, 10, 10)).astype(np.float32))
    o2.refresh(np.zeros((10, 10, 10), np.float32))
    assert np.array_equal(o1.omega, o2.omega)
    assert len(o1.omega) == k and np.all(np.diff(o1.omega.astype(np.int64)) > 0)
    counts = np.zeros(N)
    seen = set()
    for t in range(400):
        om = O.select_omega(O.randk_keys(N, 3 + (t % 2), t // 2), k)
        seen.add(om.tobytes())
        counts[om.astype(np.int64)] += 1
    assert len(seen) == 400
    expect = 400 * k / N
    chi2 = float(((counts - expect) ** 2 / expect).sum())
    # chi-square with 999 dof: mean 999, sd ~ 44.7; hypergeometric draws shrink it by 0.9
    assert 600 < chi2 < 1300, chi2


def test_randk_ties_go_to_the_lowest_index():
    """31-bit keys can collide; select_omega breaks ties by index, checked by brute force
    on keys forced to collide (N = 2^16 elements, keys reduced to 4 bits)."""
    keys = O.randk_keys(1 << 16, 11, 3) >> np.uint64(27)
    k = 5000
    om = O.select_omega(keys, k)
    order = sorted(range(len(keys)), key=lambda e: (-int(keys[e]), e))[:k]
    assert np.array_equal(om, np.array(sorted(order), np.uint32))


def _torch_adamw_run(W0, grads, wl, wd):
    p = torch.nn.Parameter(torch.from_numpy(O.decode(W0, wl.dtype).copy()))
    opt = torch.optim.AdamW([p], lr=wl.lr, betas=wl.betas, eps=wl.eps, weight_decay=wd,
                            foreach=False)
    for g in grads:
        p.grad = torch.from_numpy(O.decode(g, wl.dtype).copy())
        opt.step()
    return p.detach().numpy()


@pytest.mark.parametrize("dtype", ["f32", "c64"])
def test_weight_decay_reduces_to_adamw(dtype):
    """With full ranks and k = 0 the decayed method is AdamW (decoupled decay,
    W <- W (1 - lr wd) - lr u), checked against torch.optim.AdamW over 10 steps."""
    shape = (6, 5, 4, 3)
    wl = custom(shape, dtype, shape, 0.0, T=5, steps=10, lr=3e-2)
    gs = GradStream(wl, seed=22)
    W = init_weights(wl, seed=22) * 10
    grads = [gs.next() for _ in range(10)]
    o = O.TGradOracle(shape, shape, dtype, 0.0, 5, wl.lr, *wl.betas, wl.eps, weight_decay=0.5)
    Wo = W
    for g in grads:
        Wo = o.step(Wo, g)
    ref = _torch_adamw_run(W, grads, wl, 0.5)
    ref0 = _torch_adam_run(W, grads, wl)
    got = O.decode(Wo, dtype)
    assert np.abs(ref - ref0).max() > 100 * np.abs(got - ref).max()   # decay is visible
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel <= 1e-6, rel


def test_sparse_scale_is_a_learning_rate_on_the_sparse_part():
    """rho = 1 puts the whole gradient in the sparse part, so the update is lambda * lr
    times Adam's: the oracle with lambda = 0.25 matches torch.optim.Adam at lr / 4, and
    lambda = 0 leaves W unchanged."""
    shape = (6, 5, 4)
    wl = custom(shape, "f32", shape, 1.0, T=3, steps=8, lr=4e-3)
    gs = GradStream(wl, seed=23)
    W = init_weights(wl, seed=23)
    grads = [gs.next() for _ in range(8)]
    o = O.TGradOracle(shape, (3, 2, 2), "f32", 1.0, 3, wl.lr, *wl.betas, wl.eps,
                      sparse_scale=0.25)
    z = O.TGradOracle(shape, (3, 2, 2), "f32", 1.0, 3, wl.lr, *wl.betas, wl.eps,
                      sparse_scale=0.0)
    Wo, Wz = W, W
    for g in grads:
        Wo, Wz = o.step(Wo, g), z.step(Wz, g)
    assert np.array_equal(Wz, W)
    ref = _torch_adam_run(W, grads, custom(shape, "f32", shape, 1.0, lr=1e-3))
    rel = np.abs(O.decode(Wo, "f32") - ref).max() / np.abs(ref - W).max()
    assert rel <= 1e-5, rel


def test_remapped_moments_follow_their_element():
    """With remapped sparse moments, an element that stays in Omega across refreshes keeps
    the Adam moments of its own gradient sequence (torch.optim.Adam on that element
    alone), while Omega's other members change and shift its position; keeping moments
    by position instead gives it another element's history. Elements new to Omega start
    from zero."""
    shape = (8, 8, 8)
    N = 512
    r = rng(60)
    stay = np.array([40, 300, 301], np.int64)
    T, steps = 3, 10
    grads = []
    for t in range(steps):
        g = 1e-3 * r.standard_normal(N).astype(np.float32)
        g[stay] = 5.0 + r.standard_normal(3).astype(np.float32)
        # three more outliers, moved every refresh period
        mv = np.random.default_rng(100 + t // T).choice(np.setdiff1d(np.arange(N), stay), 3,
                                                        replace=False)
        g[mv] = 4.0 + r.standard_normal(3).astype(np.float32)
        grads.append(g.reshape(shape))
    rho = 6 / N
    kw = dict(selection="topk")
    on = O.TGradOracle(shape, (4, 4, 4), "f32", rho, T, 1e-3, 0.9, 0.999, 1e-8, remap=True, **kw)
    off = O.TGradOracle(shape, (4, 4, 4), "f32", rho, T, 1e-3, 0.9, 0.999, 1e-8, **kw)
    W = np.zeros(shape, np.float32)
    Wa, Wb = W, W
    p = torch.nn.Parameter(torch.zeros(3))
    opt = torch.optim.Adam([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, foreach=False)
    moved_new = 0
    for t, g in enumerate(grads, 1):
        old = on.omega.copy()
        Wa, Wb = on.step(Wa, g), off.step(Wb, g)
        if (t - 1) % T == 0 and t > 1:
            new_pos = [j for j, e in enumerate(on.omega) if e not in set(old.tolist())]
            moved_new += len(new_pos)
            # an element new to Omega had zero moments before this step's update: its
            # first moment is now exactly (1 - beta1) g
            for j in new_pos:
                e = int(on.omega[j])
                assert on.mS[j] == np.float32(1.0 - 0.9) * g.reshape(-1)[e]
        p.grad = torch.from_numpy(g.reshape(-1)[stay].copy())
        opt.step()
        st = opt.state[p]
        pos = np.searchsorted(on.omega, stay)
        assert np.array_equal(on.omega[pos], stay.astype(np.uint32))
        np.testing.assert_allclose(on.mS[pos], st["exp_avg"].numpy(), rtol=1e-6)
        np.testing.assert_allclose(on.vS[pos], st["exp_avg_sq"].numpy(), rtol=1e-6)
    assert moved_new > 0
    pos = np.searchsorted(off.omega, stay)
    assert not np.allclose(off.mS[pos], opt.state[p]["exp_avg"].numpy(), rtol=1e-3)


def test_variant_defaults_are_the_plain_method():
    wl = custom((8, 7, 6), "bf16", (4, 3, 3), 0.05, T=2)
    a = O.TGradOracle(wl.shape, wl.ranks, "bf16", 0.05, 2, wl.lr, *wl.betas, wl.eps)
    b = O.TGradOracle(wl.shape, wl.ranks, "bf16", 0.05, 2, wl.lr, *wl.betas, wl.eps,
                      weight_decay=0.0, sparse_scale=1.0, selection="topk", remap=False, seed=9)
    gs, W = GradStream(wl, seed=4), init_weights(wl, seed=4)
    Wa, Wb = W, W
    for _ in range(5):
        g = gs.next()
        Wa, Wb = a.step(Wa, g), b.step(Wb, g)
        assert np.array_equal(Wa, Wb)


def test_refresh_every_step_when_T_is_one():
    """T = 1: Omega and the factors are recomputed at every step."""
    wl = custom((6, 5, 4), "f32", (3, 3, 2), 0.05, T=1)
    o = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.05, 1, wl.lr, *wl.betas, wl.eps)
    calls = []
    orig = o.refresh

    def spy(G, serves=None):
        calls.append(serves)
        orig(G, serves)
    o.refresh = spy
    gs, W = GradStream(wl), init_weights(wl)
    for _ in range(4):
        W = o.step(W, gs.next())
    assert calls == [1, 2, 3, 4]


# --------------------------------------------------------------------------- low-rank-first order

def test_lowrank_first_with_k0_is_the_sparse_first_method():
    """With no sparse part the two orders are the same method: weights bit for bit."""
    wl = custom((8, 7, 6), "bf16", (4, 3, 3), 0.0, T=2)
    a = O.TGradOracle(wl.shape, wl.ranks, "bf16", 0.0, 2, wl.lr, *wl.betas, wl.eps)
    b = O.TGradOracle(wl.shape, wl.ranks, "bf16", 0.0, 2, wl.lr, *wl.betas, wl.eps,
                      order="lowrank_first")
    gs, W = GradStream(wl, seed=4), init_weights(wl, seed=4)
    Wa, Wb = W, W
    for _ in range(5):
        g = gs.next()
        Wa, Wb = a.step(Wa, g), b.step(Wb, g)
        assert np.array_equal(Wa, Wb)


@pytest.mark.parametrize("dtype", ["f32", "c64"])
def test_lowrank_first_with_full_ranks_is_dense_adam(dtype):
    """Full ranks: the low-rank part is the whole gradient, so the residual is exactly
    zero, Omega is the first k indices (all keys tie), S = 0 contributes nothing, and
    the step is dense Adam: checked against torch.optim.Adam over 10 steps."""
    shape = (6, 5, 4, 3)
    wl = custom(shape, dtype, shape, 0.2, T=5, steps=10, signal_ranks=(2, 2, 2, 2))
    gs = GradStream(wl, seed=21)
    W = init_weights(wl, seed=21)
    grads = [gs.next() for _ in range(10)]
    o = O.TGradOracle(shape, shape, dtype, 0.2, 5, wl.lr, *wl.betas, wl.eps, order="lowrank_first")
    Wo = W
    for g in grads:
        Wo = o.step(Wo, g)
        assert np.array_equal(o.omega, np.arange(o.k, dtype=np.uint32))
        assert not np.any(o.last["S"])
    ref = _torch_adam_run(W, grads, wl)
    got = O.decode(Wo, dtype)
    assert np.abs(got - ref).max() / np.abs(ref).max() <= 1e-6


def test_sparse_first_approximates_better_than_lowrank_first():
    """The pages' ablation direction (pith.science free parameters: the order is chosen
    by ablation; nullthought summary section 5: sparse first beats low-rank first): with
    1% Laplace outliers in the gradient, ||G - (L + S)|| / ||G|| after a refresh is at
    least twice as large when the Tucker factors are fitted before the outliers are
    removed."""
    wl = custom((16, 16, 8, 8), "f32", (8, 8, 4, 4), 0.05, signal_ranks=(4, 4, 2, 2))
    G = O.decode(GradStream(wl, seed=8).next(), "f32")
    err = {}
    for order in ("sparse_first", "lowrank_first"):
        o = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.05, 1, 1e-3, 0.9, 0.999, 1e-8, order=order)
        o.refresh(G)
        om = o.omega.astype(np.int64)
        base = O.residual(G, o.omega) if order == "sparse_first" else G
        L = O.reconstruct(O.project(base, o.factors), o.factors)
        S = (G if order == "sparse_first" else G - L).reshape(-1)[om]
        approx = L.reshape(-1).copy()
        approx[om] += S
        err[order] = np.linalg.norm(G.reshape(-1) - approx) / np.linalg.norm(G)
    assert err["lowrank_first"] >= 2 * err["sparse_first"], err


def test_lowrank_first_omega_is_topk_of_its_residual():
    """After a low-rank-first refresh, Omega is the k largest |G - L| (brute force by
    sorting on a small tensor), L the projection of G onto the refreshed factors."""
    wl = custom((9, 8, 7), "f32", (4, 4, 3), 0.1)
    G = O.decode(GradStream(wl, seed=2).next(), "f32")
    o = O.TGradOracle(wl.shape, wl.ranks, "f32", 0.1, 1, 1e-3, 0.9, 0.999, 1e-8, order="lowrank_first")
    o.refresh(G)
    L = O.reconstruct(O.project(G, o.factors).astype(np.float32), o.factors).astype(np.float32)
    mag = np.abs((G - L).reshape(-1)).astype(np.float64)
    order = sorted(range(mag.size), key=lambda e: (-mag[e], e))[:o.k]
    assert np.array_equal(o.omega, np.array(sorted(order), np.uint32))
    # and the factors are the HOSVD of G itself
    for n, U in enumerate(o.factors):
        Ug = O.hosvd_factor(G, n, wl.ranks[n])[0]
        assert np.allclose(U @ U.T, Ug @ Ug.T, atol=1e-6)
