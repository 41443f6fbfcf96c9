"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import numpy as np

import oracle as O
import tensor_gradient_compression_amd as tg


def make_lib(wl, T=None, rho=None, ranks=None):
    return tg.TGrad(wl.shape, ranks or wl.ranks, wl.dtype,
                    wl.sparse_ratio if rho is None else rho, T or wl.T, wl.lr, wl.betas, wl.eps)


def make_oracle(wl, T=None, rho=None, ranks=None):
    return O.TGradOracle(wl.shape, ranks or wl.ranks, wl.dtype,
                         wl.sparse_ratio if rho is None else rho, T or wl.T, wl.lr, *wl.betas, wl.eps)


def real(x, dtype):
    return O.real_view(O.decode(x, dtype)).astype(np.float64)


def weight_check(Wg, Wo, dtype, what=""):
    """Parity bar for weights. fp32 / complex64: relative max-norm <= 1e-5.
    fp16: relative max-norm <= 2e-3 (one fp16 ulp near max|W| is ~6e-4 relative, so
    legitimate rounding flips stay inside it). bf16: relative max-norm <= 2e-3, or, when
    independent fp32 updates round to different neighbours, every element within one bf16
    ulp of the oracle and at most 0.1% of the elements differing (one bf16 ulp near
    max|W| is ~4e-3 relative, above 2e-3)."""
    a, b = real(Wg, dtype), real(Wo, dtype)
    scale = np.abs(b).max()
    diff = np.abs(a - b)
    rel = diff.max() / scale if scale > 0 else diff.max()
    if dtype in ("f32", "c64"):
        assert rel <= 1e-5, f"{what} rel max-norm {rel:.3e} > 1e-5"
    elif dtype == "f16":
        assert rel <= 2e-3, f"{what} rel max-norm {rel:.3e} > 2e-3"
    else:
        if rel <= 2e-3:
            return rel
        mag = np.maximum(np.abs(a), np.abs(b))
        exp = np.floor(np.log2(np.where(mag > 0, mag, 1e-38)))
        ulp = np.exp2(exp - 7)
        assert np.all(diff <= ulp * (1 + 1e-6)), f"{what} bf16 difference above one ulp"
        frac = np.mean(diff > 0)
        assert frac <= 1e-3, f"{what} {frac:.2e} of bf16 weights differ"
    return rel


def projector(U):
    U = U.astype(np.complex128 if np.iscomplexobj(U) else np.float64)
    return U @ U.conj().T


def factor_check(lib, orc, tol=1e-4):
    """Projectors U U^H within tol (max-abs) where the eigengap makes them unique; the
    factors orthonormal to fp32 accuracy."""
    worst = 0.0
    for n, Uo in enumerate(orc.factors):
        if Uo is None:
            continue
        Ug = lib.get_factor(n)
        r = Ug.shape[1]
        G = Ug.astype(np.complex128 if np.iscomplexobj(Ug) else np.float64)
        assert np.abs(G.conj().T @ G - np.eye(r)).max() < 1e-5, f"mode {n} not orthonormal"
        if orc.gaps[n] < 1e-8:
            continue
        err = np.abs(projector(Ug) - projector(Uo)).max()
        worst = max(worst, err)
        assert err <= tol, f"mode {n}: projector error {err:.3e} (gap {orc.gaps[n]:.2e})"
    return worst


def omega_properties(keys: np.ndarray, omega: np.ndarray, k: int):
    """Complete characterisation of the top-k set with ties to the lowest index, checked
    without sorting: |Omega| = k, ascending, every selected key >= every unselected key,
    and among keys equal to the threshold the selected ones are the lowest indices."""
    assert omega.size == k
    if k == 0:
        return
    assert np.all(np.diff(omega.astype(np.int64)) > 0)
    sel = np.zeros(keys.size, bool)
    sel[omega] = True
    tau = keys[sel].min()
    if (~sel).any():
        assert keys[~sel].max() <= tau
    eq = np.flatnonzero(keys == tau)
    taken = sel[eq]
    # selected ties form a prefix of the tie indices
    if taken.size:
        first_not = np.argmin(taken) if not taken.all() else taken.size
        assert taken[:first_not].all() and not taken[first_not:].any()
