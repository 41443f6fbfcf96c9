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


def weight_check(Wg, Wo, dtype, what="", delta_backed=False, slack=0.0):
    """Parity bar for weights. fp32 / complex64: relative max-norm <= 1e-5.
    fp16: relative max-norm <= 2e-3 (one fp16 ulp near max|W| is ~6e-4 relative, so
    legitimate rounding flips stay inside it). bf16: relative max-norm <= 2e-3. One bf16
    ulp near max|W| is ~4e-3 relative, above 2e-3, so two correct fp32 updates that differ
    by rounding can round to neighbouring bf16 values. That case passes only when the
    caller has backed it with the fp32 update itself (delta_backed: every step's Delta
    checked against the oracle's and the weight update checked bit for bit against the
    rounding of W - lr Delta): then every element must be within one bf16 ulp of the
    oracle plus `slack` (the caller's bound on how far lr times the checked Delta
    difference can move W before rounding: where W - lr Delta cancels to a value far
    below both terms, that difference exceeds one ulp of the result), with at most 0.1%
    of the elements differing. Returns the criterion that passed ("max-norm" or
    "ulp+delta")."""
    a, b = real(Wg, dtype), real(Wo, dtype)
    scale = np.abs(b).max()
    diff = np.abs(a - b)
    rel = diff.max() / scale if scale > 0 else diff.max()
    if dtype in ("f32", "c64"):
        assert rel <= 1e-5, f"{what} rel max-norm {rel:.3e} > 1e-5"
        return "max-norm"
    if dtype == "f16" or rel <= 2e-3:
        assert rel <= 2e-3, f"{what} rel max-norm {rel:.3e} > 2e-3"
        return "max-norm"
    assert delta_backed, f"{what} bf16 rel max-norm {rel:.3e} > 2e-3 without the fp32-update check"
    mag = np.maximum(np.abs(a), np.abs(b))
    exp = np.floor(np.log2(np.where(mag > 0, mag, 1e-38)))
    ulp = np.exp2(exp - 7)
    assert np.all(diff <= ulp * (1 + 1e-6) + slack), f"{what} bf16 difference above one ulp"
    frac = np.mean(diff > 0)
    assert frac <= 1e-3, f"{what} {frac:.2e} of bf16 weights differ"
    return "ulp+delta"


# The fp32 update before the weight rounding, Delta = Delta_L + lambda N_S at Omega, with
# Omega and the factors pinned: relative max-norm bar against the oracle's.
DELTA_RTOL = 1e-5


class DeltaCapture:
    """A device buffer the library writes every step's fp32 update into
    (tgrad_debug_capture_delta)."""

    def __init__(self, lib, wl):
        import torch
        n = int(np.prod(wl.shape, dtype=np.int64)) * (2 if wl.dtype == "c64" else 1)
        self.buf = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        lib.capture_delta(self.buf)

    def host(self) -> np.ndarray:
        return self.buf.cpu().numpy()


def delta_rel(dg: np.ndarray, do: np.ndarray) -> float:
    """Relative max-norm of the library's Delta against the oracle's."""
    do = np.asarray(do, np.float64).reshape(-1)
    dg = np.asarray(dg, np.float64).reshape(-1)
    assert dg.shape == do.shape and np.all(np.isfinite(dg))
    scale = np.abs(do).max()
    diff = np.abs(dg - do).max()
    return diff / scale if scale > 0 else diff


def apply_check(W_prev, W_new, dg, dtype, lr, decay=1.0, what=""):
    """The weight update is exactly the rounding of fp32(W) * decay - fp32(lr) * Delta
    (one rounding per element) with the library's own Delta."""
    w32 = O.real_view(O.decode(W_prev, dtype)).copy()
    e32 = w32 * np.float32(decay) - np.float32(lr) * np.asarray(dg, np.float32)
    exp = O.encode(e32.view(np.complex64) if dtype == "c64" else e32, dtype)
    got = np.ascontiguousarray(W_new).reshape(-1)
    assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(exp).reshape(-1).view(np.uint8)), \
        f"{what}: W is not the rounding of W - lr Delta"


class CoreSplit:
    """The step's fp32 update, split where floating point is ill-conditioned.

    Adam's update of a core entry is u = (m / bc1) / (sqrt(v / bc2) + eps); at t = 1 that
    is g / (|g| + eps). Near g = 0 this map is steep (slope 1 / (4 eps) at |g| = eps) and
    at |g| >> eps it is a sign, so a core entry within rounding of zero turns the
    projection's fp32 rounding (the library) against fp64 (the oracle) into an O(1)
    difference of u, and the reconstruction spreads it over every element. Both sides
    are right to their own precision. The comparison therefore checks the path in parts:
      * the core Adam moments m, v against the oracle's (max-norm, relative 1e-5 of the
        largest): the projection and the moment update;
      * u is Adam's map of those moments on both sides (the library's kernel computes it
        in the same fp32 operation order as the oracle, which the full-rank, k = 0 runs
        pin bit for bit), so the library's u is the oracle's map of the library's moments;
      * the library's Delta against the oracle's reconstruction of that u plus the
        oracle's own lambda N_S at Omega: the reconstruction, the merge and the apply.
    The entries whose u differs from the oracle's by more than 1e-4 are counted and
    reported (steep entries)."""

    def __init__(self, orc):
        self.orc = orc

    def expected_delta(self, lib, t):
        orc = self.orc
        P = orc.P
        mC, vC, _, _ = lib.get_moments()
        for name, a, b in (("m", mC, orc.mC), ("v", vC, orc.vC)):
            scale = np.abs(b).max()
            if scale > 0:
                err = np.abs(a.astype(np.float64) - b).max() / scale
                assert err <= 1e-5, f"core {name}: rel max-norm {err:.3e} > 1e-5"
        _, _, _, _, e, bc1, bc2 = O.adam_consts(t, orc.beta1, orc.beta2, orc.eps)
        u_lib = (mC / bc1) / (np.sqrt(vC / bc2) + e)
        u_orc = orc.last["uC"]
        corr = u_lib.astype(np.float64) - u_orc.astype(np.float64)
        n_steep = int((np.abs(corr) > 1e-4).sum())
        expected = np.asarray(orc.last["delta"], np.float64)
        if np.any(corr != 0.0):
            core = corr.view(np.complex128) if P == 2 else corr
            extra = O.reconstruct(core.reshape(orc.core_shape), orc.factors)
            extra = extra.reshape(-1).view(np.float64) if P == 2 else extra.reshape(-1)
            expected = expected + extra
        return expected, n_steep, float(np.abs(corr).max()) if corr.size else 0.0


def checked_step(lib, orc, cap, W, Wo, g, wl, what, delta_tol=DELTA_RTOL, decay=1.0, G=None,
                 align=None):
    """One step on both sides with the fp32 update checked: the library's Delta against
    the oracle's (relative max-norm <= delta_tol; with `align`, a CoreSplit of this
    oracle, the core moments are checked against the oracle's and Delta against the
    oracle's reconstruction of the library's core update) and the library's weight update against the rounding of its own
    W - lr Delta (bit for bit). G: the device copy of g to step with (made here when
    None). Returns the oracle's new W and the measured relative Delta difference."""
    import torch
    W_prev = tg.to_host(W, wl.dtype)
    lib.step(W, tg.to_device(g, wl.dtype) if G is None else G)
    Wo = orc.step(Wo, g)
    torch.cuda.synchronize()
    dg = cap.host()
    apply_check(W_prev, tg.to_host(W, wl.dtype), dg, wl.dtype, wl.lr, decay, what)
    expected, n_steep, du = orc.last["delta"], 0, 0.0
    if align is not None:
        expected, n_steep, du = align.expected_delta(lib, orc.t)
    rel = delta_rel(dg, expected)
    print(f"DELTA {what}: rel {rel:.3e} (against the oracle's own Delta: "
          f"{delta_rel(dg, orc.last['delta']):.3e}; steep core entries {n_steep}, max |du| {du:.2e})")
    assert rel <= delta_tol, f"{what}: Delta rel max-norm {rel:.3e} > {delta_tol:.0e}"
    return Wo, rel


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
