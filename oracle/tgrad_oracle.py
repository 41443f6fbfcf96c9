"""CPU oracle of one TensorGRaD optimizer step (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module. It shares no code with the HIP
library: no kernels, headers, helpers, tables or constants. It is deliberately
plain and slow: numpy, float64 contractions (complex128 for complex), float32 Adam,
integer top-k keys.

Sources, cited by page and section (no code exists on the pages):
  [NT]   nullthought.net summary of "TensorGRaD: Tensor Gradient Robust Decomposition
         for Memory-Efficient Neural Operator Training", sections 二 (method overview)
         and 三 (implementation details: sparse part extracted first, Tucker on the
         residual, separate Adam updates, scatter-add after reconstruction, mixed
         precision, re-selection every T steps).
  [PITH] pith.science review of arXiv 2501.02379: "What carries the argument"
         (Tucker/HOSVD factors reused for T steps, projection to a core, Adam moments
         on the core, reconstruction by mode-wise products, COO sparse set chosen by
         top-k magnitude), "Core claim" (sparse branch first, low-rank basis on the
         residual), free parameters (lambda, T, order), and the appendix excerpts in
         its reference list: App. K (tensor notation, mode-k unfolding, stable rank,
         Tucker form), App. M Theorem 2 (project / update states / project back) and
         the tensor-low-rank parameter count, eq. (10).
  [ABS]  mlsanity.com page of arXiv 2501.02379, abstract (G = low-rank + sparse,
         mixed-precision recipe).

Readings where the pages are silent (each is listed with its reason in the design
notes): lambda = 1; k = floor(rho*N) in IEEE double; top-k key = unsigned bit pattern
of |x| (complex: bits of fl64(re^2 + im^2), NaN canonicalised), ties to the lowest
linear index; top-k and HOSVD read the refresh step's own gradient; plain truncated
HOSVD (each factor from the Gram of the full residual); eigenvectors in descending
eigenvalue order, each column scaled so its largest-magnitude entry (lowest row on
ties) is real positive; modes with r_n = I_n use the identity; moments are kept
positionally across refreshes and t is never reset; a refresh happens before the
step with (t - 1) mod T == 0; Kingma-Ba Adam with bias correction, eps outside the
root, no weight decay; complex Adam treats real and imaginary parts as independent
reals; the update is formed in fp32 and the weight rounded once per step.

Pins: tests/test_oracle_pins.py checks every function here against closed forms,
brute force, torch.optim.Adam and the identities the pages state.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "f16", "bf16", "c64")

# ----------------------------------------------------------------------------- storage


def decode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage -> float32 (complex64 for c64). Exact for every storage dtype.

    bf16 is held as uint16 bit patterns: the fp32 value has the same upper 16 bits."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "c64":
        return np.asarray(x, dtype=np.complex64)
    raise ValueError(dtype)


def _bf16_round(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN."""
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        rounded[nan] = ((bits[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return rounded


def encode(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 (complex64) -> storage, round to nearest even."""
    if dtype == "f32":
        return np.asarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(x32, dtype=np.float32).astype(np.float16)
    if dtype == "bf16":
        return _bf16_round(np.asarray(x32, dtype=np.float32))
    if dtype == "c64":
        return np.asarray(x32, dtype=np.complex64)
    raise ValueError(dtype)


def real_view(x: np.ndarray) -> np.ndarray:
    """Flat float32 view; complex64 becomes interleaved (re, im) pairs."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.complex64:
        return x.reshape(-1).view(np.float32)
    return x.reshape(-1).astype(np.float32, copy=False)


# ----------------------------------------------------------------------------- sparse part


def topk_keys(G: np.ndarray, dtype: str) -> np.ndarray:
    """Magnitude keys for top-k selection, as uint64 [NT 二: top-k gradient elements;
    PITH "What carries the argument": top-k magnitude].

    Real dtypes: the storage bit pattern with the sign bit cleared. For IEEE formats
    that orders exactly like |x| (and keeps subnormals distinct); NaN ranks above Inf.
    Complex: the bit pattern of fl64(re^2 + im^2). Both squares of fp32 values are exact
    in fp64, so the key is one correctly rounded sum; any NaN becomes the canonical
    quiet NaN so that the key does not depend on a payload."""
    flat = np.ascontiguousarray(G).reshape(-1)
    if dtype == "f32":
        return (flat.view(np.uint32) & np.uint32(0x7FFFFFFF)).astype(np.uint64)
    if dtype == "f16":
        return (flat.view(np.uint16) & np.uint16(0x7FFF)).astype(np.uint64)
    if dtype == "bf16":
        return (flat.astype(np.uint16) & np.uint16(0x7FFF)).astype(np.uint64)
    if dtype == "c64":
        re = flat.real.astype(np.float64)
        im = flat.imag.astype(np.float64)
        s = re * re + im * im
        key = s.view(np.uint64) & np.uint64(0x7FFFFFFFFFFFFFFF)
        key[np.isnan(s)] = np.uint64(0x7FF8000000000000)
        return key
    raise ValueError(dtype)


def select_omega(keys: np.ndarray, k: int) -> np.ndarray:
    """Omega = the k largest keys, ties to the lowest linear index, returned ascending
    as uint32 [NT 二/三; PITH "What carries the argument"]."""
    n = keys.size
    if k <= 0:
        return np.zeros(0, dtype=np.uint32)
    order = np.lexsort((np.arange(n, dtype=np.int64), -keys.astype(np.int64)))
    return np.sort(order[:k]).astype(np.uint32)


SPLITMIX_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(z: np.ndarray) -> np.ndarray:
    """The SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
    pseudorandom number generators", 2014; the 64-bit finaliser of Stafford's Mix13)
    applied to states z (uint64, arithmetic modulo 2^64)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def randk_keys(N: int, seed: int, t: int) -> np.ndarray:
    """Random-sampling keys for Omega (pith.science "What carries the argument": Omega is
    re-selected by top-k magnitude or by random sampling). Element e of the refresh that
    serves step t gets the top 31 bits of the SplitMix64 output for the state
    seed + gamma * (t * 2^32 + e + 1); Omega is then the k largest keys with ties to the
    lowest index, exactly as for magnitudes, i.e. a uniformly random k-subset."""
    e = np.arange(N, dtype=np.uint64)
    ctr = (np.uint64(t) << np.uint64(32)) + e + np.uint64(1)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + np.uint64(SPLITMIX_GAMMA) * ctr
    return splitmix64(z) >> np.uint64(33)


def remap_moments(omega_old: np.ndarray, omega_new: np.ndarray, m: np.ndarray, P: int) -> np.ndarray:
    """Sparse moments after a refresh when they follow their index: entry j of the new
    Omega takes the moments of the same element in the old Omega, or zero if it was not
    there (the alternative to keeping them by position)."""
    out = np.zeros(len(omega_new) * P, np.float32)
    pos = {int(x): i for i, x in enumerate(omega_old)}
    for j, x in enumerate(omega_new):
        i = pos.get(int(x))
        if i is not None:
            out[j * P:(j + 1) * P] = m[i * P:(i + 1) * P]
    return out


def gather(G32: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """S = G restricted to Omega, in Omega's order [NT 三: sparse part first]."""
    return np.ascontiguousarray(G32).reshape(-1)[omega.astype(np.int64)].copy()


def residual(G32: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """R = G with the entries at Omega set to zero [NT 三: the rest is the residual;
    PITH "Core claim": low-rank basis built on the residual]."""
    R = np.array(G32, copy=True)
    R.reshape(-1)[omega.astype(np.int64)] = 0
    return R


# ----------------------------------------------------------------------------- low-rank part


def unfold(X: np.ndarray, n: int) -> np.ndarray:
    """Mode-n unfolding: I_n x (product of the other sizes) [PITH App. K, mode-k
    unfolding]. Column order is immaterial to everything it feeds."""
    return np.moveaxis(X, n, 0).reshape(X.shape[n], -1)


def gram(R: np.ndarray, n: int) -> np.ndarray:
    """Gram_n = R_(n) R_(n)^H in float64 / complex128 [PITH: Tucker (higher-order SVD)
    factors of the residual]."""
    wide = np.complex128 if np.iscomplexobj(R) else np.float64
    Xn = unfold(R.astype(wide), n)
    return Xn @ Xn.conj().T


def canonicalize_columns(V: np.ndarray) -> np.ndarray:
    """Scale each column by a unit scalar so that its largest-|.| entry (lowest row on
    ties) is real and positive. Eigenvectors are only defined up to such a scalar; the
    pages fix none, this fixes one."""
    V = np.array(V, copy=True)
    for c in range(V.shape[1]):
        a = np.abs(V[:, c])
        i = int(np.argmax(a))
        if a[i] > 0:
            V[:, c] = V[:, c] * (np.conj(V[i, c]) / a[i])
    return V


def hosvd_factor(R: np.ndarray, n: int, r: int):
    """U(n): the r leading eigenvectors of Gram_n, descending, canonicalised, then
    stored in fp32 (complex64) as optimizer state [NT 二: Tucker part, like an SVD of
    a matrix; PITH "What carries the argument": factors U^(n); App. M: P^T P = I].

    Returns (U, eigenvalues descending, relative gap at the cut)."""
    H = gram(R, n)
    w, V = np.linalg.eigh(H)
    w = w[::-1]
    V = V[:, ::-1]
    U = canonicalize_columns(V[:, :r])
    store = np.complex64 if np.iscomplexobj(R) else np.float32
    lam1 = w[0] if w.size and w[0] > 0 else 0.0
    gap = (w[r - 1] - w[r]) / lam1 if (r < w.size and lam1 > 0) else float("inf")
    return U.astype(store), w, gap


def mode_product(X: np.ndarray, M: np.ndarray, n: int) -> np.ndarray:
    """Y = X x_n M, i.e. Y[..., j, ...] = sum_i M[j, i] X[..., i, ...] [PITH App. K,
    mode-k product]."""
    return np.moveaxis(np.tensordot(M, X, axes=([1], [n])), 0, n)


def project(R: np.ndarray, factors: Sequence[Optional[np.ndarray]]) -> np.ndarray:
    """C = R x_1 U1^H x_2 ... x_d Ud^H in float64 / complex128 [PITH App. M Theorem 2,
    step "project the gradient"; PITH "What carries the argument": gradient projected
    to a small core]. Identity modes (None) are skipped."""
    wide = np.complex128 if np.iscomplexobj(R) else np.float64
    C = R.astype(wide)
    for n, U in enumerate(factors):
        if U is not None:
            C = mode_product(C, U.astype(wide).conj().T, n)
    return C


def reconstruct(NC: np.ndarray, factors: Sequence[Optional[np.ndarray]]) -> np.ndarray:
    """Delta_L = N_C x_1 U1 x_2 ... x_d Ud in float64 / complex128 [PITH App. M
    Theorem 2, step "project back"; PITH: update reconstructed by mode-wise products]."""
    wide = np.complex128 if np.iscomplexobj(NC) else np.float64
    X = NC.astype(wide)
    for n, U in enumerate(factors):
        if U is not None:
            X = mode_product(X, U.astype(wide), n)
    return X


def lowrank_param_count(shape: Sequence[int], ranks: Sequence[int]) -> int:
    """Number of low-rank parameters kept: core (prod r_n) plus one I_n x r_n factor per
    truncated mode. For a (N, N, M, M) tensor with all ranks r this is the pages'
    eq. (10): r^4 + 2rN + 2rM [PITH reference excerpt, memory comparison]."""
    core = int(np.prod(ranks, dtype=np.int64))
    fac = sum(int(i) * int(r) for i, r in zip(shape, ranks) if r < i)
    return core + fac


# ----------------------------------------------------------------------------- Adam


def adam_consts(t: int, beta1: float, beta2: float, eps: float):
    """fp32 constants of step t: beta1, 1-beta1, beta2, 1-beta2, eps, and the bias
    corrections 1-beta^t, each computed in fp64 and rounded once to fp32."""
    f = np.float32
    return (f(beta1), f(1.0 - beta1), f(beta2), f(1.0 - beta2), f(eps),
            f(1.0 - beta1 ** t), f(1.0 - beta2 ** t))


def adam(g: np.ndarray, m: np.ndarray, v: np.ndarray, t: int, beta1: float, beta2: float,
         eps: float):
    """Kingma-Ba Adam on float32 values, every operation rounded to fp32 in this
    order [NT 二/三: Adam on each part; PITH: Adam moments live on the core; the
    reference list's Adam entry]:
        m <- b1*m + (1-b1)*g ; v <- b2*v + (1-b2)*(g*g) ; u = (m/bc1) / (sqrt(v/bc2) + eps)
    Returns (u, m, v) as new arrays."""
    b1, c1, b2, c2, e, bc1, bc2 = adam_consts(t, beta1, beta2, eps)
    g = np.asarray(g, dtype=np.float32)
    m = b1 * np.asarray(m, np.float32) + c1 * g
    v = b2 * np.asarray(v, np.float32) + c2 * (g * g)
    u = (m / bc1) / (np.sqrt(v / bc2) + e)
    return u.astype(np.float32), m.astype(np.float32), v.astype(np.float32)


# ----------------------------------------------------------------------------- optimizer


class TGradOracle:
    """State and schedule of one TensorGRaD-optimised tensor.

    refresh(G): Omega and U(n) from G [NT 三: re-select the sparse indices and the
    low-rank subspace every T steps; PITH: factors computed once and reused for T
    steps, Omega re-selected every T steps].
    step(W, G): returns the new W (storage dtype) [NT 三 step order; PITH Theorem 2]."""

    def __init__(self, shape, ranks, dtype, sparse_ratio, T, lr, beta1, beta2, eps,
                 weight_decay=0.0, sparse_scale=1.0, selection="topk", remap=False, seed=0,
                 order="sparse_first"):
        self.shape = tuple(int(s) for s in shape)
        self.ranks = tuple(int(r) for r in ranks)
        if dtype not in DTYPES:
            raise ValueError(dtype)
        self.dtype = dtype
        self.P = 2 if dtype == "c64" else 1
        self.N = int(np.prod(self.shape, dtype=np.int64))
        self.k = int(math.floor(float(sparse_ratio) * float(self.N)))
        self.T = int(T)
        self.lr, self.beta1, self.beta2, self.eps = float(lr), float(beta1), float(beta2), float(eps)
        self.core_shape = tuple(self.ranks)
        ncore = int(np.prod(self.core_shape, dtype=np.int64))
        self.mC = np.zeros(ncore * self.P, np.float32)
        self.vC = np.zeros(ncore * self.P, np.float32)
        self.mS = np.zeros(self.k * self.P, np.float32)
        self.vS = np.zeros(self.k * self.P, np.float32)
        self.omega = np.zeros(0, np.uint32)
        self.factors: List[Optional[np.ndarray]] = [None] * len(self.shape)
        self.eigvals: List[Optional[np.ndarray]] = [None] * len(self.shape)
        self.gaps: List[float] = [float("inf")] * len(self.shape)
        self.t = 0
        self.refreshed_for = 0
        self.last = {}
        # variants (defaults reproduce the plain method bit for bit)
        self.weight_decay = float(weight_decay)   # decoupled, AdamW style
        self.sparse_scale = float(sparse_scale)   # lambda in Delta[Omega] += lambda N_S
        if selection not in ("topk", "randk"):
            raise ValueError(selection)
        self.selection = selection
        self.remap = bool(remap)
        self.seed = int(seed)
        # decomposition order ([PITH] free parameters: "US -> LR", sparse then low-rank,
        # chosen by ablation; the reverse is the alternative it is compared with)
        if order not in ("sparse_first", "lowrank_first"):
            raise ValueError(order)
        self.order = order

    def refresh_due(self, t: int) -> bool:
        return (t - 1) % self.T == 0

    def refresh(self, G: np.ndarray, serves: int = None):
        """Sparse first, then HOSVD of the residual [NT 三; PITH "Core claim"]. `serves` is
        the step the new Omega and factors are first used in (default: the next one)."""
        if serves is None:
            serves = self.t + 1
        G = np.asarray(G).reshape(self.shape)
        old = self.omega
        if self.order == "lowrank_first":
            self._refresh_lowrank_first(G, serves, old)
            return
        if self.selection == "topk":
            keys = topk_keys(G, self.dtype)
        else:
            keys = randk_keys(self.N, self.seed, serves)
        self.omega = select_omega(keys, self.k)
        if self.remap:
            self.mS = remap_moments(old, self.omega, self.mS, self.P)
            self.vS = remap_moments(old, self.omega, self.vS, self.P)
        R = residual(decode(G, self.dtype), self.omega)
        self._factors_from(R)
        self.refreshed_for = serves

    def _factors_from(self, R: np.ndarray):
        for n, (I, r) in enumerate(zip(self.shape, self.ranks)):
            if r >= I:
                self.factors[n] = None
                self.eigvals[n] = None
                self.gaps[n] = float("inf")
            else:
                U, w, gap = hosvd_factor(R, n, r)
                self.factors[n], self.eigvals[n], self.gaps[n] = U, w, gap

    def lowrank_part(self, G32: np.ndarray) -> np.ndarray:
        """L = (G x_n Un^H ...) x_n Un ... with the core rounded to fp32 in between, as
        the optimizer state keeps it, and L rounded to fp32."""
        C32 = project(G32, self.factors).astype(np.complex64 if self.P == 2 else np.float32)
        return reconstruct(C32, self.factors).astype(C32.dtype)

    def _refresh_lowrank_first(self, G: np.ndarray, serves: int, old: np.ndarray):
        """Low-rank first: the Tucker factors from the HOSVD of the whole gradient, then
        Omega = the k largest entries of the fp32 residual G - L (by the same keys and tie
        rule as the sparse-first order; random sampling ignores the residual)."""
        G32 = decode(G, self.dtype)
        self._factors_from(G32)
        if self.selection == "topk":
            R32 = G32 - self.lowrank_part(G32)
            keys = topk_keys(R32, "c64" if self.P == 2 else "f32")
        else:
            keys = randk_keys(self.N, self.seed, serves)
        self.omega = select_omega(keys, self.k)
        if self.remap:
            self.mS = remap_moments(old, self.omega, self.mS, self.P)
            self.vS = remap_moments(old, self.omega, self.vS, self.P)
        self.refreshed_for = serves

    def step(self, W: np.ndarray, G: np.ndarray) -> np.ndarray:
        W = np.asarray(W).reshape(self.shape)
        G = np.asarray(G).reshape(self.shape)
        self.t += 1
        t = self.t
        if self.refresh_due(t) and self.refreshed_for != t:
            self.refresh(G, t)
        G32 = decode(G, self.dtype)
        if self.order == "lowrank_first":
            # the low-rank part of the whole gradient, then the sparse part of what it
            # leaves: S = (G - L)[Omega] in fp32
            R = G32
            L32 = self.lowrank_part(G32)
            S = gather(G32 - L32, self.omega)
        else:
            S = gather(G32, self.omega)
            R = residual(G32, self.omega)
        C = project(R, self.factors)
        C32 = C.astype(np.complex64 if self.P == 2 else np.float32)
        uC, self.mC, self.vC = adam(real_view(C32), self.mC, self.vC, t,
                                    self.beta1, self.beta2, self.eps)
        uS, self.mS, self.vS = adam(real_view(S), self.mS, self.vS, t,
                                    self.beta1, self.beta2, self.eps)
        NC = uC.view(np.complex64).reshape(self.core_shape) if self.P == 2 else uC.reshape(self.core_shape)
        DL = reconstruct(NC, self.factors)
        D = np.ascontiguousarray(DL.astype(np.complex64 if self.P == 2 else np.float32))
        Dr = real_view(D).copy()                        # fp32 (re, im interleaved)
        if self.k:
            Dr2 = Dr.reshape(-1, self.P)
            Dr2[self.omega.astype(np.int64)] += np.float32(self.sparse_scale) * uS.reshape(-1, self.P)
        W32 = real_view(decode(W, self.dtype)).copy()
        # decoupled weight decay folded into the one rounding: W (1 - lr wd) - lr Delta, the
        # factor formed in fp64 and rounded to fp32 (exactly 1 without decay)
        decay = np.float32(1.0 - self.lr * self.weight_decay)
        W32 = W32 * decay - np.float32(self.lr) * Dr
        if self.P == 2:
            Wn = encode(W32.view(np.complex64), self.dtype)
        else:
            Wn = encode(W32, self.dtype)
        self.last = dict(S=S, R=R, C=C32, uC=uC, uS=uS, delta=Dr)
        return Wn.reshape(self.shape)


def dense_adam_reference(W: np.ndarray, G: np.ndarray, m, v, t, dtype, lr, beta1, beta2, eps):
    """Plain dense Adam on a whole tensor in the same fp32 order (used by the pins: the
    method with full ranks and k = 0 reduces to it)."""
    g = real_view(decode(G, dtype))
    u, m, v = adam(g, m, v, t, beta1, beta2, eps)
    w = real_view(decode(W, dtype)).copy() - np.float32(lr) * u
    if dtype == "c64":
        return encode(w.view(np.complex64), dtype).reshape(W.shape), m, v
    return encode(w, dtype).reshape(W.shape), m, v
