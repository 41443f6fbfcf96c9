"""TensorGRaD optimizer step on AMD MI355X: Python binding of libtgrad.so.

Argument marshalling only: every step of the optimizer runs in the HIP kernels of
libtgrad.so (built in-tree by tensor_gradient_compression_amd.build). PyTorch supplies
device memory and the current stream. Loading fails loudly when the library is
missing; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtgrad.so")

F32, F16, BF16, C64 = 0, 1, 2, 3
DTYPE_CODES = {"f32": F32, "f16": F16, "bf16": BF16, "c64": C64}
OK, EINVAL, ENOMEM, EHIP, ESTATE = 0, 1, 2, 3, 4
MAX_NDIM = 8
MAX_KERNEL_IDS = 48

_lib = None


class TGradError(RuntimeError):
    pass


class Info(ctypes.Structure):
    _fields_ = [("ndim", ctypes.c_int64), ("dtype", ctypes.c_int64), ("numel", ctypes.c_int64),
                ("k", ctypes.c_int64), ("core_numel", ctypes.c_int64), ("T", ctypes.c_int64),
                ("t", ctypes.c_int64), ("shape", ctypes.c_int64 * MAX_NDIM),
                ("ranks", ctypes.c_int64 * MAX_NDIM), ("state_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("eig_sweeps_max", ctypes.c_int64),
                ("eig_unconverged", ctypes.c_int64)]


class Launch(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("modes", ctypes.c_int32),
                ("bytes_read", ctypes.c_int64), ("bytes_written", ctypes.c_int64),
                ("flops", ctypes.c_int64)]


SELECT_TOPK, SELECT_RANDK = 0, 1
SELECTIONS = {"topk": SELECT_TOPK, "randk": SELECT_RANDK}


ORDERS = {"sparse_first": 0, "lowrank_first": 1}


class Options(ctypes.Structure):
    _fields_ = [("weight_decay", ctypes.c_double), ("sparse_scale", ctypes.c_double),
                ("selection", ctypes.c_int32), ("remap_moments", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("order", ctypes.c_int32), ("reserved", ctypes.c_int32)]


# (name, restype, argtypes) of every exported symbol declared in include/tgrad.h
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = [
    ("tgrad_init", ctypes.c_int, [ctypes.POINTER(_P), ctypes.c_int, ctypes.POINTER(_I64),
                                  ctypes.POINTER(_I64), ctypes.c_int, ctypes.c_double, _I64,
                                  ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                  ctypes.c_double]),
    ("tgrad_step", ctypes.c_int, [_P, _P, _P, _P]),
    ("tgrad_refresh", ctypes.c_int, [_P, _P, _P]),
    ("tgrad_refresh_noalloc", ctypes.c_int, [_P, _P, _P]),
    ("tgrad_step_many", ctypes.c_int, [ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
                                       ctypes.c_int, _P]),
    ("tgrad_destroy", ctypes.c_int, [_P]),
    ("tgrad_status_string", ctypes.c_char_p, [ctypes.c_int]),
    ("tgrad_last_error", ctypes.c_char_p, [_P]),
    ("tgrad_get_info", ctypes.c_int, [_P, ctypes.POINTER(Info)]),
    ("tgrad_get_omega", ctypes.c_int, [_P, _P, _I64]),
    ("tgrad_get_factor", ctypes.c_int, [_P, ctypes.c_int, _P, _I64]),
    ("tgrad_get_eigvals", ctypes.c_int, [_P, ctypes.c_int, _P, _I64]),
    ("tgrad_get_moments", ctypes.c_int, [_P, _P, _P, _P, _P]),
    ("tgrad_set_omega", ctypes.c_int, [_P, _P, _I64]),
    ("tgrad_set_factor", ctypes.c_int, [_P, ctypes.c_int, _P, _I64]),
    ("tgrad_mark_refreshed", ctypes.c_int, [_P]),
    ("tgrad_debug_capture_delta", ctypes.c_int, [_P, _P]),
    ("tgrad_set_fusion", ctypes.c_int, [_P, ctypes.c_int]),
    ("tgrad_set_gram_fusion", ctypes.c_int, [_P, ctypes.c_int]),
    ("tgrad_set_pair_fusion", ctypes.c_int, [_P, ctypes.c_int]),
    ("tgrad_set_stream_overlap", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int]),
    ("tgrad_set_stream_products", ctypes.c_int, [_P, ctypes.c_int]),
    ("tgrad_default_options", None, [ctypes.POINTER(Options)]),
    ("tgrad_set_options", ctypes.c_int, [_P, ctypes.POINTER(Options)]),
    ("tgrad_get_options", ctypes.c_int, [_P, ctypes.POINTER(Options)]),
    ("tgrad_state_size", _I64, [_P]),
    ("tgrad_save_state", ctypes.c_int, [_P, _P, _I64]),
    ("tgrad_load_state", ctypes.c_int, [_P, _P, _I64]),
    ("tgrad_last_launches", ctypes.c_int, [_P, ctypes.POINTER(Launch), ctypes.c_int]),
    ("tgrad_timing_enable", ctypes.c_int, [_P, ctypes.c_int, ctypes.c_int]),
    ("tgrad_timing_read", ctypes.c_int, [_P, _P, _P, ctypes.c_int]),
    ("tgrad_timing_only", ctypes.c_int, [_P, ctypes.c_int]),
    ("tgrad_kernel_name", ctypes.c_char_p, [ctypes.c_int]),
]


def load_library(path: str = LIB_PATH):
    """Load libtgrad.so and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise TGradError(f"{path} is not built; run `python -m tensor_gradient_compression_amd.build`")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def kernel_name(i: int) -> str:
    return load_library().tgrad_kernel_name(i).decode()


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def step_many(handles, weights, grads, stream=None):
    """One step of each (handle, weight, grad) triple in one call (tgrad_step_many): the
    tensors' kernels overlap on internal streams joined back to `stream`."""
    n = len(handles)
    if len(weights) != n or len(grads) != n:
        raise ValueError("handles, weights and grads differ in length")
    for h, w, g in zip(handles, weights, grads):
        h._check_tensor(w, "weight")
        h._check_tensor(g, "grad")
    lib = load_library()
    hs = (_P * max(n, 1))(*[h._h.value for h in handles])
    ws = (_P * max(n, 1))(*[w.data_ptr() for w in weights])
    gs = (_P * max(n, 1))(*[g.data_ptr() for g in grads])
    rc = lib.tgrad_step_many(hs, ws, gs, n, TGrad._stream(stream))
    if rc != OK:
        msg = lib.tgrad_status_string(rc).decode()
        if n:
            msg += ": " + lib.tgrad_last_error(handles[0]._h).decode()
        raise TGradError(f"tgrad_step_many: {msg}")


class TGrad:
    """One TensorGRaD-optimised tensor (see include/tgrad.h for the exact semantics).

    weight and grad are device tensors (torch, contiguous) of the given shape; complex64
    for "c64", torch.bfloat16 for "bf16", float16 for "f16", float32 for "f32"."""

    def __init__(self, shape: Sequence[int], tucker_ranks: Sequence[int], dtype: str,
                 sparse_ratio: float, T: int, lr: float = 1e-3,
                 betas=(0.9, 0.999), eps: float = 1e-8):
        self._lib = load_library()
        self.shape = tuple(int(s) for s in shape)
        self.ranks = tuple(int(r) for r in tucker_ranks)
        self.dtype = dtype
        self.P = 2 if dtype == "c64" else 1
        nd = len(self.shape)
        if len(self.ranks) != nd:
            raise ValueError("shape and tucker_ranks differ in length")
        sh = (ctypes.c_int64 * nd)(*self.shape)
        rk = (ctypes.c_int64 * nd)(*self.ranks)
        h = ctypes.c_void_p()
        rc = self._lib.tgrad_init(ctypes.byref(h), nd, sh, rk, DTYPE_CODES[dtype],
                                  float(sparse_ratio), int(T), float(lr), float(betas[0]),
                                  float(betas[1]), float(eps))
        if rc != OK:
            raise TGradError(f"tgrad_init: {self._lib.tgrad_status_string(rc).decode()}")
        self._h = h
        self.info = self.get_info()
        import torch
        self.device_index = torch.cuda.current_device() if torch.cuda.is_available() else -1

    # ---------------------------------------------------------------- lifecycle
    def close(self):
        if getattr(self, "_h", None):
            self._lib.tgrad_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _check(self, rc: int, what: str):
        if rc != OK:
            msg = self._lib.tgrad_status_string(rc).decode()
            detail = self._lib.tgrad_last_error(self._h).decode() if self._h else ""
            raise TGradError(f"{what}: {msg} {detail}".strip())

    @staticmethod
    def _stream(stream):
        if stream is None:
            import torch
            return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if isinstance(stream, int):
            return ctypes.c_void_p(stream)
        return ctypes.c_void_p(stream.cuda_stream)

    def _check_tensor(self, x, what: str):
        """The library reads and writes N elements of the handle's dtype at x's address:
        refuse anything that is not exactly such a buffer on the handle's device."""
        import torch
        if not isinstance(x, torch.Tensor):
            raise ValueError(f"{what}: expected a torch.Tensor, got {type(x).__name__}")
        if not x.is_cuda:
            raise ValueError(f"{what}: must be a GPU tensor")
        if x.device.index != self.device_index:
            raise ValueError(f"{what}: on cuda:{x.device.index}, the handle is on cuda:{self.device_index}")
        if x.dtype != torch_dtype(self.dtype):
            raise ValueError(f"{what}: dtype {x.dtype}, the handle expects {torch_dtype(self.dtype)}")
        n = int(np.prod(self.shape, dtype=np.int64))
        if x.numel() != n:
            raise ValueError(f"{what}: {x.numel()} elements, the handle expects {n}")
        if not x.is_contiguous():
            raise ValueError(f"{what}: must be contiguous")

    # ---------------------------------------------------------------- hot path
    def step(self, weight, grad, stream=None):
        self._check_tensor(weight, "weight")
        self._check_tensor(grad, "grad")
        self._check(self._lib.tgrad_step(self._h, ctypes.c_void_p(weight.data_ptr()),
                                         ctypes.c_void_p(grad.data_ptr()), self._stream(stream)),
                    "tgrad_step")

    def refresh(self, grad, stream=None):
        self._check_tensor(grad, "grad")
        self._check(self._lib.tgrad_refresh(self._h, ctypes.c_void_p(grad.data_ptr()),
                                            self._stream(stream)), "tgrad_refresh")

    def refresh_noalloc(self, grad, stream=None):
        """tgrad_refresh_noalloc: the refresh with its scratch in the library's static
        device array (no allocation during the call)."""
        self._check_tensor(grad, "grad")
        self._check(self._lib.tgrad_refresh_noalloc(self._h, ctypes.c_void_p(grad.data_ptr()),
                                                    self._stream(stream)), "tgrad_refresh_noalloc")

    def capture_delta(self, delta):
        """Test hook (tgrad_debug_capture_delta): while set, every step also writes its
        fp32 update before the weight rounding into `delta` (an fp32 GPU tensor of N * P
        values); None turns it off. The tensor must outlive the steps that write it."""
        import torch
        if delta is None:
            self._check(self._lib.tgrad_debug_capture_delta(self._h, None), "tgrad_debug_capture_delta")
            self._delta = None
            return
        n = int(np.prod(self.shape, dtype=np.int64)) * self.P
        if (not isinstance(delta, torch.Tensor) or not delta.is_cuda or delta.dtype != torch.float32
                or delta.numel() != n or not delta.is_contiguous()
                or delta.device.index != self.device_index):
            raise ValueError(f"delta: needs a contiguous float32 GPU tensor of {n} values")
        self._check(self._lib.tgrad_debug_capture_delta(self._h, ctypes.c_void_p(delta.data_ptr())),
                    "tgrad_debug_capture_delta")
        self._delta = delta     # kept alive while the library may write it

    # ---------------------------------------------------------------- introspection
    def get_info(self) -> Info:
        info = Info()
        self._check(self._lib.tgrad_get_info(self._h, ctypes.byref(info)), "tgrad_get_info")
        return info

    @property
    def k(self) -> int:
        return int(self.info.k)

    @property
    def t(self) -> int:
        return int(self.get_info().t)

    def get_omega(self) -> np.ndarray:
        out = np.zeros(max(self.k, 1), np.uint32)
        self._check(self._lib.tgrad_get_omega(self._h, _ptr(out), out.size), "tgrad_get_omega")
        return out[:self.k]

    def get_factor(self, mode: int) -> np.ndarray:
        I, r = self.shape[mode], self.ranks[mode]
        out = np.zeros(I * r * self.P, np.float32)
        self._check(self._lib.tgrad_get_factor(self._h, mode, _ptr(out), out.size), "tgrad_get_factor")
        if self.P == 2:
            return out.view(np.complex64).reshape(I, r)
        return out.reshape(I, r)

    def get_eigvals(self, mode: int) -> np.ndarray:
        out = np.zeros(self.shape[mode], np.float64)
        self._check(self._lib.tgrad_get_eigvals(self._h, mode, _ptr(out), out.size), "tgrad_get_eigvals")
        return out

    def get_moments(self):
        nc = int(self.info.core_numel) * self.P
        ns = self.k * self.P
        mc, vc = np.zeros(nc, np.float32), np.zeros(nc, np.float32)
        ms, vs = np.zeros(max(ns, 1), np.float32), np.zeros(max(ns, 1), np.float32)
        self._check(self._lib.tgrad_get_moments(self._h, _ptr(mc), _ptr(vc), _ptr(ms), _ptr(vs)),
                    "tgrad_get_moments")
        return mc, vc, ms[:ns], vs[:ns]

    def set_omega(self, omega: np.ndarray):
        om = np.ascontiguousarray(omega, dtype=np.uint32)
        buf = om if om.size else np.zeros(1, np.uint32)
        self._check(self._lib.tgrad_set_omega(self._h, _ptr(buf), om.size), "tgrad_set_omega")

    def set_factor(self, mode: int, U: np.ndarray):
        if self.P == 2:
            flat = np.ascontiguousarray(U, dtype=np.complex64).reshape(-1).view(np.float32)
        else:
            flat = np.ascontiguousarray(U, dtype=np.float32).reshape(-1)
        self._check(self._lib.tgrad_set_factor(self._h, mode, _ptr(flat), flat.size), "tgrad_set_factor")

    def set_options(self, weight_decay: float = 0.0, sparse_scale: float = 1.0,
                    selection: str = "topk", remap_moments: bool = False, seed: int = 0,
                    order: str = "sparse_first"):
        """Variants of the method (include/tgrad.h, tgrad_options): decoupled weight decay,
        the sparse scale factor lambda, rand-k selection of Omega, sparse moments that
        follow their element across a refresh, and the low-rank-first decomposition
        order. The defaults are the plain method."""
        o = Options(float(weight_decay), float(sparse_scale), SELECTIONS[selection],
                    int(bool(remap_moments)), int(seed) & 0xFFFFFFFFFFFFFFFF, ORDERS[order], 0)
        self._check(self._lib.tgrad_set_options(self._h, ctypes.byref(o)), "tgrad_set_options")

    def get_options(self) -> dict:
        o = Options()
        self._check(self._lib.tgrad_get_options(self._h, ctypes.byref(o)), "tgrad_get_options")
        sel = {v: k for k, v in SELECTIONS.items()}[o.selection]
        order = {v: k for k, v in ORDERS.items()}[o.order]
        return dict(weight_decay=o.weight_decay, sparse_scale=o.sparse_scale, selection=sel,
                    remap_moments=bool(o.remap_moments), seed=o.seed, order=order)

    def set_fusion(self, enable) -> bool:
        """Select fused multi-mode launches (True or 1: default kernel choice; 2: two-mode
        workgroup tiles only; 3: two-mode slab kernels without the three-mode launches;
        4: as 1 with the two-mode reconstruction) or one launch per mode (False or 0);
        returns False when the fused form does not apply to this shape."""
        rc = self._lib.tgrad_set_fusion(self._h, int(enable))
        if rc == EINVAL and enable:
            return False
        self._check(rc, "tgrad_set_fusion")
        return True

    def set_gram_fusion(self, enable, masked: bool = False) -> bool:
        """Select the one-read Gram launch of the last three modes at a refresh (True)
        or one Gram launch per mode (False); masked: the Gram launches read the gradient
        and clear Omega's entries through its bitmask instead of reading the residual
        copy. Returns False when the one-read launch does not apply to this shape and
        dtype."""
        code = int(bool(enable)) | (2 if masked else 0)
        rc = self._lib.tgrad_set_gram_fusion(self._h, code)
        if rc == EINVAL and enable:
            return False
        self._check(rc, "tgrad_set_gram_fusion")
        return True

    def set_stream_overlap(self, adam=1, eig=True) -> None:
        """Work on the handle's second stream: the sparse values' Adam update beside the
        projection's later launches when the sparse part is large (adam=1, the default),
        whenever that applies (2) or never (0); and at a refresh, the leading modes'
        eigensolver beside the three-mode Gram launch (eig). Adam results are
        bit-identical either way; factors agree to fp64 rounding of the Grams."""
        self._check(self._lib.tgrad_set_stream_overlap(self._h, int(adam), int(bool(eig))),
                    "tgrad_set_stream_overlap")

    def set_adam_overlap(self, enable) -> None:
        """set_stream_overlap with only the Adam choice changed (eig left on)."""
        self.set_stream_overlap(adam=enable, eig=True)

    def set_pair_fusion(self, enable) -> bool:
        """Select one launch for two neighbouring leading modes of the fused plan (True)
        or one launch per mode (False); returns False when no such pair applies."""
        rc = self._lib.tgrad_set_pair_fusion(self._h, int(bool(enable)))
        if rc == EINVAL and enable:
            return False
        self._check(rc, "tgrad_set_pair_fusion")
        return True

    def set_stream_products(self, enable, max_workgroups: int = 0) -> None:
        """Single fp32 mode products on the streaming kernel where it applies (True, the
        default) or on the tiled kernel always (False); max_workgroups > 0 caps the
        streaming kernel's grid (a test hook)."""
        v = int(bool(enable))
        if v and max_workgroups:
            if max_workgroups < 0:
                raise ValueError("max_workgroups must be >= 0")
            v = int(max_workgroups) + 1
        self._check(self._lib.tgrad_set_stream_products(self._h, v), "tgrad_set_stream_products")

    def save_state(self) -> bytes:
        """The optimizer state as bytes (see tgrad_save_state)."""
        n = int(self._lib.tgrad_state_size(self._h))
        buf = np.zeros(max(n, 1), np.uint8)
        self._check(self._lib.tgrad_save_state(self._h, _ptr(buf), n), "tgrad_save_state")
        return buf[:n].tobytes()

    def load_state(self, state: bytes):
        """Restore a state written by save_state of a handle of the same shape."""
        buf = np.frombuffer(state, np.uint8).copy()
        self._check(self._lib.tgrad_load_state(self._h, _ptr(buf), buf.size), "tgrad_load_state")

    def mark_refreshed(self):
        self._check(self._lib.tgrad_mark_refreshed(self._h), "tgrad_mark_refreshed")

    def last_launches(self):
        """[(kernel name, modes, bytes read, bytes written, flops)] of the last step or
        refresh call, in issue order (tgrad_last_launches)."""
        n = self._lib.tgrad_last_launches(self._h, None, 0)
        if n < 0:
            raise TGradError("tgrad_last_launches: invalid handle")
        arr = (Launch * max(n, 1))()
        self._lib.tgrad_last_launches(self._h, arr, n)
        return [(kernel_name(l.kernel), [m for m in range(MAX_NDIM) if (l.modes >> m) & 1],
                 int(l.bytes_read), int(l.bytes_written), int(l.flops)) for l in arr[:n]]

    # ---------------------------------------------------------------- timing
    def timing_enable(self, enable: bool = True, max_records: int = 100000):
        self._check(self._lib.tgrad_timing_enable(self._h, int(enable), int(max_records)),
                    "tgrad_timing_enable")

    def timing_only(self, name=None):
        """Time only the launches of the kernel called name (None: every launch)."""
        kid = -1
        if name is not None:
            ids = [i for i in range(MAX_KERNEL_IDS) if kernel_name(i) == name]
            if not ids:
                raise ValueError(f"no kernel called {name!r}")
            kid = ids[0]
        self._check(self._lib.tgrad_timing_only(self._h, kid), "tgrad_timing_only")

    def timing_read(self):
        """{kernel name: (launches, total ms)} since the last read."""
        n = np.zeros(MAX_KERNEL_IDS, np.int64)
        ms = np.zeros(MAX_KERNEL_IDS, np.float64)
        self._check(self._lib.tgrad_timing_read(self._h, _ptr(n), _ptr(ms), MAX_KERNEL_IDS),
                    "tgrad_timing_read")
        out = {}
        for i in range(MAX_KERNEL_IDS):
            if n[i]:
                out[kernel_name(i)] = (int(n[i]), float(ms[i]))
        return out


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "c64": torch.complex64}[dtype]


def to_device(x: np.ndarray, dtype: str, device="cuda"):
    """Storage-convention numpy array (see synth) -> contiguous device tensor."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device).contiguous()


def to_host(t, dtype: str) -> np.ndarray:
    """Device tensor -> storage-convention numpy array."""
    import torch
    c = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return c.view(torch.int16).numpy().view(np.uint16).copy()
    return c.numpy().copy()
