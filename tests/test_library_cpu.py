"""CPU-only checks of the C ABI: the library loads, exports every function that
include/tgrad.h declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re

import pytest

import tensor_gradient_compression_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgrad.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tgrad_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tg.LIB_PATH):
        from tensor_gradient_compression_amd import build
        build.build(verbose=False)
    return tg.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("tgrad_init", "tgrad_step", "tgrad_refresh", "tgrad_destroy"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    bound = {name for name, _, _ in tg.SIGNATURES}
    assert set(_declared()) == bound


def test_status_strings_and_kernel_names(lib):
    for code in range(5):
        assert lib.tgrad_status_string(code)
    assert lib.tgrad_status_string(99) == b"unknown status"
    assert tg.kernel_name(0) == "topk_init"
    assert tg.kernel_name(1000) == ""


def test_destroy_null_is_noop(lib):
    assert lib.tgrad_destroy(None) == tg.OK


def _init(lib, shape, ranks, dtype=0, rho=0.05, T=10, lr=1e-3, b1=0.9, b2=0.999, eps=1e-8):
    h = ctypes.c_void_p()
    nd = len(shape)
    sh = (ctypes.c_int64 * max(nd, 1))(*shape)
    rk = (ctypes.c_int64 * max(nd, 1))(*ranks)
    rc = lib.tgrad_init(ctypes.byref(h), nd, sh, rk, dtype, rho, T, lr, b1, b2, eps)
    return rc, h


@pytest.mark.parametrize("kw", [
    dict(shape=(), ranks=()),                               # ndim 0
    dict(shape=(2,) * 9, ranks=(1,) * 9),                   # ndim 9
    dict(shape=(4, 4), ranks=(5, 4)),                       # rank > size
    dict(shape=(4, 4), ranks=(0, 4)),                       # rank 0
    dict(shape=(129, 4), ranks=(8, 4)),                     # factor mode too large
    dict(shape=(4, 4), ranks=(2, 2), dtype=7),              # dtype
    dict(shape=(4, 4), ranks=(2, 2), rho=1.5),              # rho > 1
    dict(shape=(4, 4), ranks=(2, 2), rho=-0.1),
    dict(shape=(4, 4), ranks=(2, 2), T=0),                  # T < 1
    dict(shape=(4, 4), ranks=(2, 2), b1=1.0),               # beta1 = 1
    dict(shape=(4, 4), ranks=(2, 2), eps=-1.0),
    dict(shape=(4, 4), ranks=(2, 2), lr=-1.0),
    dict(shape=(65536, 65536), ranks=(65536, 65536)),       # N = 2^32
    dict(shape=(3, 5, 64), ranks=(3, 5, 16)),               # r_n > N / I_n = 15
    dict(shape=(50,), ranks=(2,)),                          # one mode: N / I_n = 1
    dict(shape=(2, 40), ranks=(2, 3)),                      # 3 > 80 / 40
])
def test_init_rejects_invalid_arguments(lib, kw):
    rc, h = _init(lib, **kw)
    assert rc == tg.EINVAL
    assert not h.value


@pytest.mark.parametrize("kw", [
    dict(shape=(3, 5, 64), ranks=(3, 5, 15)),               # r_n = N / I_n
    dict(shape=(50,), ranks=(1,)),
    dict(shape=(2, 40), ranks=(1, 2)),
    dict(shape=(128, 4), ranks=(4, 4)),                     # a factor mode of 128
    dict(shape=(128, 4), ranks=(4, 4), dtype=3),            # a complex factor mode of 128
])
def test_rank_bound_is_inclusive(lib, kw):
    """r_n up to the rank of the mode-n unfolding, N / I_n, passes argument validation:
    without a device the call then fails at the device query (TGRAD_EHIP), never with
    TGRAD_EINVAL; on a machine with a GPU it succeeds."""
    rc, h = _init(lib, **kw)
    assert rc in (tg.OK, tg.EHIP), rc
    if h.value:
        lib.tgrad_destroy(h)


def test_info_layout():
    """tgrad_info: 7 + 2 * 8 + 2 + 2 int64 fields, matching the ctypes mirror."""
    assert ctypes.sizeof(tg.Info) == (7 + 2 * tg.MAX_NDIM + 4) * 8


def test_null_handle_calls_are_einval(lib):
    assert lib.tgrad_debug_capture_delta(None, None) == tg.EINVAL
    assert lib.tgrad_step(None, None, None, None) == tg.EINVAL
    assert lib.tgrad_refresh(None, None, None) == tg.EINVAL
    assert lib.tgrad_get_omega(None, None, 0) == tg.EINVAL
    assert lib.tgrad_mark_refreshed(None) == tg.EINVAL
    assert lib.tgrad_timing_enable(None, 1, 10) == tg.EINVAL
    assert lib.tgrad_set_stream_products(None, 1) == tg.EINVAL
    assert lib.tgrad_set_stream_overlap(None, 1, 1) == tg.EINVAL
    assert lib.tgrad_set_pair_fusion(None, 1) == tg.EINVAL
    assert lib.tgrad_set_gram_fusion(None, 1) == tg.EINVAL


def test_default_options_are_the_plain_method(lib):
    """tgrad_default_options is host-only; the ctypes layout matches the C struct
    (two doubles, two int32, one uint64, two int32: 40 bytes)."""
    assert ctypes.sizeof(tg.Options) == 40
    o = tg.Options(7.0, 7.0, 5, 5, 5, 5, 5)
    lib.tgrad_default_options(ctypes.byref(o))
    assert (o.weight_decay, o.sparse_scale, o.selection, o.remap_moments, o.seed, o.order,
            o.reserved) == (0.0, 1.0, tg.SELECT_TOPK, 0, 0, 0, 0)
    assert lib.tgrad_set_options(None, ctypes.byref(o)) == tg.EINVAL
    assert lib.tgrad_get_options(None, ctypes.byref(o)) == tg.EINVAL


def test_step_many_argument_checks_need_no_device(lib):
    """tgrad_step_many validates its arguments before any device work: n = 0 is a no-op,
    a negative count or NULL arrays are EINVAL."""
    P = ctypes.c_void_p
    assert lib.tgrad_step_many(None, None, None, 0, None) == tg.OK
    assert lib.tgrad_step_many(None, None, None, -1, None) == tg.EINVAL
    assert lib.tgrad_step_many(None, None, None, 2, None) == tg.EINVAL
    hs = (P * 1)(None)
    assert lib.tgrad_step_many(hs, hs, hs, 1, None) == tg.EINVAL


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures the step on one GPU: --gpus 2 prints one JSON error line and
    exits with status 2 before importing torch or touching a device."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
