"""The C-ABI library loads, exports every function include/cfm.h declares, and
rejects bad arguments on the host with the documented status codes (these
calls return before any HIP call, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cfm.h")
LIB = os.path.join(ROOT, "calibration_free_channel_amd", "libcfm.so")

OK, EINVAL, EUNSUP, EWS = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "libcfm.so not built (python calibration_free_channel_amd/build.py)"
    return ctypes.CDLL(LIB)


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("sketch_build", "lowrank_build", "moe_select_forward", "moe_dense_forward"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_python_binding_covers_the_header():
    from calibration_free_channel_amd import _lib
    assert set(_lib.EXPORTED) == set(_declared())


def _sel(lib, T=1, K=2, E=8, I=128, H=256, k=23, c=46, r=8, ptr=FAKE, ws=FAKE, wsb=1 << 40, A=FAKE):
    f = lib.moe_select_forward
    f.restype = ctypes.c_int
    P = ptr
    return f(P, P, P, T, K, P, P, P, E, I, H, P, P, P, P, P, A, A, k, c, r, P, None, None, None,
             ws, ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(H=96), EUNSUP),            # not a power of two
    (dict(H=32), EUNSUP),            # too small
    (dict(H=16384), EUNSUP),         # too large
    (dict(k=47), EUNSUP),            # k > c
    (dict(c=129), EUNSUP),           # c > I
    (dict(r=129), EUNSUP),           # r > min(H, I)
    (dict(k=-1), EUNSUP),
    (dict(K=0), EINVAL),
    (dict(K=65), EUNSUP),
    (dict(T=-1), EINVAL),
    (dict(E=0), EINVAL),
    (dict(ptr=None), EINVAL),        # null arrays
    (dict(A=None), EINVAL),          # r > 0 needs the map
    (dict(ws=None), EWS),
    (dict(wsb=16), EWS),
])
def test_select_forward_rejects(lib, kw, code):
    assert _sel(lib, **kw) == code
    lib.cfm_last_error.restype = ctypes.c_char_p
    assert lib.cfm_last_error().decode() != ""


def _sel_ex(lib, flags, T=1, K=2, E=8, I=128, H=256, k=23, c=46, r=8, ptr=FAKE, ws=FAKE, wsb=1 << 40):
    f = lib.moe_select_forward_ex
    f.restype = ctypes.c_int
    P = ptr
    return f(P, P, P, T, K, P, P, P, E, I, H, P, P, P, P, P, P, P, k, c, r, ctypes.c_uint(flags), P, None,
             None, None, ws, ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("flags,kw,code", [
    (2, {}, EINVAL),                 # undefined flag bit
    (0x80000000, {}, EINVAL),
    (1, dict(k=47), EUNSUP),         # the variant keeps every other check
    (1, dict(ptr=None), EINVAL),
    (1, dict(wsb=16), EWS),
    (0, dict(wsb=16), EWS),
    (1, dict(T=0, ptr=None, ws=None), OK),
])
def test_select_forward_ex_flags(lib, flags, kw, code):
    assert _sel_ex(lib, flags, **kw) == code


def _sel_thr(lib, tau, flags=0, T=1, K=2, E=8, I=128, H=256, c=46, r=8, ptr=FAKE, ws=FAKE, wsb=1 << 40):
    f = lib.moe_select_forward_threshold
    f.restype = ctypes.c_int
    P = ptr
    return f(P, P, P, T, K, P, P, P, E, I, H, P, P, P, P, P, P, P, ctypes.c_float(tau), c, r,
             ctypes.c_uint(flags), P, None, None, None, None, ws, ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("tau,flags,kw,code", [
    (float("nan"), 0, {}, EINVAL),
    (-1.0, 0, {}, EINVAL),
    (float("-inf"), 0, {}, EINVAL),
    (1.0, 2, {}, EINVAL),                # undefined flag bit
    (1.0, 0, dict(c=129), EUNSUP),       # c > I
    (1.0, 0, dict(r=129), EUNSUP),
    (1.0, 0, dict(ptr=None), EINVAL),
    (1.0, 1, dict(ptr=None), EINVAL),
    (1.0, 0, dict(wsb=16), EWS),
    (1.0, 0, dict(T=0, ptr=None, ws=None), OK),
    (float("inf"), 1, dict(T=0, ptr=None, ws=None), OK),
    (-0.0, 0, dict(T=0, ptr=None, ws=None), OK),
])
def test_select_forward_threshold_rejects(lib, tau, flags, kw, code):
    assert _sel_thr(lib, tau, flags, **kw) == code


def test_select_forward_empty_batch_is_a_noop(lib):
    assert _sel(lib, T=0, ptr=None, ws=None) == OK


def test_select_forward_r0_needs_no_map(lib):
    # with r = 0 a null map is fine; the call then fails only on the tiny workspace
    assert _sel(lib, r=0, A=None, wsb=16) == EWS


def test_workspace_queries(lib):
    lib.select_workspace.restype = ctypes.c_size_t
    lib.dense_workspace.restype = ctypes.c_size_t
    lib.lowrank_workspace.restype = ctypes.c_size_t
    assert lib.select_workspace(1, 8, 128, 768, 2048, 138, 276, 64) > 0
    assert lib.select_workspace(1, 8, 128, 768, 2048, 300, 276, 64) == 0   # k > c
    assert lib.dense_workspace(16, 8, 128, 768, 2048) > 0
    assert lib.lowrank_workspace(128, 768, 2048, 64) >= 128 * 768 * 768 * 8
    assert lib.lowrank_workspace(8, 128, 256, 200) == 0


def test_sketch_build_rejects(lib):
    f = lib.sketch_build
    f.restype = ctypes.c_int
    P = FAKE
    assert f(P, P, 8, 128, 100, P, P, P, P, P, None) == EUNSUP
    assert f(None, P, 8, 128, 256, P, P, P, P, P, None) == EINVAL
    assert f(P, P, 0, 128, 256, P, P, P, P, P, None) == EINVAL


def test_lowrank_build_rejects(lib):
    f = lib.lowrank_build
    f.restype = ctypes.c_int
    P = FAKE
    assert f(P, 8, 128, 256, 129, P, P, P, ctypes.c_size_t(1 << 40), None) == EUNSUP
    assert f(P, 8, 128, 256, 8, P, P, None, ctypes.c_size_t(0), None) == EWS
    assert f(P, 8, 128, 256, 0, None, None, None, ctypes.c_size_t(0), None) == OK   # r = 0: nothing to do


def test_dense_forward_rejects(lib):
    f = lib.moe_dense_forward
    f.restype = ctypes.c_int
    P = FAKE
    assert f(P, P, P, 1, 2, P, P, P, 8, 128, 100, P, P, ctypes.c_size_t(1 << 40), None) == EUNSUP
    assert f(P, P, P, 1, 2, P, P, P, 8, 128, 256, P, None, ctypes.c_size_t(0), None) == EWS
    assert f(None, P, P, 1, 2, P, P, P, 8, 128, 256, P, P, ctypes.c_size_t(1 << 40), None) == EINVAL


def test_forward_path_switch(lib):
    f = lib.cfm_set_forward_path
    f.restype = ctypes.c_int
    assert f(5) == EINVAL and f(-1) == EINVAL
    prev = f(4)
    assert f(3) == 4                        # 4: per-pair with the screen inside the single launch
    f(prev)
    prev = f(2)
    try:
        assert f(2) == 2
        # the grouped pass needs r to be a multiple of 8: refused before any HIP call
        assert _sel(lib, r=6) == EUNSUP
        assert _sel(lib, r=8, wsb=16) == EWS
        # dense: H a multiple of 64 suffices
        d = lib.moe_dense_forward
        d.restype = ctypes.c_int
        assert d(FAKE, FAKE, FAKE, 1, 2, FAKE, FAKE, FAKE, 8, 128, 192, FAKE, FAKE, ctypes.c_size_t(16), None) == EWS
        assert f(1) == 2
        assert _sel(lib, r=6, wsb=16) == EWS
        assert f(3) == 1 and f(1) == 3          # per-pair without the batch-1 instance
    finally:
        f(prev)


def test_workspace_covers_both_passes(lib):
    lib.select_workspace.restype = ctypes.c_size_t
    lib.dense_workspace.restype = ctypes.c_size_t
    # grouped regions follow the per-pair layout, so a batch of 16 needs more than the per-pair pass alone
    one = lib.select_workspace(1, 8, 128, 768, 2048, 100, 200, 64)
    many = lib.select_workspace(16, 8, 128, 768, 2048, 100, 200, 64)
    assert many > 16 * 8 * 768 * (8 + 4 + 4 + 2)      # per-pair exchange words plus grouped activations
    assert many > one
    assert lib.dense_workspace(16, 8, 128, 768, 2048) > 16 * 8 * 768 * 8


def _layer(lib, E=8, K=2, eps=1e-6, ptr=FAKE, T=1, wsb=1 << 40, flags=0):
    f = lib.moe_layer_forward
    f.restype = ctypes.c_int
    P = ptr
    return f(P, P, ctypes.c_float(eps), P, 0, T, K, P, P, P, E, 128, 256, P, P, P, P, P, P, P, 23, 46, 8,
             ctypes.c_uint(flags), P, None, None, None, FAKE, ctypes.c_size_t(wsb), None)


@pytest.mark.parametrize("kw,code", [
    (dict(E=2048), EUNSUP),          # the envelope's router covers at most 1024 experts
    (dict(E=4, K=5), EUNSUP),        # K > E
    (dict(eps=-1.0), EINVAL),
    (dict(eps=float("nan")), EINVAL),
    (dict(ptr=None), EINVAL),
    (dict(flags=4), EINVAL),
    (dict(wsb=16), EWS),
    (dict(T=0, ptr=None), OK),
])
def test_layer_forward_rejects(lib, kw, code):
    assert _layer(lib, **kw) == code


def test_layer_dense_forward_rejects(lib):
    f = lib.moe_layer_dense_forward
    f.restype = ctypes.c_int
    P = FAKE
    args = lambda eps, wsb: (P, P, ctypes.c_float(eps), P, 0, 1, 2, P, P, P, 8, 128, 256, P, None, None, None, P,
                             ctypes.c_size_t(wsb), None)
    assert f(*args(-1.0, 1 << 40)) == EINVAL
    assert f(*args(1e-6, 16)) == EWS

