"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching a device."""
from __future__ import annotations

import ctypes

import pytest

import bit_weight_only_packed_amd as Q


@pytest.fixture(scope="module")
def L():
    try:
        return Q.lib()
    except ImportError as e:  # the build step must have run first
        pytest.fail(str(e))


def test_exports_every_declared_symbol(L):
    names = Q.declared_symbols()
    assert {"qgemv_create", "qgemv_run", "qmlp_run", "qgemv_destroy", "qg_last_error",
            "qgemv_debug_unpack", "qgemv_debug_dequant", "qgemv_debug_operand", "qgemv_debug_trellis",
            "qgemv_weight_bytes", "qg_stream_read"} <= set(names)
    assert "qgemv_set_launch" not in names    # launch choices are fixed at create
    for n in names:
        assert hasattr(L, n), n


def _desc(**kw):
    d = Q._Desc()
    d.K, d.N, d.group_size, d.format, d.bits = 512, 512, 128, 0, 3
    d.codes, d.scales = 0x100000, 0x200000      # never dereferenced: validation fails first
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("kw,frag", [
    (dict(K=500), "K"), (dict(K=0), "K"), (dict(N=20), "N"), (dict(group_size=16), "group_size"),
    (dict(group_size=96), "group_size"), (dict(format=1, group_size=64), "group_size"),
    (dict(codes=0), "codes"), (dict(scales=0x200004), "aligned"), (dict(format=7), "format"),
    (dict(format=1, codebook=None), "codebook"),
])
def test_create_rejects_bad_descriptor(L, kw, frag):
    h = ctypes.c_void_p(1)
    d = _desc(**kw)
    st = L.qgemv_create(ctypes.byref(h), ctypes.byref(d), 8, None)
    assert st == Q.QG_ERR_INVALID_ARG
    assert h.value is None
    assert frag in L.qg_last_error().decode()


@pytest.mark.parametrize("cls,launch,frag", [(0, (0, 17, 0), "16 waves"), (1, (9, 0, 0), "8 tile groups"),
                                              (2, (0, 0, 64), "63 K slices"), (1, (-1, 0, 0), "negative")])
def test_create_rejects_bad_launch_override(L, cls, launch, frag):
    d = _desc()
    d.launch[cls] = Q._Launch(*launch)
    h = ctypes.c_void_p()
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(d), 8, None) == Q.QG_ERR_INVALID_ARG
    assert frag in L.qg_last_error().decode()


@pytest.mark.parametrize("pins", [Q.PIN_M1_PERGROUP | Q.PIN_M1_RUNS, Q.PIN_XS_T1 | Q.PIN_XS_T2,
                                  Q.PIN_PARTIALS | Q.PIN_WORDS])
def test_create_rejects_conflicting_pins(L, pins):
    d = _desc(pins=pins)
    h = ctypes.c_void_p()
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(d), 8, None) == Q.QG_ERR_INVALID_ARG
    assert "pins" in L.qg_last_error().decode()


@pytest.mark.parametrize("max_M", [0, 33, -1])
def test_create_rejects_bad_max_m(L, max_M):
    h = ctypes.c_void_p()
    d = _desc()
    assert L.qgemv_create(ctypes.byref(h), ctypes.byref(d), max_M, None) == Q.QG_ERR_INVALID_ARG


def test_null_arguments(L):
    d = _desc()
    assert L.qgemv_create(None, ctypes.byref(d), 8, None) == Q.QG_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    assert L.qgemv_create(ctypes.byref(h), None, 8, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_run(None, 0x1000, 1, 0x2000, None) == Q.QG_ERR_INVALID_ARG
    assert L.qmlp_run(None, None, None, 0x1000, 1, 0x2000, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_debug_unpack(None, 0x1000, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_debug_dequant(None, 0x1000, None, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_debug_trellis(None, 0x1000, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_debug_operand(None, 0x1000, None, None, None) == Q.QG_ERR_INVALID_ARG
    assert L.qg_stream_read(None, 1024, None) == Q.QG_ERR_INVALID_ARG
    assert L.qg_stream_read(0x1000, 1000, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_weight_bytes(None, None) == Q.QG_ERR_INVALID_ARG
    assert L.qgemv_destroy(None) == Q.QG_OK
    assert L.qg_last_error() == b""


def test_bad_col_bits_rejected_before_device(L):
    import numpy as np
    cb = np.full(512, 3, dtype=np.uint8)
    cb[7] = 5
    d = _desc(bits=0, col_bits=cb.ctypes.data)
    h = ctypes.c_void_p()
    st = L.qgemv_create(ctypes.byref(h), ctypes.byref(d), 8, None)
    # either the device check (no GPU here) or the width check rejects it; never OK
    assert st in (Q.QG_ERR_INVALID_ARG, Q.QG_ERR_UNSUPPORTED)


def test_binding_constants_match_the_header():
    """Every status code, format, flag and pin the binding passes to the
    library has the value include/qgemv.h declares (read from the header's
    enumerators, `1u << n` forms evaluated)."""
    import re
    text = open(Q.HEADER_PATH).read()
    decl = {}
    for name, expr in re.findall(r"\b(QG_[A-Z0-9_]+)\s*=\s*(-?\d+u?(?:\s*<<\s*\d+)?)", text):
        m = re.fullmatch(r"(-?\d+)u?(?:\s*<<\s*(\d+))?", expr.strip())
        decl[name] = int(m.group(1)) << int(m.group(2) or 0)
    pairs = {"QG_OK": Q.QG_OK, "QG_ERR_INVALID_ARG": Q.QG_ERR_INVALID_ARG, "QG_ERR_UNSUPPORTED": Q.QG_ERR_UNSUPPORTED,
             "QG_ERR_DEVICE": Q.QG_ERR_DEVICE, "QG_ERR_OOM": Q.QG_ERR_OOM,
             "QG_FMT_UNIFORM": Q.FMT_UNIFORM, "QG_FMT_TRELLIS3": Q.FMT_TRELLIS3, "QG_FMT_MXFP4": Q.FMT_MXFP4,
             "QG_FMT_MXFP6": Q.FMT_MXFP6, "QG_FLAG_X_PREROTATED": Q.FLAG_X_PREROTATED,
             "QG_FLAG_BATCH_INVARIANT": Q.FLAG_BATCH_INVARIANT, "QG_PIN_M1_PERGROUP": Q.PIN_M1_PERGROUP,
             "QG_PIN_M1_RUNS": Q.PIN_M1_RUNS, "QG_PIN_PARTIALS": Q.PIN_PARTIALS, "QG_PIN_WORDS": Q.PIN_WORDS,
             "QG_PIN_XS_T1": Q.PIN_XS_T1, "QG_PIN_XS_T2": Q.PIN_XS_T2,
             "QG_PIN_TRELLIS_ROT_LAUNCH": Q.PIN_TRELLIS_ROT_LAUNCH, "QG_PIN_TRELLIS_BAND": Q.PIN_TRELLIS_BAND,
             "QG_GROUP": Q.GROUP}
    for name, value in pairs.items():
        assert decl.get(name) == value, (name, decl.get(name), value)
    # every pin and flag the header declares is known to the binding
    assert {n for n in decl if n.startswith(("QG_PIN_", "QG_FLAG_", "QG_FMT_"))} <= set(pairs)
