"""The allocation-free entry point (qgemv_run_noalloc): through the C ABI, its
outputs equal qgemv_run's bit for bit (the same kernels and launch plans, the
workspace in the library's static scratch array instead of the handle) and
match the oracle, on two calls in a row, the second with a smaller input, for
the M = 1 GEMVs, the verify GEMM and the trellis product; a run whose
workspace exceeds the array is refused before anything is enqueued."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, dev_u16, say  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def noalloc(lin, x):
    """qgemv_run_noalloc through the C ABI (no Python wrapper involved)."""
    L = Q.lib()
    f = L.qgemv_run_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    y = torch.full((x.shape[0], lin.N), float("nan"), dtype=torch.float16, device="cuda")
    st = f(lin.handle, x.data_ptr(), int(x.shape[0]), y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if st != 0:
        raise Q.QGError(st, L.qg_last_error().decode())
    return y


def _pair(lin, x_np, ref):
    x = dev_f16(x_np)
    y_ref = lin.run(x)
    y_na = noalloc(lin, x)
    torch.cuda.synchronize()
    err = O.normwise_rel_err(y_na.cpu().numpy().astype(np.float64), ref)
    say("noalloc err", err, "run err", O.normwise_rel_err(y_ref.cpu().numpy().astype(np.float64), ref))
    assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16))
    assert err <= TOL, err


@pytest.mark.parametrize("pins", [0, Q.PIN_M1_RUNS, Q.PIN_M1_PERGROUP | Q.PIN_PARTIALS])
def test_m1_two_calls_second_smaller(pins):
    big = Uniform(4096, 9216, 3, cfg_id=150, pins=pins)
    small = Uniform(272, 2560, 4, cfg_id=151, pins=pins)
    say("noalloc m1", pins)
    xb = S.activations(1, 9216, cfg_id=150)
    _pair(big.lin, xb, O.gemv_uniform_rows(xb, big.words, big.scales, 4096, 9216, 3, np.arange(4096)))
    xs = S.activations(1, 2560, cfg_id=151)
    _pair(small.lin, xs, small.ref(xs))


@pytest.mark.parametrize("M1,M2", [(32, 8), (16, 3)])
def test_verify_two_calls_second_smaller(M1, M2):
    u = Uniform(1024, 5120, 3, cfg_id=152)
    for M in (M1, M2):
        say("noalloc verify", M)
        x = S.activations(M, 5120, cfg_id=152, tensor_id=M)
        _pair(u.lin, x, u.ref(x))


def test_verify_gate_up_shape_full_rows():
    N, K = 17408, 5120
    w = S.uniform_code_words(N, K, 3, cfg_id=153)
    sc = S.scales(N, K, cfg_id=153)
    from _gpu import dev_words
    lin = Q.QLinear(dev_words(w), dev_f16(sc), K, N, bits=3, max_M=32)
    for M in (32, 1):
        x = S.activations(M, K, cfg_id=153, tensor_id=M)
        xd = dev_f16(x)
        a, b = lin.run(xd), noalloc(lin, xd)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        rows = np.arange(0, N, 97)
        err = O.normwise_rel_err(b.cpu().numpy().astype(np.float64)[:, rows],
                                 O.gemv_uniform_rows(x, w, sc, N, K, 3, rows))
        assert err <= TOL, err


@pytest.mark.parametrize("M1,M2", [(8, 1), (1, 2)])
def test_trellis_two_calls(M1, M2):
    N, K = 400, 2560
    cb = S.codebook(cfg_id=154)
    words, scales = S.trellis_words(N, K, cfg_id=154), S.scales(N, K, cfg_id=154)
    for pins in (0, Q.PIN_TRELLIS_ROT_LAUNCH | Q.PIN_PARTIALS):
        lin = Q.QLinear(dev_u16(words), dev_f16(scales), K, N, trellis=True, codebook=dev_f16(cb), max_M=8, pins=pins)
        for M in (M1, M2):
            say("noalloc trellis", pins, M)
            x = S.activations(M, K, cfg_id=154, tensor_id=M)
            _pair(lin, x, O.gemv_trellis(x, words, cb, scales, N, K))


def test_too_large_is_refused_before_any_work():
    N, K = 69632, 5120                     # 4 x gate|up stacked at 32 rows: partials beyond the static array
    w = S.uniform_code_words(N, K, 3, cfg_id=155)
    from _gpu import dev_words
    lin = Q.QLinear(dev_words(w), dev_f16(S.scales(N, K, cfg_id=155)), K, N, bits=3, max_M=32)
    x = dev_f16(S.activations(32, K, cfg_id=155))
    with pytest.raises(Q.QGError) as e:
        noalloc(lin, x)
    assert e.value.status == Q.QG_ERR_INVALID_ARG and "scratch" in str(e.value)
    y = noalloc(lin, x[:1].contiguous())   # one row fits
    torch.cuda.synchronize()
    assert torch.equal(y, lin.run(x[:1].contiguous()))
