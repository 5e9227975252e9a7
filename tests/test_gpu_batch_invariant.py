"""Batch-invariant rows (QG_FLAG_BATCH_INVARIANT): row m of a run of M rows is
bit-identical to that row run alone, for every M up to max_M -- at 2, 3 and 4
bits and several widths, through fixed-point words and through fp32 partials,
in the fused MLP, through the allocation-free entry point, at the full
27B-class gate/up and down shapes -- and every output still matches the oracle
within the normwise budget.  Repeats are bit-identical as everywhere."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, dev_words, say  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


MS = (1, 2, 3, 7, 8, 15, 16, 17, 24, 31, 32)


def _bits(t):
    return t.view(torch.int16)


def _rows_alone(run, x, n_rows):
    ys = [run(x[m:m + 1]) for m in range(n_rows)]
    torch.cuda.synchronize()
    return torch.cat(ys)


def _assert_invariant(run, x, alone, Ms=MS):
    for M in Ms:
        y = run(x[:M])
        torch.cuda.synchronize()
        same = torch.equal(_bits(y), _bits(alone[:M]))
        if not same:
            bad = (_bits(y) != _bits(alone[:M])).nonzero()[:5].tolist()
            pytest.fail(f"M={M}: rows differ from the rows run alone at {bad}")


# (N, K, bits or None for mixed, pins): K = 5120 and 17408 take several K slices
CASES = [
    (400, 5120, 3, 0),
    (256, 5120, 2, 0),
    (272, 5120, 4, Q.PIN_PARTIALS),
    (256, 17408, 3, 0),
    (208, 17408, 3, Q.PIN_PARTIALS),
    (480, 1536, None, 0),
    (1040, 640, 3, Q.PIN_XS_T2),
]


@pytest.mark.parametrize("N,K,bits,pins", CASES)
def test_rows_equal_rows_alone(N, K, bits, pins):
    cb = None if bits is not None else S.column_bits(N, 0.3, 4, cfg_id=170, tensor_id=S.T_MASK)
    m = Uniform(N, K, bits if bits else 3, col_bits=cb, cfg_id=170, tid=N % 7, pins=pins, batch_invariant=True)
    x_np = S.activations(32, K, cfg_id=171, tensor_id=K % 11)
    x = dev_f16(x_np)
    say("invariant", N, K, bits, pins)
    alone = _rows_alone(m.lin.run, x, 32)
    _assert_invariant(m.lin.run, x, alone)
    err = O.normwise_rel_err(alone.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("err", err)
    assert err <= TOL, err
    # repeats
    assert torch.equal(_bits(m.lin.run(x)), _bits(m.lin.run(x)))


def test_plain_handle_is_not_invariant_but_flagged_one_matches_it_in_tolerance():
    """The default handle's M = 1 GEMV and verify GEMM round differently; the
    flagged handle's single rows agree with the default handle's within the
    budget (both against the oracle)."""
    N, K = 512, 5120
    m = Uniform(N, K, 3, cfg_id=172, batch_invariant=True)
    plain = m.relinked()
    x_np = S.activations(1, K, cfg_id=172)
    x = dev_f16(x_np)
    a, b = m.lin.run(x), plain.run(x)
    torch.cuda.synchronize()
    r = m.ref(x_np)
    for y in (a, b):
        assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64), r) <= TOL


def test_mlp_rows_equal_rows_alone():
    H, I = 1024, 5120
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=173, tensor_id=S.T_MASK)
    cb_dn = S.column_bits(H, 0.2, 2, cfg_id=173, tensor_id=S.T_MASK + 100)
    wg = S.mixed_code_words(cb_gu, H, cfg_id=173, tensor_id=S.T_CODES)
    wu = S.mixed_code_words(cb_gu, H, cfg_id=173, tensor_id=S.T_CODES + 10)
    wd = S.mixed_code_words(cb_dn, I, cfg_id=173, tensor_id=S.T_CODES + 20)
    sg = S.scales(I, H, cfg_id=173, tensor_id=S.T_SCALE)
    su = S.scales(I, H, cfg_id=173, tensor_id=S.T_SCALE + 10)
    sd = S.scales(H, I, cfg_id=173, tensor_id=S.T_SCALE + 20)
    mk = lambda w, s, k, n, cb: Q.QLinear(dev_words(w), dev_f16(s), k, n, col_bits=cb, max_M=32, batch_invariant=True)
    g, u, d = mk(wg, sg, H, I, cb_gu), mk(wu, su, H, I, cb_gu), mk(wd, sd, I, H, cb_dn)
    x_np = S.activations(32, H, cfg_id=174)
    x = dev_f16(x_np)
    run = lambda xx: Q.mlp(g, u, d, xx)
    say("invariant mlp")
    alone = _rows_alone(run, x, 32)
    _assert_invariant(run, x, alone, Ms=(1, 2, 8, 16, 17, 32))
    h = O.silu(O.gemv_mixed(x_np, wg, sg, cb_gu, H)) * O.gemv_mixed(x_np, wu, su, cb_gu, H)
    r = O.gemv_mixed(h, wd, sd, cb_dn, I)
    err = O.normwise_rel_err(alone.cpu().numpy().astype(np.float64), r)
    say("mlp err", err)
    assert err <= TOL, err


def test_mlp_flags_must_agree():
    H, I = 256, 512
    a = Uniform(I, H, 3, cfg_id=175, tid=0, batch_invariant=True)
    b = Uniform(I, H, 3, cfg_id=175, tid=1)
    c = Uniform(H, I, 3, cfg_id=175, tid=2, batch_invariant=True)
    with pytest.raises(Q.QGError):
        Q.mlp(a.lin, b.lin, c.lin, dev_f16(S.activations(1, H, cfg_id=175)))


def test_noalloc_rows_equal_rows_alone():
    N, K = 320, 5120
    m = Uniform(N, K, 3, cfg_id=176, batch_invariant=True)
    L = Q.lib()
    f = L.qgemv_run_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int

    def run(xx):
        y = torch.empty((xx.shape[0], N), dtype=torch.float16, device="cuda")
        st = f(m.lin.handle, xx.data_ptr(), int(xx.shape[0]), y.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, L.qg_last_error().decode()
        return y

    x = dev_f16(S.activations(32, K, cfg_id=176))
    alone = _rows_alone(m.lin.run, x, 32)  # the handle's own workspace
    _assert_invariant(run, x, alone, Ms=(1, 5, 16, 32))


def test_batch_entry_point_runs_flagged_handles_invariantly():
    a = Uniform(256, 5120, 3, cfg_id=177, tid=0, batch_invariant=True)
    b = Uniform(512, 5120, 3, cfg_id=177, tid=1, batch_invariant=True)
    x = dev_f16(S.activations(1, 5120, cfg_id=177))
    ya, yb = Q.run_batch([a.lin, b.lin], [x, x])
    torch.cuda.synchronize()
    assert torch.equal(_bits(ya), _bits(a.lin.run(x)))
    assert torch.equal(_bits(yb), _bits(b.lin.run(x)))


def test_trellis_refuses_the_flag():
    cbk = dev_f16(S.codebook(cfg_id=S.CFG_TRELLIS))
    N, K = 64, 256
    tw = S.trellis_words(N, K, cfg_id=178)
    ts = S.scales(N, K, cfg_id=178)
    dtw = torch.from_numpy(np.ascontiguousarray(tw).view(np.int16).copy()).cuda()
    with pytest.raises(Q.QGError):
        Q.QLinear(dtw, dev_f16(ts), K, N, trellis=True, codebook=cbk, max_M=8, batch_invariant=True)


@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_full_size_rows_equal_rows_alone(N, K):
    """The gate/up and down shapes at 3 bits: every row count's rows equal the
    rows run alone (all columns, bitwise); sampled columns against the oracle."""
    m = Uniform(N, K, 3, cfg_id=S.CFG_DECODE, tid=3, batch_invariant=True)
    x_np = S.activations(32, K, cfg_id=179)
    x = dev_f16(x_np)
    say("invariant full", N, K)
    alone = _rows_alone(m.lin.run, x, 32)
    _assert_invariant(m.lin.run, x, alone, Ms=(1, 2, 8, 16, 17, 32))
    rows = np.sort(np.random.default_rng(179).choice(N, 96, replace=False))
    err = O.normwise_rel_err(alone.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("err", err)
    assert err <= TOL, err
