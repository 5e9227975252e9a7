"""MXFP4 weights (E2M1 elements, one UE8M0 exponent byte per 32): the
elements, exact weights and the verify GEMM's operand are bit-exact against
the oracle; products match the oracle within the normwise budget at every row
count (both tile groupings and hand-overs, narrow and long matrices, exponents
spread far apart within a group); a NaN exponent byte makes exactly its
columns NaN; the prefill route, the batch entry point and batch-invariant rows
work; the full 27B-class gate/up shape on sampled columns."""
from __future__ import annotations

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


class MX:
    def __init__(self, N, K, cfg=210, tid=0, lo=116, hi=124, **kw):
        self.N, self.K = N, K
        self.words = S.uniform_code_words(N, K, 4, cfg_id=cfg, tensor_id=S.T_CODES + tid)
        self.e8 = S.mx_scales(N, K, cfg_id=cfg, tensor_id=S.T_SCALE + tid, lo=lo, hi=hi)
        self.dw = dev_words(self.words)
        self.de = torch.from_numpy(self.e8.copy()).cuda()
        self.lin = Q.QLinear(self.dw, self.de, K, N, mxfp4=True, max_M=32, **kw)

    def codes(self):
        return O.unpack_uniform(self.words, self.N, self.K, 4)

    def ref(self, x, rows=None):
        return O.gemv_mxfp4(x, self.words, self.e8, self.N, self.K, rows)


def test_decode_bit_exact():
    m = MX(400, 1536, lo=100, hi=140)
    codes = m.codes()
    np.testing.assert_array_equal(m.lin.debug_unpack().cpu().numpy(), codes)
    w, q = m.lin.debug_dequant()
    np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), O.dequant_mxfp4(codes, m.e8))
    lut = np.array([O.e2m1_value(c) for c in range(16)])
    np.testing.assert_array_equal(q.cpu().numpy().astype(np.float64), lut[codes])
    # the verify GEMM's operand: element * 2^-14 * 2^-(e_max - e) rounded once to fp16
    c, b, wo = m.lin.debug_operand()
    np.testing.assert_array_equal(c.cpu().numpy(), codes)
    e = m.e8.astype(np.int64)
    emax = e.reshape(m.N, -1, 4).max(axis=2)
    de = np.repeat(np.repeat(emax, 4, axis=1) - e, 32, axis=1)
    want = (lut[codes] * 2.0 ** (-14 - de)).astype(np.float16)
    np.testing.assert_array_equal(b.cpu().numpy().view(np.uint16), want.view(np.uint16))
    wexp = want.astype(np.float64) * 2.0 ** (np.repeat(emax, 128, axis=1) - 113)
    np.testing.assert_array_equal(wo.cpu().numpy().astype(np.float64), wexp.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("N,K", [(400, 1536), (128, 5120), (256, 17408)])
@pytest.mark.parametrize("M", [1, 2, 8, 17, 32])
def test_products(N, K, M):
    m = MX(N, K, tid=N % 9)
    x_np = S.activations(M, K, cfg_id=211, tensor_id=M)
    y = m.lin.run(dev_f16(x_np))
    y2 = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("mxfp4", N, K, M, err)
    assert err <= TOL, err


@pytest.mark.parametrize("pins", [Q.PIN_XS_T1 | Q.PIN_PARTIALS, Q.PIN_XS_T2 | Q.PIN_WORDS])
@pytest.mark.parametrize("M", [8, 32])
def test_verify_variants_and_spread_exponents(pins, M):
    m = MX(528, 5120, tid=3, lo=96, hi=127, pins=pins)  # 31 binades within groups, outputs within fp16
    x_np = S.activations(M, m.K, cfg_id=212, tensor_id=M)
    y = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("mxfp4 spread", pins, M, err)
    assert err <= TOL, err


@pytest.mark.parametrize("M", [1, 8])
def test_nan_exponent(M):
    N, K = 256, 1024
    m = MX(N, K, tid=4)
    e8 = m.e8.copy()
    e8[37, 5] = 255
    m.de.copy_(torch.from_numpy(e8))
    lin = Q.QLinear(m.dw, m.de, K, N, mxfp4=True, max_M=32)
    x_np = S.activations(M, K, cfg_id=213)
    y = lin.run(dev_f16(x_np)).cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(y[:, 37]))
    ok = np.ones(N, dtype=bool)
    ok[37] = False
    assert np.all(np.isfinite(y[:, ok]))
    m.e8 = e8
    assert O.normwise_rel_err(y[:, ok], m.ref(x_np)[:, ok]) <= TOL


def test_prefill():
    m = MX(400, 1536, tid=5)
    x_np = S.activations(80, m.K, cfg_id=214)
    ws = torch.zeros(m.lin.prefill_workspace()[1], dtype=torch.uint8, device="cuda")
    y = m.lin.run_prefill(dev_f16(x_np), workspace=ws)
    torch.cuda.synchronize()
    got = ws[32 << 20:(32 << 20) + m.N * m.K * 2].view(torch.float16).cpu().numpy().reshape(m.N, m.K)
    # values equal bit for bit except the sign of zero (E2M1 code 8 is -0; the
    # route's fp16 weight of it may be +0, which multiplies the same)
    want = O.dequant_mxfp4(m.codes(), m.e8).astype(np.float16)
    np.testing.assert_array_equal(got.astype(np.float64), want.astype(np.float64))
    nz = want != 0
    np.testing.assert_array_equal(got.view(np.uint16)[nz], want.view(np.uint16)[nz])
    assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np)) <= TOL


def test_batch_and_invariant_rows():
    a = MX(256, 1536, tid=6)
    u = Uniform(400, 1536, 3, cfg_id=215)
    xs_np = [S.activations(1, 1536, cfg_id=215, tensor_id=i) for i in range(2)]
    ya, yu = Q.run_batch([a.lin, u.lin], [dev_f16(x) for x in xs_np])
    torch.cuda.synchronize()
    assert O.normwise_rel_err(ya.cpu().numpy().astype(np.float64), a.ref(xs_np[0])) <= TOL
    assert O.normwise_rel_err(yu.cpu().numpy().astype(np.float64), u.ref(xs_np[1])) <= TOL
    inv = MX(272, 5120, tid=7, batch_invariant=True)
    x = dev_f16(S.activations(32, 5120, cfg_id=216))
    alone = torch.cat([inv.lin.run(x[i:i + 1]) for i in range(32)])
    for M in (1, 7, 16, 17, 32):
        assert torch.equal(inv.lin.run(x[:M]).view(torch.int16), alone[:M].view(torch.int16)), M


def test_refusals():
    g = MX(128, 256, tid=8)
    d = MX(256, 128, tid=9)
    with pytest.raises(Q.QGError):  # the fused MLP takes uniform codes only
        Q.mlp(g.lin, g.lin, d.lin, dev_f16(S.activations(1, 256, cfg_id=217)))
    L = Q.lib()
    desc = Q._Desc()
    desc.K, desc.N, desc.group_size, desc.format, desc.bits = 256, 128, 128, Q.FMT_MXFP4, 4
    desc.codes, desc.scales = g.dw.data_ptr(), g.de.data_ptr()
    h = Q.ctypes.c_void_p()
    assert L.qgemv_create(Q.ctypes.byref(h), Q.ctypes.byref(desc), 8, None) == Q.QG_ERR_INVALID_ARG  # group 128
    desc.group_size, desc.bits = 32, 3
    assert L.qgemv_create(Q.ctypes.byref(h), Q.ctypes.byref(desc), 8, None) == Q.QG_ERR_INVALID_ARG  # 3 bits


@pytest.mark.parametrize("M", [1, 32])
def test_full_size_gate_shape(M):
    m = MX(17408, 5120, cfg=S.CFG_DECODE, tid=10)
    x_np = S.activations(M, m.K, cfg_id=218, tensor_id=M)
    y = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(218 + M).choice(m.N, 96, replace=False))
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("mxfp4 full", M, err)
    assert err <= TOL, err


@pytest.mark.parametrize("M,chunked", [(32, True), (33, False)])
def test_prefill_crossover(M, chunked):
    """Outside the measured shapes the crossover is the generic rule halved for
    MX elements: 32 rows on 4096x4096 (64 at group 128).  Up to it the rows run
    as the verify GEMM and leave the caller's workspace untouched; past it they
    are dequantised there.  Both match the oracle on sampled columns."""
    m = MX(4096, 4096, tid=9)
    x_np = S.activations(M, m.K, cfg_id=215, tensor_id=M)
    ws = torch.full((m.lin.prefill_workspace()[1],), 0x5A, dtype=torch.uint8, device="cuda")
    y = m.lin.run_prefill(dev_f16(x_np), workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws == 0x5A).all()) == chunked
    rows = np.random.default_rng(M).choice(m.N, 64, replace=False)
    assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows)) <= TOL
