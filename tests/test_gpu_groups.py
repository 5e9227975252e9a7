"""Scale groups of 64 and 32 (W4A16 g64 / g32 and the 2- and 3-bit codes
alike): the decode is bit-exact against the oracle (codes, exact w and q16,
and the verify GEMM's scaled operand 2 (c - o) s rounded once to fp16); the
products match the oracle within the normwise budget at every row count, on
both M = 1 kernels, both tile groupings and both hand-overs, several widths,
the fused MLP, the prefill route, the batch entry point and batch-invariant
rows; at the full 27B-class gate/up shape on sampled columns."""
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


def _mat(gs, bits, N=400, K=1536, cfg=190, tid=0, **kw):
    cb = None if bits else S.column_bits(N, 0.3, 4, cfg_id=cfg, tensor_id=S.T_MASK + tid)
    return Uniform(N, K, bits or 3, col_bits=cb, cfg_id=cfg, tid=tid, group_size=gs, **kw)


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("bits", [2, 3, 4, None])
def test_decode_bit_exact(gs, bits):
    m = _mat(gs, bits, tid=gs + (bits or 0))
    assert m.scales.shape == (m.N, m.K // gs)
    codes = m.codes()
    np.testing.assert_array_equal(m.lin.debug_unpack().cpu().numpy(), codes)
    w, q = m.lin.debug_dequant()
    wr = m.w()
    np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), wr)
    o = 0.5 * (2.0 ** (np.asarray(m.col_bits)[:, None] if bits is None else bits) - 1)
    np.testing.assert_array_equal(q.cpu().numpy().astype(np.float64), codes - o)
    # the verify GEMM's operand: 2 (c - o) s rounded once to fp16 (RNE), w its half
    c, b, wo = m.lin.debug_operand()
    np.testing.assert_array_equal(c.cpu().numpy(), codes)
    want = (2.0 * wr).astype(np.float16)
    np.testing.assert_array_equal(b.cpu().numpy().view(np.uint16), want.view(np.uint16))
    np.testing.assert_array_equal(wo.cpu().numpy(), want.astype(np.float32) * np.float32(0.5))


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("bits", [2, 3, 4, None])
@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
def test_m1_gemv(gs, bits, kernel):
    pins = Q.PIN_M1_PERGROUP if kernel == "pergroup" else Q.PIN_M1_RUNS
    m = _mat(gs, bits, K=2560, tid=3, pins=pins)
    x_np = S.activations(1, m.K, cfg_id=191, tensor_id=gs)
    y = m.lin.run(dev_f16(x_np))
    y2 = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("m1", gs, bits, kernel, err)
    assert err <= TOL, err


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("M", [2, 8, 17, 32])
@pytest.mark.parametrize("pins", [0, Q.PIN_XS_T1 | Q.PIN_PARTIALS, Q.PIN_XS_T2 | Q.PIN_WORDS])
def test_verify_gemm(gs, M, pins):
    m = _mat(gs, 4, N=528, K=5120, tid=5, pins=pins)
    x_np = S.activations(M, m.K, cfg_id=192, tensor_id=M)
    y = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("verify", gs, M, pins, err)
    assert err <= TOL, err


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("bits", [2, 3, None])
def test_verify_gemm_widths(gs, bits):
    m = _mat(gs, bits, N=400, K=1536, tid=6)
    x_np = S.activations(24, m.K, cfg_id=193, tensor_id=gs)
    y = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np)) <= TOL


@pytest.mark.parametrize("gs", [64, 32])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_mlp(gs, M):
    H, I = 1024, 2560
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=194, tensor_id=S.T_MASK)
    cb_dn = S.column_bits(H, 0.2, 2, cfg_id=194, tensor_id=S.T_MASK + 100)
    wg = S.mixed_code_words(cb_gu, H, cfg_id=194, tensor_id=S.T_CODES)
    wu = S.mixed_code_words(cb_gu, H, cfg_id=194, tensor_id=S.T_CODES + 10)
    wd = S.mixed_code_words(cb_dn, I, cfg_id=194, tensor_id=S.T_CODES + 20)
    sg = S.scales(I, H, cfg_id=194, tensor_id=S.T_SCALE, group=gs)
    su = S.scales(I, H, cfg_id=194, tensor_id=S.T_SCALE + 10, group=gs)
    sd = S.scales(H, I, cfg_id=194, tensor_id=S.T_SCALE + 20, group=gs)
    mk = lambda w, s, k, n, cb: Q.QLinear(dev_words(w), dev_f16(s), k, n, col_bits=cb, max_M=32, group_size=gs)
    g, u, d = mk(wg, sg, H, I, cb_gu), mk(wu, su, H, I, cb_gu), mk(wd, sd, I, H, cb_dn)
    x_np = S.activations(M, H, cfg_id=195, tensor_id=M)
    out = Q.mlp(g, u, d, dev_f16(x_np))
    torch.cuda.synchronize()
    h = O.silu(O.gemv_mixed(x_np, wg, sg, cb_gu, H)) * O.gemv_mixed(x_np, wu, su, cb_gu, H)
    err = O.normwise_rel_err(out.cpu().numpy().astype(np.float64), O.gemv_mixed(h, wd, sd, cb_dn, I))
    say("mlp", gs, M, err)
    assert err <= TOL, err


@pytest.mark.parametrize("gs", [64, 32])
def test_prefill(gs):
    m = _mat(gs, 4, N=400, K=1536, tid=7)
    x_np = S.activations(96, m.K, cfg_id=196)
    ws = torch.zeros(m.lin.prefill_workspace()[1], dtype=torch.uint8, device="cuda")
    y = m.lin.run_prefill(dev_f16(x_np), workspace=ws)
    torch.cuda.synchronize()
    got = ws[32 << 20:(32 << 20) + m.N * m.K * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(m.N, m.K)
    np.testing.assert_array_equal(got, m.w().astype(np.float16).view(np.uint16))
    assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np)) <= TOL


def test_batch_mixes_group_sizes():
    mats = [_mat(128, 3, N=256, K=1536, tid=8), _mat(64, 4, N=400, K=1536, tid=9), _mat(32, 2, N=128, K=2560, tid=10)]
    xs_np = [S.activations(1, m.K, cfg_id=197, tensor_id=i) for i, m in enumerate(mats)]
    ys = Q.run_batch([m.lin for m in mats], [dev_f16(x) for x in xs_np])
    torch.cuda.synchronize()
    for m, y, x in zip(mats, ys, xs_np):
        assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x)) <= TOL


def test_batch_invariant_rows():
    m = _mat(32, 4, N=272, K=5120, tid=11, batch_invariant=True)
    x = dev_f16(S.activations(32, m.K, cfg_id=198))
    alone = torch.cat([m.lin.run(x[i:i + 1]) for i in range(32)])
    for M in (1, 5, 16, 17, 32):
        assert torch.equal(m.lin.run(x[:M]).view(torch.int16), alone[:M].view(torch.int16)), M


def test_bad_group_sizes():
    m = _mat(32, 3, N=64, K=256, tid=12)
    for gs in (16, 96, 256):
        with pytest.raises(Q.QGError):
            Q.QLinear(m.dw, m.ds, 256, 64, bits=3, max_M=8, group_size=gs)
    cbk = dev_f16(S.codebook(cfg_id=S.CFG_TRELLIS))
    tw = S.trellis_words(64, 256, cfg_id=199)
    dtw = torch.from_numpy(np.ascontiguousarray(tw).view(np.int16).copy()).cuda()
    with pytest.raises(Q.QGError):
        Q.QLinear(dtw, dev_f16(S.scales(64, 256, cfg_id=199, group=64)), 256, 64, trellis=True, codebook=cbk,
                  max_M=8, group_size=64)


@pytest.mark.parametrize("M", [1, 8, 32])
def test_full_size_w4_g32(M):
    """W4A16 at group 32 on the gate/up shape (5120 -> 17408), sampled columns."""
    m = _mat(32, 4, N=17408, K=5120, cfg=S.CFG_DECODE, tid=13)
    x_np = S.activations(M, m.K, cfg_id=200, tensor_id=M)
    y = m.lin.run(dev_f16(x_np))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(200 + M).choice(m.N, 96, replace=False))
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("w4 g32 full", M, err)
    assert err <= TOL, err


@pytest.mark.parametrize("M,chunked", [(32, True), (33, False)])
def test_prefill_crossover(M, chunked):
    """Outside the measured shapes the crossover is the generic rule times 3/4
    for groups of 64 or 32: 32 rows on 4096x4096 (64 at group 128).  Up to it
    the rows run as the verify GEMM and leave the caller's workspace
    untouched; past it they are dequantised there.  Both match the oracle."""
    m = _mat(32, 4, N=4096, K=4096, tid=11)
    x_np = S.activations(M, m.K, cfg_id=197, tensor_id=M)
    ws = torch.full((m.lin.prefill_workspace()[1],), 0x5A, dtype=torch.uint8, device="cuda")
    y = m.lin.run_prefill(dev_f16(x_np), workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws == 0x5A).all()) == chunked
    rows = np.random.default_rng(M).choice(m.N, 64, replace=False)
    assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows)) <= TOL
