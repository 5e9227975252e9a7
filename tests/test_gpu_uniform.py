"""GPU parity of the uniform / per-column-width path against the CPU oracle,
through the C ABI: bit-exact unpacked codes and dequantised weights, matmul
outputs within the normwise 2e-3 budget, bit-identical repeats."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, run_np, say, sha  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_tiny_reference_config():
    """K = N = 512, M = 1, 3-bit codes uniform in 0..7, seed 0."""
    say("tiny reference config")
    N = K = 512
    words = S.uniform_code_words(N, K, 3, seed=0, cfg_id=S.CFG_TINY)
    sc = S.scales(N, K, seed=0, cfg_id=S.CFG_TINY)
    x = S.activations(1, K, seed=0, cfg_id=S.CFG_TINY)
    from _gpu import dev_words
    lin = Q.QLinear(dev_words(words), dev_f16(sc), K, N, bits=3, max_M=1)
    y = run_np(lin, x)
    r = O.gemv_uniform(x, words, sc, N, K, 3)
    err = O.normwise_rel_err(y, r)
    say("tiny err", err)
    assert err <= TOL
    codes = lin.debug_unpack().cpu().numpy()
    np.testing.assert_array_equal(codes, O.unpack_uniform(words, N, K, 3))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 1280)])
def test_debug_unpack_and_dequant_bit_exact(bits, N, K):
    say("debug exact", bits, N, K)
    u = Uniform(N, K, bits, cfg_id=51)
    codes = u.lin.debug_unpack().cpu().numpy()
    np.testing.assert_array_equal(codes, u.codes())
    w, q = u.lin.debug_dequant()
    w = w.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(w, u.w())                     # exact in fp32
    qo = (u.codes() - O.code_offset(bits)).astype(np.float16)   # c - o is exact in fp16
    np.testing.assert_array_equal(q.cpu().numpy(), qo)


def test_debug_exact_mixed_widths():
    N, K = 160, 512
    cb = S.column_bits(N, 0.3, 4, cfg_id=52)
    cb[::7] = 2
    say("debug exact mixed", np.bincount(cb))
    u = Uniform(N, K, col_bits=cb, cfg_id=52)
    np.testing.assert_array_equal(u.lin.debug_unpack().cpu().numpy(), u.codes())
    w, q = u.lin.debug_dequant()
    np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), u.w())


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 1280)])
def test_debug_operand_bit_exact(bits, N, K):
    """The verify GEMM's decode into the matrix-core operand (decode_off1 and
    its offset constant, the functions the verify kernel runs): codes read back
    out of the operand registers, the operand's fp16 bits (c * 2^-23 = the
    integer 2c) and the dequantised weight rebuilt from them, all bit-exact."""
    say("operand exact", bits, N, K)
    u = Uniform(N, K, bits, cfg_id=51)
    c, b, w = u.lin.debug_operand()
    np.testing.assert_array_equal(c.cpu().numpy(), u.codes())
    np.testing.assert_array_equal(b.cpu().numpy().view(np.uint16), (2 * u.codes()).astype(np.uint16))
    np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), u.w())


def test_debug_operand_mixed_widths():
    N, K = 160, 512
    cb = S.column_bits(N, 0.3, 4, cfg_id=52)
    cb[::7] = 2
    u = Uniform(N, K, col_bits=cb, cfg_id=52)
    c, b, w = u.lin.debug_operand()
    np.testing.assert_array_equal(c.cpu().numpy(), u.codes())
    np.testing.assert_array_equal(b.cpu().numpy().view(np.uint16), (2 * u.codes()).astype(np.uint16))
    np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), u.w())


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("M", [1, 2, 5, 8, 16, 17, 32])
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (272, 1280)])
def test_matmul_parity(bits, M, N, K):
    say("parity", bits, M, N, K)
    u = Uniform(N, K, bits, cfg_id=53)
    x = S.activations(M, K, cfg_id=53, tensor_id=100 + M)
    y = run_np(u.lin, x)
    err = O.normwise_rel_err(y, u.ref(x))
    assert err <= TOL, err


@pytest.mark.parametrize("M", [1, 3, 8, 32])
def test_mixed_width_parity(M):
    N, K = 336, 768
    cb = S.column_bits(N, 0.2, 4, cfg_id=54)
    cb[5::11] = 2
    say("mixed parity", M)
    u = Uniform(N, K, col_bits=cb, cfg_id=54)
    x = S.activations(M, K, cfg_id=54, tensor_id=100 + M)
    assert O.normwise_rel_err(run_np(u.lin, x), u.ref(x)) <= TOL


@pytest.mark.parametrize("M,tiles,waves,splits", [
    (1, 1, 4, 1), (1, 2, 2, 1), (1, 1, 1, 3), (1, 2, 4, 5), (1, 1, 4, 10), (1, 1, 2, 16), (1, 1, 8, 1), (1, 2, 8, 2),
    (8, 1, 4, 1), (8, 2, 2, 2), (8, 4, 4, 3), (8, 1, 1, 7), (8, 2, 4, 10), (8, 1, 8, 1),
    (32, 1, 4, 1), (32, 2, 2, 4), (32, 4, 4, 2), (32, 4, 1, 1), (32, 2, 4, 9), (32, 2, 8, 1),
])
def test_launch_shapes(M, tiles, waves, splits):
    """Every launch geometry gives oracle-matching, repeatable results (ragged
    tile sets, uneven K slices, slices with fewer groups than waves)."""
    N, K = 400, 1280
    say("launch", M, tiles, waves, splits)
    cls = 0 if M == 1 else (1 if M <= 16 else 2)
    u = Uniform(N, K, 3, cfg_id=55, launch={cls: (tiles, waves, splits)})
    x = S.activations(M, K, cfg_id=55, tensor_id=100 + M)
    xd = dev_f16(x)
    y1 = u.lin.run(xd)
    y2 = u.lin.run(xd)
    torch.cuda.synchronize()
    assert sha(y1) == sha(y2)
    assert O.normwise_rel_err(y1.cpu().numpy().astype(np.float64), u.ref(x)) <= TOL


@pytest.mark.parametrize("M", [1, 8, 32])
def test_repeat_bit_identical(M):
    N, K = 1024, 5120
    say("repeat", M)
    u = Uniform(N, K, 3, cfg_id=56)
    x = dev_f16(S.activations(M, K, cfg_id=56))
    hs = {sha(u.lin.run(x)) for _ in range(10)}
    assert len(hs) == 1
    # a second handle over the same bytes gives the same bits
    v = Q.QLinear(u.dw, u.ds, K, N, bits=3, max_M=32)
    assert sha(v.run(x)) in hs


def test_error_paths_on_device():
    u = Uniform(64, 256, 3, cfg_id=57, max_M=8)
    x = dev_f16(S.activations(9, 256, cfg_id=57))
    with pytest.raises(Q.QGError) as e:
        u.lin.run(x)                                  # M = 9 > max_M
    assert e.value.status == Q.QG_ERR_INVALID_ARG
    xb = torch.zeros(2 * 256 + 1, dtype=torch.float16, device="cuda")[1:].view(2, 256)
    with pytest.raises(Q.QGError):
        u.lin.run(xb)                                 # misaligned x
    with pytest.raises(Q.QGError):
        u.relinked(launch={0: (1, 17, 1)})           # M = 1: at most 16 waves
    with pytest.raises(Q.QGError):
        u.relinked(launch={1: (9, 0, 1)})            # M > 1: at most 8 tile groups


@pytest.mark.parametrize("max_M", [1, 2, 5, 17])
def test_every_row_count_up_to_max_M(max_M):
    """A handle sized for max_M rows runs every M <= max_M: the workspace sized
    at create covers whichever kernel, K slices and hand-over each row count
    takes (per-group GEMV in fixed-point K slices at M = 1, x-in-LDS GEMM with
    partials or words above), repeats are bit-identical, sampled rows match."""
    N, K = 4096, 9216
    say("row counts up to", max_M)
    u = Uniform(N, K, 3, cfg_id=58, max_M=max_M)
    rows = np.random.default_rng(max_M).choice(N, 48, replace=False)
    for M in range(1, max_M + 1):
        x = S.activations(M, K, cfg_id=58, tensor_id=700 + M)
        xd = dev_f16(x)
        y1 = u.lin.run(xd)
        y2 = u.lin.run(xd)
        torch.cuda.synchronize()
        assert sha(y1) == sha(y2)
        r = O.gemv_uniform_rows(x, u.words, u.scales, N, K, 3, rows)
        err = O.normwise_rel_err(y1.cpu().numpy().astype(np.float64)[:, rows], r)
        assert err <= TOL, (M, err)
