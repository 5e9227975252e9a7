"""GPU parity of the bitshift-trellis path (3 bits/weight, 65536-entry fp16
codebook, Walsh-Hadamard-rotated activations) against the CPU oracle, through
the C ABI: bit-exact states and dequantised weights from the checking entry
points, outputs within the normwise 2e-3 budget at M = 1 (vector-ALU GEMV)
and M = 2..32 (the banded matrix-core GEMM), pre-rotated
input, bit-identical repeats and sampled columns of the 27B-class shapes."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, dev_f16, dev_u16, say, sha  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def codebook():
    cb = S.codebook(cfg_id=S.CFG_TRELLIS)
    return cb, dev_f16(cb)


class Trellis:
    def __init__(self, N, K, cb, cfg_id=80, max_M=32, prerotated=False, pins=0):
        self.N, self.K = N, K
        self.words = S.trellis_words(N, K, cfg_id=cfg_id)
        self.scales = S.scales(N, K, cfg_id=cfg_id)
        self.cb = cb[0]
        self.dw = dev_u16(self.words)
        self.ds = dev_f16(self.scales)
        self.lin = Q.QLinear(self.dw, self.ds, K, N, trellis=True, codebook=cb[1], max_M=max_M,
                             prerotated=prerotated, pins=pins)

    def ref(self, x, prerotated=False):
        return O.gemv_trellis(x, self.words, self.cb, self.scales, self.N, self.K, prerotated=prerotated)


def _run(lin, x):
    y = lin.run(dev_f16(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (160, 1280)])
def test_states_and_dequant_bit_exact(N, K, codebook):
    say("trellis exact", N, K)
    t = Trellis(N, K, codebook)
    st = t.lin.debug_trellis().cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(st, O.trellis_states(t.words, N, K))
    w, _ = t.lin.debug_dequant(with_q16=False)
    ref = O.trellis_dequant(O.trellis_states(t.words, N, K), t.cb, t.scales)
    np.testing.assert_array_equal(w.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M", [1, 2, 8, 16, 17, 32])
@pytest.mark.parametrize("N,K", [(16, 128), (96, 640), (272, 1536), (512, 512)])
def test_product_parity(M, N, K, codebook):
    say("trellis product", M, N, K)
    t = Trellis(N, K, codebook, cfg_id=81)
    x = S.activations(M, K, cfg_id=81, tensor_id=200 + M)
    y = _run(t.lin, x)
    err = O.normwise_rel_err(y, t.ref(x))
    say("trellis err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("M", [1, 8])
def test_prerotated_input(M, codebook):
    say("trellis prerotated", M)
    N, K = 128, 1024
    t = Trellis(N, K, codebook, cfg_id=82, prerotated=True)
    xr = O.rotate(S.activations(M, K, cfg_id=82)).astype(np.float16)
    y = _run(t.lin, xr)
    err = O.normwise_rel_err(y, t.ref(xr, prerotated=True))
    say("prerotated err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("M", [1, 8, 32])
def test_repeat_bit_identical(M, codebook):
    say("trellis repeat", M)
    t = Trellis(320, 2560, codebook, cfg_id=83)
    x = dev_f16(S.activations(M, 2560, cfg_id=83))
    h0 = sha(t.lin.run(x))
    for _ in range(10):
        assert sha(t.lin.run(x)) == h0


@pytest.mark.parametrize("K,N", [(5120, 5120), (5120, 1024), (5120, 17408), (17408, 5120)])
@pytest.mark.parametrize("M", [1, 8])
def test_full_size_sampled_columns(K, N, M, codebook):
    say("trellis full size", K, N, M)
    t = Trellis(N, K, codebook, cfg_id=S.CFG_TRELLIS, max_M=8)
    x = S.activations(M, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_X + M)
    y = _run(t.lin, x)
    # whole 16-row tile rows: the first, the last and six random ones
    blocks = np.unique(np.concatenate([[0, N // 16 - 1], np.random.default_rng(7).choice(N // 16, 6, replace=False)]))
    rows = (16 * blocks[:, None] + np.arange(16)[None, :]).reshape(-1)
    r = O.gemv_trellis_rows(x, t.words, t.cb, t.scales, N, K, rows)
    err = O.normwise_rel_err(y[:, rows], r)
    say("full size err", err)
    assert err <= TOL, err
    assert np.isfinite(y).all()


@pytest.mark.parametrize("handover", ["words", "partials"])
@pytest.mark.parametrize("M", [2, 8, 17, 32])
@pytest.mark.parametrize("N,K", [(48, 384), (400, 2560)])
def test_banded_gemm_handovers(handover, M, N, K, codebook):
    """The banded GEMM (x fragments shared through LDS) with its K slices
    meeting in fixed-point words (the default where they fit) or, pinned, in
    partials with a count."""
    say("trellis gemm", handover, M, N, K)
    t = Trellis(N, K, codebook, cfg_id=86, pins=Q.PIN_PARTIALS if handover == "partials" else 0)
    x = S.activations(M, K, cfg_id=86, tensor_id=500 + M)
    y1 = _run(t.lin, x)
    y2 = _run(t.lin, x)
    assert np.array_equal(y1, y2)
    err = O.normwise_rel_err(y1, t.ref(x))
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("handover", ["words", "partials"])
@pytest.mark.parametrize("N,K", [(16, 2048), (48, 2048), (400, 2560), (5120, 2048), (4112, 4096), (112, 17408)])
def test_gemv_handovers_both(handover, N, K, codebook):
    """The M = 1 trellis GEMV with both row-block hand-overs, forced: the
    fixed-point words (one atomic per output and wave) and the partials with an
    arrival count.  The shapes give one to 16 waves per row block, one to three
    units per wave, ranges that start and end inside row blocks, and (112 x
    17408: 136 waves meet in one row block, more than the words count) the
    partials either way.  The two largest are checked on sampled row blocks."""
    say("trellis gemv", handover, N, K)
    t = Trellis(N, K, codebook, cfg_id=87, pins=Q.PIN_PARTIALS if handover == "partials" else 0)
    x = S.activations(1, K, cfg_id=87, tensor_id=600)
    y1 = _run(t.lin, x)
    y2 = _run(t.lin, x)
    assert np.array_equal(y1, y2)
    if N * K <= (1 << 22):
        err = O.normwise_rel_err(y1, t.ref(x))
    else:
        blocks = np.unique(np.concatenate([[0, N // 16 - 1], np.random.default_rng(8).choice(N // 16, 6, replace=False)]))
        rows = (16 * blocks[:, None] + np.arange(16)[None, :]).reshape(-1)
        err = O.normwise_rel_err(y1[:, rows], O.gemv_trellis_rows(x, t.words, t.cb, t.scales, N, K, rows))
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("N,K", [(48, 384), (400, 2560), (1040, 5120), (96, 16384)])
def test_gemv_rotation_in_kernel(N, K, codebook):
    """The M = 1 GEMV that rotates x itself into LDS gives the same bits as the
    separate rotation launch followed by the GEMV (both compute the same fp16
    rotated values), and matches the oracle."""
    t = Trellis(N, K, codebook, cfg_id=88)
    tl = Trellis(N, K, codebook, cfg_id=88, pins=Q.PIN_TRELLIS_ROT_LAUNCH)
    x = S.activations(1, K, cfg_id=88, tensor_id=700)
    say("trellis rotation", N, K)
    y_launch = _run(tl.lin, x)
    y_kernel = _run(t.lin, x)
    assert np.array_equal(y_launch, y_kernel)
    if N * K <= (1 << 22):
        err = O.normwise_rel_err(y_kernel, t.ref(x))
        say("err", err)
        assert err <= TOL, err


@pytest.mark.parametrize("handover", ["words", "partials"])
@pytest.mark.parametrize("M", [2, 3, 5, 8])
@pytest.mark.parametrize("N,K", [(48, 128), (48, 384), (400, 2560), (24576, 1280), (5120, 17408)])
def test_staged_slice_kernel_matches_band(handover, M, N, K, codebook):
    """2..8 rows: the kernel that stages its K slice's x once (no per-group
    barrier) gives the same bits as the band kernel (pinned), which stages x
    group by group, on the same rotated x: both sum the same MFMA products in
    group order.  With x as given, it rotates x in LDS and matches the oracle.
    Shapes: one group (a single K slice, direct stores), one group per slice,
    5 groups per slice (two K slices) and 11 or 12 (12 slices, x slices of up
    to 96 pieces at 8 rows); the largest checked on sampled row blocks."""
    hp = Q.PIN_PARTIALS if handover == "partials" else 0
    x = S.activations(M, K, cfg_id=89, tensor_id=800 + M)
    xr = O.rotate(x).astype(np.float16)
    say("trellis staged slice", handover, M, N, K)
    tp = Trellis(N, K, codebook, cfg_id=89, max_M=8, prerotated=True, pins=hp)
    tbp = Trellis(N, K, codebook, cfg_id=89, max_M=8, prerotated=True, pins=hp | Q.PIN_TRELLIS_BAND)
    assert np.array_equal(_run(tp.lin, xr), _run(tbp.lin, xr))
    del tp, tbp
    t = Trellis(N, K, codebook, cfg_id=89, max_M=8, pins=hp)
    y = _run(t.lin, x)
    if N * K <= (1 << 22):
        err = O.normwise_rel_err(y, t.ref(x))
    else:
        blocks = np.unique(np.concatenate([[0, N // 16 - 1], np.random.default_rng(9).choice(N // 16, 4, replace=False)]))
        rows = (16 * blocks[:, None] + np.arange(16)[None, :]).reshape(-1)
        err = O.normwise_rel_err(y[:, rows], O.gemv_trellis_rows(x, t.words, t.cb, t.scales, N, K, rows))
    say("err", err)
    assert err <= TOL, err
