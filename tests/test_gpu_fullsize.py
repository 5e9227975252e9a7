"""Parity at the full decode / verify / MLP sizes, in the launch configuration
the benchmark times (the library's own choice), on sampled output columns that
the oracle computes one by one: every tile edge class (first, last, a seeded
random sample), all rows M."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, dev_f16, dev_words, say  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sample(N, n=80, seed=0):
    rng = np.random.default_rng([seed, N])
    pick = rng.choice(N, size=n, replace=False)
    return np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), pick]))


# one matrix of each distinct layer-set shape, generated exactly as the benchmark does
_SHAPES = {"qo": 0, "kv": 1, "gateup": 4, "down": 6}


@pytest.fixture(scope="module")
def decode_handles():
    out = {}
    for name, i in _SHAPES.items():
        sh = S.LAYER_SET[i]
        N, K = sh["N"], sh["K"]
        w = S.uniform_code_words(N, K, 3, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 10 * i)
        sc = S.scales(N, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 10 * i)
        lin = Q.QLinear(dev_words(w), dev_f16(sc), K, N, bits=3, max_M=32)
        out[name] = (lin, w, sc, N, K)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M", [1, 8, 16, 32])
@pytest.mark.parametrize("name", list(_SHAPES))
def test_decode_and_verify_full_size(decode_handles, name, M):
    lin, w, sc, N, K = decode_handles[name]
    say("full size", name, N, K, "M", M)
    x = S.activations(M, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + M)
    y = lin.run(dev_f16(x))
    torch.cuda.synchronize()
    rows = _sample(N)
    r = O.gemv_uniform_rows(x, w, sc, N, K, 3, rows)
    yy = y.cpu().numpy().astype(np.float64)[:, rows]
    err = O.normwise_rel_err(yy, r)
    say("err", err)
    assert err <= TOL, err
    assert np.all(np.isfinite(y.cpu().numpy()))


@pytest.mark.parametrize("M", [1, 32])
def test_mlp_full_size_mixed(M):
    H, I = S.MLP["hidden"], S.MLP["inter"]
    say("mlp full size", M)
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK)
    cb_dn = S.column_bits(H, 0.2, 2, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK + 100)
    wg = S.mixed_code_words(cb_gu, H, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES)
    wu = S.mixed_code_words(cb_gu, H, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES + 10)
    wd = S.mixed_code_words(cb_dn, I, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES + 20)
    sg = S.scales(I, H, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE)
    su = S.scales(I, H, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE + 10)
    sd = S.scales(H, I, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE + 20)
    assert wg.nbytes + wu.nbytes + wd.nbytes + sg.nbytes + su.nbytes + sd.nbytes == 106_676_736
    g = Q.QLinear(dev_words(wg), dev_f16(sg), H, I, col_bits=cb_gu, max_M=32)
    u = Q.QLinear(dev_words(wu), dev_f16(su), H, I, col_bits=cb_gu, max_M=32)
    d = Q.QLinear(dev_words(wd), dev_f16(sd), I, H, col_bits=cb_dn, max_M=32)
    x = S.activations(M, H, cfg_id=S.CFG_MLP, tensor_id=S.T_X + M)
    out = Q.mlp(g, u, d, dev_f16(x))
    torch.cuda.synchronize()
    # the oracle needs every intermediate value for any output column: h in blocks
    h = np.empty((M, I))
    for b in range(0, I, 2048):
        rr = np.arange(b, min(I, b + 2048))
        gg = O.gemv_mixed(x, wg, sg, cb_gu, H, rr)
        uu = O.gemv_mixed(x, wu, su, cb_gu, H, rr)
        h[:, rr] = O.silu(gg) * uu
    rows = _sample(H)
    r = O.gemv_mixed(h, wd, sd, cb_dn, I, rows)
    err = O.normwise_rel_err(out.cpu().numpy().astype(np.float64)[:, rows], r)
    say("mlp full err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("M", [1, 8, 32])
@pytest.mark.parametrize("name,N", [("qkv", 7168), ("gateup", 34816)])
def test_stacked_sibling_shapes(name, N, M):
    """The sibling projections stacked into one matrix (q|k|v: 7168 x 5120,
    gate|up: 34816 x 5120), each with its own tuned launch, on sampled
    columns."""
    K = 5120
    say("stacked", name, N, "M", M)
    w = S.uniform_code_words(N, K, 3, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 900)
    sc = S.scales(N, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 900)
    lin = Q.QLinear(dev_words(w), dev_f16(sc), K, N, bits=3, max_M=32)
    x = S.activations(M, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + 50 + M)
    xd = dev_f16(x)
    y = lin.run(xd)
    y2 = lin.run(xd)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows = _sample(N, n=96, seed=5)
    r = O.gemv_uniform_rows(x, w, sc, N, K, 3, rows)
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], r)
    say("err", err)
    assert err <= TOL, err
    lin.close()
