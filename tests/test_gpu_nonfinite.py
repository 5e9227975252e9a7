"""Non-finite activations reach the outputs on every hand-over path: a NaN in a
row of x makes that row's outputs NaN (and leaves the other rows finite), an
infinity makes them non-finite -- through the fixed-point words (which count
non-finite contributions), the fp32 partials, the exchange words of the fused
pass and the direct stores."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import qg_synth as S  # noqa: E402
from _gpu import Uniform, dev_f16, dev_u16, say  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cls(M):
    return 0 if M == 1 else (1 if M <= 16 else 2)


# (pins, launch override of the M's class) per hand-over path
PATHS = {
    "m1-pergroup-one-slice": (Q.PIN_M1_PERGROUP, (0, 0, 1)),
    "m1-pergroup-words": (Q.PIN_M1_PERGROUP, (0, 0, 3)),
    "m1-pergroup-partials": (Q.PIN_M1_PERGROUP | Q.PIN_PARTIALS, (0, 0, 3)),
    "m1-runs-words": (Q.PIN_M1_RUNS, (4, 0, 0)),
    "m1-runs-one-wave": (Q.PIN_M1_RUNS, (1, 0, 0)),
    "xs-one-slice": (0, (0, 0, 1)),
    "xs-words": (Q.PIN_WORDS, (0, 0, 3)),
    "xs-partials": (Q.PIN_PARTIALS, (0, 0, 3)),
}


@pytest.mark.parametrize("value", ["nan", "inf"])
@pytest.mark.parametrize("path", list(PATHS))
def test_uniform_paths(path, value):
    M = 1 if path.startswith("m1") else 8
    pins, launch = PATHS[path]
    N, K = 272, 2560
    u = Uniform(N, K, 3, cfg_id=130, pins=pins, launch={_cls(M): launch})
    x = S.activations(M, K, cfg_id=130)
    x[0, 777] = np.float16(value)
    say("nonfinite", path, value)
    y = u.lin.run(dev_f16(x)).float().cpu().numpy()
    if value == "nan":
        assert np.isnan(y[0]).all()
    else:
        assert not np.isfinite(y[0]).any()
    assert np.isfinite(y[1:]).all()


@pytest.mark.parametrize("M", [1, 8])
def test_fused_mlp(M):
    H, I = 512, 1408
    g = Uniform(I, H, 3, cfg_id=131, tid=0)
    up = Uniform(I, H, 3, cfg_id=131, tid=1)
    d = Uniform(H, I, 3, cfg_id=131, tid=2)
    x = S.activations(M, H, cfg_id=131)
    x[0, 5] = np.float16("nan")
    out = Q.mlp(g.lin, up.lin, d.lin, dev_f16(x)).float().cpu().numpy()
    assert np.isnan(out[0]).all()
    assert np.isfinite(out[1:]).all()


@pytest.mark.parametrize("partials", [False, True])
@pytest.mark.parametrize("M", [1, 8])
def test_trellis(M, partials):
    N, K = 400, 2560
    cb = dev_f16(S.codebook(cfg_id=S.CFG_TRELLIS))
    lin = Q.QLinear(dev_u16(S.trellis_words(N, K, cfg_id=132)), dev_f16(S.scales(N, K, cfg_id=132)), K, N,
                    trellis=True, codebook=cb, max_M=8, pins=Q.PIN_PARTIALS if partials else 0)
    x = S.activations(M, K, cfg_id=132)
    x[0, 300] = np.float16("nan")
    y = lin.run(dev_f16(x)).float().cpu().numpy()
    assert np.isnan(y[0]).all()      # the rotation spreads the NaN over its whole 128-group
    assert np.isfinite(y[1:]).all()
