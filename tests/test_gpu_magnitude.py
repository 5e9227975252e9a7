"""Scale invariance: GPU parity when the activations are far from unit size.

The M = 1 GEMVs stage x in fp16 with a power-of-two block exponent per 32
values (so small activations keep all their bits), and the fused MLP keeps its
intermediate h in fp32 (rounded once with a block exponent for the matrix
cores).  Each case is checked at the normwise 2e-3 budget against the fp64
oracle, on both M = 1 kernels, 2-, 3- and 4-bit codes, several widths, the
verify GEMM and the fused MLP, with x = fp16(N(0,1) * 2^p) for p = -13, -10
and +6 (|x| up to about 2^8), and with outliers mixed into small activations.
Where the true outputs themselves fall below fp16's normal range (the MLP at
2^-13, whose outputs scale with x^2 and land among fp16's few subnormals),
each output may also be one fp16 spacing off: an fp16 result cannot be closer
than that."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, say  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402

M1_PIN = {"pergroup": Q.PIN_M1_PERGROUP, "runs": Q.PIN_M1_RUNS}


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def scaled_x(M, K, p, cfg, tid, outliers=False):
    """fp16(N(0,1) * 2^p); with outliers, every 97th value is +-2^8 instead."""
    x = S.activations(M, K, cfg_id=cfg, tensor_id=tid).astype(np.float64) * 2.0 ** p
    if outliers:
        x[:, ::97] = np.where(np.arange(x[:, ::97].size).reshape(x[:, ::97].shape) % 2, 256.0, -256.0)
    return x.astype(np.float16)


def fp16_ulp(r):
    """Spacing of fp16 values at |r| (2^-24 in the subnormal range)."""
    a = np.abs(np.asarray(r, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


def _run(lin, x):
    y = lin.run(dev_f16(x))
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("p", [-13, -10, 6])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
def test_m1_gemv_scale_invariant(kernel, bits, p):
    N, K = 272, 2560
    say("m1 magnitude", kernel, bits, p)
    u = Uniform(N, K, bits, cfg_id=120, pins=M1_PIN[kernel])
    x = scaled_x(1, K, p, 120, 10 + bits)
    r = u.ref(x)
    err = O.normwise_rel_err(_run(u.lin, x), r)
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("p", [-13, -10, 6])
@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
def test_m1_gemv_scale_invariant_mixed_widths_and_k_slices(kernel, p):
    N, K = 464, 9216
    cb = S.column_bits(N, 0.2, 4, cfg_id=121)
    cb[3::13] = 2
    say("m1 magnitude mixed", kernel, p)
    u = Uniform(N, K, col_bits=cb, cfg_id=121, pins=M1_PIN[kernel], launch={0: (0, 0, 3)} if kernel == "pergroup" else None)
    x = scaled_x(1, K, p, 121, 20)
    err = O.normwise_rel_err(_run(u.lin, x), u.ref(x))
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_m1_gemv_outliers_among_small_values(kernel, bits):
    N, K = 272, 2560
    u = Uniform(N, K, bits, cfg_id=122, pins=M1_PIN[kernel])
    x = scaled_x(1, K, -10, 122, 30, outliers=True)
    err = O.normwise_rel_err(_run(u.lin, x), u.ref(x))
    say("outliers err", kernel, bits, err)
    assert err <= TOL, err


@pytest.mark.parametrize("p", [-13, 6])
@pytest.mark.parametrize("M", [8, 32])
def test_verify_gemm_scale_invariant(M, p):
    N, K = 400, 2560
    u = Uniform(N, K, 3, cfg_id=123)
    x = scaled_x(M, K, p, 123, 40 + M)
    err = O.normwise_rel_err(_run(u.lin, x), u.ref(x))
    say("verify magnitude", M, p, err)
    assert err <= TOL, err


@pytest.mark.parametrize("p", [-13, -10, 3])
@pytest.mark.parametrize("M", [1, 8, 32])
@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
def test_mlp_scale_invariant(kernel, M, p):
    """The fused MLP: gate/up, h = SiLU(g) * u in fp32, down."""
    H, I = 640, 1408
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=124, tensor_id=S.T_MASK)
    cb_dn = S.column_bits(H, 0.2, 2, cfg_id=124, tensor_id=S.T_MASK + 100)
    pins = M1_PIN[kernel]
    g = Uniform(I, H, col_bits=cb_gu, cfg_id=124, tid=0, pins=pins)
    u = Uniform(I, H, col_bits=cb_gu, cfg_id=124, tid=1, pins=pins)
    d = Uniform(H, I, col_bits=cb_dn, cfg_id=124, tid=2, pins=pins)
    x = scaled_x(M, H, p, 124, 50 + M)
    out = Q.mlp(g.lin, u.lin, d.lin, dev_f16(x))
    torch.cuda.synchronize()
    r = O.mlp(x, g.w(), u.w(), d.w())
    assert np.abs(r).max() < 30000.0
    y = out.cpu().numpy().astype(np.float64)
    err = O.normwise_rel_err(y, r)
    slack = np.abs(y - r) - fp16_ulp(r)
    say("mlp magnitude", kernel, M, p, "err", err, "beyond one fp16 spacing", slack.max() / np.abs(r).max())
    assert np.all(slack <= TOL * np.abs(r).max()), (err, slack.max())
