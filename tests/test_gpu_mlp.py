"""GPU parity of the fused MLP (gate and up in one launch, SiLU(g)*u kept as
fp16, then down) against the fp64 oracle, which rounds nothing in between.
Per-column widths: a shared 4/3-bit mask for gate and up, a 2/3-bit mask for
down."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, say, sha  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _mlp(H, I, cfg, uniform_bits=None):
    if uniform_bits is None:
        cb_gu = S.column_bits(I, 0.2, 4, cfg_id=cfg, tensor_id=S.T_MASK)
        cb_dn = S.column_bits(H, 0.2, 2, cfg_id=cfg, tensor_id=S.T_MASK + 100)
        g = Uniform(I, H, col_bits=cb_gu, cfg_id=cfg, tid=0)
        u = Uniform(I, H, col_bits=cb_gu, cfg_id=cfg, tid=1)
        d = Uniform(H, I, col_bits=cb_dn, cfg_id=cfg, tid=2)
    else:
        g = Uniform(I, H, uniform_bits, cfg_id=cfg, tid=0)
        u = Uniform(I, H, uniform_bits, cfg_id=cfg, tid=1)
        d = Uniform(H, I, uniform_bits, cfg_id=cfg, tid=2)
    return g, u, d


@pytest.mark.parametrize("M", [1, 2, 8, 17, 32])
@pytest.mark.parametrize("H,I", [(256, 512), (640, 1408)])
def test_mlp_mixed_parity(M, H, I):
    say("mlp mixed", M, H, I)
    g, u, d = _mlp(H, I, cfg=70)
    x = S.activations(M, H, cfg_id=70, tensor_id=100 + M)
    out = Q.mlp(g.lin, u.lin, d.lin, dev_f16(x))
    torch.cuda.synchronize()
    r = O.mlp(x, g.w(), u.w(), d.w())
    err = O.normwise_rel_err(out.cpu().numpy().astype(np.float64), r)
    say("mlp err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mlp_uniform_parity(bits):
    say("mlp uniform", bits)
    g, u, d = _mlp(384, 768, cfg=71, uniform_bits=bits)
    x = S.activations(4, 384, cfg_id=71)
    out = Q.mlp(g.lin, u.lin, d.lin, dev_f16(x))
    torch.cuda.synchronize()
    r = O.mlp(x, g.w(), u.w(), d.w())
    assert O.normwise_rel_err(out.cpu().numpy().astype(np.float64), r) <= TOL


def test_mlp_zero_input_gives_zero():
    g, u, d = _mlp(256, 512, cfg=72)
    out = Q.mlp(g.lin, u.lin, d.lin, torch.zeros((3, 256), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_mlp_repeat_bit_identical():
    g, u, d = _mlp(640, 1408, cfg=73)
    x = dev_f16(S.activations(8, 640, cfg_id=73))
    hs = {sha(Q.mlp(g.lin, u.lin, d.lin, x)) for _ in range(10)}
    assert len(hs) == 1


def test_mlp_shape_mismatch_rejected():
    g, u, d = _mlp(256, 512, cfg=74)
    other = Uniform(512, 256, 3, cfg_id=74, tid=5)      # widths differ from gate's
    x = dev_f16(S.activations(1, 256, cfg_id=74))
    with pytest.raises(Q.QGError) as e:
        Q.mlp(g.lin, other.lin, d.lin, x)
    assert e.value.status == Q.QG_ERR_INVALID_ARG
    with pytest.raises(Q.QGError):
        Q.mlp(g.lin, u.lin, g.lin, x)                  # down's K must be gate's N


@pytest.mark.parametrize("mixed", [False, True])
def test_three_quad_plans(mixed):
    """The fused gate/up pass at K = 5120 and a several-width matrix at
    K = 17408 run 3 quads per wave: the MLP (one width and mixed widths)
    against the oracle, and the several-width long-K GEMV on its own."""
    H, I = 5120, 1024
    if mixed:
        cb_gu = S.column_bits(I, 0.25, 4, cfg_id=171, tensor_id=S.T_MASK)
        g = Uniform(I, H, col_bits=cb_gu, cfg_id=171, tid=0)
        u = Uniform(I, H, col_bits=cb_gu, cfg_id=171, tid=1)
        d = Uniform(H, I, col_bits=S.column_bits(H, 0.25, 2, cfg_id=171, tensor_id=S.T_MASK + 1), cfg_id=171, tid=2)
    else:
        g, u, d = (Uniform(I, H, 3, cfg_id=172, tid=0), Uniform(I, H, 3, cfg_id=172, tid=1),
                   Uniform(H, I, 3, cfg_id=172, tid=2))
    x_np = S.activations(1, H, cfg_id=173 + mixed)
    y = Q.mlp(g.lin, u.lin, d.lin, dev_f16(x_np)).cpu().numpy().astype(np.float64)
    ref = O.mlp(x_np, g.w(), u.w(), d.w())
    err = O.normwise_rel_err(y, ref)
    say("mlp 3-quad", mixed, err)
    assert err <= TOL, err
    if mixed:
        cb = S.column_bits(640, 0.3, 4, cfg_id=175, tensor_id=S.T_MASK)
        m = Uniform(640, 17408, col_bits=cb, cfg_id=175, tid=3)
        xl = S.activations(1, 17408, cfg_id=175)
        yl = m.lin.run(dev_f16(xl)).cpu().numpy().astype(np.float64)
        assert O.normwise_rel_err(yl, m.ref(xl)) <= TOL
