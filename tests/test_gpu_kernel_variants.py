"""Every kernel variant the dispatcher can pick, forced through its switch on
shapes small enough for a full oracle comparison: the two M = 1 GEMVs (per-group
and per-tile-run) and the two verify GEMMs (per-wave K split and shared-x), on
one and several code widths, single matrices and the fused gate/up pass, each
checked against the oracle and for bit-identical repeats."""
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


def _check(lin, x_np, ref):
    x = dev_f16(x_np)
    y1 = lin.run(x)
    y2 = lin.run(x)
    torch.cuda.synchronize()
    assert sha(y1) == sha(y2)
    err = O.normwise_rel_err(y1.cpu().numpy().astype(np.float64), ref)
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
@pytest.mark.parametrize("N,K,bits", [(16, 128, 3), (272, 1280, 2), (528, 2560, 4), (96, 9216, 3)])
def test_m1_kernels(kernel, N, K, bits, monkeypatch):
    monkeypatch.setenv("QG_M1_KERNEL", kernel)
    say("m1", kernel, N, K, bits)
    u = Uniform(N, K, bits, cfg_id=90)
    x = S.activations(1, K, cfg_id=90, tensor_id=300)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
def test_m1_kernels_mixed_widths(kernel, monkeypatch):
    monkeypatch.setenv("QG_M1_KERNEL", kernel)
    N, K = 464, 1536
    cb = S.column_bits(N, 0.2, 4, cfg_id=91)
    cb[3::13] = 2
    say("m1 mixed", kernel)
    u = Uniform(N, K, col_bits=cb, cfg_id=91)
    x = S.activations(1, K, cfg_id=91, tensor_id=300)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("gemm", ["v1", "v2"])
@pytest.mark.parametrize("M", [2, 8, 16, 17, 32])
@pytest.mark.parametrize("N,K,bits", [(48, 384, 3), (272, 1280, 2), (528, 2560, 4)])
def test_gemm_kernels(gemm, M, N, K, bits, monkeypatch):
    monkeypatch.setenv("QG_GEMM", gemm)
    say("gemm", gemm, M, N, K, bits)
    u = Uniform(N, K, bits, cfg_id=92)
    x = S.activations(M, K, cfg_id=92, tensor_id=300 + M)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("gemm", ["v1", "v2"])
@pytest.mark.parametrize("M,tiles,waves,splits", [(8, 1, 4, 1), (8, 2, 8, 3), (32, 1, 8, 5), (32, 4, 4, 2),
                                                  (32, 2, 8, 1), (17, 2, 4, 4)])
def test_gemm_launch_shapes(gemm, M, tiles, waves, splits, monkeypatch):
    monkeypatch.setenv("QG_GEMM", gemm)
    N, K = 400, 2560
    say("gemm launch", gemm, M, tiles, waves, splits)
    u = Uniform(N, K, 3, cfg_id=93)
    u.lin.set_launch(M, tiles, waves, splits)
    x = S.activations(M, K, cfg_id=93, tensor_id=300 + M)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("kernel,gemm", [("pergroup", "v1"), ("runs", "v2")])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_fused_mlp_variants(kernel, gemm, M, monkeypatch):
    monkeypatch.setenv("QG_M1_KERNEL", kernel)
    monkeypatch.setenv("QG_GEMM", gemm)
    H, I = 512, 1408
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=94, tensor_id=S.T_MASK)
    cb_dn = S.column_bits(H, 0.2, 2, cfg_id=94, tensor_id=S.T_MASK + 100)
    g = Uniform(I, H, col_bits=cb_gu, cfg_id=94, tid=0)
    up = Uniform(I, H, col_bits=cb_gu, cfg_id=94, tid=1)
    d = Uniform(H, I, col_bits=cb_dn, cfg_id=94, tid=2)
    say("mlp variant", kernel, gemm, M)
    x = S.activations(M, H, cfg_id=94, tensor_id=400 + M)
    xd = dev_f16(x)
    o1 = Q.mlp(g.lin, up.lin, d.lin, xd)
    o2 = Q.mlp(g.lin, up.lin, d.lin, xd)
    torch.cuda.synchronize()
    assert sha(o1) == sha(o2)
    err = O.normwise_rel_err(o1.cpu().numpy().astype(np.float64), O.mlp(x, g.w(), up.w(), d.w()))
    say("mlp err", err)
    assert err <= TOL, err
