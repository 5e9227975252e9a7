"""Every kernel and hand-over the planner can pick, forced through the
create-time pins and launch overrides on shapes small enough for a full oracle
comparison: the two M = 1 GEMVs (per-group and per-tile-run), the per-group
GEMV's K slices meeting in fixed-point words or partials, the verify GEMM with
one- and two-tile groups and both K-slice hand-overs, on one and several code
widths, single matrices and the fused gate/up pass, each checked against the
oracle and for bit-identical repeats."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, dev_words, run_np, say, sha  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402

M1_PIN = {"pergroup": Q.PIN_M1_PERGROUP, "runs": Q.PIN_M1_RUNS}
XS_PIN = {"xs": 0, "xs-t1": Q.PIN_XS_T1, "xs-t2": Q.PIN_XS_T2}


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cls(M):
    return 0 if M == 1 else (1 if M <= 16 else 2)


def _check(lin, x_np, ref):
    x = dev_f16(x_np)
    y1 = lin.run(x)
    y2 = lin.run(x)
    torch.cuda.synchronize()
    assert sha(y1) == sha(y2)
    err = O.normwise_rel_err(y1.cpu().numpy().astype(np.float64), ref)
    say("err", err)
    assert err <= TOL, err


def _mlp_check(g, up, d, x_np):
    xd = dev_f16(x_np)
    o1 = Q.mlp(g.lin, up.lin, d.lin, xd)
    o2 = Q.mlp(g.lin, up.lin, d.lin, xd)
    torch.cuda.synchronize()
    assert sha(o1) == sha(o2)
    err = O.normwise_rel_err(o1.cpu().numpy().astype(np.float64), O.mlp(x_np, g.w(), up.w(), d.w()))
    say("mlp err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
@pytest.mark.parametrize("N,K,bits", [(16, 128, 3), (272, 1280, 2), (528, 2560, 4), (96, 9216, 3)])
def test_m1_kernels(kernel, N, K, bits):
    say("m1", kernel, N, K, bits)
    u = Uniform(N, K, bits, cfg_id=90, pins=M1_PIN[kernel])
    x = S.activations(1, K, cfg_id=90, tensor_id=300)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("handover", ["words", "partials"])
@pytest.mark.parametrize("splits", [2, 3, 5])
@pytest.mark.parametrize("mixed", [False, True])
def test_m1_pergroup_k_slices(handover, splits, mixed):
    """Per-group M = 1 GEMV in K slices that meet in fixed-point words (the
    default for long K) or, pinned, in partials with an arrival count."""
    N, K = 464, 9216
    kw = dict(col_bits=S.column_bits(N, 0.2, 2, cfg_id=99)) if mixed else dict(bits=3)
    say("m1 k slices", handover, splits, mixed)
    pins = Q.PIN_M1_PERGROUP | (Q.PIN_PARTIALS if handover == "partials" else 0)
    u = Uniform(N, K, cfg_id=99, pins=pins, launch={0: (1, 0, splits)}, **kw)
    x = S.activations(1, K, cfg_id=99, tensor_id=300)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
def test_m1_kernels_mixed_widths(kernel):
    N, K = 464, 1536
    cb = S.column_bits(N, 0.2, 4, cfg_id=91)
    cb[3::13] = 2
    say("m1 mixed", kernel)
    u = Uniform(N, K, col_bits=cb, cfg_id=91, pins=M1_PIN[kernel])
    x = S.activations(1, K, cfg_id=91, tensor_id=300)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("gemm", ["xs", "xs-t1", "xs-t2"])
@pytest.mark.parametrize("M", [2, 8, 16, 17, 32])
@pytest.mark.parametrize("N,K,bits", [(48, 384, 3), (272, 1280, 2), (528, 2560, 4)])
def test_gemm_tile_groups(gemm, M, N, K, bits):
    """The verify GEMM with its own tile-group choice and with one- and
    two-tile groups pinned."""
    say("gemm", gemm, M, N, K, bits)
    u = Uniform(N, K, bits, cfg_id=92, pins=XS_PIN[gemm])
    x = S.activations(M, K, cfg_id=92, tensor_id=300 + M)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("gemm", ["xs-t1", "xs-t2"])
@pytest.mark.parametrize("M,tiles,waves,splits", [(8, 1, 4, 1), (8, 2, 8, 3), (32, 1, 8, 5), (32, 4, 4, 2),
                                                  (32, 2, 8, 1), (17, 2, 4, 4), (5, 0, 3, 7)])
def test_gemm_launch_shapes(gemm, M, tiles, waves, splits):
    N, K = 400, 2560
    say("gemm launch", gemm, M, tiles, waves, splits)
    u = Uniform(N, K, 3, cfg_id=93, pins=XS_PIN[gemm], launch={_cls(M): (tiles, waves, splits)})
    x = S.activations(M, K, cfg_id=93, tensor_id=300 + M)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("kernel", ["pergroup", "runs"])
@pytest.mark.parametrize("M", [1, 8, 32])
def test_fused_mlp_variants(kernel, M):
    """The fused MLP with either M = 1 kernel pinned on all three handles (the
    gate's pins steer the gate/up pass, the down's the down pass)."""
    H, I = 512, 1408
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=94, tensor_id=S.T_MASK)
    cb_dn = S.column_bits(H, 0.2, 2, cfg_id=94, tensor_id=S.T_MASK + 100)
    pins = M1_PIN[kernel]
    g = Uniform(I, H, col_bits=cb_gu, cfg_id=94, tid=0, pins=pins)
    up = Uniform(I, H, col_bits=cb_gu, cfg_id=94, tid=1, pins=pins)
    d = Uniform(H, I, col_bits=cb_dn, cfg_id=94, tid=2, pins=pins)
    say("mlp variant", kernel, M)
    _mlp_check(g, up, d, S.activations(M, H, cfg_id=94, tensor_id=400 + M))


@pytest.mark.parametrize("mixed", [False, True])
@pytest.mark.parametrize("splits", [0, 2, 3])
@pytest.mark.parametrize("handover", ["words", "partials"])
def test_m1_gate_up_pair_k_slices(mixed, splits, handover):
    """M = 1 per-group gate/up pass, one matrix per workgroup: in one K slice
    (the two workgroups of a tile meet in an exchange word) and in K slices
    (they meet in the partials); the down pass in words or partials."""
    H, I = 2048, 1408
    cb_gu = S.column_bits(I, 0.2, 4, cfg_id=96, tensor_id=S.T_MASK) if mixed else None
    kw = dict(col_bits=cb_gu) if mixed else dict(bits=3)
    pins = Q.PIN_M1_PERGROUP | (Q.PIN_PARTIALS if handover == "partials" else 0)
    launch = {0: (1, 0, splits)} if splits else None
    g = Uniform(I, H, cfg_id=96, tid=0, pins=pins, launch=launch, **kw)
    up = Uniform(I, H, cfg_id=96, tid=1, pins=pins, launch=launch, **kw)
    d = Uniform(H, I, bits=4, cfg_id=96, tid=2, pins=pins, launch={0: (1, 0, 3)})
    say("mlp pair", mixed, splits, handover)
    _mlp_check(g, up, d, S.activations(1, H, cfg_id=96, tensor_id=401))


@pytest.mark.parametrize("handover", ["partials", "words"])
@pytest.mark.parametrize("tiles", ["xs-t1", "xs-t2"])
@pytest.mark.parametrize("M", [2, 8, 17, 32])
def test_gemm_xs_handovers(handover, tiles, M):
    """Verify GEMM with its K slices pinned to meet through partials and an
    arrival count or through fixed-point words, with one- and two-tile groups,
    uniform and several widths, and the fused MLP (gate/up pass and the down
    pass with per-(row, group) factors); repeats are bit-identical."""
    hp = Q.PIN_PARTIALS if handover == "partials" else Q.PIN_WORDS
    N, K = 400, 3072
    say("gemm xs handover", handover, tiles, M)
    u = Uniform(N, K, 3, cfg_id=97, pins=hp | XS_PIN[tiles], launch={_cls(M): (2, 0, 4)})
    x = S.activations(M, K, cfg_id=97, tensor_id=300 + M)
    _check(u.lin, x, u.ref(x))
    cb = S.column_bits(N, 0.2, 4, cfg_id=97)
    v = Uniform(N, K, col_bits=cb, cfg_id=97, pins=hp | XS_PIN[tiles], launch={_cls(M): (2, 0, 3)})
    _check(v.lin, x, v.ref(x))
    H, I = 2048, 1408
    g = Uniform(I, H, bits=3, cfg_id=98, tid=0, pins=hp, launch={_cls(M): (2, 0, 2)})
    up = Uniform(I, H, bits=3, cfg_id=98, tid=1, pins=hp)
    d = Uniform(H, I, bits=3, cfg_id=98, tid=2, pins=hp | XS_PIN[tiles], launch={_cls(M): (2, 0, 2)})
    _mlp_check(g, up, d, S.activations(M, H, cfg_id=98, tensor_id=400 + M))


@pytest.mark.parametrize("M", [3, 16, 32])
def test_gemm_xs_mixed_widths(M):
    """Verify GEMM over three width segments (its workgroups never span two)."""
    N, K = 464, 4608
    cb = S.column_bits(N, 0.2, 4, cfg_id=95)
    cb[3::13] = 2
    say("gemm xs mixed", M)
    u = Uniform(N, K, col_bits=cb, cfg_id=95)
    x = S.activations(M, K, cfg_id=95, tensor_id=300 + M)
    _check(u.lin, x, u.ref(x))


@pytest.mark.parametrize("M", [8, 32])
@pytest.mark.parametrize("N,K", [(5120, 5120), (1024, 5120), (17408, 5120), (5120, 17408)])
def test_gemm_xs_decode_shapes(M, N, K):
    """Verify GEMM at the full 27B-class layer shapes, in its own launch
    choice, on sampled output columns the oracle computes one by one."""
    say("gemm xs full", M, N, K)
    w = S.uniform_code_words(N, K, 3, cfg_id=96)
    sc = S.scales(N, K, cfg_id=96)
    lin = Q.QLinear(dev_words(w), dev_f16(sc), K, N, bits=3, max_M=32)
    x = S.activations(M, K, cfg_id=96, tensor_id=300 + M)
    y1 = run_np(lin, x)
    y2 = run_np(lin, x)
    assert np.array_equal(y1, y2)
    rng = np.random.default_rng([96, N])
    rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, size=64, replace=False)]))
    r = O.gemv_uniform_rows(x, w, sc, N, K, 3, rows)
    err = O.normwise_rel_err(y1[:, rows], r)
    say("err", err)
    assert err <= TOL, err
    lin.close()
