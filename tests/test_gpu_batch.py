"""Several independent products in one call (qgemv_run_batch): at M = 1 all of
them run in one launch.  Each output matches the oracle within the normwise
budget, repeats are bit-identical, siblings may share one x, several code
widths mix, other row counts run entry by entry exactly as qgemv_run does; at
the full 27B-class layer set on sampled columns too."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, dev_words, say, sha  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# a small layer set: (N, K) of q, k, v, o, gate, up, down
SMALL = [(512, 640), (128, 640), (128, 640), (640, 512), (1408, 640), (1408, 640), (640, 1408)]


def _layer(bits=3, mixed=False, cfg=160):
    out = []
    for i, (N, K) in enumerate(SMALL):
        if mixed:
            cb = S.column_bits(N, 0.25, 2 + 2 * (i % 2), cfg_id=cfg, tensor_id=S.T_MASK + i)
            out.append(Uniform(N, K, col_bits=cb, cfg_id=cfg, tid=i))
        else:
            out.append(Uniform(N, K, bits, cfg_id=cfg, tid=i))
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_layer_set_one_launch(bits):
    mats = _layer(bits)
    xs_np = [S.activations(1, K, cfg_id=161, tensor_id=i) for i, (N, K) in enumerate(SMALL)]
    xs = [dev_f16(x) for x in xs_np]
    say("batch layer", bits)
    ys = Q.run_batch([m.lin for m in mats], xs)
    ys2 = Q.run_batch([m.lin for m in mats], xs)
    torch.cuda.synchronize()
    for i, m in enumerate(mats):
        assert sha(ys[i]) == sha(ys2[i])
        err = O.normwise_rel_err(ys[i].cpu().numpy().astype(np.float64), m.ref(xs_np[i]))
        say(i, err)
        assert err <= TOL, (i, err)


def test_mixed_widths_and_shared_x():
    mats = _layer(mixed=True, cfg=162)
    q, k, v = mats[0], mats[1], mats[2]
    x_np = S.activations(1, 640, cfg_id=162)
    x = dev_f16(x_np)
    ys = Q.run_batch([q.lin, k.lin, v.lin], [x, x, x])     # siblings reading one x
    torch.cuda.synchronize()
    for m, y in zip((q, k, v), ys):
        assert O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np)) <= TOL


def test_pinned_partials_and_long_k():
    a = Uniform(400, 9216, 3, cfg_id=163, pins=Q.PIN_PARTIALS | Q.PIN_M1_PERGROUP, launch={0: (0, 0, 8)})
    b = Uniform(96, 17408, 2, cfg_id=164)
    xa, xb = S.activations(1, 9216, cfg_id=163), S.activations(1, 17408, cfg_id=164)
    ys = Q.run_batch([a.lin, b.lin], [dev_f16(xa), dev_f16(xb)])
    torch.cuda.synchronize()
    assert O.normwise_rel_err(ys[0].cpu().numpy().astype(np.float64), a.ref(xa)) <= TOL
    assert O.normwise_rel_err(ys[1].cpu().numpy().astype(np.float64), b.ref(xb)) <= TOL


@pytest.mark.parametrize("M", [2, 8, 32])
def test_other_row_counts_run_entry_by_entry(M):
    mats = _layer(3, cfg=165)
    xs = [dev_f16(S.activations(M, K, cfg_id=165, tensor_id=i)) for i, (N, K) in enumerate(SMALL)]
    ys = Q.run_batch([m.lin for m in mats], xs)
    for m, x, y in zip(mats, xs, ys):
        assert sha(y) == sha(m.lin.run(x))


def test_bad_arguments():
    mats = _layer(3, cfg=166)
    x = dev_f16(S.activations(1, 640, cfg_id=166))
    with pytest.raises(Q.QGError) as e:
        Q.run_batch([mats[0].lin, mats[0].lin], [x, x])        # one handle twice: one workspace
    assert e.value.status == Q.QG_ERR_INVALID_ARG
    with pytest.raises(Q.QGError):
        Q.run_batch([m.lin for m in mats] * 2, [x] * 14)       # more than 8 entries


def test_full_size_layer_set_sampled():
    say("batch full layer set")
    mats, xs_np = [], []
    for i, sh in enumerate(S.LAYER_SET):
        N, K = sh["N"], sh["K"]
        w = S.uniform_code_words(N, K, 3, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 10 * i)
        sc = S.scales(N, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 10 * i)
        mats.append((Q.QLinear(dev_words(w), dev_f16(sc), K, N, bits=3, max_M=32), w, sc, N, K))
        xs_np.append(S.activations(1, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + 60 + i))
    xs = [dev_f16(x) for x in xs_np]
    ys = Q.run_batch([m[0] for m in mats], xs)
    ys2 = Q.run_batch([m[0] for m in mats], xs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    for i, (lin, w, sc, N, K) in enumerate(mats):
        assert torch.equal(ys[i], ys2[i])
        rows = np.unique(np.concatenate([np.arange(16), np.arange(N - 16, N), rng.choice(N, 48, replace=False)]))
        err = O.normwise_rel_err(ys[i].cpu().numpy().astype(np.float64)[:, rows],
                                 O.gemv_uniform_rows(xs_np[i], w, sc, N, K, 3, rows))
        say(S.LAYER_SET[i]["name"], err)
        assert err <= TOL, (i, err)


@pytest.mark.parametrize("bits", [2, 3, 4, 0])
def test_wide_batch_three_quads_per_wave(bits):
    """From 1024 tiles in one batch the launch runs 3 quads per wave: two wide
    matrices (one K slice with a ragged last quad; two K slices meeting in
    fixed-point words), every code width and several widths mixed, against the
    oracle on sampled columns (first and last tiles included)."""
    shapes = [(8192, 4736), (8192, 7168)]  # 37 groups (ragged quad), 56 groups (2 slices)
    mats, xs_np = [], []
    for i, (N, K) in enumerate(shapes):
        if bits == 0:
            cb = S.column_bits(N, 0.3, 2 + 2 * i, cfg_id=167, tensor_id=S.T_MASK + i)
            mats.append(Uniform(N, K, col_bits=cb, cfg_id=167, tid=i))
        else:
            mats.append(Uniform(N, K, bits, cfg_id=167, tid=i))
        xs_np.append(S.activations(1, K, cfg_id=167, tensor_id=10 + i))
    xs = [dev_f16(x) for x in xs_np]
    say("wide batch", bits)
    ys = Q.run_batch([m.lin for m in mats], xs)
    ys2 = Q.run_batch([m.lin for m in mats], xs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(167 + bits)
    for i, (m, (N, K)) in enumerate(zip(mats, shapes)):
        assert sha(ys[i]) == sha(ys2[i])
        rows = np.unique(np.concatenate([np.arange(32), np.arange(N - 32, N), rng.choice(N, 64, replace=False)]))
        err = O.normwise_rel_err(ys[i].cpu().numpy().astype(np.float64)[:, rows], m.ref(xs_np[i], rows))
        say(i, err)
        assert err <= TOL, (i, err)
