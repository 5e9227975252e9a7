"""The prefill route (qgemv_run_prefill): the fp16 weights it builds equal the
oracle's exact weights rounded once to fp16 (RNE), bit for bit, at 2, 3 and 4
bits and several widths; the products match the oracle within the normwise
budget for row counts from 1 to 2048 (ragged ones too), with the whole matrix
in the workspace and cut into column chunks; repeats are bit-identical; the
full 27B-class gate/up and down shapes at 512 rows on sampled columns; bad
arguments are refused."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle as O  # noqa: E402
import qg_synth as S  # noqa: E402
from _gpu import TOL, Uniform, dev_f16, say  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402

GEMM_WS = 32 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu_present():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _weights_f16(ws, N, K):
    return ws[GEMM_WS:GEMM_WS + N * K * 2].view(torch.int16).view(N, K).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("bits", [2, 3, 4, None])
def test_fp16_weights_bit_exact(bits):
    N, K = 400, 640
    cb = None if bits else S.column_bits(N, 0.3, 2, cfg_id=180, tensor_id=S.T_MASK)
    m = Uniform(N, K, bits or 3, col_bits=cb, cfg_id=180, tid=bits or 9)
    lo, full = m.lin.prefill_workspace()
    assert full == GEMM_WS + N * K * 2
    assert lo == (GEMM_WS + 16 * K * 2 if bits else full)
    ws = torch.zeros(full, dtype=torch.uint8, device="cuda")
    x = dev_f16(S.activations(3, K, cfg_id=180))
    m.lin.run_prefill(x, workspace=ws)
    torch.cuda.synchronize()
    got = _weights_f16(ws, N, K)
    want = m.w().astype(np.float16).view(np.uint16)  # exact fp64 w rounded once (RNE)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (bits, bad[:5])


@pytest.mark.parametrize("M", [1, 64, 200, 1024])
@pytest.mark.parametrize("bits", [3, None])
def test_products_match_oracle(M, bits):
    N, K = 528, 1536
    cb = None if bits else S.column_bits(N, 0.2, 4, cfg_id=181, tensor_id=S.T_MASK)
    m = Uniform(N, K, bits or 3, col_bits=cb, cfg_id=181, tid=M % 5)
    x_np = S.activations(M, K, cfg_id=181, tensor_id=M)
    x = dev_f16(x_np)
    say("prefill", M, bits)
    y = m.lin.run_prefill(x)
    y2 = m.lin.run_prefill(x)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("chunk_tiles", [1, 7, 33])
def test_column_chunks(chunk_tiles):
    """A workspace too small for the whole matrix: the columns go through in
    chunks of 16-column multiples (the last one ragged)."""
    N, K, M = 1040, 1024, 96
    m = Uniform(N, K, 3, cfg_id=182, tid=chunk_tiles)
    ws = torch.empty(GEMM_WS + chunk_tiles * 16 * K * 2 + 100, dtype=torch.uint8, device="cuda")
    x_np = S.activations(M, K, cfg_id=182)
    y = m.lin.run_prefill(dev_f16(x_np), workspace=ws)
    torch.cuda.synchronize()
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64), m.ref(x_np))
    say("chunks", chunk_tiles, err)
    assert err <= TOL, err


def test_long_prompt_2048_rows():
    N, K, M = 1024, 5120, 2048
    m = Uniform(N, K, 3, cfg_id=183)
    x_np = S.activations(M, K, cfg_id=183)
    y = m.lin.run_prefill(dev_f16(x_np))
    torch.cuda.synchronize()
    rows = np.arange(0, N, 7)
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("2048 rows err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("N,K", [(17408, 5120), (5120, 17408)])
def test_full_size_shapes_sampled(N, K):
    M = 512
    m = Uniform(N, K, 3, cfg_id=S.CFG_DECODE, tid=4)
    x_np = S.activations(M, K, cfg_id=184)
    say("prefill full", N, K)
    y = m.lin.run_prefill(dev_f16(x_np))
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(184).choice(N, 64, replace=False))
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("err", err)
    assert err <= TOL, err


def test_bad_arguments():
    m = Uniform(64, 256, 3, cfg_id=185)
    x = dev_f16(S.activations(8, 256, cfg_id=185))
    lo, full = m.lin.prefill_workspace()
    with pytest.raises(Q.QGError):
        m.lin.run_prefill(x, workspace=torch.empty(lo - 16, dtype=torch.uint8, device="cuda"))
    with pytest.raises(Q.QGError):
        m.lin.run_prefill(x[:0], workspace=torch.empty(full, dtype=torch.uint8, device="cuda"))
    cbk = dev_f16(S.codebook(cfg_id=S.CFG_TRELLIS))
    tw = S.trellis_words(64, 256, cfg_id=185)
    dtw = torch.from_numpy(np.ascontiguousarray(tw).view(np.int16).copy()).cuda()
    t = Q.QLinear(dtw, dev_f16(S.scales(64, 256, cfg_id=185)), 256, 64, trellis=True, codebook=cbk, max_M=8)
    with pytest.raises(Q.QGError):
        t.prefill_workspace()


@pytest.mark.parametrize("N,K,M", [(17408, 5120, 128), (5120, 5120, 63), (5120, 17408, 200), (1024, 5120, 64),
                                   (4096, 4096, 50)])
def test_chunked_rows_below_the_crossover(N, K, M):
    """Up to the crossover (measured on the 27B-class shapes, as (N, K):
    128 rows on (17408, 5120), 224 on (5120, 17408), 64 on (5120, 5120) and
    (1024, 5120); elsewhere 32 rows per 2048 of sqrt(N K)) the rows run as the
    verify GEMM, 32 at a time: the result equals qgemv_run on each 32-row
    block bit for bit (the last block ragged), matches the oracle on sampled
    columns, and leaves the caller's workspace untouched."""
    m = Uniform(N, K, 3, cfg_id=185, tid=M)
    x_np = S.activations(M, K, cfg_id=185, tensor_id=M)
    x = dev_f16(x_np)
    lo, _ = m.lin.prefill_workspace()
    ws = torch.full((lo,), 0x5A, dtype=torch.uint8, device="cuda")
    say("chunked prefill", N, K, M)
    y = m.lin.run_prefill(x, workspace=ws)
    parts = [m.lin.run(x[r0:r0 + 32]) for r0 in range(0, M, 32)]
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), torch.cat(parts).view(torch.int16))
    assert bool((ws == 0x5A).all())
    rows = np.random.default_rng(M).choice(N, 64, replace=False)
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("err", err)
    assert err <= TOL, err


@pytest.mark.parametrize("N,K,M", [(17408, 5120, 129), (1024, 5120, 65), (4096, 4096, 65)])
def test_route_above_the_crossover(N, K, M):
    """One row past the crossover the weights are dequantised into the
    caller's workspace and multiplied there; the result matches the oracle on
    sampled columns."""
    m = Uniform(N, K, 3, cfg_id=186, tid=M)
    x_np = S.activations(M, K, cfg_id=186, tensor_id=M)
    _, full = m.lin.prefill_workspace()
    ws = torch.full((full,), 0x5A, dtype=torch.uint8, device="cuda")
    say("prefill route", N, K, M)
    y = m.lin.run_prefill(dev_f16(x_np), workspace=ws)
    torch.cuda.synchronize()
    assert not bool((ws == 0x5A).all())
    rows = np.random.default_rng(M).choice(N, 64, replace=False)
    err = O.normwise_rel_err(y.cpu().numpy().astype(np.float64)[:, rows], m.ref(x_np, rows))
    say("err", err)
    assert err <= TOL, err
