"""Runs captured in a HIP graph: every replay equals the eager result (replays
interleaved with eager work and synchronisations)."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import qg_synth as S  # noqa: E402
from _gpu import Uniform, dev_f16, say, sha  # noqa: E402
import bit_weight_only_packed_amd as Q  # noqa: E402


@pytest.mark.parametrize("M,splits", [(1, 1), (1, 4), (8, 1), (8, 3), (32, 2)])
def test_graph_replays_match_eager(M, splits):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    say("graph", M, splits)
    N, K = 1024, 5120
    u = Uniform(N, K, 3, cfg_id=60, launch={0 if M == 1 else (1 if M <= 16 else 2): (0, 0, splits)})
    x = dev_f16(S.activations(M, K, cfg_id=60))
    y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    eager = sha(u.lin.run(x))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        u.lin.run(x, out=y)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        u.lin.run(x, out=y)
    for i in range(5):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert sha(y) == eager, i
        other = u.lin.run(x)               # eager work between replays
        torch.cuda.synchronize()
        assert sha(other) == eager


def test_graph_mlp_replays_match_eager():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H, I = 256, 512
    cb = S.column_bits(I, 0.2, 4, cfg_id=61)
    cbd = S.column_bits(H, 0.2, 2, cfg_id=61, tensor_id=S.T_MASK + 100)
    g_ = Uniform(I, H, col_bits=cb, cfg_id=61, tid=0)
    u_ = Uniform(I, H, col_bits=cb, cfg_id=61, tid=1)
    d_ = Uniform(H, I, col_bits=cbd, cfg_id=61, tid=2)
    for M in (1, 8):
        x = dev_f16(S.activations(M, H, cfg_id=61))
        out = torch.empty((M, H), dtype=torch.float16, device="cuda")
        eager = sha(Q.mlp(g_.lin, u_.lin, d_.lin, x))
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            Q.mlp(g_.lin, u_.lin, d_.lin, x, out=out)
        torch.cuda.current_stream().wait_stream(s)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            Q.mlp(g_.lin, u_.lin, d_.lin, x, out=out)
        for i in range(4):
            out.zero_()
            gr.replay()
            torch.cuda.synchronize()
            assert sha(out) == eager, (M, i)
