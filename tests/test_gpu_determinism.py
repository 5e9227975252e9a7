"""Bit-identical results across processes: a fresh Python process builds its
own handles over the same seeded bytes and its outputs hash to the same
SHA-256 as this process's, for the M = 1 GEMV, the verify GEMM at 8 and 32
rows, the fused MLP and the trellis product (the pages' "bit-exact repeatable"
outputs and determinism tests)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _hashes():
    """SHA-256 of every case's output, computed in this process."""
    import hashlib

    import numpy as np

    import bit_weight_only_packed_amd as Q
    import qg_synth as S

    def dw(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32).copy()).cuda()

    def df(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).copy()).cuda()

    def h(t):
        torch.cuda.synchronize()
        return hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()

    out = {}
    N, K = 4096, 5120
    lin = Q.QLinear(dw(S.uniform_code_words(N, K, 3, cfg_id=140)), df(S.scales(N, K, cfg_id=140)), K, N, bits=3)
    for M in (1, 8, 32):
        out[f"uniform_M{M}"] = h(lin.run(df(S.activations(M, K, cfg_id=140, tensor_id=M))))
    H, I = 1024, 2816
    g = Q.QLinear(dw(S.uniform_code_words(I, H, 3, cfg_id=141, tensor_id=1)), df(S.scales(I, H, cfg_id=141, tensor_id=1)),
                  H, I, bits=3)
    u = Q.QLinear(dw(S.uniform_code_words(I, H, 3, cfg_id=141, tensor_id=2)), df(S.scales(I, H, cfg_id=141, tensor_id=2)),
                  H, I, bits=3)
    d = Q.QLinear(dw(S.uniform_code_words(H, I, 2, cfg_id=141, tensor_id=3)), df(S.scales(H, I, cfg_id=141, tensor_id=3)),
                  I, H, bits=2)
    for M in (1, 8):
        out[f"mlp_M{M}"] = h(Q.mlp(g, u, d, df(S.activations(M, H, cfg_id=141, tensor_id=M))))
    tw = torch.from_numpy(S.trellis_words(N, K, cfg_id=142).view(np.int16).copy()).cuda()
    t = Q.QLinear(tw, df(S.scales(N, K, cfg_id=142)), K, N, trellis=True, codebook=df(S.codebook(cfg_id=142)), max_M=8)
    for M in (1, 8):
        out[f"trellis_M{M}"] = h(t.run(df(S.activations(M, K, cfg_id=142, tensor_id=M))))
    return out


def test_hashes_match_a_fresh_process():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mine = _hashes()
    print("this process:", json.dumps(mine), flush=True)
    code = ("import json, sys; sys.path.insert(0, %r); sys.path.insert(0, %r); "
            "import test_gpu_determinism as T; print(json.dumps(T._hashes()))" % (HERE, os.path.dirname(HERE)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    theirs = json.loads(r.stdout.strip().splitlines()[-1])
    print("fresh process:", json.dumps(theirs), flush=True)
    assert theirs == mine
