"""Shared helpers of the GPU tests: upload the seeded inputs, build handles,
compare against the oracle.  Imported only by tests marked ``gpu``."""
from __future__ import annotations

import hashlib
import sys

import numpy as np
import torch

import bit_weight_only_packed_amd as Q
import oracle as O
import qg_synth as S

TOL = 2e-3  # max |y - r| / max |r|, fp32 accumulate vs fp64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_words(w: np.ndarray) -> torch.Tensor:
    """uint32 numpy words -> int32 CUDA tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(w).view(np.int32).copy()).cuda()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).cuda()


def dev_f16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).copy()).cuda()


class Uniform:
    """A seeded uniform-code (or per-column width) matrix with its handle."""

    def __init__(self, N, K, bits=3, col_bits=None, cfg_id=50, tid=0, max_M=32, pins=0, launch=None,
                 batch_invariant=False, group_size=128):
        self.N, self.K = N, K
        self.bits = bits
        self.col_bits = col_bits
        if col_bits is None:
            self.words = S.uniform_code_words(N, K, bits, cfg_id=cfg_id, tensor_id=S.T_CODES + 10 * tid)
        else:
            self.words = S.mixed_code_words(col_bits, K, cfg_id=cfg_id, tensor_id=S.T_CODES + 10 * tid)
        self.group_size = group_size
        self.scales = S.scales(N, K, cfg_id=cfg_id, tensor_id=S.T_SCALE + 10 * tid, group=group_size)
        self.dw = dev_words(self.words)
        self.ds = dev_f16(self.scales)
        self.lin = Q.QLinear(self.dw, self.ds, K, N, bits=bits, col_bits=col_bits, max_M=max_M, pins=pins,
                             launch=launch, batch_invariant=batch_invariant, group_size=group_size)

    def relinked(self, pins=0, launch=None, max_M=32, batch_invariant=False):
        """A second handle over the same device bytes, with other pins / launch overrides."""
        return Q.QLinear(self.dw, self.ds, self.K, self.N, bits=self.bits, col_bits=self.col_bits, max_M=max_M,
                         pins=pins, launch=launch, batch_invariant=batch_invariant, group_size=self.group_size)

    def codes(self, rows=None):
        if self.col_bits is None:
            c = O.unpack_uniform(self.words, self.N, self.K, self.bits)
            return c if rows is None else c[rows]
        return O.unpack_mixed(self.words, self.col_bits, self.K, rows)

    def w(self, rows=None):
        rr = np.arange(self.N) if rows is None else np.asarray(rows)
        bits = self.bits if self.col_bits is None else np.asarray(self.col_bits)[rr]
        return O.dequant_uniform(self.codes(rr), self.scales[rr], bits)

    def ref(self, x, rows=None):
        return O.matmul(x, self.w(rows))


def run_np(lin, x_np):
    x = dev_f16(x_np)
    y = lin.run(x)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def sha(t: torch.Tensor) -> str:
    return hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()
