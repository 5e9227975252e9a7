"""Seeded synthetic inputs for the packed low-bit weight-only GEMV / verify GEMM.

This module only draws random numbers in the shapes, dtypes and distributions of
the workloads; it holds none of the method's arithmetic (no packing, unpacking,
dequantisation, rotation or product).  Both the CPU oracle (tests, bench
baseline) and the GPU path read the very same arrays, so the two sides agree on
every input bit.

Every tensor draws from its own NumPy PCG64 stream seeded by
``SeedSequence([seed, cfg_id, tensor_id])``.

Packed code words are drawn as uniformly random 32-bit words.  The canonical
packing (b-bit fields laid end to end, 128 codes per group filling exactly
4*b words, no padding) is a bijection between word patterns and code arrays,
so uniformly random words are exactly iid uniform codes in 0..2**b-1 -- the
"codes uniform in 0..7" of the 3-bit workload -- without this module having to
pack anything.
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# tensor ids (one random stream per tensor kind; matrix index is added on top)
T_X, T_SCALE, T_CODES, T_MASK, T_TRELLIS, T_CODEBOOK = 1, 2, 3, 4, 5, 6


def _rng(seed: int, cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, cfg_id, tensor_id]))


def activations(M: int, K: int, *, seed: int = 0, cfg_id: int = 0, tensor_id: int = T_X) -> np.ndarray:
    """fp16 activations x[M][K], iid N(0,1) drawn in fp64 then rounded (RNE)."""
    r = _rng(seed, cfg_id, tensor_id)
    return r.standard_normal((M, K)).astype(np.float16)


def scales(N: int, K: int, *, seed: int = 0, cfg_id: int = 0, tensor_id: int = T_SCALE,
           sigma: float = 0.02, floor: float = 1e-3, group: int = GROUP) -> np.ndarray:
    """fp16 per-group scales s[N][K/group] = fp16(|N(0, sigma)| + floor)."""
    assert K % GROUP == 0 and group in (32, 64, 128)
    r = _rng(seed, cfg_id, tensor_id)
    v = np.abs(r.standard_normal((N, K // group))) * sigma + floor
    return v.astype(np.float16)


def mx_scales(N: int, K: int, *, seed: int = 0, cfg_id: int = 0, tensor_id: int = T_SCALE, lo: int = 116,
              hi: int = 124) -> np.ndarray:
    """UE8M0 block-scale bytes [N][K/32], uniform integers in [lo, hi]
    (2^-11 .. 2^-3 by default: the magnitudes of LLM weight blocks)."""
    assert K % 32 == 0 and 0 <= lo <= hi <= 255
    r = _rng(seed, cfg_id, tensor_id)
    return r.integers(lo, hi + 1, size=(N, K // 32)).astype(np.uint8)


def code_words(n_words: int, *, seed: int = 0, cfg_id: int = 0, tensor_id: int = T_CODES) -> np.ndarray:
    """``n_words`` uniformly random uint32 words (canonical packed code stream)."""
    r = _rng(seed, cfg_id, tensor_id)
    return r.integers(0, 2**32, size=n_words, dtype=np.uint64).astype(np.uint32)


def uniform_code_words(N: int, K: int, bits: int, **kw) -> np.ndarray:
    """Code stream for an N x K matrix with ``bits`` bits for every column
    (6: the MXFP6 element stream)."""
    assert K % GROUP == 0 and bits in (2, 3, 4, 6)
    return code_words(N * K * bits // 32, **kw)


def column_bits(N: int, frac: float, minor_bits: int, major_bits: int = 3, *, seed: int = 0,
                cfg_id: int = 0, tensor_id: int = T_MASK) -> np.ndarray:
    """Per-column bit widths: exactly round(frac*N) columns, chosen by a seeded
    permutation, get ``minor_bits``; the rest get ``major_bits``."""
    r = _rng(seed, cfg_id, tensor_id)
    n_minor = int(round(frac * N))
    pick = r.permutation(N)[:n_minor]
    cb = np.full(N, major_bits, dtype=np.uint8)
    cb[pick] = minor_bits
    return cb


def mixed_code_words(col_bits: np.ndarray, K: int, **kw) -> np.ndarray:
    """Code stream for per-column bit widths (row n holds K*col_bits[n]/32 words)."""
    assert K % GROUP == 0
    return code_words(int(np.sum(col_bits.astype(np.int64))) * K // 32, **kw)


def trellis_words(N: int, K: int, *, seed: int = 0, cfg_id: int = 0, tensor_id: int = T_TRELLIS) -> np.ndarray:
    """Trellis tiles: uint16[N/16][K/16][48], uniformly random bits (768 bits per 16x16 tile)."""
    assert N % 16 == 0 and K % 16 == 0
    r = _rng(seed, cfg_id, tensor_id)
    return r.integers(0, 2**16, size=(N // 16, K // 16, 48), dtype=np.uint32).astype(np.uint16)


def codebook(*, seed: int = 0, cfg_id: int = 0, tensor_id: int = T_CODEBOOK) -> np.ndarray:
    """65536-entry fp16 codebook, iid N(0,1) rounded to fp16."""
    r = _rng(seed, cfg_id, tensor_id)
    return r.standard_normal(65536).astype(np.float16)


# ---------------------------------------------------------------------------
# Named workloads (27B-class dense layer shapes; K x N = in x out features)
# ---------------------------------------------------------------------------
TINY = {"name": "tiny", "K": 512, "N": 512}
LAYER_SET = [
    {"name": "q", "K": 5120, "N": 5120},
    {"name": "k", "K": 5120, "N": 1024},
    {"name": "v", "K": 5120, "N": 1024},
    {"name": "o", "K": 5120, "N": 5120},
    {"name": "gate", "K": 5120, "N": 17408},
    {"name": "up", "K": 5120, "N": 17408},
    {"name": "down", "K": 17408, "N": 5120},
]
DISTINCT_SHAPES = [
    {"name": "qo", "K": 5120, "N": 5120},
    {"name": "kv", "K": 5120, "N": 1024},
    {"name": "gateup", "K": 5120, "N": 17408},
    {"name": "down", "K": 17408, "N": 5120},
]
MLP = {"hidden": 5120, "inter": 17408, "frac": 0.2, "gate_up_minor": 4, "down_minor": 2}

# config ids used to seed the streams of each workload
CFG_TINY, CFG_DECODE, CFG_VERIFY, CFG_MLP, CFG_TRELLIS = 0, 1, 2, 3, 4
