"""CPU oracle for the packed low-bit weight-only GEMV / verify GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or helper
with the HIP library; the only thing both sides share is the seeded input
generator (``qg_synth``), which holds no arithmetic of the method.

What is computed, and where it comes from
-----------------------------------------
The method is "dequantise the packed weights, then multiply by the fp16
activations" -- the weight-only low-bit GEMV that runs a single-request decode
step (one activation row) and the speculative-decode verify pass (8..32 rows);
see "OrcaSAQ2-27B on AMD Radeon -- ROCm runtime" (intro: EXL3 trellis weights at
~3.2 bits/weight, GEMM kernels on vector ALUs) and "Qwen3.8-27B on a 16 GB RX
9070 XT" (section "What we added on top of upstream": WMMA GEMV for verifying 8
drafted tokens, batched verify up to 32 rows, fused MLP).  Block formats with a
per-block fp16 scale over 128 elements and an unsigned-code offset are the
"Format / Block / Scale / Leaf encoding" table of "The Rock8".  The pages give no
bit layout, so the conventions below are this library's, stated once here:

* W is [N][K] (out x in features), y[m][n] = sum_k x[m][k] * w[n][k].
* Uniform b-bit codes (b in 2,3,4), one fp16 scale per 128 consecutive k of a
  row: w = (c - o_b) * s with o_b = (2**b - 1)/2 (3.5 for 3 bits).
* Canonical packed stream: per row n, per group g, 4*b little-endian uint32
  words at word index (n*G + g)*4*b; in-group code j sits in stream bits
  [b*j, b*j + b), stream bit t being bit (t mod 32) of word t//32.  Per-column
  bit widths concatenate the rows' streams in row order.
* Bitshift trellis: 16x16 tiles (16 rows n x 16 columns k), 48 uint16 words =
  768 bits per tile, stream bit t = bit (15 - t mod 16) of word t//16 (MSB
  first); weight i = 16*r + c of the tile (r = n - 16*tn, c = k - 16*tk) has
  state_i = the cyclic 16-bit window starting at stream bit 3*i, and
  w = codebook[state_i] * s[n][k//128].
* Rotation: normalised 128-point Walsh-Hadamard transform of x per 128-group,
  Sylvester (natural) order, H[i][j] = (-1)**popcount(i & j) / sqrt(128).
* MLP: out = down(SiLU(gate(x)) * up(x)), SiLU(z) = z / (1 + exp(-z)).
* MXFP4 ("The Rock8", format table, MXFP4 row: blocks of 32 elements in 17
  bytes, OCP E2M1 leaves -- 2 exponent bits, 1 mantissa bit -- nibble-packed,
  and one UE8M0 scale byte per block, value 2**(e - 127)): element codes in the
  4-bit canonical stream above, scales uint8 [N][K/32];
  w = e2m1(c) * 2**(e - 127).  E2M1 read as a binary float with exponent bias
  1: sign bit 3, exponent bits 2..1, mantissa bit 0; exponent 0 is subnormal
  (0.5 * m).  E8M0 = 255 is NaN.
* MXFP6 ("The Rock8", format table, MXFP6 row: blocks of 32 elements in 25
  bytes, OCP E3M2 leaves -- 3 exponent bits, 2 mantissa bits -- four values per
  three bytes, one UE8M0 scale byte per block): element codes in the 6-bit
  canonical stream (the uniform stream above with b = 6: 24 words per row and
  group, element j at stream bits [6j, 6j + 6), so bytes 3i..3i+2 hold elements
  4i..4i+3), scales uint8 [N][K/32]; w = e3m2(c) * 2**(e - 127).  E3M2 read as
  a binary float with exponent bias 3: sign bit 5, exponent bits 4..2, mantissa
  bits 1..0; exponent 0 is subnormal (m / 16); no infinities or NaN.

All floating point is fp64 and no intermediate is rounded.  Dequantised weights
are exact (fp16 scale times a code offset has at most 15 significant bits), and
the matrix product uses NumPy's float64 matmul as a library primitive.
"""
from __future__ import annotations

import numpy as np

GROUP = 128


# ---------------------------------------------------------------------------
# uniform b-bit codes
# ---------------------------------------------------------------------------
def code_offset(bits: int) -> float:
    """o_b = (2**b - 1) / 2: the code value that maps to weight zero."""
    return (2 ** bits - 1) / 2.0


def _stream_bits_lsb(words: np.ndarray) -> np.ndarray:
    """uint32 words -> bit array, bit t = bit (t mod 32) of word t//32."""
    w = np.ascontiguousarray(words, dtype="<u4")
    return np.unpackbits(w.view(np.uint8), bitorder="little")


def unpack_uniform(words: np.ndarray, N: int, K: int, bits: int) -> np.ndarray:
    """Canonical packed stream -> codes int64[N][K] (every column ``bits`` wide)."""
    assert K % GROUP == 0 and bits in (2, 3, 4, 6)
    G = K // GROUP
    words = np.asarray(words, dtype=np.uint32).reshape(-1)
    assert words.size == N * G * 4 * bits
    b = _stream_bits_lsb(words).reshape(N, G, GROUP, bits).astype(np.int64)
    weights = (1 << np.arange(bits, dtype=np.int64))
    return (b * weights).sum(axis=-1).reshape(N, K)


def pack_uniform(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of :func:`unpack_uniform` (codes[N][K] -> canonical words)."""
    codes = np.asarray(codes, dtype=np.int64)
    N, K = codes.shape
    assert K % GROUP == 0 and codes.min() >= 0 and codes.max() < 2 ** bits
    b = ((codes[..., None] >> np.arange(bits)) & 1).astype(np.uint8).reshape(-1)
    return np.packbits(b, bitorder="little").view("<u4").astype(np.uint32)


def row_word_offsets(col_bits: np.ndarray, K: int) -> np.ndarray:
    """Word offset of each row's stream when rows have different bit widths."""
    per_row = np.asarray(col_bits, dtype=np.int64) * (K // 32)
    return np.concatenate([[0], np.cumsum(per_row)])


def unpack_mixed(words: np.ndarray, col_bits: np.ndarray, K: int, rows=None) -> np.ndarray:
    """Per-column bit widths: row n's stream has K*col_bits[n]/32 words, rows in
    order.  Returns codes int64[len(rows)][K] for the requested rows."""
    words = np.asarray(words, dtype=np.uint32).reshape(-1)
    off = row_word_offsets(col_bits, K)
    rows = np.arange(len(col_bits)) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), K), dtype=np.int64)
    for i, n in enumerate(rows):
        b = int(col_bits[n])
        out[i] = unpack_uniform(words[off[n]:off[n + 1]], 1, K, b)[0]
    return out


def scale_group(K: int, scales: np.ndarray, N: int) -> int:
    """The scale group size gs of an [N][K/gs] scale array: 128, or 64 / 32
    ("The Rock8", dormant-capabilities table: int4 weight-only at group 128, 64
    and 32; one fp16 scale per gs consecutive k of a row)."""
    per_row = np.asarray(scales).size // N
    assert per_row * N == np.asarray(scales).size and K % per_row == 0
    gs = K // per_row
    assert gs in (32, 64, 128), gs
    return gs


def dequant_uniform(codes: np.ndarray, scales: np.ndarray, bits) -> np.ndarray:
    """w[n][k] = (c[n][k] - o_b) * s[n][k // gs] in fp64 (exact); gs is the
    scale group the scale array's shape gives (128, 64 or 32).

    ``bits`` is an int (all rows) or an array of per-row widths."""
    codes = np.asarray(codes, dtype=np.float64)
    N, K = codes.shape
    gs = scale_group(K, scales, N)
    s = np.repeat(np.asarray(scales, dtype=np.float64).reshape(N, K // gs), gs, axis=1)
    if np.ndim(bits) == 0:
        o = code_offset(int(bits))
    else:
        o = ((2.0 ** np.asarray(bits, dtype=np.float64) - 1.0) / 2.0)[:, None]
    return (codes - o) * s


# ---------------------------------------------------------------------------
# bitshift trellis
# ---------------------------------------------------------------------------
def trellis_states(words16: np.ndarray, N: int, K: int) -> np.ndarray:
    """Trellis tiles uint16[N/16][K/16][48] -> states uint16[N][K].

    state_i = sum_{u<16} bit[(3i + u) mod 768] * 2**(15 - u), stream bits taken
    MSB first from each uint16 word."""
    t = np.asarray(words16, dtype=np.uint16).reshape(N // 16, K // 16, 48)
    be = t.astype(">u2").view(np.uint8).reshape(N // 16, K // 16, 96)
    bits = np.unpackbits(be, axis=-1, bitorder="big").astype(np.int64)  # [..., 768]
    i = np.arange(256)[:, None]
    u = np.arange(16)[None, :]
    idx = (3 * i + u) % 768                                            # [256][16]
    win = bits[:, :, idx]                                              # [tn][tk][256][16]
    st = (win << (15 - u)).sum(axis=-1)                                # [tn][tk][256]
    st = st.reshape(N // 16, K // 16, 16, 16)                          # [tn][tk][r][c]
    return st.transpose(0, 2, 1, 3).reshape(N, K).astype(np.uint16)


def trellis_dequant(states: np.ndarray, codebook: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """w[n][k] = codebook[state[n][k]] * s[n][k//128] in fp64 (exact)."""
    N, K = states.shape
    cb = np.asarray(codebook, dtype=np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float64).reshape(N, K // GROUP), GROUP, axis=1)
    return cb[states.astype(np.int64)] * s


def hadamard128() -> np.ndarray:
    """Normalised Sylvester Walsh-Hadamard matrix, H[i][j] = (-1)^popcount(i&j) / sqrt(128)."""
    i = np.arange(GROUP)
    pc = np.array([bin(v).count("1") for v in range(GROUP)])
    sign = 1.0 - 2.0 * (pc[(i[:, None] & i[None, :])] & 1)
    return sign * 2.0 ** -3.5


def rotate(x: np.ndarray) -> np.ndarray:
    """x'[m][128g + j] = sum_i H[j][i] x[m][128g + i] (per 128-group), fp64."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    H = hadamard128()
    xg = x.reshape(M, K // GROUP, GROUP)
    return np.einsum("ji,mgi->mgj", H, xg).reshape(M, K)


# ---------------------------------------------------------------------------
# MXFP4: E2M1 elements, UE8M0 block scales (blocks of 32 along k)
# ---------------------------------------------------------------------------
MX_BLOCK = 32


def e2m1_value(code: int) -> float:
    """An E2M1 element: sign bit 3, two exponent bits (bias 1), one mantissa bit."""
    code = int(code)
    sign = -1.0 if (code >> 3) & 1 else 1.0
    e, m = (code >> 1) & 3, code & 1
    if e == 0:
        return sign * 0.5 * m                      # subnormal: 2^(1-1) * (0 + m/2)
    return sign * 2.0 ** (e - 1) * (1.0 + 0.5 * m)


def e8m0_value(e: int) -> float:
    """A UE8M0 scale byte: 2^(e - 127); 255 is NaN."""
    e = int(e)
    return float("nan") if e == 255 else 2.0 ** (e - 127)


def dequant_mxfp4(codes: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """w[n][k] = e2m1(c[n][k]) * 2^(e8[n][k // 32] - 127) in fp64 (exact)."""
    codes = np.asarray(codes, dtype=np.int64)
    N, K = codes.shape
    lut = np.array([e2m1_value(c) for c in range(16)])
    sc = np.array([e8m0_value(e) for e in range(256)])
    s = np.repeat(sc[np.asarray(e8, dtype=np.int64).reshape(N, K // MX_BLOCK)], MX_BLOCK, axis=1)
    return lut[codes] * s


def gemv_mxfp4(x, words, e8, N: int, K: int, rows=None) -> np.ndarray:
    """y = x * dequant(W)^T for MXFP4 weights (optionally some output columns)."""
    rows = np.arange(N) if rows is None else np.asarray(rows)
    words = np.asarray(words, dtype=np.uint32).reshape(N, -1)
    codes = unpack_uniform(words[rows].reshape(-1), len(rows), K, 4)
    return matmul(x, dequant_mxfp4(codes, np.asarray(e8).reshape(N, -1)[rows]))


# ---------------------------------------------------------------------------
# MXFP6: E3M2 elements, UE8M0 block scales (blocks of 32 along k)
# ---------------------------------------------------------------------------
def e3m2_value(code: int) -> float:
    """An E3M2 element: sign bit 5, three exponent bits (bias 3), two mantissa bits."""
    code = int(code)
    sign = -1.0 if (code >> 5) & 1 else 1.0
    e, m = (code >> 2) & 7, code & 3
    if e == 0:
        return sign * 2.0 ** (1 - 3) * (m / 4.0)   # subnormal
    return sign * 2.0 ** (e - 3) * (1.0 + m / 4.0)


def dequant_mxfp6(codes: np.ndarray, e8: np.ndarray) -> np.ndarray:
    """w[n][k] = e3m2(c[n][k]) * 2^(e8[n][k // 32] - 127) in fp64 (exact)."""
    codes = np.asarray(codes, dtype=np.int64)
    N, K = codes.shape
    lut = np.array([e3m2_value(c) for c in range(64)])
    sc = np.array([e8m0_value(e) for e in range(256)])
    s = np.repeat(sc[np.asarray(e8, dtype=np.int64).reshape(N, K // MX_BLOCK)], MX_BLOCK, axis=1)
    return lut[codes] * s


def gemv_mxfp6(x, words, e8, N: int, K: int, rows=None) -> np.ndarray:
    """y = x * dequant(W)^T for MXFP6 weights (optionally some output columns)."""
    rows = np.arange(N) if rows is None else np.asarray(rows)
    words = np.asarray(words, dtype=np.uint32).reshape(N, -1)
    codes = unpack_uniform(words[rows].reshape(-1), len(rows), K, 6)
    return matmul(x, dequant_mxfp6(codes, np.asarray(e8).reshape(N, -1)[rows]))


# ---------------------------------------------------------------------------
# products
# ---------------------------------------------------------------------------
def matmul(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """r[m][n] = sum_k x[m][k] w[n][k] in fp64 (x taken at its exact fp16 value)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def gemv_uniform(x, words, scales, N: int, K: int, bits: int) -> np.ndarray:
    """y = x * dequant(W)^T for uniform b-bit codes."""
    return matmul(x, dequant_uniform(unpack_uniform(words, N, K, bits), scales, bits))


def gemv_uniform_rows(x, words, scales, N: int, K: int, bits: int, rows) -> np.ndarray:
    """Same as :func:`gemv_uniform` restricted to output columns ``rows`` (for
    spot checks of large shapes).  Returns [M][len(rows)]."""
    G = K // GROUP
    wpr = G * 4 * bits
    words = np.asarray(words, dtype=np.uint32).reshape(N, wpr)
    rows = np.asarray(rows)
    codes = unpack_uniform(words[rows].reshape(-1), len(rows), K, bits)
    s = np.asarray(scales).reshape(N, -1)[rows]
    return matmul(x, dequant_uniform(codes, s, bits))


def gemv_mixed(x, words, scales, col_bits, K: int, rows=None) -> np.ndarray:
    """y = x * dequant(W)^T with per-column bit widths (optionally some columns)."""
    N = len(col_bits)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    codes = unpack_mixed(words, col_bits, K, rows)
    s = np.asarray(scales).reshape(N, -1)[rows]
    return matmul(x, dequant_uniform(codes, s, np.asarray(col_bits)[rows]))


def gemv_trellis(x, words16, codebook, scales, N: int, K: int, prerotated: bool = False) -> np.ndarray:
    """y = rotate(x) * W^T with trellis-coded W (x used as given if prerotated)."""
    xr = np.asarray(x, dtype=np.float64) if prerotated else rotate(x)
    w = trellis_dequant(trellis_states(words16, N, K), codebook, scales)
    return matmul(xr, w)


def gemv_trellis_rows(x, words16, codebook, scales, N: int, K: int, rows, prerotated: bool = False) -> np.ndarray:
    """Same as :func:`gemv_trellis` restricted to output rows ``rows`` (spot
    checks of large shapes: only the 16-row tile rows holding them are
    decoded).  Returns [M][len(rows)]."""
    rows = np.asarray(rows)
    xr = np.asarray(x, dtype=np.float64) if prerotated else rotate(x)
    tiles = np.asarray(words16, dtype=np.uint16).reshape(N // 16, K // 16, 48)
    blocks = np.unique(rows // 16)
    st = trellis_states(tiles[blocks].reshape(-1), 16 * len(blocks), K)       # [16*nb][K]
    pos = {int(b): i for i, b in enumerate(blocks)}
    sel = np.array([16 * pos[int(n) // 16] + int(n) % 16 for n in rows])
    s = np.asarray(scales).reshape(N, K // GROUP)[rows]
    return matmul(xr, trellis_dequant(st[sel], codebook, s))


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def mlp(x, w_gate, w_up, w_down) -> np.ndarray:
    """out = (SiLU(x W_g^T) * (x W_u^T)) W_d^T in fp64, nothing rounded."""
    g = matmul(x, w_gate)
    u = matmul(x, w_up)
    return matmul(silu(g) * u, w_down)


# ---------------------------------------------------------------------------
# comparison
# ---------------------------------------------------------------------------
def normwise_rel_err(y: np.ndarray, r: np.ndarray) -> float:
    """max |y - r| / max |r| over the whole output tensor."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = np.max(np.abs(r))
    num = np.max(np.abs(y - r))
    if den == 0.0:
        return float(num)
    return float(num / den)
