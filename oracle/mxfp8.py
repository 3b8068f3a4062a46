"""MXFP8 codecs and grouped quantize / dequantize / requantize / dbias (CPU oracle).

TEST INFRASTRUCTURE ONLY: used by tests, the smoke check and the CPU
baseline of the benchmark; never by the product path.

Definitions followed
--------------------
* Element format E4M3 (OCP 8-bit floating point, "FN" variant; OCP MX v1.0
  section 5.3): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
  Exponent field 0 is subnormal (m * 2^-9); code 0x7F / 0xFF is NaN; the
  largest finite magnitude is 448 = 1.75 * 2^8.  There is no infinity.
* Scale format E8M0 (OCP MX v1.0 section 5.4): an unsigned 8-bit biased
  exponent, value 2^(u - 127); 0xFF is NaN.
* Block conversion (OCP MX v1.0 section 6.3): for a block of 32 values the
  shared exponent is X = floor(log2(max |v|)) - emax_elem with emax_elem = 8
  for E4M3, and each element is stored as the E4M3 value nearest to v / 2^X.
  Rounding is to nearest with ties to the even code; magnitudes beyond 448
  saturate to 448.  A block whose values are all zero gets the smallest
  scale (2^-127, byte 0).  The sign of a zero is kept (-0 -> 0x80).
* Row-wise blocks run along the contraction (hidden) dimension: 1 x 32
  ("row-wise quanted input", Description of "[Pytorch] Add support for
  row-wise quanted input for grouped gemm", PR #3244).
* Column-wise blocks run along the token dimension inside each expert's
  group of rows: 32 x 1.  The column-wise copy is made by dequantizing the
  row-wise data and quantizing it again column-wise only (same page,
  Description and the Greptile Summary flowchart: Dequantize ->
  Columnwise-only requantize -> Wgrad grouped GEMM).  It is stored
  transposed: the column-wise copy of a [T, K] tensor is a [K, T] byte array
  with [K, T/32] scales, i.e. exactly the row-wise encoding of the
  transposed tensor's blocks.
* Scale tensor shape (round_up(T, 128), round_up(K/32, 4)) (same page, review
  thread on ``scale_shape``); the same review establishes per-expert
  128-token alignment and hidden % 512 == 0, under which the padding is
  empty.
* Bias gradient: the per-expert sum over token rows of the dequantized
  (high-precision) gradient (same page, Greptile Summary: "Bias and
  routing-scale reductions" fed from the Dequantize node).
"""

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # floor(log2(448))
E4M3_MIN_NORMAL_EXP = -6
E4M3_MANT_BITS = 3
E8M0_BIAS = 127
SCALE_EXP_MIN = -127
SCALE_EXP_MAX = 127
ROW_ALIGN = 128        # per-expert token alignment
HIDDEN_ALIGN = 512     # hidden-size alignment


# ----------------------------------------------------------------------------
# codecs
# ----------------------------------------------------------------------------

def decode_e4m3(codes):
    """E4M3 (FN) byte -> float64 value, from the bit fields."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = b >> 7
    e = (b >> 3) & 0xF
    m = b & 0x7
    subnormal = m * 2.0 ** -9
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def decode_e8m0(u):
    """E8M0 byte -> float64 scale 2^(u-127); 0xFF is NaN."""
    u = np.asarray(u, dtype=np.uint8).astype(np.int64)
    return np.where(u == 255, np.nan, np.exp2(u - float(E8M0_BIAS)))


def shared_exponent(amax):
    """X = floor(log2(amax)) - 8, exactly, clamped to the E8M0 range.

    floor(log2 a) is taken from the binary exponent (frexp: a = f * 2^p with
    0.5 <= f < 1, so floor(log2 a) = p - 1), never from a floating log2.
    amax == 0 gives the smallest exponent, -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, p = np.frexp(amax)
    x = np.where(amax > 0, (p - 1) - E4M3_EMAX, SCALE_EXP_MIN)
    return np.clip(x, SCALE_EXP_MIN, SCALE_EXP_MAX).astype(np.int64)


def encode_e4m3(y):
    """Exact float64 value -> nearest E4M3 byte, ties to even, saturating.

    The representable E4M3 magnitudes below 2^-6 are the multiples of 2^-9;
    in the binade [2^e, 2^(e+1)) with e >= -6 they are the multiples of
    2^(e-3).  y is divided by that spacing (exact, a power of two), rounded
    to an integer with ties to even (np.rint), multiplied back, clipped to
    448 and turned into a code.  The integer's parity is the code's last
    mantissa bit, so ties-to-even on the integer is ties-to-even on the code.
    """
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.abs(y)
    _, p = np.frexp(a)
    e = np.where(a > 0, p - 1, E4M3_MIN_NORMAL_EXP)
    e = np.maximum(e, E4M3_MIN_NORMAL_EXP)
    spacing = np.exp2((e - E4M3_MANT_BITS).astype(np.float64))
    v = np.rint(a / spacing) * spacing
    v = np.minimum(v, E4M3_MAX)
    code = _magnitude_code(v)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def _magnitude_code(v):
    """Representable magnitude (0 <= v <= 448) -> 7-bit E4M3 code."""
    _, p = np.frexp(v)
    ev = p - 1
    sub = v < 2.0 ** E4M3_MIN_NORMAL_EXP
    code_sub = v / 2.0 ** -9
    frac = np.where(sub, 1.0, v / np.exp2(ev.astype(np.float64)))  # in [1, 2)
    code_norm = (ev + 7) * 8 + (frac - 1.0) * 8
    code = np.where(sub, code_sub, code_norm)
    code_i = code.astype(np.int64)
    assert np.all(code_i == code), "value is not an E4M3 grid point"
    return code_i


# ----------------------------------------------------------------------------
# block quantization
# ----------------------------------------------------------------------------

def quantize_blocks_lastdim(x):
    """Quantize every run of 32 consecutive values along the last axis.

    x: float64 [R, C] with C % 32 == 0 (values exactly representable: bf16 or
    dequantized MXFP8).  Returns (codes uint8 [R, C], scale bytes uint8
    [R, C/32]).
    """
    x = np.asarray(x, dtype=np.float64)
    r, c = x.shape
    assert c % BLOCK == 0
    blocks = x.reshape(r, c // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=2)
    xexp = shared_exponent(amax)
    y = np.ldexp(blocks, -xexp[..., None])        # v / 2^X, exact
    q = encode_e4m3(y).reshape(r, c)
    s = (xexp + E8M0_BIAS).astype(np.uint8)
    return q, s


def check_splits(m_splits, total):
    m = [int(v) for v in m_splits]
    assert all(v >= 0 and v % ROW_ALIGN == 0 for v in m), "splits must be multiples of 128"
    assert sum(m) == total, "splits must sum to the token count"
    return m


def quantize_rowwise(x):
    """Row-wise (1 x 32 along K) MXFP8 of a [T, K] tensor -> ([T,K], [T,K/32])."""
    return quantize_blocks_lastdim(x)


def quantize_colwise(x, m_splits):
    """Column-wise (32 x 1 along tokens, within each expert group) MXFP8.

    x: float64 [T, K].  Returns the transposed physical copy
    (codes uint8 [K, T], scales uint8 [K, T/32]).  Blocks are taken group by
    group, 32 rows at a time from the group's first row.
    """
    x = np.asarray(x, dtype=np.float64)
    t, k = x.shape
    m = check_splits(m_splits, t)
    q = np.zeros((k, t), dtype=np.uint8)
    s = np.zeros((k, t // BLOCK), dtype=np.uint8)
    row = 0
    for mg in m:
        for i in range(mg // BLOCK):
            r0 = row + i * BLOCK
            blk = x[r0:r0 + BLOCK, :]                 # [32, K]: one block per column
            amax = np.abs(blk).max(axis=0)
            xexp = shared_exponent(amax)
            y = np.ldexp(blk, -xexp[None, :])
            q[:, r0:r0 + BLOCK] = encode_e4m3(y).T
            s[:, r0 // BLOCK] = (xexp + E8M0_BIAS).astype(np.uint8)
        row += mg
    return q, s


def dequantize_lastdim(q, s):
    """Codes [R, C] with scales [R, C/32] (blocks along the last axis) -> float64."""
    q = np.asarray(q)
    r, c = q.shape
    vals = decode_e4m3(q).reshape(r, c // BLOCK, BLOCK)
    return (vals * decode_e8m0(s)[..., None]).reshape(r, c)


def dequantize_rowwise(q_row, s_row):
    """Row-wise MXFP8 [T, K] -> float64 [T, K]."""
    return dequantize_lastdim(q_row, s_row)


def dequantize_colwise(q_col, s_col):
    """Transposed column-wise copy ([K, T], [K, T/32]) -> logical float64 [T, K]."""
    return dequantize_lastdim(q_col, s_col).T


def requant_colwise(q_row, s_row, m_splits):
    """Dequantize the row-wise data, then quantize column-wise only."""
    return quantize_colwise(dequantize_rowwise(q_row, s_row), m_splits)


def grouped_dbias(q_row, s_row, m_splits):
    """dbias[g, :] = sum over the rows of group g of the dequantized tensor.

    Returns float64 [G, K]; an empty group's row is zero.
    """
    xh = dequantize_rowwise(q_row, s_row)
    t, k = xh.shape
    m = check_splits(m_splits, t)
    out = np.zeros((len(m), k), dtype=np.float64)
    row = 0
    for g, mg in enumerate(m):
        if mg:
            out[g] = xh[row:row + mg].sum(axis=0)
        row += mg
    return out


def grouped_scaled_bias_grad(q_row, s_row, m_splits, scales, bias):
    """Gradients of a bias scaled by each row's routing scale.

    Reading (the pages name "scaled-bias gradient reductions" and "bias and
    routing-scale reductions" taken from the dequantized gradient, "[Pytorch]
    Add support for row-wise quanted input for grouped gemm", Greptile Summary
    and its flowchart, without formulas): the forward adds s_r * b_g to the
    output row r of expert g, so with dY the dequantized output gradient
        dbias[g, n] = sum over rows r of g of s_r * dY[r, n]
        dscales[r]  = sum over n of dY[r, n] * b[g, n]
    Returns float64 (dbias [G, N], dscales [T]); an empty group's dbias row is
    zero.  scales: [T]; bias: [G, N] (both taken as given, float64).
    """
    xh = dequantize_rowwise(q_row, s_row)
    t, n = xh.shape
    m = check_splits(m_splits, t)
    s = np.asarray(scales, dtype=np.float64)
    b = np.asarray(bias, dtype=np.float64)
    dbias = np.zeros((len(m), n), dtype=np.float64)
    dscales = np.zeros(t, dtype=np.float64)
    row = 0
    for g, mg in enumerate(m):
        if mg:
            rows = slice(row, row + mg)
            dbias[g] = (s[rows, None] * xh[rows]).sum(axis=0)
            dscales[rows] = xh[rows] @ b[g]
        row += mg
    return dbias, dscales


def scale_shape(total_tokens, cols):
    """Shape of the row-wise scale tensor: (round_up(T,128), round_up(K/32,4))."""
    def round_up(v, mult):
        return (v + mult - 1) // mult * mult
    return (round_up(total_tokens, 128), round_up(cols // BLOCK, 4))


# ----------------------------------------------------------------------------
# bf16 helpers (for comparing bf16 outputs)
# ----------------------------------------------------------------------------

def round_to_bf16(x):
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits: x = f * 2^p (0.5 <= f < 1), so the bf16
    value is rint(f * 2^8) * 2^(p-8).  Finite, normal-range inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    f, p = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(f, 8)), p - 8)


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (the ulp of the bf16 value x)."""
    x = np.asarray(x, dtype=np.float64)
    _, p = np.frexp(np.abs(x))
    ulp = np.ldexp(1.0, p - 8)
    return np.where(x == 0, np.ldexp(1.0, -133), ulp)
