"""CPU oracle for the BitNet b1.58 BitLinear projection y = (W~ . x~) * gamma * beta.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import this module.  The HIP library never calls
it, and it shares no code with the HIP library.

Source of every formula: the page "BitNet b1.58: Mathematical Foundations of
1.58-Bit Ternary Quantization, Absmean Scaling, and Multiplication-Free LLM
Architectures" (llms.blog), cited below as [B158] with its section names.

The oracle is written for obviousness, not speed: one numpy expression per
formula, exact rational arithmetic where a rounding decides an integer, and a
library float64 matrix product only where every partial sum is an integer far
below 2^53 (so the product is exact in any summation order).

Readings taken where the page leaves a step open (each is listed with its
reason in the design notes):
  * epsilon = 1e-5 (fp32) is added to gamma before dividing W, and to the
    absmax before dividing 127, as the two quantiser formulas print it; the
    rescale of the output uses gamma and the absmax without epsilon, as the
    rescale formula prints it.
  * floor(z + 0.5) is evaluated exactly (round half up), after z itself has
    been rounded to fp32 by a correctly rounded fp32 division/multiplication.
  * gamma is the exact mean of |W| rounded once to the nearest fp32 (ties to
    even); the page gives the mean, not a summation order.
  * Activations use one absmax per token (the page allows per-token or
    per-tensor) and the symmetric range [-127, 127] (Q_b - 1 = 127).  The
    4-bit activations that "The End of Matrix Multiplications" names (A4,
    no formula there) take the same formula with Q_b = 2^(4-1): the range
    [-7, 7] and x_scale = beta / 7.
  * The per-token reciprocal 127 / (absmax + eps) is formed in fp32 first and
    each element is multiplied by it (one fp32 multiply per element).
  * RMS normalisation before the quantiser ([B158] section 2 names it and
    cites Zhang and Sennrich's "Root Mean Square Layer Normalization"):
    y_k = x_k / sqrt(mean_k x_k^2 + eps) * g_k with a gain vector g, no
    centring, eps the quantisers' 1e-5 inside the root; the mean of squares is
    exact and rounded once to fp32, then an fp32 add, a correctly rounded fp32
    square root and reciprocal r, and per element fl32(fl32(x_k r) g_k).

Every function here is pinned by the CPU tests (closed forms, brute force,
invariants, a hand-derived worked example); none is "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

EPS = np.float32(1e-5)       # [B158] section 2, weight and activation quantisers
QMAX = 127                   # Q_b - 1 for 8-bit symmetric activations, [B158] section 2
_ROW_CHUNK_ELEMS = 1 << 24   # bounds temporaries on large tensors


# --------------------------------------------------------------------------
# Exact rounding of a rational to fp32
# --------------------------------------------------------------------------
def f32_nearest(q: Fraction) -> np.float32:
    """The fp32 value nearest to the rational q, ties to even (IEEE RNE).

    Covers subnormal results; results beyond the fp32 range become +-inf.
    """
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    # e = floor(log2(a))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    lsb = max(e, -126) - 23            # exponent of the last significand bit
    scaled = a / (Fraction(2) ** lsb)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    value = Fraction(n) * (Fraction(2) ** lsb)
    if value >= Fraction(2) ** 128:
        out = np.float32(np.inf)
    else:
        out = np.float32(float(value))  # exactly representable: no second rounding
    return np.float32(-out) if neg else out


# --------------------------------------------------------------------------
# Weight quantisation: absmean scale and RoundClip to {-1, 0, +1}
# --------------------------------------------------------------------------
def exact_abs_sum(W: np.ndarray) -> Fraction:
    """sum_ij |W_ij| as an exact rational.

    Each finite fp32 |w| equals sig * 2^(max(e,1) - 150) where e is the biased
    exponent field and sig the significand (with the implicit bit when e > 0).
    Significands are summed per exponent: each chunk's per-exponent total is an
    integer below 2^48, so float64 bincount adds them exactly; chunk totals are
    then added as Python integers.
    """
    flat = np.abs(np.ascontiguousarray(W, dtype=np.float32)).reshape(-1)
    totals = [0] * 256
    for s in range(0, flat.size, _ROW_CHUNK_ELEMS):
        bits = flat[s:s + _ROW_CHUNK_ELEMS].view(np.uint32)
        e = (bits >> np.uint32(23)).astype(np.int64)
        frac = (bits & np.uint32(0x7FFFFF)).astype(np.int64)
        sig = np.where(e > 0, frac | 0x800000, frac)
        eb = np.maximum(e, 1)
        part = np.bincount(eb, weights=sig.astype(np.float64), minlength=256)
        for b in np.nonzero(part)[0]:
            totals[int(b)] += int(part[b])
    num = sum(t << (b - 1) for b, t in enumerate(totals) if t)   # units of 2^-149
    return Fraction(num, 1 << 149)


def absmean_gamma(W: np.ndarray) -> np.float32:
    """gamma = (1 / (d_out d_in)) sum_ij |W_ij|  ([B158] section 2, absmean scaling).

    Exact mean, rounded once to fp32.
    """
    N, K = W.shape
    if N * K == 0:
        raise ValueError("empty weight")
    return f32_nearest(exact_abs_sum(W) / (N * K))


def round_clip(z: np.ndarray, a: int, b: int) -> np.ndarray:
    """RoundClip(z, a, b) = max(a, min(b, floor(z + 0.5)))  ([B158] section 2).

    z is fp32; z + 0.5 is formed in float64, where it is exact.
    """
    zz = np.asarray(z, dtype=np.float32).astype(np.float64)
    r = np.floor(zz + 0.5)
    return np.clip(r, a, b).astype(np.int64)


def ternarize(W: np.ndarray, gamma: np.float32) -> np.ndarray:
    """W~_ij = RoundClip(W_ij / (gamma + eps), -1, 1)  ([B158] section 2).

    gamma + eps is an fp32 add; W / (gamma + eps) a correctly rounded fp32
    division.  Returns int8 in {-1, 0, +1}.
    """
    W = np.ascontiguousarray(W, dtype=np.float32)
    g = np.float32(np.float32(gamma) + EPS)
    out = np.empty(W.shape, dtype=np.int8)
    rows = max(1, _ROW_CHUNK_ELEMS // max(1, W.shape[1]))
    with np.errstate(over="ignore", under="ignore"):
        for r in range(0, W.shape[0], rows):
            z = W[r:r + rows] / g
            out[r:r + rows] = round_clip(z, -1, 1).astype(np.int8)
    return out


# --------------------------------------------------------------------------
# 2-bit packing (format BLT2-v1)
# --------------------------------------------------------------------------
def pack_codes(Wt: np.ndarray) -> np.ndarray:
    """Pack ternary W~ [N][K] into bytes [N][K/4].

    Format (this library's own; the page names 2-bit registers, [B158]
    section 6): code c = W~ + 1 in {0, 1, 2}.  Row n is K/16 little-endian
    32-bit words; word g holds k = 16g + t (t = 0..15), and weight t = 4j + i
    sits in byte i of the word at bits 2j..2j+1.
    """
    Wt = np.asarray(Wt)
    N, K = Wt.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    c = (Wt.astype(np.int64) + 1)
    if c.min(initial=0) < 0 or c.max(initial=0) > 2:
        raise ValueError("not ternary")
    c = c.reshape(N, K // 16, 4, 4)          # axes: n, g, j, i  (k = 16g + 4j + i)
    byte = np.zeros((N, K // 16, 4), dtype=np.int64)  # axes: n, g, i
    for j in range(4):
        byte |= c[:, :, j, :] << (2 * j)
    return byte.reshape(N, K // 4).astype(np.uint8)


def unpack_codes(P: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_codes: bytes [N][K/4] -> int8 W~ [N][K]."""
    P = np.asarray(P, dtype=np.uint8)
    N = P.shape[0]
    b = P.reshape(N, K // 16, 4).astype(np.int64)     # n, g, i
    c = np.empty((N, K // 16, 4, 4), dtype=np.int64)  # n, g, j, i
    for j in range(4):
        c[:, :, j, :] = (b >> (2 * j)) & 3
    if (c == 3).any():
        raise ValueError("code 3 is not part of the format")
    return (c.reshape(N, K) - 1).astype(np.int8)


# --------------------------------------------------------------------------
# Base-3 packing, five weights per byte (format BLT3-v1)
# --------------------------------------------------------------------------
BLT3_PIECE = 80   # weights per 16-byte piece (four words of 20)


def base3_row_bytes(K: int) -> int:
    """Bytes of one BLT3-v1 row: K rounded up to whole 80-weight pieces."""
    return 16 * ((K + BLT3_PIECE - 1) // BLT3_PIECE)


def pack_codes_base3(Wt: np.ndarray) -> np.ndarray:
    """Pack ternary W~ [N][K] into bytes [N][base3_row_bytes(K)].

    [B158] section 4, "Memory Bandwidth and Latency Bounds": five ternary
    values fit one byte because 3^5 = 243 < 256.  The layout is this
    library's own (the page gives none): code c = W~ + 1; a row is padded with
    W~ = 0 to a multiple of 80 weights; little-endian 32-bit word g of the row
    holds k = 20g + 4j + b (j = 0..4, b = 0..3) in its byte b, which stores
    the base-3 number Nb = sum_j c_{20g+4j+b} 3^(4-j) (j = 0 the leading
    digit) as the byte ceil(256 Nb / 243).
    """
    Wt = np.asarray(Wt)
    N, K = Wt.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    c0 = Wt.astype(np.int64) + 1
    if c0.min(initial=0) < 0 or c0.max(initial=0) > 2:
        raise ValueError("not ternary")
    Kp = base3_row_bytes(K) * 5
    c = np.ones((N, Kp), dtype=np.int64)
    c[:, :K] = c0
    c = c.reshape(N, Kp // 20, 5, 4)                  # axes: n, g, j, b
    num = np.zeros((N, Kp // 20, 4), dtype=np.int64)  # axes: n, g, b
    for j in range(5):
        num += c[:, :, j, :] * 3 ** (4 - j)
    byte = (256 * num + 242) // 243                   # ceil(256 Nb / 243)
    return byte.reshape(N, Kp // 5).astype(np.uint8)


def unpack_codes_base3(P: np.ndarray, K: int) -> np.ndarray:
    """Inverse of pack_codes_base3: bytes -> int8 W~ [N][K].

    A byte B read as the fraction B / 256 approximates Nb / 243, the five
    digits after the point in base 3; multiplying by 3 moves the next digit
    into bits 8 and up: for j = 0..4, B = 3 B, digit j = B >> 8, B = B & 255.
    """
    P = np.asarray(P, dtype=np.uint8)
    N = P.shape[0]
    Kp = base3_row_bytes(K) * 5
    b0 = P.reshape(N, Kp // 20, 4).astype(np.int64)    # n, g, b
    x = b0
    c = np.empty((N, Kp // 20, 5, 4), dtype=np.int64)  # n, g, j, b
    for j in range(5):
        x = 3 * x
        c[:, :, j, :] = x >> 8
        x = x & 255
    # 13 of the 256 byte values are never written: re-encode and compare
    num = sum(c[:, :, j, :] * 3 ** (4 - j) for j in range(5))
    if ((256 * num + 242) // 243 != b0).any():
        raise ValueError("byte outside the format")
    c = c.reshape(N, Kp)
    if (c[:, K:] != 1).any():
        raise ValueError("padding weights must be zero")
    return (c[:, :K] - 1).astype(np.int8)


# --------------------------------------------------------------------------
# RMS normalisation of the activations (before the quantiser)
# --------------------------------------------------------------------------
def exact_sum_squares(X: np.ndarray) -> list:
    """Per row, the exact sum of x_k^2 as a Fraction.

    Every fp32 value is an integer multiple of 2^-149, so x = n 2^-149 with an
    integer n and sum x^2 = (sum n^2) 2^-298: a Python-integer sum, exact.
    """
    X = np.ascontiguousarray(X, dtype=np.float32)
    out = []
    for row in X:
        m, e = np.frexp(row.astype(np.float64))          # row = m 2^e, 0.5 <= |m| < 1
        ints = (m * 2.0 ** 24).astype(np.int64)          # exact: 24 significant bits
        total = 0
        for n, ee in zip(ints.tolist(), e.tolist()):
            if n:
                sh = ee - 24 + 149                       # x = n 2^(e-24) = v 2^-149
                v = n << sh if sh >= 0 else n >> -sh     # exact: x is a multiple of 2^-149
                total += v * v
        out.append(Fraction(total, 1 << 298))
    return out


def mean_square(X: np.ndarray) -> np.ndarray:
    """Per row, the mean of squares sum_k x_k^2 / K: the exact rational,
    rounded once to fp32 (nearest, ties to even).  fp32 [M]."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    K = X.shape[1]
    return np.array([f32_nearest(s / K) for s in exact_sum_squares(X)], dtype=np.float32)


def rmsnorm(X: np.ndarray, g: np.ndarray):
    """RMS-normalised activations ([B158] section 2; the normalisation of the
    reference it cites), fp32 [M][K], and the per-token reciprocal r [M].

    ms = fl32(exact mean of x^2);  d = fl32(sqrt(fl32(ms + eps)));  r = fl32(1 / d);
    y_k = fl32(fl32(x_k r) g_k).
    """
    X = np.ascontiguousarray(X, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    ms = mean_square(X)
    d = np.sqrt(ms + EPS)                                # fp32 add, correctly rounded fp32 sqrt
    r = np.float32(1.0) / d                              # correctly rounded fp32 division
    Y = (X * r[:, None]) * g[None, :]                    # two fp32 multiplies per element
    return Y.astype(np.float32), r.astype(np.float32)


# --------------------------------------------------------------------------
# Activation quantisation: per-token absmax to int8
# --------------------------------------------------------------------------
def act_qmax(bits: int) -> int:
    """Q_b - 1 for b-bit symmetric activations: Q_b = 2^(b - 1) levels per sign
    ([B158] section 2 gives it for b = 8; b = 4 is the "A4" of the W1A4KV2
    combination named by "The End of Matrix Multiplications: Welcome to
    Addition", which prints no quantiser of its own)."""
    if bits not in (4, 8):
        raise ValueError("activation bits must be 8 or 4")
    return 2 ** (bits - 1) - 1


def quantize_activations(X: np.ndarray, bits: int = 8):
    """Per-token absmax quantisation ([B158] section 2, absmax scaling), b = 8
    (int8) by default or b = 4 (values in [-7, 7], still one per byte).

    beta_m = max_k |X_mk|;  X~_mk = RoundClip(X_mk * (Qm / (beta_m + eps)), -Qm, Qm),
    Qm = 2^(b-1) - 1.  Returns (X~ int8 [M][K], x_scale fp32 [M] = beta/Qm,
    x_sum int64 [M], beta fp32 [M]).
    """
    qm = act_qmax(bits)
    X = np.ascontiguousarray(X, dtype=np.float32)
    beta = np.abs(X).max(axis=1) if X.shape[1] else np.zeros(X.shape[0], np.float32)
    inv = np.float32(qm) / (beta + EPS)               # fp32 add, fp32 divide
    q = X * inv[:, None]                              # one fp32 multiply per element
    Xq = round_clip(q, -qm, qm).astype(np.int8)
    x_scale = beta / np.float32(qm)                   # fp32 divide
    x_sum = Xq.astype(np.int64).sum(axis=1)
    return Xq, x_scale.astype(np.float32), x_sum, beta.astype(np.float32)


# --------------------------------------------------------------------------
# Integer accumulation  X~ W~^T  (add/subtract only)
# --------------------------------------------------------------------------
def integer_matmul(Wt: np.ndarray, Xq: np.ndarray) -> np.ndarray:
    """acc[m][n] = sum_k W~[n][k] X~[m][k]  ([B158] section 2, linear transformation).

    Computed with a float64 library product: every term is in [-127, 127] and
    every partial sum an integer of magnitude <= 127 K < 2^53, so the result is
    exact whatever order the library adds in.
    """
    K = Wt.shape[1]
    assert K * QMAX < 2 ** 53
    acc = Xq.astype(np.float64) @ Wt.astype(np.float64).T
    return acc.astype(np.int64)


def integer_matmul_loops(Wt: np.ndarray, Xq: np.ndarray) -> np.ndarray:
    """Same sum by explicit Python-integer loops (tiny shapes only)."""
    M, K = Xq.shape
    N = Wt.shape[0]
    out = np.zeros((M, N), dtype=np.int64)
    for m in range(M):
        xr = [int(v) for v in Xq[m]]
        for n in range(N):
            wr = Wt[n]
            s = 0
            for k in range(K):
                w = int(wr[k])
                if w == 1:
                    s += xr[k]
                elif w == -1:
                    s -= xr[k]
            out[m, n] = s
    return out


def masked_add_matmul(Wt: np.ndarray, Xq: np.ndarray) -> np.ndarray:
    """Same sum by the sign-mask / zero-mask route of [B158] section 6.

    For each weight that is not zero, the int8 activation is xor-ed with a sign
    mask (0 for +1, all ones for -1) and the mask subtracted, which negates it
    exactly when the weight is -1; zero weights are skipped.
    """
    M, K = Xq.shape
    N = Wt.shape[0]
    out = np.zeros((M, N), dtype=np.int64)
    sign = np.where(Wt < 0, np.int8(-1), np.int8(0)).astype(np.int8)   # [N][K]
    nonzero = Wt != 0
    for m in range(M):
        x = Xq[m].astype(np.int8)
        term = ((x[None, :] ^ sign).astype(np.int64) - sign.astype(np.int64))
        out[m] = np.where(nonzero, term, 0).sum(axis=1)
    return out


# --------------------------------------------------------------------------
# Rescale
# --------------------------------------------------------------------------
def rescale(acc: np.ndarray, gamma: np.float32, beta: np.ndarray, bits: int = 8) -> np.ndarray:
    """Y = (X~ W~^T) * beta * gamma / (Q_b - 1)  ([B158] section 2), in float64.

    beta is the per-token absmax (without epsilon).  Returns float64 [M][N].
    """
    return (acc.astype(np.float64) * np.float64(gamma)
            * np.asarray(beta, dtype=np.float64)[:, None] / act_qmax(bits))


# --------------------------------------------------------------------------
# The whole projection
# --------------------------------------------------------------------------
def bitlinear(W: np.ndarray, X: np.ndarray, bits: int = 8) -> dict:
    """Every intermediate of the projection for latent W [N][K] and X [M][K]
    (activations quantised to `bits` bits)."""
    gamma = absmean_gamma(W)
    Wt = ternarize(W, gamma)
    packed = pack_codes(Wt)
    Xq, x_scale, x_sum, beta = quantize_activations(X, bits)
    acc = integer_matmul(Wt, Xq)
    y = rescale(acc, gamma, beta, bits)
    return dict(gamma=gamma, Wt=Wt, packed=packed, Xq=Xq, x_scale=x_scale,
                x_sum=x_sum, beta=beta, acc=acc, y=y)
