"""AWQ oracle: statistics, scale search, group-wise INT4 (and its variants), W4A16 product.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain NumPy; float64
unless a step is defined in float32 / float16.

Notation follows "AWQ Math": W is [C_out, C_in] = [N, K], a token's activation
x is [C_in], the per-input-channel scale is s [C_in], N = 4 bits, groups of 128
input channels.  Readings of points the pages leave open are marked READING.
"""
from __future__ import annotations

import numpy as np

GROUP = 128        # "AWQ Math", "Shapes, granularity, and complexity": groups of (commonly) 128
NBITS = 4          # "AWQ Math", "Weight-only quantization and where it breaks": N-bit weights, N = 4
QMAX = (1 << NBITS) - 1   # READING: 2^N levels 0..15, so the step is range / 15
FIX_FRAC_BITS = 24        # READING: fixed-point LSB 2^-24 for the activation sums
M_FLOOR = 2.0 ** -14      # READING: floor on mean|x| so a dead channel cannot give s = 0
FP16_TINY = 2.0 ** -24    # smallest positive float16 (floor on the group step)


# --------------------------------------------------------------------------
# O1  calibration statistic: mean |x_j| over the calibration tokens
#     "AWQ Math", "Saliency is an activation property, not a weight property"
#     (channels are ranked by the average |x_j| over a calibration set) and
#     "Searching the scale" (s_X,j = average |x_j|); "AWQ > Limitations"
#     (the saliency metric is the average activation magnitude).
# --------------------------------------------------------------------------
def act_fixed_point_sums(x: np.ndarray) -> np.ndarray:
    """S_j = sum_t floor(|x_tj| * 2^24) as exact integers (int64).

    READING: the mean is taken exactly and rounded once.  Every float16 value is
    a multiple of 2^-24, so for float16 input the floor is exact and S_j * 2^-24
    is the exact column sum; bfloat16 magnitudes below 2^-17 lose the bits below
    2^-24 (a defined truncation).  ``x`` holds fp16/bf16 values as float32.
    """
    assert x.ndim == 2
    a = np.abs(x.astype(np.float64))
    assert np.all(np.isfinite(a)), "non-finite activations are outside the method's domain"
    assert a.size == 0 or a.max() < 2.0 ** 29, "|x| beyond the fixed-point range"
    fx = np.floor(a * 2.0 ** FIX_FRAC_BITS)
    # exact integer accumulation; Python ints never overflow
    S = np.zeros(x.shape[1], dtype=object)
    for t in range(0, x.shape[0], 4096):
        S = S + fx[t:t + 4096].astype(np.int64).sum(axis=0, dtype=np.int64).astype(object)
    return np.array([int(v) for v in S], dtype=object)


def act_mean_abs(x: np.ndarray) -> np.ndarray:
    """m_j = fp32( fp64(S_j) * 2^-24 / T ), S from ``act_fixed_point_sums``.

    Precondition (READING): S_j < 2^53, i.e. sum_t |x_tj| < 2^29, so the
    conversion to float64 is exact and the only roundings are the float64
    quotient and the final float32.
    """
    T = x.shape[0]
    S = act_fixed_point_sums(x)
    assert all(v < (1 << 53) for v in S), "column |x| sum exceeds 2^29 (fixed-point range)"
    s64 = np.array([float(v) for v in S], dtype=np.float64)
    return ((s64 * 2.0 ** -FIX_FRAC_BITS) / np.float64(T)).astype(np.float32)


# --------------------------------------------------------------------------
# O2  candidate scales  s_j = (s_X,j)^alpha
#     "AWQ Math", "Searching the scale": s_j = (s_X,j)^alpha, alpha in [0, 1];
#     alpha = 0 gives s = 1 everywhere, alpha = 1 gives s = s_X.
# --------------------------------------------------------------------------
def candidate_scales(m: np.ndarray, alphas: np.ndarray) -> np.ndarray:
    """S[i, j] = fp32( pow_fp64( max(m_j, 2^-14), alpha_i ) ).

    READING: no normalisation of s (a common power-of-two factor cancels
    exactly); the floor keeps dead channels finite.
    """
    base = np.maximum(np.asarray(m, dtype=np.float32).astype(np.float64), M_FLOOR)
    al = np.asarray(alphas, dtype=np.float64)
    return np.power(base[None, :], al[:, None]).astype(np.float32)


# --------------------------------------------------------------------------
# O3  group-wise asymmetric 4-bit round-to-nearest
#     "AWQ Math", "Weight-only quantization and where it breaks": Q(w) =
#     step * round(w / step), error up to step/2 per weight; "Shapes,
#     granularity, and complexity": groups of 128 input channels, each with
#     its own step and zero point; "AWQ > Benefits and Practical
#     Considerations": one scale and one zero point per 128 weights.
#     Variants the same passages name: other group sizes (64, 256), other bit
#     widths N, and the symmetric step max|w| / 2^(N-1) of the lead-in.
# --------------------------------------------------------------------------
def fp16_round_up(d: np.ndarray) -> np.ndarray:
    """Smallest float16 >= d (d float32, d >= 0), as float16.

    READING: the stored step is rounded toward +inf so that the top of the
    group range never needs a code above 15 (keeps the error <= step/2).
    """
    d = np.asarray(d, dtype=np.float32)
    h = d.astype(np.float16)                      # round to nearest even
    low = h.astype(np.float32) < d
    with np.errstate(over="ignore"):
        h = np.where(low, np.nextafter(h, np.float16(np.inf)), h)
    return h.astype(np.float16)


def code_max(bits: int = NBITS, symmetric: bool = False) -> int:
    """Largest stored code: 2^N - 1 for the asymmetric grid (2^N levels); 2^N
    for the symmetric one, whose codes run over -2^(N-1) .. 2^(N-1) (2^N + 1
    levels) and are stored shifted up by the zero point 2^(N-1)."""
    return (1 << bits) if symmetric else (1 << bits) - 1


def group_quant_params(wg: np.ndarray, bits: int = NBITS, symmetric: bool = False,
                       exclude: np.ndarray | None = None):
    """Step and zero point of each group.  ``wg`` float32 [..., G, group].

    Asymmetric (the default; scale and zero point per group, "AWQ > Benefits
    and Practical Considerations"):
      lo = min(0, min w'), hi = max(0, max w')          READING: range holds 0
      d  = fp32( fp32(hi - lo) / (2^N - 1) )             2^N levels, 15 intervals at N = 4
      z  = clamp( rint( fp32(-lo / D) ), 0, 2^N - 1 )    integer zero point
    Symmetric ("AWQ Math", "Weight-only quantization and where it breaks":
    step = max|w| / 2^(N-1), Q(w) = step * round(w / step)):
      d  = fp32( max|w'| / 2^(N-1) )                     exact: a power-of-two divisor
      z  = 2^(N-1)                                       codes stored shifted by z
    Both: step (fp16) = round-up(d), at least 2^-24; D = fp32(step).
    ``exclude`` (bool, broadcast against wg): weights kept in 16-bit, left out
    of the min / max (a group with none left has lo = hi = 0).
    Returns (D float32, step float16, z float32, d float32).
    """
    wg = np.asarray(wg, dtype=np.float32)
    assert np.all(np.isfinite(wg)), "non-finite weights are outside the method's domain"
    assert 2 <= bits <= (7 if symmetric else 8), "codes must fit one byte"
    ex = np.zeros(wg.shape, dtype=bool) if exclude is None else np.broadcast_to(exclude, wg.shape)
    if symmetric:
        amax = np.max(np.where(ex, np.float32(0), np.abs(wg)), axis=-1)
        d = amax / np.float32(1 << (bits - 1))
    else:
        lo = np.minimum(np.where(ex, np.float32(np.inf), wg).min(axis=-1), np.float32(0))
        hi = np.maximum(np.where(ex, np.float32(-np.inf), wg).max(axis=-1), np.float32(0))
        d = (hi - lo) / np.float32((1 << bits) - 1)
    step = fp16_round_up(np.maximum(d, np.float32(FP16_TINY)))
    assert np.all(np.isfinite(step)), "group range exceeds the float16 step range"
    D = step.astype(np.float32)
    if symmetric:
        z = np.full(D.shape, 1 << (bits - 1), dtype=np.float32)
    else:
        z = np.clip(np.rint((-lo) / D), 0, (1 << bits) - 1).astype(np.float32)
    return D, step, z, d


def quantize_codes(wg: np.ndarray, D: np.ndarray, z: np.ndarray, cmax: int = QMAX) -> np.ndarray:
    """q = clamp( rint( fp32(w' / D) ) + z, 0, cmax ) as uint8 (cmax from
    ``code_max``).  round() is round-half-to-even (READING)."""
    wg = np.asarray(wg, dtype=np.float32)
    q = np.rint(wg / D[..., None]) + z[..., None]
    return np.clip(q, 0, cmax).astype(np.uint8)


def dequantize(q: np.ndarray, D: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Grid value D * (q - z) in float64 (exact: an fp16 value times a 4-bit integer)."""
    return D.astype(np.float64)[..., None] * (q.astype(np.float64) - z.astype(np.float64)[..., None])


def scale_columns(W: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W' = W diag(s): column j (input channel j) times s_j, in W's dtype
    ("AWQ Math", "The equivalent transform: scale up W, scale down x")."""
    W = np.asarray(W)
    return W * np.asarray(s).astype(W.dtype)[None, :]


def unscale_activation(x: np.ndarray, s: np.ndarray) -> np.ndarray:
    """x' = diag(s)^-1 x for x [..., K], in float64 (same passage)."""
    return np.asarray(x, dtype=np.float64) / np.asarray(s).astype(np.float64)


def quantize_layer(W: np.ndarray, s: np.ndarray | None = None, group: int = GROUP,
                   bits: int = NBITS, symmetric: bool = False, keep: np.ndarray | None = None):
    """Quantize W' = W * diag(s) ("AWQ Math", "The equivalent transform").

    W float32 [N, K] holding fp16/bf16 values; s float32 [K] or None (s = 1,
    plain round-to-nearest).  Groups are ``group`` consecutive input channels
    of one row ("AWQ Math", "Shapes, granularity, and complexity"); ``bits`` and
    ``symmetric`` select the grid (``group_quant_params``).  Returns dict with
    codes q uint8 [N, K], step float16 [N, G], D float32 [N, G], z uint8
    [N, G], d float32 [N, G] (pre-rounding step), wp float32 [N, K] (the
    scaled weights).  ``keep`` (bool [K], optional): input channels kept in
    16-bit, left out of their groups' ranges (their codes are computed but
    not used).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % group == 0, "K must be a multiple of the group size"
    wp = W if s is None else scale_columns(W, np.asarray(s, dtype=np.float32))
    wg = wp.reshape(N, K // group, group)
    ex = None if keep is None else np.asarray(keep, dtype=bool).reshape(1, K // group, group)
    D, step, z, d = group_quant_params(wg, bits, symmetric, ex)
    q = quantize_codes(wg, D, z, code_max(bits, symmetric)).reshape(N, K)
    return {"q": q, "step": step, "D": D, "z": z.astype(np.uint8), "d": d, "wp": wp}


def pack_codes(q: np.ndarray) -> np.ndarray:
    """8 codes per int32 along K: code of k = 8c + j sits in bits [4j, 4j+4) of
    word c (READING: the plainest sequential order).  q uint8 [N, K] -> int32 [N, K/8]."""
    N, K = q.shape
    assert K % 8 == 0
    q8 = q.reshape(N, K // 8, 8).astype(np.uint32)
    word = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        word |= q8[:, :, j] << np.uint32(4 * j)
    return word.view(np.int32)


def unpack_codes(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words).view(np.uint32)
    N, C = w.shape
    out = np.empty((N, C, 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(N, C * 8)


# --------------------------------------------------------------------------
# O4/O5  scale search: loss of every candidate, then the argmin
#     "AWQ Math", "Searching the scale": alpha* = argmin || W x -
#     Q(W diag(s)) diag(s)^-1 x ||, measured as the mean squared error over
#     the calibration activations; a small grid of alpha; forward passes only.
# --------------------------------------------------------------------------
def _dequantized_weight(W: np.ndarray, s: np.ndarray, group: int = GROUP,
                        bits: int = NBITS, symmetric: bool = False,
                        keep: np.ndarray | None = None) -> np.ndarray:
    """W_hat = Q(W diag(s)) diag(s)^-1 in float64; kept channels are W itself."""
    r = quantize_layer(W, s, group, bits, symmetric, keep)
    N, K = W.shape
    G = K // group
    grid = dequantize(r["q"].reshape(N, G, group), r["D"], r["z"].astype(np.float32))
    Wh = unscale_activation(grid.reshape(N, K), np.asarray(s, dtype=np.float32))
    if keep is not None:
        Wh = np.where(np.asarray(keep, dtype=bool)[None, :], np.asarray(W, dtype=np.float64), Wh)
    return Wh


def search_losses(W: np.ndarray, X: np.ndarray, S: np.ndarray, group: int = GROUP,
                  t_chunk: int = 4096, *, bits: int = NBITS, symmetric: bool = False,
                  keep: np.ndarray | None = None) -> np.ndarray:
    """L_i = (1 / (T N)) * sum_t sum_n ( sum_k (W - W_hat_i)[n, k] x_t[k] )^2.

    READING: the objective is the mean squared error (same argmin as the norm);
    the target is the unrounded W x; W_hat_i uses the stored fp16 step, so the
    loss scores exactly what is deployed.  W float32 [N, K], X float32 [T, K],
    S float32 [n_alpha, K]; ``bits`` / ``symmetric`` select the quantizer's
    grid; ``keep`` marks channels kept in 16-bit (no error).  float64 throughout.
    """
    W = np.asarray(W, dtype=np.float32)
    X = np.asarray(X, dtype=np.float32)
    N, K = W.shape
    T = X.shape[0]
    out = np.empty(S.shape[0], dtype=np.float64)
    W64 = W.astype(np.float64)
    for i in range(S.shape[0]):
        E = W64 - _dequantized_weight(W, S[i], group, bits, symmetric, keep)
        acc = 0.0
        for t0 in range(0, T, t_chunk):
            P = X[t0:t0 + t_chunk].astype(np.float64) @ E.T
            acc += float(np.sum(P * P))
        out[i] = acc / (float(T) * float(N))
    return out


def _pow2_row_exponent(a: np.ndarray) -> np.ndarray:
    """Per row, p such that max|a_row| * 2^p < 2^14 (p = 14 - e with
    max = f 2^e, f in [0.5, 1)); 0 for an all-zero row."""
    mx = np.max(np.abs(a), axis=1).astype(np.float32)
    _, e = np.frexp(mx)
    return np.where(mx > 0, 14 - e.astype(np.int64), 0)


def _round_rows_fp16(a32: np.ndarray):
    """(fp16(a * 2^p_row) as float64, p_row): the exact power-of-two row scale
    keeps each row inside float16's normal range before rounding."""
    p = _pow2_row_exponent(a32)
    scaled = np.ldexp(a32, p[:, None].astype(np.int32)).astype(np.float32)
    return scaled.astype(np.float16).astype(np.float64), p


def search_losses_operand_model(W: np.ndarray, X: np.ndarray, S: np.ndarray,
                                x_is_fp16: bool = True, group: int = GROUP,
                                t_chunk: int = 4096, *, bits: int = NBITS,
                                symmetric: bool = False,
                                keep: np.ndarray | None = None) -> np.ndarray:
    """The same losses as ``search_losses``, scored in the precision of a
    matrix-core evaluation, so that the chosen index -- an integer decided by
    floating point -- is taken in the precision that evaluation uses.

    READING (the pages fix no precision for the search): the error of each
    weight is formed in float32 as E = W - fp32(fp32(D (q - z)) * r) with
    r = fp32(1 / s), the product with diag(s)^-1 as "AWQ Math" writes it
    ("The equivalent transform") and as the fused product applies it; each row
    of E is scaled by an exact power of two 2^p (row max below 2^14) and
    rounded to float16; calibration tokens that are not float16 already
    (bfloat16 input) get the same treatment per token; the products and sums
    are then exact (float64 here), and the scales are undone exactly.
    """
    W = np.asarray(W, dtype=np.float32)
    X = np.asarray(X, dtype=np.float32)
    N, K = W.shape
    T = X.shape[0]
    if x_is_fp16:
        Xh = X.astype(np.float64)
        assert np.array_equal(X.astype(np.float16).astype(np.float32), X)
        px = np.zeros(T, dtype=np.int64)
    else:
        Xh, px = _round_rows_fp16(X)
    out = np.empty(S.shape[0], dtype=np.float64)
    for i in range(S.shape[0]):
        s = np.asarray(S[i], dtype=np.float32)
        r = quantize_layer(W, s, group, bits, symmetric, keep)
        Dk = np.repeat(r["D"], group, axis=1)                       # float32 [N, K]
        zk = np.repeat(r["z"].astype(np.float32), group, axis=1)
        grid = Dk * (r["q"].astype(np.float32) - zk)                # exact in float32
        r = (np.float32(1) / s).astype(np.float32)                  # fp32(1 / s), IEEE division
        E32 = W - grid * r[None, :]                                 # float32 product, subtraction
        if keep is not None:
            E32 = np.where(np.asarray(keep, dtype=bool)[None, :], np.float32(0), E32)
        Eh, pe = _round_rows_fp16(E32)
        acc = 0.0
        for t0 in range(0, T, t_chunk):
            P = Xh[t0:t0 + t_chunk] @ Eh.T                          # [t, N], scaled by 2^(px + pe)
            P = np.ldexp(P, -(px[t0:t0 + t_chunk, None] + pe[None, :]).astype(np.int32))
            acc += float(np.sum(P * P))
        out[i] = acc / (float(T) * float(N))
    return out


def choose_candidate(losses: np.ndarray) -> int:
    """Lowest index among the minimal finite losses; NaN is never chosen
    (READING); all-NaN is an error."""
    L = np.asarray(losses, dtype=np.float64)
    ok = ~np.isnan(L)
    if not np.any(ok):
        raise ValueError("every candidate loss is NaN")
    best = np.min(L[ok])
    return int(np.flatnonzero(ok & (L == best))[0])


def search_scales(W: np.ndarray, X: np.ndarray, m: np.ndarray, alphas: np.ndarray,
                  group: int = GROUP, operand_model: str | None = None, *,
                  bits: int = NBITS, symmetric: bool = False, keep: np.ndarray | None = None):
    """Full search: candidate scales, losses, argmin.  Returns
    (best index, s* float32 [K], 1/s* float32 [K], losses float64 [n]).
    operand_model: None scores exactly (float64); "fp16" / "fp16-scaled-x"
    score with ``search_losses_operand_model`` (calibration tokens already
    float16, or rounded to float16 per token)."""
    S = candidate_scales(m, alphas)
    if operand_model is None:
        L = search_losses(W, X, S, group, bits=bits, symmetric=symmetric, keep=keep)
    else:
        L = search_losses_operand_model(W, X, S, operand_model == "fp16", group,
                                        bits=bits, symmetric=symmetric, keep=keep)
    i = choose_candidate(L)
    s = S[i]
    return i, s, (np.float32(1.0) / s).astype(np.float32), L


# --------------------------------------------------------------------------
# O7  fused W4A16 product
#     "AWQ > Benefits and Practical Considerations": the dequantization
#     unpacks 4-bit integers, applies the group scale and zero point, and
#     optionally the per-channel inverse scale if it was not folded into the
#     preceding layer; fused with the matrix multiply.
# --------------------------------------------------------------------------
def w4a16_matmul(x: np.ndarray, words: np.ndarray, step: np.ndarray, zeros: np.ndarray,
                 inv_s: np.ndarray | None = None, group: int = GROUP) -> np.ndarray:
    """y[m, n] = sum_k D[n, g(k)] (q[n, k] - z[n, g(k)]) x[m, k] r[k], r = inv_s or 1.

    x float32 [M, K] holding fp16/bf16 values; words int32 [N, K/8]; step
    float16 [N, G]; zeros uint8 [N, G].  Accumulated in float64.
    """
    q = unpack_codes(words)
    N, K = q.shape
    G = K // group
    Wd = dequantize(q.reshape(N, G, group), np.asarray(step).astype(np.float32),
                    np.asarray(zeros).astype(np.float32)).reshape(N, K)
    xr = np.asarray(x, dtype=np.float32).astype(np.float64)
    if inv_s is not None:
        xr = xr * np.asarray(inv_s, dtype=np.float32).astype(np.float64)[None, :]
    return xr @ Wd.T


def w4a16_matmul_rows(x, words, step, zeros, rows, inv_s=None, group: int = GROUP):
    """Same product restricted to output columns ``rows`` (output channels are
    independent), for sampled checks of large layers."""
    rows = np.asarray(rows)
    return w4a16_matmul(x, np.asarray(words)[rows], np.asarray(step)[rows],
                        np.asarray(zeros)[rows], inv_s, group)


# --------------------------------------------------------------------------
# O8  folding the activation scaling into the producer of x
#     "AWQ Math", "The equivalent transform: scale up W, scale down x": the
#     division of x_j by s_j can be folded backward into the previous layer,
#     for example the preceding LayerNorm or linear; "AWQ > Benefits and
#     Practical Considerations": the product applies 1/s only when it is not
#     already fused into the preceding layer.
#     READING: each folded value is dt(float32(v) / float32(s)) -- one IEEE
#     binary32 division, then round-to-nearest-even to the storage type.
# --------------------------------------------------------------------------
def round_bf16(a: np.ndarray) -> np.ndarray:
    """Finite float32 values rounded to bfloat16 (8 significant bits),
    nearest with ties to even, returned as float32: add half of the dropped
    low 16 bits of the binary32 pattern, plus one when the kept part is odd,
    then clear them."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    odd = (b >> 16) & 1
    r = ((b + 0x7FFF + odd) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(a))


def round_storage(a32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values rounded to the storage type ('f16', 'bf16', 'f32')."""
    a32 = np.asarray(a32, dtype=np.float32)
    if dtype == "f16":
        return a32.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        return round_bf16(a32)
    return a32


def fold_scales(v: np.ndarray, s: np.ndarray, axis: int = 1, dtype: str = "f16") -> np.ndarray:
    """v [rows, cols] float32 holding dtype values.  axis 1: column j divided
    by s[j] (a LayerNorm's gain and bias, a bias: 1 x K rows); axis 0: row i
    divided by s[i] (a preceding linear's weight [K, C_in], whose row i
    produces x_i).  Returns the folded values as float32."""
    v32 = np.asarray(v, dtype=np.float32)
    s32 = np.asarray(s, dtype=np.float32)
    q = v32 / (s32[None, :] if axis == 1 else s32[:, None])   # IEEE binary32 division
    return round_storage(q, dtype)


# --------------------------------------------------------------------------
# O9  the mixed-precision baseline AWQ replaces
#     "AWQ vs. GPTQ: Understanding Weight Quantization Principles", sections
#     on the central insight (the salient weights are those of the channels
#     with large activation magnitudes; protecting about 1 % of them greatly
#     reduces the degradation) and on per-channel scaling (keeping them in a
#     higher precision works but gives a mixed-precision model); "AWQ Math",
#     "Weight-only quantization and where it breaks" (keep the important
#     weights in FP16 and quantize the rest).
#     READING: the n_keep channels with the largest mean |x_j|, ties to the
#     lower index; they are left out of their groups' ranges and carry no
#     error (``keep`` of quantize_layer and the search losses).
# --------------------------------------------------------------------------
def salient_channels(m: np.ndarray, n_keep: int) -> np.ndarray:
    """bool [K]: True for the n_keep channels of largest m (stable order)."""
    m = np.asarray(m, dtype=np.float32)
    order = np.argsort(-m.astype(np.float64), kind="stable")
    keep = np.zeros(m.shape[0], dtype=bool)
    keep[order[:n_keep]] = True
    return keep


# --------------------------------------------------------------------------
# The pages' textbook lead-in quantizer, used only to reproduce their worked
# example: "AWQ Math", "Weight-only quantization and where it breaks"
# (Q(w) = step * round(w / step), step = max|w| / 2^(N-1)).
# --------------------------------------------------------------------------
def symmetric_rtn(w: np.ndarray, step: float) -> np.ndarray:
    w = np.asarray(w, dtype=np.float64)
    return step * np.rint(w / step)
