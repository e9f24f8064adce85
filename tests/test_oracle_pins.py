"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks an oracle function against something other than itself: a
value printed on the pages (fixtures under tests/golden/), a closed form, an
invariant, a special case that reduces to a textbook quantity, or brute force
on tiny inputs.  None of these needs a GPU.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _fp16_values(a):
    return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)


# ---------------------------------------------------------------- transform
def test_equivalent_transform_exact_in_fp64():
    """W' x' = W x in full precision ("AWQ Math", "The equivalent transform")."""
    g = _rng(1)
    for N, K in [(7, 256), (64, 512), (3, 128)]:
        W = g.standard_normal((N, K))
        x = g.standard_normal(K) * np.where(g.random(K) < 0.05, 20.0, 1.0)
        s = np.exp(g.uniform(-3, 3, K))
        y = W @ x
        y2 = O.scale_columns(W, s) @ O.unscale_activation(x, s)
        assert np.max(np.abs(y2 - y)) / np.max(np.abs(y)) <= 1e-12


def test_transform_direction_on_grid_weights():
    """Weights that sit on the 16-level grid after W diag(s) quantize without
    loss, so the search loss is zero: pins that s multiplies W's columns before
    quantizing and divides them after.  With s = 2^e the products are exact."""
    g = _rng(2)
    N, K = 4, 256
    e = g.integers(-3, 4, K)
    s = np.ldexp(np.float32(1), e).astype(np.float32)
    D = np.float32(2.0 ** -6)
    q = g.integers(0, 16, (N, K))
    q[:, ::128] = 0
    q[:, 1::128] = 15
    z = 7
    Wp = (D * (q - z)).astype(np.float32)            # on the grid, 0 at code 7
    W = (Wp / s[None, :]).astype(np.float32)
    r = O.quantize_layer(W, s)
    assert np.array_equal(r["q"], q.astype(np.uint8))
    assert np.all(r["z"] == z)
    X = g.standard_normal((5, K)).astype(np.float32)
    L = O.search_losses(W, X, s[None, :])
    assert L[0] == 0.0
    # the opposite direction (dividing the columns first) is not lossless
    L_wrong = O.search_losses(W, X, (1.0 / s)[None, :].astype(np.float32))
    assert L_wrong[0] > 0.0


# ---------------------------------------------------------------- quantizer
def _bound_ok(wp, D, q, z):
    err = np.abs(wp.astype(np.float64) - D.astype(np.float64)[..., None]
                 * (q.astype(np.float64) - z.astype(np.float64)[..., None]))
    return np.all(err <= D.astype(np.float64)[..., None] * (0.5 + 2.0 ** -18)), err


@pytest.mark.parametrize("kind", ["normal", "uniform", "outlier", "positive", "negative",
                                  "constant", "zeros", "tiny", "ties"])
def test_rounding_error_at_most_half_step(kind):
    """Per-weight error <= step/2 ("AWQ Math", "Weight-only quantization and
    where it breaks"); the fp32 division adds at most 15 * 2^-24 steps."""
    g = _rng(3)
    G = 2000
    if kind == "normal":
        w = g.standard_normal((G, 128)) * 0.02
    elif kind == "uniform":
        w = g.uniform(-1, 1, (G, 128))
    elif kind == "outlier":
        w = g.standard_normal((G, 128)) * 0.02
        w[:, 5] *= 40
    elif kind == "positive":
        w = np.abs(g.standard_normal((G, 128))) + 0.5
    elif kind == "negative":
        w = -np.abs(g.standard_normal((G, 128))) - 0.5
    elif kind == "constant":
        w = np.repeat(g.standard_normal((G, 1)), 128, axis=1)
    elif kind == "zeros":
        w = np.zeros((G, 128))
    elif kind == "tiny":
        w = g.standard_normal((G, 128)) * 1e-7
    else:  # values on half-steps of a power-of-two grid
        w = (g.integers(-30, 31, (G, 128)) + 0.5) * 2.0 ** -8
        w[:, 0] = -7.5 * 2.0 ** -6
        w[:, 1] = 7.5 * 2.0 ** -6
    wp = _fp16_values(w)
    D, step, z, d = O.group_quant_params(wp)
    q = O.quantize_codes(wp, D, z)
    ok, err = _bound_ok(wp, D, q, z)
    assert ok, float(np.max(err / D[..., None]))
    assert np.all(D >= d) and np.all(D >= 2.0 ** -24)


def test_round_to_nearest_step_would_break_the_bound():
    """The reading that rounds the stored step up is needed: rounding it to
    nearest instead lets the top of some ranges need code 16, which exceeds the
    half-step bound.  Pins that the oracle really rounds up."""
    g = _rng(4)
    wp = _fp16_values(g.standard_normal((20000, 128)) * 0.02)
    lo = np.minimum(wp.min(-1), 0)
    hi = np.maximum(wp.max(-1), 0)
    d = (hi - lo) / np.float32(15)
    D_rne = d.astype(np.float16).astype(np.float32)
    z = np.clip(np.rint(-lo / D_rne), 0, 15)
    q = np.clip(np.rint(wp / D_rne[:, None]) + z[:, None], 0, 15)
    err = np.abs(wp - D_rne[:, None] * (q - z[:, None])) / D_rne[:, None]
    assert err.max() > 0.5 + 1e-3
    D, _, zz, _ = O.group_quant_params(wp)
    ok, _ = _bound_ok(wp, D, O.quantize_codes(wp, D, zz), zz)
    assert ok


def test_fp16_round_up_brute_force():
    """Smallest float16 >= d, checked against the sorted list of every finite
    positive float16."""
    allh = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    g = _rng(5)
    d = np.concatenate([
        g.uniform(0, 1, 20000).astype(np.float32) * np.float32(2.0) ** g.integers(-26, 15, 20000),
        allh[g.integers(0, allh.size, 2000)],          # exact fp16 values map to themselves
        np.float32([2.0 ** -25, 2.0 ** -24, 65504.0, 1.0, 3.0e-8]),
    ]).astype(np.float32)
    got = O.fp16_round_up(d).astype(np.float32)
    idx = np.searchsorted(allh, d, side="left")
    assert np.array_equal(got, allh[idx])


def test_exactly_sixteen_levels_and_full_code_range():
    """N = 4 bits give 2^N = 16 levels; a dense sweep over a group's range hits
    every code; the group minimum maps to code 0 when the range is negative."""
    g = _rng(6)
    for _ in range(50):
        lo, hi = -g.uniform(0.1, 3), g.uniform(0.1, 3)
        wp = _fp16_values(np.linspace(lo, hi, 128))[None, :]
        D, _, z, _ = O.group_quant_params(wp)
        q = O.quantize_codes(wp, D, z)
        assert q.min() == 0 and q.max() <= 15 and q[0, np.argmin(wp)] == 0
        levels = np.unique(O.dequantize(np.arange(16, dtype=np.uint8)[None, :], D, z))
        assert levels.size == 16
        assert set(np.unique(q).tolist()) >= set(range(1, 15))


def test_codes_are_nearest_level_brute_force():
    """Every code is the level nearest to fp32(w'/D) - by exhaustive search over
    the 16 codes in exact rational arithmetic, ties to the even quotient."""
    g = _rng(7)
    wp = _fp16_values(g.standard_normal((40, 128)) * g.uniform(0.001, 2, (40, 1)))
    D, _, z, _ = O.group_quant_params(wp)
    q = O.quantize_codes(wp, D, z)
    for gi in range(wp.shape[0]):
        zz = int(z[gi])
        for k in range(0, 128, 3):
            quo = Fraction(float(np.float32(wp[gi, k]) / np.float32(D[gi])))
            best = None
            for c in range(16):
                dist = abs(quo - (c - zz))
                key = (dist, (c - zz) % 2)   # ties: even integer (c - z)
                if best is None or key < best[0]:
                    best = (key, c)
            assert q[gi, k] == best[1]


def test_zero_is_exact_and_zero_point_in_range():
    g = _rng(8)
    wp = _fp16_values(g.standard_normal((500, 128)))
    wp[:, 17] = 0.0
    D, _, z, _ = O.group_quant_params(wp)
    q = O.quantize_codes(wp, D, z)
    assert np.all(z <= 15) and np.all(z >= 0)
    assert np.all(q[:, 17] == z)


def test_mean_round_fraction_is_quarter():
    """E[RoundErr] ~ 0.25 with RoundErr in [0, 0.5] ("AWQ Math", "Why scaling
    shrinks the error that matters"; fixture worked_example.json)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    g = _rng(9)
    wp = g.uniform(-1, 1, (8000, 128)).astype(np.float32)
    D, _, z, _ = O.group_quant_params(wp)
    q = O.quantize_codes(wp, D, z)
    frac = np.abs(wp / D[:, None] - (q.astype(np.float32) - z[:, None]))
    assert frac.max() <= ex["round_fraction_range"][1] + 1e-5
    # the two extremes of each group set the grid (for symmetric data they sit
    # near half-steps); the statistic is about the weights inside the range
    inner = np.ones_like(frac, dtype=bool)
    inner[np.arange(wp.shape[0]), np.argmin(wp, 1)] = False
    inner[np.arange(wp.shape[0]), np.argmax(wp, 1)] = False
    assert abs(frac[inner].mean() - ex["mean_round_fraction"]) < 0.002


def test_worked_example():
    """The pages' worked example: 4 bits, group max 1.0 -> step 1/8; a salient
    weight 0.1 with |x| = 10 has expected output error 0.3125; scaling the
    channel by 2 (group max unchanged) gives 0.15625.  Expectations are over
    the rounding fraction, so they are checked by Monte Carlo with the pages'
    symmetric quantizer and with the oracle's code/dequantize steps at the same
    step (zero point 8)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    step = ex["group_max_abs"] / 2 ** (ex["bits"] - 1)
    assert step == ex["step"]
    assert math.isclose(step * ex["mean_round_fraction"] * ex["mean_abs_activation"], ex["err_before"])
    g = _rng(10)
    w = g.uniform(-0.25, 0.25, 2_000_000)          # weights spread over several steps
    x = ex["mean_abs_activation"]
    s = ex["scale"]
    e1 = np.mean(np.abs(O.symmetric_rtn(w, step) - w)) * x
    e2 = np.mean(np.abs(O.symmetric_rtn(w * s, step) - w * s)) * x / s
    assert abs(e1 - ex["err_before"]) / ex["err_before"] < 0.01
    assert abs(e2 - ex["err_after"]) / ex["err_after"] < 0.01
    # same expectation through the oracle's asymmetric code path at step 1/8
    D = np.full(1, step, dtype=np.float32)
    z = np.full(1, 8, dtype=np.float32)
    for sc, want in [(1.0, ex["err_before"]), (s, ex["err_after"])]:
        wp = (w * sc).astype(np.float32)[None, :]
        q = O.quantize_codes(wp, D, z)
        e = np.mean(np.abs(O.dequantize(q, D, z)[0] - wp[0])) * x / sc
        assert abs(e - want) / want < 0.01


def test_idempotent_on_dequantized_weights():
    """Re-quantizing D (q - z) returns the same step, zero point and codes when
    both end codes occur in the group."""
    g = _rng(11)
    wp = _fp16_values(g.standard_normal((3000, 128)) * 0.05)
    D, step, z, _ = O.group_quant_params(wp)
    q = O.quantize_codes(wp, D, z)
    full = (q.min(-1) == 0) & (q.max(-1) == 15)
    assert full.mean() > 0.5
    back = O.dequantize(q, D, z).astype(np.float32)
    D2, step2, z2, _ = O.group_quant_params(back)
    q2 = O.quantize_codes(back, D2, z2)
    assert np.array_equal(step2[full], step[full])
    assert np.array_equal(z2[full], z[full])
    assert np.array_equal(q2[full], q[full])


def test_power_of_two_scale_invariance():
    """s -> 2^k s leaves codes and zero points unchanged, multiplies the step by
    2^k and leaves the dequantized weights and the loss unchanged (the
    transform is exact for powers of two and the step has no over/underflow)."""
    g = _rng(12)
    N, K, T = 6, 384, 9
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    X = _fp16_values(g.standard_normal((T, K)))
    s = np.exp(g.uniform(-1, 1, K)).astype(np.float32)
    base = O.quantize_layer(W, s)
    L0 = O.search_losses(W, X, s[None, :])[0]
    for k in (-3, 3):
        s2 = (s * np.float32(2.0 ** k)).astype(np.float32)
        r = O.quantize_layer(W, s2)
        assert np.array_equal(r["q"], base["q"]) and np.array_equal(r["z"], base["z"])
        assert np.array_equal(r["D"], base["D"] * np.float32(2.0 ** k))
        assert O.search_losses(W, X, s2[None, :])[0] == L0


# ---------------------------------------------------------------- packing
def test_pack_layout_and_round_trip():
    q = np.array([[0, 1, 2, 3, 4, 5, 6, 7], [15] * 8], dtype=np.uint8)
    w = O.pack_codes(q)
    assert w.dtype == np.int32
    assert int(w[0, 0]) == 0x76543210
    assert int(w[1, 0]) == -1
    g = _rng(13)
    q = g.integers(0, 16, (37, 256)).astype(np.uint8)
    assert np.array_equal(O.unpack_codes(O.pack_codes(q)), q)


def test_storage_size_matches_pages():
    """~4x smaller than FP16 with one scale and one zero point per 128 weights
    ("AWQ > Benefits and Practical Considerations"; storage_figures.json)."""
    fx = json.load(open(os.path.join(GOLDEN, "storage_figures.json")))
    N, K = 256, 1024
    r = O.quantize_layer(np.zeros((N, K), np.float32))
    nbytes = O.pack_codes(r["q"]).nbytes + r["step"].nbytes + r["z"].nbytes
    assert nbytes == N * K // 2 + 3 * N * K // fx["group"]
    ratio = (2 * N * K) / nbytes
    assert abs(ratio - 16 / 4.1875) < 1e-12 and abs(ratio - fx["approx_reduction"]) < 0.25
    # 70B-shaped stack: 80 x (q, k, v, o, gate, up, down) of the workload
    per_layer = 8192 * 8192 * 2 + 1024 * 8192 * 2 + 28672 * 8192 * 3
    packed_gb = 80 * per_layer * (0.5 + 3 / 128) / 1e9
    assert abs(packed_gb - 35.83) < 0.01
    lo, hi = fx["models_gb"]["70B"]
    assert packed_gb < hi and 80 * per_layer * 2 / 1e9 < lo * 1.0


# ---------------------------------------------------------------- statistics
def test_mean_abs_closed_forms():
    g = _rng(14)
    T, K = 300, 40
    X = np.zeros((T, K), np.float32)
    X[:, 0] = -3.25                                  # constant column
    X[:, 1] = g.integers(-50, 51, T)                 # integer-valued column
    X[:, 2:] = _fp16_values(g.standard_normal((T, K - 2)) * 5)
    m = O.act_mean_abs(X)
    assert m[0] == np.float32(3.25)
    assert m[1] == np.float32(np.abs(X[:, 1]).astype(np.int64).sum() / T)
    for j in range(K):   # every column equals the correctly rounded sum / T
        want = np.float32(math.fsum(np.abs(X[:, j].astype(np.float64))) / T)
        assert m[j] == want


def test_mean_abs_bf16_truncation_only_below_2_pow_minus_17():
    # bf16-valued data whose magnitudes are >= 2^-17 are multiples of 2^-24: exact
    g = _rng(15)
    v = (g.standard_normal((64, 16)) * 4).astype(np.float32)
    v = (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # bf16 values
    v[np.abs(v) < 2.0 ** -17] = 0
    m = O.act_mean_abs(v)
    for j in range(16):
        assert m[j] == np.float32(math.fsum(np.abs(v[:, j].astype(np.float64))) / 64)
    tiny = np.full((4, 1), 2.0 ** -30, np.float32)
    assert O.act_mean_abs(tiny)[0] == 0.0
    # below 2^-24 the fixed point truncates (toward zero), it does not round
    frac = np.full((8, 1), 1.5 * 2.0 ** -25, np.float32)      # 0.75 LSB
    assert O.act_mean_abs(frac)[0] == 0.0
    assert O.act_fixed_point_sums(np.full((8, 1), 1.75 * 2.0 ** -24, np.float32))[0] == 8


# ---------------------------------------------------------------- scales
def test_candidate_scale_special_cases():
    """alpha = 0 gives s = 1 (plain quantization); alpha = 1 gives s = s_X
    ("AWQ Math", "Searching the scale")."""
    g = _rng(16)
    m = np.abs(g.standard_normal(300)).astype(np.float32)
    m[:3] = [0.0, 1e-9, 2.0 ** -14]
    S = O.candidate_scales(m, np.array([0.0, 1.0, 0.5]))
    assert np.all(S[0] == 1.0)
    assert np.array_equal(S[1], np.maximum(m, np.float32(2.0 ** -14)))
    assert np.array_equal(S[2], np.sqrt(np.maximum(m, 2.0 ** -14).astype(np.float64)).astype(np.float32))
    r1 = O.quantize_layer(_fp16_values(g.standard_normal((4, 256))), S[0, :256])
    r0 = O.quantize_layer(_fp16_values(g.standard_normal((4, 256))) * 0 + r1["wp"], None)
    assert np.array_equal(r0["q"], r1["q"])


# ---------------------------------------------------------------- loss + search
def _loss_by_loops(W, X, s):
    """Independent tiny-size loss: for each token, the layer output W x and the
    quantized layer's output computed as Q(W diag(s)) (diag(s)^-1 x), each
    with explicit Python loops over the unpacked codes; squared difference
    averaged over tokens and outputs."""
    N, K = W.shape
    r = O.quantize_layer(W, s)
    q, D, z = r["q"], r["D"], r["z"]
    tot = 0.0
    for t in range(X.shape[0]):
        xs = [float(X[t, k]) / float(s[k]) for k in range(K)]
        for n in range(N):
            y = math.fsum(float(W[n, k]) * float(X[t, k]) for k in range(K))
            yq = math.fsum(float(D[n, k // 128]) * (int(q[n, k]) - int(z[n, k // 128])) * xs[k]
                           for k in range(K))
            tot += (y - yq) ** 2
    return tot / (X.shape[0] * N)


def _fp32_correctly_rounded(v):
    """The float32 nearest to the Decimal v > 0 (ties: even), and the distance
    from v to the nearest float32 rounding boundary relative to v."""
    import decimal
    c = np.float32(float(v))
    cands = {c, np.nextafter(c, np.float32(np.inf)), np.nextafter(c, np.float32(0))}
    # neighbours of every candidate, so that the bracketing pair is present
    cands |= {np.nextafter(x, np.float32(np.inf)) for x in list(cands)}
    cands |= {np.nextafter(x, np.float32(0)) for x in list(cands)}
    ordered = sorted(cands, key=lambda x: (abs(decimal.Decimal(float(x)) - v), int(np.array(x).view(np.uint32)) & 1))
    best = ordered[0]
    lo = max((x for x in cands if decimal.Decimal(float(x)) <= v), key=lambda x: float(x))
    hi = min((x for x in cands if decimal.Decimal(float(x)) >= v), key=lambda x: float(x))
    mid = (decimal.Decimal(float(lo)) + decimal.Decimal(float(hi))) / 2
    margin = abs(v - mid) / v if lo != hi else decimal.Decimal(1)
    return best, margin


def test_candidate_scales_against_decimal_powers():
    """s = fp32(max(m, 2^-14)^alpha) at every alpha = i / 19 (the grid of the
    workloads) against m^alpha = exp(alpha ln m) evaluated in 50-digit decimal
    arithmetic, independent of the float64 pow the oracle uses: bit-exact
    after correct rounding to float32, except where the exact power lies
    within 2^-40 (relative) of a float32 rounding boundary, where a correctly
    rounded float64 result may legitimately fall on either side."""
    import decimal
    ctx = decimal.Context(prec=50)
    g = _rng(161)
    m = np.concatenate([np.abs(g.standard_normal(40)) * 3, np.exp(g.uniform(-12, 4, 40)),
                        [0.0, 1e-9, 2.0 ** -14, 1.0, 2.0, 0.5, 20.0]]).astype(np.float32)
    alphas = np.arange(20, dtype=np.float64) / np.float64(19)
    S = O.candidate_scales(m, alphas)
    checked = skipped = 0
    for j, mj in enumerate(m):
        base = decimal.Decimal(float(max(np.float64(mj), 2.0 ** -14)))
        ln = base.ln(ctx)
        for i, a in enumerate(alphas):
            v = (decimal.Decimal(float(a)) * ln).exp(ctx)          # alpha exactly as stored in float64
            want, margin = _fp32_correctly_rounded(v)
            if margin < decimal.Decimal(2) ** -40:
                skipped += 1
                continue
            assert S[i, j] == want, (j, i, float(mj), float(a), S[i, j], want)
            checked += 1
    assert checked >= 0.99 * len(m) * len(alphas) and skipped <= 2
    # a float32 pow, or a product in place of the power, fails this pin
    bad = np.power(np.maximum(m, np.float32(2.0 ** -14))[None, :], alphas.astype(np.float32)[:, None])
    assert not np.array_equal(bad.astype(np.float32), S)


def test_search_loss_against_loops_and_gram_form():
    g = _rng(17)
    N, K, T = 3, 256, 6
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    X = _fp16_values(g.standard_normal((T, K)) * np.where(np.arange(K) % 50 == 3, 20, 1))
    m = O.act_mean_abs(X)
    alphas = np.arange(20) / 19.0
    S = O.candidate_scales(m, alphas)
    L = O.search_losses(W, X, S)
    for i in (0, 7, 19):
        ref = _loss_by_loops(W, X, S[i])
        assert abs(L[i] - ref) <= 1e-9 * ref
    # Gram form: sum_n e_n^T (X^T X) e_n -- the same sum regrouped
    for i in (3, 11):
        r = O.quantize_layer(W, S[i])
        grid = r["D"].astype(np.float64).repeat(128, 1) * (r["q"].astype(np.float64)
                                                            - r["z"].astype(np.float64).repeat(128, 1))
        E = W.astype(np.float64) - grid / S[i].astype(np.float64)
        Gm = X.astype(np.float64).T @ X.astype(np.float64)
        ref = np.einsum("nk,kl,nl->", E, Gm, E) / (T * N)
        assert abs(L[i] - ref) <= 1e-10 * ref


def test_search_loss_identity_calibration_is_frobenius():
    """With X = I (each token activates one channel) the loss is ||E||_F^2 / (T N)."""
    g = _rng(18)
    N, K = 5, 128
    W = _fp16_values(g.standard_normal((N, K)) * 0.1)
    X = np.eye(K, dtype=np.float32)
    r = O.quantize_layer(W, None)
    E = W.astype(np.float64) - O.dequantize(r["q"].reshape(N, 1, K), r["D"],
                                            r["z"].astype(np.float32)).reshape(N, K)
    L = O.search_losses(W, X, np.ones((1, K), np.float32))
    assert abs(L[0] - np.sum(E * E) / (K * N)) <= 1e-14


def test_search_tiny_layers_brute_force():
    """Search on tiny layers: the chosen index is the minimum of the loss vector
    (lowest index on ties), never worse than alpha = 0 (plain round-to-nearest),
    and a brute-force per-channel scale over the boosted channels can only do
    as well or better than the one-knob family."""
    for seed in range(4):
        g = _rng(100 + seed)
        K = 128 * (1 + seed % 2)
        N, T = 2 + seed % 3, 8 + 4 * seed
        b = np.ones(K, np.float32)
        boosted = g.choice(K, 2, replace=False)
        b[boosted] = 20.0
        W = _fp16_values(g.standard_normal((N, K)) * 0.02)
        X = _fp16_values(g.standard_normal((T, K)) * b)
        m = O.act_mean_abs(X)
        alphas = np.arange(20) / 19.0
        i, s, inv, L = O.search_scales(W, X, m, alphas)
        assert L[i] == np.min(L) and np.all(L[:i] > L[i])
        assert L[i] <= L[0]
        assert np.array_equal(s, O.candidate_scales(m, alphas)[i])
        assert np.array_equal(inv, (np.float32(1) / s).astype(np.float32))
        cands = []
        for a in (1, 2, 4, 8):
            for c in (1, 2, 4, 8):
                v = np.ones(K, np.float32)
                v[boosted[0]], v[boosted[1]] = a, c
                cands.append(v)
        Lb = O.search_losses(W, X, np.array(cands))
        assert np.min(Lb) <= L[0]          # s = 1 is in the brute-force set


def test_argmin_ties_and_nan():
    assert O.choose_candidate(np.array([3.0, 1.0, 1.0, 2.0])) == 1
    assert O.choose_candidate(np.array([np.nan, 5.0, np.nan, 4.0])) == 3
    with pytest.raises(ValueError):
        O.choose_candidate(np.array([np.nan, np.nan]))


# ---------------------------------------------------------------- W4A16 product
def test_w4a16_special_cases():
    g = _rng(19)
    N, K = 9, 384
    q = g.integers(0, 16, (N, K)).astype(np.uint8)
    step = _fp16_values(g.uniform(1e-3, 1e-1, (N, K // 128))).astype(np.float16)
    z = g.integers(0, 16, (N, K // 128)).astype(np.uint8)
    words = O.pack_codes(q)
    # q == z everywhere -> y == 0 exactly
    qz = np.repeat(z, 128, axis=1)
    x = _fp16_values(g.standard_normal((3, K)))
    assert np.all(O.w4a16_matmul(x, O.pack_codes(qz), step, z) == 0.0)
    # one-hot x picks one dequantized column exactly
    for k in (0, 129, 383):
        e = np.zeros((1, K), np.float32)
        e[0, k] = 1.0
        y = O.w4a16_matmul(e, words, step, z)[0]
        want = step[:, k // 128].astype(np.float64) * (q[:, k].astype(np.float64) - z[:, k // 128])
        assert np.array_equal(y, want)


def test_w4a16_equals_quantized_layer_times_scaled_input():
    """The fused product over the packed format equals the quantized layer
    Q(W diag(s)) applied to diag(s)^-1 x, rebuilt from the unpacked codes."""
    g = _rng(20)
    N, K, M = 12, 512, 4
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    s = np.exp(g.uniform(-2, 2, K)).astype(np.float32)
    r = O.quantize_layer(W, s)
    words = O.pack_codes(r["q"])
    x = _fp16_values(g.standard_normal((M, K)))
    inv = (np.float32(1) / s).astype(np.float32)
    y = O.w4a16_matmul(x, words, r["step"], r["z"], inv)
    Wq = np.zeros((N, K))
    for n in range(N):
        for k in range(K):
            Wq[n, k] = float(r["step"][n, k // 128]) * (int(r["q"][n, k]) - int(r["z"][n, k // 128]))
    ref = (x.astype(np.float64) * inv.astype(np.float64)) @ Wq.T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    rows = np.array([0, 5, 11])
    assert np.allclose(O.w4a16_matmul_rows(x, words, r["step"], r["z"], rows, inv), y[:, rows],
                       rtol=0, atol=1e-15)
    # with s = 1 it approximates the unquantized layer W x within the 4-bit error
    r1 = O.quantize_layer(W, None)
    y1 = O.w4a16_matmul(x, O.pack_codes(r1["q"]), r1["step"], r1["z"])
    yw = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.max(np.abs(y1 - yw)) < 0.25 * np.max(np.abs(yw))


# ---------------------------------------------------------------- scoring precision model
def test_operand_model_within_rounding_bound_of_exact():
    """Scoring with fp16-rounded errors stays within the rounding bound of the
    exact loss (fp16 unit roundoff 2^-11 on E, plus the float32 formation of
    E), on tiny layers with outlier channels."""
    g = _rng(30)
    for seed in range(3):
        N, K, T = 3 + seed, 256, 9 + seed
        W = _fp16_values(g.standard_normal((N, K)) * 0.02)
        X = _fp16_values(g.standard_normal((T, K)) * np.where(np.arange(K) % 37 == 1, 20, 1))
        S = O.candidate_scales(O.act_mean_abs(X), np.arange(20) / 19.0)
        Lm = O.search_losses_operand_model(W, X, S)
        Le = O.search_losses(W, X, S)
        for i in range(20):
            r = O.quantize_layer(W, S[i])
            grid = O.dequantize(r["q"].reshape(N, 2, 128), r["D"], r["z"].astype(np.float32)).reshape(N, K)
            Wh = O.unscale_activation(grid, S[i])
            E = W.astype(np.float64) - Wh
            A = np.abs(E) @ np.abs(X.astype(np.float64)).T
            C = (np.abs(W) + np.abs(Wh)) @ np.abs(X.astype(np.float64)).T
            B = 2.0 ** -11 * A + 2.0 ** -22 * C
            P = E @ X.astype(np.float64).T
            bound = np.sum(2 * np.abs(P) * B + B * B) / (T * N)
            assert abs(Lm[i] - Le[i]) <= bound


def test_operand_model_exact_when_errors_are_representable():
    """With s = 1 and weights on a coarse dyadic grid the errors have few
    significant bits, so rounding them to fp16 changes nothing."""
    g = _rng(31)
    N, K, T = 4, 256, 7
    W = (g.integers(-40, 41, (N, K)) * 2.0 ** -9).astype(np.float32)
    W[:, 0], W[:, 128] = -40 * 2.0 ** -9, 40 * 2.0 ** -9
    X = _fp16_values(g.standard_normal((T, K)))
    S = np.ones((1, K), np.float32)
    assert O.search_losses_operand_model(W, X, S)[0] == O.search_losses(W, X, S)[0]


def test_operand_model_token_scaling_is_exact_for_fp16_tokens():
    """Per-token power-of-two scaling then fp16 rounding is exact for tokens
    that are already fp16 values of moderate range, so both token treatments
    score identically; bf16-valued tokens also convert exactly."""
    g = _rng(32)
    N, K, T = 5, 384, 11
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    X = _fp16_values(g.standard_normal((T, K)) * 3)
    S = O.candidate_scales(O.act_mean_abs(X), np.array([0.0, 0.5, 1.0]))
    a = O.search_losses_operand_model(W, X, S, x_is_fp16=True)
    b = O.search_losses_operand_model(W, X, S, x_is_fp16=False)
    assert np.array_equal(a, b)
    Xb = (X.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # bf16 values
    c = O.search_losses_operand_model(W, Xb, S, x_is_fp16=False)
    d = O.search_losses_operand_model(W, Xb.astype(np.float16).astype(np.float32), S, x_is_fp16=True)
    assert np.array_equal(c, d)


def test_operand_model_row_exponent():
    from oracle.awq import _pow2_row_exponent
    a = np.array([[0.75, -3.0], [0.0, 0.0], [2.0 ** -30, 1e-31], [40000.0, 1.0]], np.float32)
    p = _pow2_row_exponent(a)
    for row, pi in zip(a, p):
        mx = np.max(np.abs(row))
        if mx == 0:
            assert pi == 0
        else:
            assert 2.0 ** 13 <= mx * 2.0 ** pi < 2.0 ** 14


# ---------------------------------------------------------------------------
# O8  folding 1/s into the producer of x ("AWQ Math", "The equivalent
# transform: scale up W, scale down x")
# ---------------------------------------------------------------------------
def test_round_bf16_matches_library_cast_including_ties():
    """bfloat16 rounding against torch's float -> bfloat16 cast (a library
    routine the oracle does not use), with exact ties in both directions."""
    torch = pytest.importorskip("torch")
    g = np.random.Generator(np.random.PCG64(80))
    a = (g.standard_normal(20000) * np.exp(g.uniform(-20, 20, 20000))).astype(np.float32)
    bits = g.integers(0, 1 << 16, 2000).astype(np.uint32) << 16
    ties = (bits | 0x8000).view(np.float32)                       # exactly halfway
    ties = ties[np.isfinite(ties)]
    for v in (a, ties):
        want = torch.from_numpy(v.copy()).to(torch.bfloat16).float().numpy()
        assert np.array_equal(O.round_bf16(v).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_fold_by_powers_of_two_and_one_is_exact(dtype):
    g = np.random.Generator(np.random.PCG64(81))
    v = O.round_storage(g.uniform(-4, 4, (3, 256)).astype(np.float32), dtype)
    s = (2.0 ** g.integers(-3, 4, 256)).astype(np.float32)
    assert np.array_equal(O.fold_scales(v, s, 1, dtype), (v / s[None, :]).astype(np.float32))
    assert np.array_equal(O.fold_scales(v, np.ones(256, np.float32), 1, dtype), v)
    s0 = (2.0 ** g.integers(-3, 4, 3)).astype(np.float32)
    assert np.array_equal(O.fold_scales(v, s0, 0, dtype), (v / s0[:, None]).astype(np.float32))


@pytest.mark.parametrize("dtype,u", [("f16", 2.0 ** -11), ("bf16", 2.0 ** -8), ("f32", 2.0 ** -24)])
def test_fold_gives_the_scaled_activation(dtype, u):
    """The fold reproduces x / s through the producer of x, in fp64 up to the
    rounding of the folded values: a LayerNorm x = n * gamma + beta (gain and
    bias folded along axis 1) and a preceding linear x = W_prev u (rows of
    W_prev folded along axis 0)."""
    g = np.random.Generator(np.random.PCG64(82))
    K, C = 384, 200
    s = np.exp(g.uniform(-2, 2, K)).astype(np.float32)
    n = g.standard_normal(K)
    gamma = O.round_storage(g.uniform(0.5, 1.5, K).astype(np.float32), dtype)
    beta = O.round_storage(g.uniform(-0.2, 0.2, K).astype(np.float32), dtype)
    gf = O.fold_scales(gamma[None, :], s, 1, dtype)[0].astype(np.float64)
    bf = O.fold_scales(beta[None, :], s, 1, dtype)[0].astype(np.float64)
    x = n * gamma + beta
    xf = n * gf + bf
    bound = (u + 2.0 ** -24) * 1.01 * (np.abs(n * gamma) + np.abs(beta)) / s
    assert np.all(np.abs(xf - x / s) <= bound)
    W = O.round_storage(g.standard_normal((K, C)).astype(np.float32) * 0.05, dtype)
    uu = g.standard_normal(C)
    Wf = O.fold_scales(W, s, 0, dtype).astype(np.float64)
    y = W.astype(np.float64) @ uu
    yf = Wf @ uu
    bound = (u + 2.0 ** -24) * 1.01 * (np.abs(W.astype(np.float64)) @ np.abs(uu)) / s
    assert np.all(np.abs(yf - y / s) <= bound)
    # dividing columns instead of rows gives something else
    assert not np.allclose(O.fold_scales(W, s[:C], 1, dtype), Wf)



# ------------------------------------------------------- quantizer variants
def _nearest_code_brute(quo, zz, cmax):
    """Code c in 0..cmax whose level c - z is nearest to the rational quo,
    ties to the even integer c - z."""
    best = None
    for c in range(cmax + 1):
        key = (abs(quo - (c - zz)), (c - zz) % 2)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_symmetric_step_is_the_worked_example():
    """The symmetric variant reproduces the pages' worked example: 4 bits and a
    group whose largest magnitude is 1.0 give the step 1/8 (zero point 8,
    codes -8 .. 8 around it); through the whole layer quantizer, a channel with
    |x| = 10 then carries output error 0.3125, and scaling it by 2 (group
    maximum unchanged) gives 0.15625 ("AWQ Math", "A worked numeric example";
    fixture worked_example.json)."""
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    g = _rng(60)
    R, grp = 4000, 128
    W = g.uniform(-0.25, 0.25, (R, 2 * grp)).astype(np.float32)
    W[:, 0] = ex["group_max_abs"]                 # each group's largest magnitude
    W[:, grp] = -ex["group_max_abs"]
    for sc, want in [(1.0, ex["err_before"]), (ex["scale"], ex["err_after"])]:
        s = np.full(2 * grp, sc, np.float32)
        s[0] = s[grp] = 1.0                        # the maxima stay where they are
        r = O.quantize_layer(W, s, grp, bits=ex["bits"], symmetric=True)
        assert np.all(r["D"] == ex["step"]) and np.all(r["z"] == 8)
        assert np.all(r["q"][:, 0] == 16) and np.all(r["q"][:, grp] == 0)
        Wh = O.dequantize(r["q"].reshape(R, 2, grp), r["D"], r["z"].astype(np.float32)).reshape(R, -1)
        e = np.abs(Wh - r["wp"].astype(np.float64))[:, np.r_[1:grp, grp + 1:2 * grp]]
        got = e.mean() * ex["mean_abs_activation"] / sc
        assert abs(got - want) / want < 0.01


@pytest.mark.parametrize("bits", [2, 3, 5, 7])
def test_symmetric_levels_brute_force(bits):
    """Symmetric grid: 2^N + 1 levels D (q - 2^(N-1)), the group's extreme
    magnitude maps to the end code when max|w| / 2^(N-1) is an fp16 value, and
    every code is the nearest level (exhaustive, exact rationals)."""
    g = _rng(61 + bits)
    half = 1 << (bits - 1)
    cmax = O.code_max(bits, True)
    assert cmax == 2 * half
    wp = _fp16_values(g.standard_normal((30, 128)) * g.uniform(0.01, 2, (30, 1)))
    D, _, z, d = O.group_quant_params(wp, bits, True)
    assert np.all(z == half) and np.all(D >= d)
    q = O.quantize_codes(wp, D, z, cmax)
    assert q.max() <= cmax
    ok, _ = _bound_ok(wp, D, q, z)
    assert ok
    for gi in range(wp.shape[0]):
        for k in range(0, 128, 5):
            quo = Fraction(float(np.float32(wp[gi, k]) / np.float32(D[gi])))
            assert q[gi, k] == _nearest_code_brute(quo, half, cmax)
    # a power-of-two maximum: the step is exact and the extremes use both ends
    v = np.linspace(-1, 1, 1025).astype(np.float32)[None, :]
    Dv, _, zv, _ = O.group_quant_params(v, bits, True)
    qv = O.quantize_codes(v, Dv, zv, cmax)
    assert Dv[0] == np.float32(1.0 / half) and qv[0, 0] == 0 and qv[0, -1] == cmax
    assert np.unique(qv).size == cmax + 1


@pytest.mark.parametrize("bits", [2, 3, 5, 8])
def test_asymmetric_bits_levels_bound_and_nearest(bits):
    """N-bit asymmetric grid: 2^N levels, a dense sweep reaches both end codes,
    the half-step bound holds, and codes are the nearest level."""
    g = _rng(70 + bits)
    cmax = O.code_max(bits, False)
    assert cmax == (1 << bits) - 1
    for _ in range(20):
        lo, hi = -g.uniform(0.1, 3), g.uniform(0.1, 3)
        wp = _fp16_values(np.linspace(lo, hi, 128))[None, :]
        D, _, z, _ = O.group_quant_params(wp, bits)
        q = O.quantize_codes(wp, D, z, cmax)
        assert q[0, 0] == 0 and q.max() <= cmax and q.max() >= cmax - 1
        levels = np.unique(O.dequantize(np.arange(cmax + 1, dtype=np.uint8)[None, :], D, z))
        assert levels.size == cmax + 1
    wp = _fp16_values(g.standard_normal((40, 128)) * g.uniform(0.001, 2, (40, 1)))
    D, _, z, d = O.group_quant_params(wp, bits)
    assert np.all(D >= d) and np.all(z <= cmax)
    q = O.quantize_codes(wp, D, z, cmax)
    ok, _ = _bound_ok(wp, D, q, z)
    assert ok
    for gi in range(0, 40, 3):
        for k in range(0, 128, 7):
            quo = Fraction(float(np.float32(wp[gi, k]) / np.float32(D[gi])))
            assert q[gi, k] == _nearest_code_brute(quo, int(z[gi]), cmax)


@pytest.mark.parametrize("group", [64, 256])
def test_group_size_slices_and_wider_step(group):
    """Group g of row n is input channels [g * group, (g + 1) * group) of that
    row, quantized on its own ("AWQ Math", "Shapes, granularity, and
    complexity"); checked slice by slice with explicit indexing.  A group of
    256 never has a smaller step than either of its 128-halves, and the same
    step when both halves span the same range ("CPU-SLM implications and
    common pitfalls": larger groups widen the step)."""
    g = _rng(80 + group)
    N, K = 5, 1024
    W = _fp16_values(g.standard_normal((N, K)) * 0.03)
    W[:, 7] *= 30
    s = np.exp(g.uniform(-1, 1, K)).astype(np.float32)
    r = O.quantize_layer(W, s, group)
    wp = O.scale_columns(W, s)
    for n in range(N):
        for gi in range(K // group):
            sl = wp[n, gi * group:(gi + 1) * group][None, :]
            D, step, z, _ = O.group_quant_params(sl)
            assert r["D"][n, gi] == D[0] and r["z"][n, gi] == z[0]
            assert np.array_equal(r["q"][n, gi * group:(gi + 1) * group], O.quantize_codes(sl, D, z)[0])
    if group == 256:
        r128 = O.quantize_layer(W, s, 128)
        assert np.all(r["D"] >= np.maximum(r128["D"][:, 0::2], r128["D"][:, 1::2]))
        V = W.copy()
        V[:, 128:256] = V[:, 0:128][:, ::-1]       # second half: same values, same range
        ra, rb = O.quantize_layer(V, None, 256), O.quantize_layer(V, None, 128)
        assert np.array_equal(ra["D"][:, 0], rb["D"][:, 0]) and np.array_equal(rb["D"][:, 0], rb["D"][:, 1])


def _loss_by_loops_q(W, X, s, group, bits, symmetric):
    """Like the loop loss above, for any group size and grid."""
    N, K = W.shape
    r = O.quantize_layer(W, s, group, bits, symmetric)
    q, D, z = r["q"], r["D"], r["z"]
    tot = 0.0
    for t in range(X.shape[0]):
        xs = [float(X[t, k]) / float(s[k]) for k in range(K)]
        for n in range(N):
            y = math.fsum(float(W[n, k]) * float(X[t, k]) for k in range(K))
            yq = math.fsum(float(D[n, k // group]) * (int(q[n, k]) - int(z[n, k // group])) * xs[k]
                           for k in range(K))
            tot += (y - yq) ** 2
    return tot / (X.shape[0] * N)


@pytest.mark.parametrize("group,bits,symmetric", [(64, 4, False), (256, 3, False), (128, 4, True),
                                                  (64, 8, False), (128, 2, True)])
def test_search_loss_variants_against_loops(group, bits, symmetric):
    g = _rng(90 + group + bits)
    N, K, T = 3, 256, 5
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    X = _fp16_values(g.standard_normal((T, K)) * np.where(np.arange(K) % 50 == 3, 20, 1))
    S = O.candidate_scales(O.act_mean_abs(X), np.arange(20) / 19.0)
    L = O.search_losses(W, X, S, group, bits=bits, symmetric=symmetric)
    for i in (0, 9, 19):
        ref = _loss_by_loops_q(W, X, S[i], group, bits, symmetric)
        assert abs(L[i] - ref) <= 1e-9 * ref
    # more bits never give a coarser grid: the plain (s = 1) loss falls with N
    if not symmetric and bits < 8:
        L8 = O.search_losses(W, X, S[:1], group, bits=8)
        assert L8[0] < L[0]
    Lm = O.search_losses_operand_model(W, X, S, True, group, bits=bits, symmetric=symmetric)
    assert np.all(np.abs(Lm - L) <= 2e-3 * L)


# ------------------------------------------------ mixed-precision baseline
def test_salient_channels_rank_brute_force():
    """The n most salient channels by mean |x| ("AWQ vs. GPTQ", the central
    insight: saliency follows the activation magnitude), by an explicit rank
    count: rank_j = #{i: m_i > m_j} + #{i < j: m_i = m_j}, kept when rank_j < n."""
    g = _rng(120)
    for K in (128, 515, 1024):
        m = g.integers(0, 40, K).astype(np.float32) * np.float32(0.25)   # many ties
        for n in (0, 1, max(1, K // 100), K // 3, K):
            keep = O.salient_channels(m, n)
            assert keep.sum() == n
            for j in range(0, K, 7):
                rank = sum(1 for i in range(K) if m[i] > m[j] or (m[i] == m[j] and i < j))
                assert keep[j] == (rank < n)


def test_keep_all_is_lossless_and_keep_none_is_plain():
    g = _rng(121)
    N, K, T = 3, 256, 7
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    X = _fp16_values(g.standard_normal((T, K)))
    S = O.candidate_scales(O.act_mean_abs(X), np.array([0.0, 0.5]))
    assert np.all(O.search_losses(W, X, S, keep=np.ones(K, bool)) == 0.0)
    assert np.array_equal(O.search_losses(W, X, S, keep=np.zeros(K, bool)), O.search_losses(W, X, S))
    Lm = O.search_losses_operand_model(W, X, S, keep=np.ones(K, bool))
    assert np.all(Lm == 0.0)


def _loss_by_loops_keep(W, X, s, keep, group=128):
    """Loop loss with kept channels exact and every group's range taken over
    the weights left after removing the kept ones (explicit deletion)."""
    N, K = W.shape
    wp = O.scale_columns(W, s)
    tot = 0.0
    Wh = np.zeros((N, K))
    for n in range(N):
        for gi in range(K // group):
            idx = np.arange(gi * group, (gi + 1) * group)
            rest = idx[~keep[idx]]
            sub = wp[n, rest][None, :] if rest.size else np.zeros((1, 1), np.float32)
            D, _, z, _ = O.group_quant_params(sub)
            q = O.quantize_codes(wp[n, idx][None, :], D, z)[0]
            for t, k in enumerate(idx):
                Wh[n, k] = float(W[n, k]) if keep[k] else float(D[0]) * (int(q[t]) - int(z[0])) / float(s[k])
    for t in range(X.shape[0]):
        for n in range(N):
            y = math.fsum(float(W[n, k]) * float(X[t, k]) for k in range(K))
            yq = math.fsum(Wh[n, k] * float(X[t, k]) for k in range(K))
            tot += (y - yq) ** 2
    return tot / (X.shape[0] * N)


def test_keep_excludes_channels_from_the_range():
    """Kept channels carry no error and do not set their groups' steps: with
    the outlier channels kept, the steps shrink to the rest's range; the loss
    matches explicit loops; and on a layer whose boosted channels are the
    salient ones, keeping 1 % of the channels lowers the loss against plain
    round-to-nearest ("AWQ vs. GPTQ", protecting about 1 % of the salient
    weights reduces the degradation)."""
    g = _rng(122)
    N, K, T = 4, 512, 9
    W = _fp16_values(g.standard_normal((N, K)) * 0.02)
    boosted = np.array([5, 200, 301, 450, 470])
    W[:, boosted] *= 25                          # outlier weights on the boosted channels
    b = np.ones(K, np.float32)
    b[boosted] = 30.0
    X = _fp16_values(g.standard_normal((T, K)) * b)
    m = O.act_mean_abs(X)
    keep = O.salient_channels(m, len(boosted))
    assert set(np.flatnonzero(keep)) == set(boosted.tolist())
    r0 = O.quantize_layer(W, None)
    rk = O.quantize_layer(W, None, keep=keep)
    assert np.all(rk["D"] <= r0["D"]) and np.any(rk["D"] < r0["D"])
    S = O.candidate_scales(m, np.array([0.0, 0.4]))
    L = O.search_losses(W, X, S, keep=keep)
    for i in range(2):
        ref = _loss_by_loops_keep(W, X, S[i], keep)
        assert abs(L[i] - ref) <= 1e-9 * ref
    assert L[0] < O.search_losses(W, X, S[:1])[0]
