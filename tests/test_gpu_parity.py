"""GPU vs oracle parity for every step of the hot path, through the C ABI.

Sizes are small enough for the oracle to finish in seconds but span several
tiles, ragged tails and both dtypes.  Integer and byte outputs (statistics,
codes, packed words, fp16 steps, zero points, the chosen candidate and its
scales) must be bit-exact; products are held to max|err| / max|ref| <= 2e-3, where for 16-bit outputs
the output's own rounding (half an ulp) is not counted;
search losses to a bound derived from the operand rounding (gpu_util).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_util import GEMM_TOL, f32, gpu, rel_max_err
from tests.search_check import check_search_outputs

pytestmark = pytest.mark.gpu

awq = pytest.importorskip("weight_only_int4_stats_amd")
F16, BF16 = torch.float16, torch.bfloat16


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.lib()


def _act(T, K, dtype, seed, boost=20.0, tiny=False):
    x = WL.random_matrix((T, K), torch.float32, seed)
    x[:, ::97] *= boost
    if tiny:
        x[:, 1::53] *= 1e-7
    return x.to(dtype)


# ------------------------------------------------------------- statistics
@pytest.mark.parametrize("T,K,dtype,ld_pad", [
    (64, 512, F16, 0), (77, 4096, F16, 0), (64, 11008, F16, 0), (1, 128, F16, 0),
    (200, 384, BF16, 0), (1000, 8192, BF16, 0), (333, 1024, F16, 64), (96, 2048, BF16, 8),
])
def test_act_stats_bit_exact(T, K, dtype, ld_pad):
    x = _act(T, K, dtype, seed=T * 7 + K, tiny=(dtype == BF16))
    if ld_pad:
        big = torch.zeros((T, K + ld_pad), dtype=dtype)
        big[:, :K] = x
        xg = gpu(big)[:, :K]
    else:
        xg = gpu(x)
    m = awq.awq_act_stats(xg)
    torch.cuda.synchronize()
    ref = O.act_mean_abs(f32(x))
    assert np.array_equal(m.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------- quantize + pack
@pytest.mark.parametrize("N,K,dtype,with_s", [
    (512, 512, F16, False), (37, 4096, F16, True), (300, 11008, BF16, True),
    (5, 128, F16, True), (129, 1024, BF16, False), (64, 384, F16, True),
])
def test_quantize_pack_bit_exact(N, K, dtype, with_s):
    W = WL.random_matrix((N, K), torch.float32, seed=N + K, scale=0.02)
    W[:, 3::101] *= 30.0                      # outliers inside some groups
    W[0, :128] = 0.0                          # an all-zero group
    W[1, 128 % K:128 % K + 128] = 0.75        # a constant group (or row 1 start)
    W = W.to(dtype)
    s = None
    if with_s:
        g = np.random.Generator(np.random.PCG64(N * K))
        s = torch.from_numpy(np.exp(g.uniform(-2.5, 2.5, K)).astype(np.float32))
    dbg = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")
    q, sc, z = awq.awq_quantize_pack(gpu(W), None if s is None else gpu(s), scales_f32_dbg=dbg)
    torch.cuda.synchronize()
    r = O.quantize_layer(f32(W), None if s is None else s.numpy())
    assert np.array_equal(dbg.cpu().numpy().view(np.uint32), r["d"].view(np.uint32))
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), r["step"].view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), r["z"])
    assert np.array_equal(q.cpu().numpy(), O.pack_codes(r["q"]))


# ------------------------------------------------------------- W4A16 product
def _random_packed(N, K, seed, step_lo=2e-4, step_hi=4e-3):
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.integers(0, 16, (N, K)).astype(np.uint8)
    step = g.uniform(step_lo, step_hi, (N, K // 128)).astype(np.float16)
    z = g.integers(0, 16, (N, K // 128)).astype(np.uint8)
    return O.pack_codes(q), step, z


def _run_product(M, N, K, dtype, ydt, with_r, seed):
    words, step, z = _random_packed(N, K, seed)
    x = _act(M, K, dtype, seed + 1)
    r = None
    if with_r:
        g = np.random.Generator(np.random.PCG64(seed + 2))
        r = (np.float32(1) / np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)).astype(np.float32)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)),
                           out_dtype=ydt)
    torch.cuda.synchronize()
    ref = O.w4a16_matmul(f32(x), words, step, z, r)
    return f32(y), ref


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r", [
    (1, 512, 512, F16, F16, False), (1, 11008, 4096, F16, F16, True),
    (1, 1000, 11008, F16, torch.float32, True), (1, 333, 128, BF16, BF16, False),
    (1, 257, 384, F16, torch.float32, False), (2, 4096, 4096, BF16, torch.float32, True),
    (3, 700, 2048, F16, F16, True), (8, 11008, 4096, F16, F16, False),
    (8, 1024, 11008, BF16, torch.float32, True), (5, 96, 1024, F16, torch.float32, False),
    (1, 64, 28672, F16, torch.float32, True), (4, 130, 28672, BF16, BF16, False),
])
def test_gemv_parity(M, N, K, dtype, ydt, with_r):
    y, ref = _run_product(M, N, K, dtype, ydt, with_r, seed=M * 1000 + N + K)
    err = rel_max_err(y, ref, ydt)
    print(f"gemv M={M} N={N} K={K} {dtype} -> {ydt}: rel max err {err:.3e}")
    assert err <= GEMM_TOL


def _sampled_product(M, N, K, dtype, ydt, with_r, seed, group=128):
    """Random packed layer (words drawn directly), sampled output channels
    against the oracle (channels are independent)."""
    g = np.random.Generator(np.random.PCG64(seed))
    words = g.integers(-2 ** 31, 2 ** 31, (N, K // 8), dtype=np.int64).astype(np.int32)
    step = g.uniform(2e-4, 4e-3, (N, K // group)).astype(np.float16)
    z = g.integers(0, 16, (N, K // group)).astype(np.uint8)
    x = _act(M, K, dtype, seed + 1)
    r = (np.float32(1) / np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)).astype(np.float32) if with_r else None
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)),
                           out_dtype=ydt, group_size=group)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, N, max(1, N // 300)), np.arange(N - 40, N),
                                     g.integers(0, N, 100)]))
    ref = O.w4a16_matmul_rows(f32(x), words, step, z, rows, r, group)
    return rel_max_err(f32(y)[:, rows], ref, ydt), len(rows)


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r", [
    (2, 28672, 8192, BF16, BF16, True),        # per-CU skinny, 7 row tiles per block
    (3, 100000, 1024, F16, F16, True),         # 25 row tiles per block: waves run two items
    (8, 10240, 8192, F16, F16, True),          # 8 staged pieces per thread (K = 8192)
    (12, 5000, 2048, BF16, torch.float32, True),  # 3 token phases per thread
    (16, 3000, 4096, F16, F16, False),         # 16 tokens, activations fill LDS
    (5, 11008, 4096, F16, F16, True),
    (8, 2000, 16384, F16, torch.float32, True),  # activations staged in two passes
    (16, 700, 11008, BF16, BF16, False),       # ragged K slices, passes of 3712 channels
])
def test_skinny_product_parity(M, N, K, dtype, ydt, with_r):
    """2 <= M <= 16: the skinny matrix-core products."""
    err, nrow = _sampled_product(M, N, K, dtype, ydt, with_r, seed=7 * M + N + K)
    print(f"skinny M={M} N={N} K={K} {dtype} -> {ydt}: rel max err {err:.3e} on {nrow} channels")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r,group", [
    (8, 3000, 11008, F16, F16, True, 128),        # two passes of 43 units, one tile per block
    (16, 3000, 8192, BF16, torch.float32, True, 128),  # K fits the threads, not LDS: two passes
    (2, 8192, 28672, F16, F16, False, 128),       # four passes, two tiles per block
    (12, 1500, 20608, F16, torch.float32, True, 64),   # eight passes, the last one shorter
    (5, 2000, 16640, BF16, BF16, True, 256),      # groups of 256 over three passes
    (4, 63488, 8448, F16, torch.float32, True, 256),   # 16 tiles per block: one item per wave
])
def test_skinny_product_passes(M, N, K, dtype, ydt, with_r, group):
    """2..16 tokens whose activations do not fit LDS (or the block's threads)
    at once: the 2..16-token product stages them in passes of whole 128-channel
    units, and every wave runs the units of its slice that fall in the pass."""
    err, nrow = _sampled_product(M, N, K, dtype, ydt, with_r, seed=3 * M + N + K + group, group=group)
    print(f"skinny passes M={M} N={N} K={K} g={group}: rel max err {err:.3e} on {nrow} channels")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r,group", [
    (2, 40000, 8192, F16, F16, True, 128),        # two row chunks, one pass each
    (8, 20000, 8192, BF16, torch.float32, True, 64),   # two row chunks, passes, groups of 64
    (16, 17000, 16384, F16, BF16, False, 128),    # two row chunks, five passes
])
def test_skinny_product_row_chunks(M, N, K, dtype, ydt, with_r, group):
    """2..16 tokens on layers whose rows hold more steps and zero points than
    one launch of the 2..16-token product stages: it runs on row chunks, one
    launch each, writing disjoint output columns."""
    err, nrow = _sampled_product(M, N, K, dtype, ydt, with_r, seed=5 * M + N + K + group, group=group)
    print(f"skinny row chunks M={M} N={N} K={K} g={group}: rel max err {err:.3e} on {nrow} channels")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,ks", [(8, 3000, 11008, (5503, 5504, 5631, 11007)),
                                      (16, 3000, 8192, (0, 4095, 4096, 8191))])
def test_skinny_one_hot_exact_passes(M, N, K, ks):
    """One-hot tokens on either side of a pass boundary are exact on the
    staged-in-passes product too (every output equals step * (q - z))."""
    words, step, z = _random_packed(N, K, 23 + M)
    for k in ks:
        x = torch.zeros((M, K), dtype=F16)
        x[:, k] = 1.0
        y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                               gpu(torch.from_numpy(z)), out_dtype=torch.float32)
        ref = O.w4a16_matmul(f32(x), words, step, z)
        assert np.array_equal(f32(y), ref.astype(np.float32)), (M, N, K, k)


@pytest.mark.parametrize("N,K,dtype,ydt,with_r", [
    (6400, 4224, BF16, BF16, True),          # ragged second K slice (4 of 128 chunks)
    (6145, 8320, F16, torch.float32, False),  # 3 K slices, 2 staged pieces per thread
    (6200, 28672, BF16, torch.float32, True),  # 7 K slices, 4 staged pieces per thread
    (12000, 4096, F16, F16, False),
    (300, 30720, F16, F16, True),             # K beyond the row-block kernel, few rows per block
    (10240, 8192, F16, F16, True),            # 70B q|k|v fused: 2 K slices, one staged piece, rows in pairs
    (8192, 28672, BF16, torch.float32, False),  # 70B down-projection: 7 K slices, four rows in flight
])
def test_gemv_batch1_per_cu_parity(N, K, dtype, ydt, with_r):
    """Batch-1 shapes served by the one-block-per-compute-unit kernel (many
    rows, or K past the row-block kernel's staging)."""
    err, nrow = _sampled_product(1, N, K, dtype, ydt, with_r, seed=N + K)
    print(f"gemv batch 1 N={N} K={K} {dtype} -> {ydt}: rel max err {err:.3e} on {nrow} channels")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r", [
    (9, 300, 512, F16, torch.float32, False), (32, 4096, 4096, F16, F16, True),
    (100, 1000, 1024, BF16, torch.float32, True), (256, 512, 8192, BF16, BF16, False),
    (130, 257, 384, F16, torch.float32, True), (8, 64, 65536, F16, torch.float32, False),
])
def test_gemm_parity(M, N, K, dtype, ydt, with_r):
    y, ref = _run_product(M, N, K, dtype, ydt, with_r, seed=M * 1000 + N + K)
    err = rel_max_err(y, ref, ydt)
    print(f"gemm M={M} N={N} K={K} {dtype} -> {ydt}: rel max err {err:.3e}")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r", [
    (24, 3000, 4096, F16, torch.float32, True),   # 188 row blocks x 2 slices, summed; ragged rows
    (20, 4090, 2048, BF16, BF16, False),          # 256 row blocks, one slice; ragged last tile and tokens
    (17, 300, 4096, F16, torch.float32, True),    # 19 row blocks x 4 slices of 8 units, summed
])
def test_small_batch_single_tile_blocks(M, N, K, dtype, ydt, with_r):
    """17..32 tokens on layers of at most one 16-row tile per compute unit
    (one tile per block), with and without the cross-slice sum, on ragged
    rows and tokens, against the oracle."""
    y, ref = _run_product(M, N, K, dtype, ydt, with_r, seed=M * 1000 + N + K)
    err = rel_max_err(y, ref, ydt)
    print(f"small batch M={M} N={N} K={K} {dtype} -> {ydt}: rel max err {err:.3e}")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r,group", [
    (2048, 8092, 256, BF16, torch.float32, True, 128),   # 256-wide tiles only, ragged last tile
    (2000, 25000, 256, F16, BF16, False, 128),           # 768 wide + 32 half-width tiles, ragged m and n
    (2048, 28672, 128, BF16, F16, True, 128),            # the 70B up-projection's cut, K of one group
    (1100, 14000, 512, F16, torch.float32, True, 64),    # groups of 64 across the cut
    (300, 5000, 1024, BF16, BF16, False, 256),           # few tiles: half-width tiles only
])
def test_gemm_tile_widths(M, N, K, dtype, ydt, with_r, group):
    """The tiled GEMM cuts the columns into 256-wide tiles and 128-wide ones
    so that the last round of tiles on the compute units is not left half
    empty; sampled output channels on both sides of the cut and in the ragged
    tails against the oracle."""
    err, nrow = _sampled_product(M, N, K, dtype, ydt, with_r, seed=3 * M + N + K, group=group)
    print(f"gemm M={M} N={N} K={K} g={group} {dtype} -> {ydt}: rel max err {err:.3e} on {nrow} channels")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,ydt", [
    (100, 300, 1024, F16),          # half-width tiles only
    (130, 700, 512, torch.float32),
    (2048, 8092, 256, BF16),        # 256-wide tiles, ragged last tile
])
def test_gemm_unaligned_output(M, N, K, ydt):
    """The tiled GEMM into an output whose start is not 16-byte aligned (one
    element into a wider buffer): every element is stored on its own, the
    neighbours stay untouched; sampled channels against the oracle."""
    words, step, z = _random_packed_g(N, K, M + N + K, 128)
    x = _act(M, K, BF16, M + 7)
    big = torch.full((M, N + 9), 5.0, dtype=ydt, device="cuda")
    y = big[:, 1:N + 1]
    awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                       gpu(torch.from_numpy(z)), y=y)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.PCG64(N))
    rows = np.unique(np.concatenate([np.arange(0, N, max(1, N // 200)), np.arange(N - 20, N),
                                     g.integers(0, N, 50)]))
    ref = O.w4a16_matmul_rows(f32(x), words, step, z, rows, None, 128)
    assert rel_max_err(f32(y.cpu())[:, rows], ref, ydt) <= GEMM_TOL
    assert torch.all(big[:, 0] == 5.0).item() and torch.all(big[:, N + 1:] == 5.0).item()


def test_product_special_cases():
    """q == z gives 0; a one-hot x picks the dequantized column.  The GEMV
    accumulates exact int4 x activation products, so the one-hot column is
    exact there and q == z leaves only the rounding of the zero-point sum.  The
    matrix-core paths for 17 or more tokens form each operand as one fused
    step * q - fp16(step * z), so q == z leaves the rounding of fp16(step * z)
    (at most 2^-11 of it) and, with power-of-two steps (step * z exact in
    fp16), everything is exact.  The 2..16-token product multiplies the codes
    themselves and applies step and zero point in fp32, so its one-hot
    columns are exact with any step."""
    N, K = 200, 1024
    words, step, z = _random_packed(N, K, 5)
    qz = np.repeat(z, 128, axis=1)
    x = _act(40, K, F16, 6)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(O.pack_codes(qz))),
                           gpu(torch.from_numpy(step)), gpu(torch.from_numpy(z)),
                           out_dtype=torch.float32)
    zd = step.astype(np.float64) * z.astype(np.float64)                      # [N, G]
    bound = 2.0 ** -11 * np.abs(f32(x)).astype(np.float64).reshape(40, K // 128, 128).sum(-1) @ zd.T
    assert np.all(np.abs(f32(y)) <= bound * (1 + 1e-3) + 1e-30)
    pow2_step = np.ldexp(np.float16(1), np.random.Generator(np.random.PCG64(9)).integers(
        -12, -5, step.shape)).astype(np.float16)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(O.pack_codes(qz))),
                           gpu(torch.from_numpy(pow2_step)), gpu(torch.from_numpy(z)),
                           out_dtype=torch.float32)
    assert torch.count_nonzero(y).item() == 0
    y1 = awq.awq_w4a16_gemm(gpu(x[:1]), gpu(torch.from_numpy(O.pack_codes(qz))),
                            gpu(torch.from_numpy(step)), gpu(torch.from_numpy(z)),
                            out_dtype=torch.float32)
    bound = 2.0 ** -20 * 1040 * float(np.max(step.astype(np.float32))) * float(np.abs(f32(x[:1])).sum())
    assert float(y1.abs().max()) <= bound
    pow2 = np.ldexp(np.float16(1), np.random.Generator(np.random.PCG64(8)).integers(
        -12, -5, step.shape)).astype(np.float16)
    # 2..16 tokens: the zero point enters the accumulator as -z sum X and the step
    # multiplies in fp32, so a one-hot token is exact with any step
    for M, k, st in ((1, 0, step), (1, 777, step), (33, 130, pow2), (17, 1023, pow2),
                     (8, 5, step), (4, 1000, step), (16, 129, step)):
        x = torch.zeros((M, K), dtype=F16)
        x[:, k] = 1.0
        y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(st)),
                               gpu(torch.from_numpy(z)), out_dtype=torch.float32)
        ref = O.w4a16_matmul(f32(x), words, st, z)
        assert np.array_equal(f32(y), ref.astype(np.float32))


# ------------------------------------------------------------- scale search
def _check_search(W, X, dtype, n_alpha=20, group=128, bits=4, sym=False, keep=None, alphas=None):
    """Statistic bit-exact; every loss against the exact fp64 loss of the
    definition, the chosen index against its argmin, s and 1/s bit-exact
    (tests/search_check.py: tolerances, ill-posed seeds, the operand-precision
    oracle as a second check).  group / bits / sym select the quantizer
    variant; keep (bool [K]) the channels kept in 16-bit.  Returns the GPU
    losses."""
    alphas = WL.alpha_grid(n_alpha) if alphas is None else alphas
    m = awq.awq_act_stats(gpu(X))
    kept = None if keep is None else gpu(torch.from_numpy(keep.astype(np.uint8)))
    s, inv, L, best = awq.awq_search_scales(gpu(W), gpu(X), m, gpu(torch.from_numpy(alphas)), group,
                                            bits=bits, symmetric=sym, kept=kept)
    torch.cuda.synchronize()
    s, inv, L, best = s.cpu().numpy(), inv.cpu().numpy(), L.cpu().numpy(), int(best.cpu()[0])
    m_ref = O.act_mean_abs(f32(X))
    assert np.array_equal(m.cpu().numpy().view(np.uint32), m_ref.view(np.uint32))
    check_search_outputs(L, best, s, inv, f32(W), f32(X), m_ref, alphas, dtype == F16, group, bits,
                         sym, keep)
    return L


def test_search_single_linear_512():
    w = WL.workload(1)
    _check_search(WL.weight(w), WL.calibration(w), F16)


@pytest.mark.parametrize("N,K,T,dtype,ld_pad,wseed", [(300, 1024, 200, F16, 0, 300), (130, 768, 77, BF16, 0, 130),
                                                        (64, 4096, 64, F16, 0, 64), (2500, 256, 520, F16, 24, 2500),
                                                        (1100, 128, 300, BF16, 8, 1100),
                                                        (300, 256, 4096, F16, 0, 300), (200, 384, 3000, BF16, 8, 200),
                                                        (256, 1024, 8192, F16, 0, 259)])
def test_search_ragged(N, K, T, dtype, ld_pad, wseed):
    """Ragged token and row tiles; 2500 rows = 10 tiles of 256, two tile bands
    of the contraction's order, the second narrower; padded token rows.  The
    last three shapes (T well above K) take the Gram form of the loss: ragged
    token chunks, a ragged tile of G (384 = 256 + 128) and bf16 tokens.  (The
    last shape's weight seed 259: with seed 256 its two best exact losses lie
    3.2e-5 apart, too close to decide.)"""
    W = WL.random_matrix((N, K), torch.float32, seed=wseed, scale=0.02).to(dtype)
    X = gpu(_act(T, K + ld_pad, dtype, seed=T))[:, :K]     # strided view on the device
    _check_search(W, X, dtype)


def test_search_single_candidate_and_endpoints():
    """n_alpha = 1 and the endpoints: alpha = 0 gives s = 1 exactly, alpha = 1
    gives s = max(m, 2^-14) exactly."""
    w = WL.workload(1)
    W, X = gpu(WL.weight(w)), gpu(WL.calibration(w))
    m = awq.awq_act_stats(X)
    for a, want in ((0.0, None), (1.0, "m")):
        al = torch.tensor([a], dtype=torch.float64, device="cuda")
        s, inv, L, best = awq.awq_search_scales(W, X, m, al)
        torch.cuda.synchronize()
        assert int(best.cpu()[0]) == 0
        if want is None:
            assert torch.all(s == 1.0).item() and torch.all(inv == 1.0).item()
        else:
            assert torch.equal(s, torch.clamp(m, min=2.0 ** -14))


def test_quantized_layer_end_to_end_c1():
    """stats -> search -> quantize with s -> GEMV with 1/s, against the oracle
    chain on the same inputs."""
    w = WL.workload(1)
    W, X = WL.weight(w), WL.calibration(w)
    x = WL.decode_input(w, 1)
    m = awq.awq_act_stats(gpu(X))
    al = gpu(torch.from_numpy(WL.alpha_grid(20)))
    s, inv, _, _ = awq.awq_search_scales(gpu(W), gpu(X), m, al)
    q, sc, z = awq.awq_quantize_pack(gpu(W), s)
    y = awq.awq_w4a16_gemm(gpu(x), q, sc, z, inv, out_dtype=torch.float32)
    torch.cuda.synchronize()
    i_ref, s_ref, inv_ref, _ = O.search_scales(f32(W), f32(X), O.act_mean_abs(f32(X)),
                                               WL.alpha_grid(20))
    r = O.quantize_layer(f32(W), s_ref)
    words = O.pack_codes(r["q"])
    assert np.array_equal(q.cpu().numpy(), words)
    ref = O.w4a16_matmul(f32(x), words, r["step"], r["z"], inv_ref)
    assert rel_max_err(f32(y), ref) <= GEMM_TOL
    # and the quantized layer tracks the unquantized one
    yw = f32(x).astype(np.float64) @ f32(W).astype(np.float64).T
    assert rel_max_err(ref, yw) < 0.1


def test_determinism():
    w = WL.workload(1)
    W, X = gpu(WL.weight(w)), gpu(WL.calibration(w))
    al = gpu(torch.from_numpy(WL.alpha_grid(20)))
    outs = []
    for _ in range(2):
        m = awq.awq_act_stats(X)
        s, inv, L, best = awq.awq_search_scales(W, X, m, al)
        q, sc, z = awq.awq_quantize_pack(W, s)
        xx = gpu(WL.prefill_input(w, 64))
        y = awq.awq_w4a16_gemm(xx, q, sc, z, inv)
        y1 = awq.awq_w4a16_gemm(xx[:1], q, sc, z, inv)
        torch.cuda.synchronize()
        outs.append([t.cpu().clone() for t in (m, s, L, q, sc, z, y, y1)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_pipeline_graph_replay():
    """The whole path (statistic, search, quantize + pack, batch-1 and 64-token
    products on the 512 x 512 linear) captured in one HIP graph with
    preallocated outputs and workspaces: every replay, with eager work and
    synchronisations between them, gives bit-identical outputs to the eager
    run (no call allocates, synchronises or records a memset)."""
    w = WL.workload(1)
    W, X = gpu(WL.weight(w)), gpu(WL.calibration(w))
    al = gpu(torch.from_numpy(WL.alpha_grid(20)))
    xx = gpu(WL.prefill_input(w, 64))
    N, K, T = w.N, w.K, w.T
    dev = W.device
    ws_st = torch.empty(awq.awq_workspace_bytes(awq.AWQ_OP_ACT_STATS, 0, N, K, T), dtype=torch.uint8, device=dev)
    ws_se = torch.empty(awq.awq_workspace_bytes(awq.AWQ_OP_SEARCH, 0, N, K, T, 20), dtype=torch.uint8, device=dev)
    ws_g = torch.empty(max(1, awq.awq_workspace_bytes(awq.AWQ_OP_GEMM, 64, N, K)), dtype=torch.uint8, device=dev)
    m = torch.empty(K, dtype=torch.float32, device=dev)
    s = torch.empty(K, dtype=torch.float32, device=dev)
    inv = torch.empty(K, dtype=torch.float32, device=dev)
    L = torch.empty(20, dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    q = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    sc = torch.empty((N, K // 128), dtype=torch.float16, device=dev)
    z = torch.empty((N, K // 128), dtype=torch.uint8, device=dev)
    y = torch.empty((64, N), dtype=torch.float16, device=dev)
    y1 = torch.empty((1, N), dtype=torch.float32, device=dev)

    def run():
        awq.awq_act_stats(X, m, ws=ws_st)
        awq.awq_search_scales(W, X, m, al, s_out=s, inv_s_out=inv, loss_out=L, best_idx_out=best, ws=ws_se)
        awq.awq_quantize_pack(W, s, qweight=q, scales=sc, zeros=z)
        awq.awq_w4a16_gemm(xx, q, sc, z, inv, y=y, ws=ws_g)
        awq.awq_w4a16_gemm(xx[:1], q, sc, z, inv, y=y1)

    outs = (m, s, inv, L, best, q, sc, z, y, y1)
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    st = torch.cuda.Stream()
    run()                                     # warm-up on the capture stream's device
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()                         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {rep}"


# ---------------------------------------------------------------------------
# folding 1/s into the producer of x ("AWQ Math", "The equivalent transform:
# scale up W, scale down x") and the shared-input search of q, k and v
# ---------------------------------------------------------------------------
_FOLD_DT = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols,ld,axis", [(1, 4096, 4096, 1), (37, 300, 304, 1), (37, 300, 304, 0),
                                               (1000, 513, 513, 0), (3, 1, 1, 1)])
def test_fold_scales_bit_exact(dtype, rows, cols, ld, axis):
    g = np.random.Generator(np.random.PCG64(rows * 7 + cols + axis))
    full = torch.from_numpy(g.uniform(-3, 3, (rows, ld)).astype(np.float32)).to(dtype)
    s = np.exp(g.uniform(-3, 3, cols if axis == 1 else rows)).astype(np.float32)
    v = gpu(full)
    awq.awq_fold_scales(v[:, :cols], gpu(torch.from_numpy(s)), axis=axis)
    torch.cuda.synchronize()
    want = O.fold_scales(f32(full)[:, :cols], s, axis, _FOLD_DT[dtype])
    got = f32(v.cpu())
    assert np.array_equal(got[:, :cols].view(np.uint32), want.view(np.uint32))
    assert np.array_equal(got[:, cols:], f32(full)[:, cols:])      # padding untouched


def test_shared_input_search_and_fold_c3():
    """q, k and v of a decoder layer read one input: one search on their
    row-concatenated W gives one s for all three; 1/s folded into the
    preceding LayerNorm's gain and bias leaves the products without inv_s, and
    they match the unfolded layer."""
    X = WL.calibration(WL.workload(3, "q"))
    assert torch.equal(X, WL.calibration(WL.workload(3, "v")))          # the shared input
    W = torch.cat([WL.weight(WL.workload(3, "q"))[:256], WL.weight(WL.workload(3, "k"))[:128],
                   WL.weight(WL.workload(3, "v"))[:128]])
    _check_search(W, X, F16)                                                 # search parity
    m = awq.awq_act_stats(gpu(X))
    al = gpu(torch.from_numpy(WL.alpha_grid(20)))
    s, inv, _, _ = awq.awq_search_scales(gpu(W), gpu(X), m, al)
    q, sc, z = awq.awq_quantize_pack(gpu(W), s)
    g = np.random.Generator(np.random.PCG64(33))
    K = W.shape[1]
    gamma = torch.from_numpy(g.uniform(0.5, 1.5, K).astype(np.float16))
    beta = torch.from_numpy(g.uniform(-0.1, 0.1, K).astype(np.float16))
    gf, bf = gpu(gamma.clone()), gpu(beta.clone())
    awq.awq_fold_scales(gf, s)
    awq.awq_fold_scales(bf, s)
    torch.cuda.synchronize()
    s_np = s.cpu().numpy()
    assert np.array_equal(f32(gf.cpu()), O.fold_scales(f32(gamma)[None, :], s_np, 1, "f16")[0])
    assert np.array_equal(f32(bf.cpu()), O.fold_scales(f32(beta)[None, :], s_np, 1, "f16")[0])
    # a normalized decode batch through the LayerNorm's affine part, folded and not
    n = g.standard_normal((8, K)).astype(np.float32)
    x = torch.from_numpy((n * f32(gamma) + f32(beta)).astype(np.float16))
    xf = torch.from_numpy((n * f32(gf.cpu()) + f32(bf.cpu())).astype(np.float16))
    words, step, zeros = q.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy()
    inv_np = inv.cpu().numpy()
    ref = O.w4a16_matmul(f32(x), words, step, zeros, inv_np)                # the unfolded layer
    for M in (1, 8):
        y = awq.awq_w4a16_gemm(gpu(xf[:M]), q, sc, z, None, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert rel_max_err(f32(y), O.w4a16_matmul(f32(xf[:M]), words, step, zeros, None)) <= GEMM_TOL
        assert rel_max_err(f32(y), ref[:M]) <= GEMM_TOL



# ------------------------------------------------------------- quantizer variants
def _variant_layer(N, K, dtype, seed, with_s):
    W = WL.random_matrix((N, K), torch.float32, seed=seed, scale=0.02)
    W[:, 3::101] *= 30.0                      # outliers inside some groups
    W[0, :64] = 0.0                           # an all-zero group (every group size starts it)
    W[1, :] = -0.4                            # a constant negative row
    W = W.to(dtype)
    s = None
    if with_s:
        g = np.random.Generator(np.random.PCG64(seed + 5))
        s = torch.from_numpy(np.exp(g.uniform(-2.5, 2.5, K)).astype(np.float32))
    return W, s


@pytest.mark.parametrize("group", [64, 256])
@pytest.mark.parametrize("N,K,dtype,with_s", [
    (37, 4096, F16, True), (300, 11008 - 11008 % 256, BF16, True), (129, 1024, BF16, False),
    (5, 256, F16, True), (64, 768, F16, False),
])
def test_quantize_pack_groups_bit_exact(group, N, K, dtype, with_s):
    """awq_quantize_pack with groups of 64 and 256: packed words, steps, zero
    points and the unrounded steps bit-exact."""
    W, s = _variant_layer(N, K, dtype, N + K + group, with_s)
    dbg = torch.empty((N, K // group), dtype=torch.float32, device="cuda")
    q, sc, z = awq.awq_quantize_pack(gpu(W), None if s is None else gpu(s), group, scales_f32_dbg=dbg)
    torch.cuda.synchronize()
    r = O.quantize_layer(f32(W), None if s is None else s.numpy(), group)
    assert sc.shape == (N, K // group)
    assert np.array_equal(dbg.cpu().numpy().view(np.uint32), r["d"].view(np.uint32))
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), r["step"].view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), r["z"])
    assert np.array_equal(q.cpu().numpy(), O.pack_codes(r["q"]))


VARIANTS = [(128, 4, False), (64, 3, False), (256, 2, False), (128, 8, False), (64, 5, False),
            (64, 4, True), (128, 7, True), (256, 2, True), (128, 3, True)]


@pytest.mark.parametrize("group,bits,sym", VARIANTS)
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_quantize_codes_bit_exact(group, bits, sym, dtype):
    """awq_quantize_codes: every grid of the family (N bits, asymmetric or
    symmetric, groups of 64 / 128 / 256), codes, steps and zero points
    bit-exact; for 4-bit asymmetric the codes are those awq_quantize_pack packs."""
    N, K = 203, 1536
    W, s = _variant_layer(N, K, dtype, 7 * bits + group + (1000 if sym else 0), True)
    c, sc, z = awq.awq_quantize_codes(gpu(W), gpu(s), group, bits, sym)
    torch.cuda.synchronize()
    r = O.quantize_layer(f32(W), s.numpy(), group, bits, sym)
    assert np.array_equal(c.cpu().numpy(), r["q"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), r["step"].view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), r["z"])
    assert int(c.max()) <= O.code_max(bits, sym)
    if bits == 4 and not sym:
        q, _, _ = awq.awq_quantize_pack(gpu(W), gpu(s), group)
        assert np.array_equal(q.cpu().numpy(), O.pack_codes(c.cpu().numpy()))


@pytest.mark.parametrize("group,bits,sym", [(64, 4, False), (256, 4, False), (128, 3, False),
                                            (64, 8, False), (128, 4, True), (256, 3, True)])
@pytest.mark.parametrize("N,K,T,dtype", [(300, 1024, 200, F16), (130, 768, 3000, BF16)])
def test_search_variants(group, bits, sym, N, K, T, dtype):
    """The search scores the quantizer variant it is given: every loss, the
    chosen index and s as for the 4-bit grid (the first shape takes the
    direct form of the loss, the second the Gram form)."""
    W = WL.random_matrix((N, K), torch.float32, seed=N + bits, scale=0.02).to(dtype)
    X = _act(T, K, dtype, seed=T + group)
    _check_search(W, X, dtype, group=group, bits=bits, sym=sym)


def _random_packed_g(N, K, seed, group):
    g = np.random.Generator(np.random.PCG64(seed))
    q = g.integers(0, 16, (N, K)).astype(np.uint8)
    step = g.uniform(2e-4, 4e-3, (N, K // group)).astype(np.float16)
    z = g.integers(0, 16, (N, K // group)).astype(np.uint8)
    return O.pack_codes(q), step, z


@pytest.mark.parametrize("group", [64, 256])
@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r", [
    (1, 1000, 4096, F16, F16, True), (1, 11008, 4096, BF16, torch.float32, False),
    (1, 257, 768, F16, torch.float32, True), (3, 700, 2048, F16, F16, True),
    (8, 4096, 11008 - 11008 % 256, BF16, torch.float32, True), (16, 96, 1024, F16, torch.float32, False),
    (40, 600, 2560, F16, F16, True), (300, 520, 1024, BF16, torch.float32, False),
])
def test_product_groups_parity(group, M, N, K, dtype, ydt, with_r):
    """The fused product with groups of 64 and 256, on every path (batch-1
    GEMV, skinny matrix-core product, tiled GEMM)."""
    words, step, z = _random_packed_g(N, K, M * 1000 + N + K + group, group)
    x = _act(M, K, dtype, M + K)
    r = None
    if with_r:
        g = np.random.Generator(np.random.PCG64(K + group))
        r = (np.float32(1) / np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)).astype(np.float32)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)),
                           out_dtype=ydt, group_size=group)
    torch.cuda.synchronize()
    ref = O.w4a16_matmul(f32(x), words, step, z, r, group)
    err = rel_max_err(f32(y), ref, ydt)
    print(f"product g={group} M={M} N={N} K={K}: rel max err {err:.3e}")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("M", [1, 4, 16, 40])
def test_product_group64_odd_units(M):
    """Groups of 64 with K = 64 * odd (not whole 128-channel units): batch 1
    runs the GEMV, larger batches the tiled GEMM."""
    N, K, group = 333, 64 * 23, 64
    words, step, z = _random_packed_g(N, K, 77 + M, group)
    x = _act(M, K, F16, 5 + M)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), out_dtype=torch.float32, group_size=group)
    torch.cuda.synchronize()
    ref = O.w4a16_matmul(f32(x), words, step, z, None, group)
    assert rel_max_err(f32(y), ref) <= GEMM_TOL


@pytest.mark.parametrize("group", [64, 256])
def test_group_end_to_end(group):
    """Statistics -> search -> quantize -> products with one group size: the
    search's s, the packed layer and the product at M = 1 and 8 against the
    oracle on the same inputs."""
    w = WL.workload(1)
    W, X = WL.weight(w), WL.calibration(w)
    _check_search(W, X, F16, group=group)
    m = awq.awq_act_stats(gpu(X))
    al = gpu(torch.from_numpy(WL.alpha_grid(20)))
    s, inv, _, _ = awq.awq_search_scales(gpu(W), gpu(X), m, al, group)
    q, sc, z = awq.awq_quantize_pack(gpu(W), s, group)
    torch.cuda.synchronize()
    r = O.quantize_layer(f32(W), s.cpu().numpy(), group)
    assert np.array_equal(q.cpu().numpy(), O.pack_codes(r["q"]))
    xs = X[:8]
    for M in (1, 8):
        y = awq.awq_w4a16_gemm(gpu(xs[:M]), q, sc, z, inv, out_dtype=torch.float32, group_size=group)
        torch.cuda.synchronize()
        ref = O.w4a16_matmul(f32(xs[:M]), q.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy(),
                             inv.cpu().numpy(), group)
        assert rel_max_err(f32(y), ref) <= GEMM_TOL


# ------------------------------------------------------------- mixed-precision baseline
@pytest.mark.parametrize("K,n_keep,ties", [(4096, 41, False), (512, 5, True), (11008, 110, False),
                                           (128, 0, False), (384, 384, True), (1000, 1, True)])
def test_salient_channels_bit_exact(K, n_keep, ties):
    """awq_salient_channels on the GPU's own statistic: the mask equals the
    oracle's on the same (bit-exact) statistic, ties included (pairs of equal
    columns)."""
    x = _act(64, K, F16, seed=K + n_keep)
    if ties:
        x[:, 1::2] = x[:, 0::2]
    m = awq.awq_act_stats(gpu(x))
    kept = awq.awq_salient_channels(m, n_keep)
    torch.cuda.synchronize()
    ref = O.salient_channels(O.act_mean_abs(f32(x)), n_keep)
    got = kept.cpu().numpy()
    assert got.max(initial=0) <= 1 and np.array_equal(got.astype(bool), ref)


@pytest.mark.parametrize("N,K,T,dtype,group", [(300, 1024, 200, F16, 128), (130, 768, 3000, BF16, 128),
                                               (256, 1024, 300, F16, 64), (200, 512, 2500, F16, 256)])
def test_search_with_kept_channels(N, K, T, dtype, group):
    """The mixed-precision baseline: 1 % of the channels (the most salient)
    kept in 16-bit, the rest round-to-nearest (alpha = 0), and the search with
    those channels kept, against the oracle (direct and Gram forms of the
    loss); keeping them lowers the plain loss on this outlier layer."""
    W = WL.random_matrix((N, K), torch.float32, seed=N + K, scale=0.02)
    W[:, ::97] *= 10.0                         # outlier weights on the boosted channels
    W = W.to(dtype)
    X = _act(T, K, dtype, seed=T + K)
    n_keep = max(1, K // 100)
    keep = O.salient_channels(O.act_mean_abs(f32(X)), n_keep)
    kept_gpu = awq.awq_salient_channels(awq.awq_act_stats(gpu(X)), n_keep)
    assert np.array_equal(kept_gpu.cpu().numpy().astype(bool), keep)
    L_mixed = _check_search(W, X, dtype, group=group, keep=keep, alphas=np.array([0.0]))
    L_rtn = _check_search(W, X, dtype, group=group, alphas=np.array([0.0]))
    assert L_mixed[0] < L_rtn[0]
    _check_search(W, X, dtype, group=group, keep=keep)


@pytest.mark.parametrize("ydt", [F16, BF16, torch.float32])
def test_gemm_strided_output_ragged_tail(ydt):
    """Tiled GEMM into a strided output (row pitch 1024, N = 1001): the
    16-byte stores of whole row pieces, the element stores of the last
    partial piece, and the padding left untouched."""
    M, N, K = 70, 1001, 1024
    words, step, z = _random_packed_g(N, K, 991, 128)
    x = _act(M, K, F16, 17)
    big = torch.full((M, 1024), 7.0, dtype=ydt, device="cuda")
    y = big[:, :N]
    awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                       gpu(torch.from_numpy(z)), y=y)
    torch.cuda.synchronize()
    ref = O.w4a16_matmul(f32(x), words, step, z)
    assert rel_max_err(f32(y.cpu()), ref, ydt) <= GEMM_TOL
    assert torch.all(big[:, N:] == 7.0).item()


@pytest.mark.parametrize("M,N", [(1, 1), (1, 3), (2, 5), (17, 2), (40, 65)])
def test_product_single_group_64(M, N):
    """K = 64 with groups of 64: one group per row; the tiled GEMM then runs a
    single 64-channel stage, and tiny N leaves most of a tile empty."""
    K, group = 64, 64
    words, step, z = _random_packed_g(N, K, 500 + M * 10 + N, group)
    x = _act(M, K, F16, 9 + M)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), out_dtype=torch.float32, group_size=group)
    torch.cuda.synchronize()
    ref = O.w4a16_matmul(f32(x), words, step, z, None, group)
    assert rel_max_err(f32(y), ref) <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,dtype,ydt,with_r,group", [
    (17, 4096, 4096, F16, F16, True, 128),        # one 16-row tile per block, 256 blocks
    (24, 11008, 4096, BF16, torch.float32, True, 128),   # 43 rows in 3 tiles per block
    (20, 13000, 1024, F16, F16, True, 128),        # 50 or 51 rows in 4 tiles per block
    (56, 9000, 1024, BF16, torch.float32, False, 128),   # four token groups, two rounds of blocks
    (32, 4096, 11008, F16, torch.float32, True, 128),    # 4-tile blocks, 86 units over 4 uneven slices
    (48, 1000, 2560, BF16, BF16, False, 64),       # 2 K slices, groups of 64
    (64, 777, 8192, F16, torch.float32, True, 256),     # 8 K slices of 2-tile blocks, groups of 256
    (33, 64, 128, F16, torch.float32, False, 128),  # one unit, four row blocks
    (17, 10, 256, BF16, torch.float32, True, 128),   # fewer rows than one tile
    (40, 3000, 28672, BF16, F16, True, 128),       # long K: 224 units over 4 slices, 2-tile blocks
])
def test_small_batch_product_parity(M, N, K, dtype, ydt, with_r, group):
    """17 <= M <= 64: the memory-bound small-batch product (row blocks of up to
    four tiles; small layers split over K, the slices' partial sums added in
    slice order by a second kernel)."""
    words, step, z = _random_packed_g(N, K, M * 31 + N + K + group, group)
    x = _act(M, K, dtype, M + N)
    r = None
    if with_r:
        g = np.random.Generator(np.random.PCG64(K + M))
        r = (np.float32(1) / np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)).astype(np.float32)
    ldy = N + 40
    big = torch.full((M, ldy), 9.0, dtype=ydt, device="cuda")
    awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                       gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)),
                       y=big[:, :N], group_size=group)
    torch.cuda.synchronize()
    ref = O.w4a16_matmul(f32(x), words, step, z, r, group)
    err = rel_max_err(f32(big[:, :N].cpu()), ref, ydt)
    print(f"small batch M={M} N={N} K={K} g={group}: rel max err {err:.3e}")
    assert err <= GEMM_TOL
    assert torch.all(big[:, N:] == 9.0).item()
    # bit-identical on a second call (fixed order of the slice sums)
    again = torch.empty((M, N), dtype=ydt, device="cuda")
    awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                       gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)),
                       y=again, group_size=group)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.uint8), big[:, :N].contiguous().view(torch.uint8))


@pytest.mark.parametrize("M,N,K,dtype,with_r,pad", [
    (8, 11008, 4096, F16, True, 64),            # loader/stager schedule
    (5, 4096, 4096, BF16, False, 8),            # one tile per block
    (16, 3000, 2048, F16, True, 136),           # 16 tokens, odd row pitch in 16-byte units
])
def test_skinny_product_strided_activations(M, N, K, dtype, with_r, pad):
    """2..16 tokens from a strided activation view (row pitch K + pad): the
    staging reads each token row at its own pitch."""
    g = np.random.Generator(np.random.PCG64(M * 31 + N + pad))
    words = g.integers(-2 ** 31, 2 ** 31, (N, K // 8), dtype=np.int64).astype(np.int32)
    step = g.uniform(2e-4, 4e-3, (N, K // 128)).astype(np.float16)
    z = g.integers(0, 16, (N, K // 128)).astype(np.uint8)
    x = _act(M, K, dtype, M + K + pad)
    big = torch.zeros((M, K + pad), dtype=dtype)
    big[:, :K] = x
    r = (np.float32(1) / np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)).astype(np.float32) if with_r else None
    y = awq.awq_w4a16_gemm(gpu(big)[:, :K], gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, N, max(1, N // 300)), np.arange(N - 40, N)]))
    ref = O.w4a16_matmul_rows(f32(x), words, step, z, rows, r)
    assert rel_max_err(f32(y)[:, rows], ref) <= GEMM_TOL


@pytest.mark.parametrize("M,N,K", [(8, 5000, 2048), (2, 11008, 4096), (16, 9000, 1024)])
def test_skinny_one_hot_exact_split_path(M, N, K):
    """Blocks of two or more 16-row tiles take the loader/stager schedule of
    the 2..16-token product.  A one-hot token is exact there too: the codes
    enter the matrix cores exactly, the zero point's sum is exact and the
    step multiplies in fp32, so every output equals step * (q - z)."""
    words, step, z = _random_packed(N, K, 11 + M)
    for k in (0, K // 2 + 3, K - 1):
        x = torch.zeros((M, K), dtype=F16)
        x[:, k] = 1.0
        y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                               gpu(torch.from_numpy(z)), out_dtype=torch.float32)
        ref = O.w4a16_matmul(f32(x), words, step, z)
        assert np.array_equal(f32(y), ref.astype(np.float32)), (M, N, K, k)


@pytest.mark.parametrize("M,N,K", [(4, 4096, 4096), (2, 8192, 8192), (8, 3000, 4224), (5, 11008, 3968)])
def test_skinny_one_hot_exact_lds_ring(M, N, K):
    """The 2..16-token product with the packed words copied through LDS in
    whole 128-byte row pieces (unit pairs): one-hot tokens stay exact, also
    where the unit count is odd (the last pair holds one unit) and where the
    loader/stager split is on (K = 3968)."""
    words, step, z = _random_packed(N, K, 41 + M)
    for k in (0, 127, 128, K - 129, K - 1):
        x = torch.zeros((M, K), dtype=F16)
        x[:, k] = 1.0
        y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                               gpu(torch.from_numpy(z)), out_dtype=torch.float32)
        ref = O.w4a16_matmul(f32(x), words, step, z)
        assert np.array_equal(f32(y), ref.astype(np.float32)), (M, N, K, k)


@pytest.mark.parametrize("nbytes,blocks,unroll", [(1024, 1, 1), (23601152, 256, 4), (3 * 1024 * 1037, 300, 8),
                                                  (64 * 1024, 1000, 2)])
def test_read_stream_xor(nbytes, blocks, unroll):
    """The streaming-read diagnostic reads every word once: the XOR over its
    blocks equals the XOR of the buffer (integer, bit-exact), including a
    ragged last step and more blocks than units."""
    g = np.random.Generator(np.random.PCG64(nbytes + blocks))
    words = g.integers(-2 ** 31, 2 ** 31, nbytes // 4, dtype=np.int64).astype(np.int32)
    bx = awq.awq_read_stream(gpu(torch.from_numpy(words)), blocks, unroll)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(bx.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words.view(np.uint32))

