"""awq_w4a16_gemm_noalloc (the product for callers that cannot allocate)
against awq_w4a16_gemm, through the C ABI: the same kernels, so the outputs
must be bit-identical, and both within the product's bar of the oracle.  Two
calls in a row share the library's scratch array, the second with a smaller
input; a batch-1 and a batch-8 call take the paths that need no scratch."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests.gpu_util import GEMM_TOL, f32, gpu, rel_max_err

pytestmark = pytest.mark.gpu

awq = pytest.importorskip("weight_only_int4_stats_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    awq.lib()


def _layer(M, N, K, dtype, seed, with_r):
    g = np.random.Generator(np.random.PCG64(seed))
    words = g.integers(-2 ** 31, 2 ** 31, (N, K // 8), dtype=np.int64).astype(np.int32)
    step = g.uniform(2e-4, 4e-3, (N, K // 128)).astype(np.float16)
    z = g.integers(0, 16, (N, K // 128)).astype(np.uint8)
    x = WL.random_matrix((M, K), torch.float32, seed + 1).to(dtype)
    r = (np.float32(1) / np.exp(g.uniform(-1.5, 1.5, K)).astype(np.float32)).astype(np.float32) if with_r else None
    return words, step, z, x, r


@pytest.mark.parametrize("cases", [
    # (M, N, K, x dtype, y dtype, 1/s): the second call is smaller than the first
    [(300, 1000, 2048, torch.float16, torch.float32, True), (100, 520, 1024, torch.bfloat16, torch.bfloat16, False)],
    [(1, 4096, 4096, torch.float16, torch.float16, True), (8, 1100, 2048, torch.float16, torch.float32, False)],
])
def test_noalloc_matches_workspace_entry_point(cases):
    for M, N, K, xdt, ydt, with_r in cases:
        words, step, z, x, r = _layer(M, N, K, xdt, M * 7 + N + K, with_r)
        args = (gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                gpu(torch.from_numpy(z)), None if r is None else gpu(torch.from_numpy(r)))
        y_ws = awq.awq_w4a16_gemm(*args, out_dtype=ydt)
        y_na = torch.full((M, N), 3.0, dtype=ydt, device="cuda")
        awq.awq_w4a16_gemm_noalloc(*args, y=y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.uint8), y_ws.view(torch.uint8)), (M, N, K)
        ref = O.w4a16_matmul(f32(x), words, step, z, r)
        err = rel_max_err(f32(y_na), ref, ydt)
        print(f"noalloc M={M} N={N} K={K}: bit-identical to the workspace call, rel max err {err:.3e}")
        assert err <= GEMM_TOL


def test_noalloc_rejects_scratch_beyond_the_limit():
    """2048 tokens through 28672 -> 8192 with groups of 64 need more scratch
    than the array holds: AWQ_ERR_UNSUPPORTED before any launch."""
    M, N, K = 2048, 8192, 28672
    need = awq.awq_workspace_bytes(awq.AWQ_OP_GEMM, M, N, K, 0, 0)
    assert need > awq._abi.AWQ_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    sc = torch.zeros((N, K // 64), dtype=torch.float16, device="cuda")
    z = torch.zeros((N, K // 64), dtype=torch.uint8, device="cuda")
    y = torch.full((M, N), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(awq.AwqError) as e:
        awq.awq_w4a16_gemm_noalloc(x, q, sc, z, y=y, group_size=64)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert torch.all(y == 5.0).item()
