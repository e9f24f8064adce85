"""Parity at the benchmark's full sizes, in the launch configurations bench.py
times: the Llama-7B MLP up-projection (K=4096, N=11008, fp16, 65536
calibration tokens) and the Llama-70B MLP up-projection prefill (K=8192,
N=28672, bf16, M=2048).

The statistic, codes, steps and zero points are compared in full.  Products
are compared on sampled output channels (output channels are independent, so
a sample is an exact check of those channels).  The search is checked on a
row slice against the oracle at the full token count, and at full size
through properties that hold at any size.
"""
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


@pytest.fixture(scope="module")
def up7b():
    w = WL.workload(2)
    W, X = WL.weight(w), WL.calibration(w)
    m_ref = O.act_mean_abs(f32(X))
    return w, W, X, m_ref


def _sample_rows(N, step, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    rows = np.unique(np.concatenate([np.arange(0, N, step), g.integers(0, N, 64),
                                     np.arange(N - 5, N)]))
    return rows


def test_full_act_stats_bit_exact(up7b):
    w, W, X, m_ref = up7b
    m = awq.awq_act_stats(gpu(X))
    torch.cuda.synchronize()
    assert np.array_equal(m.cpu().numpy().view(np.uint32), m_ref.view(np.uint32))


def test_full_quantize_pack_and_decode(up7b):
    """Quantize the full layer with oracle scales (alpha = 10/19), bit-exact;
    then the batch-1 and batch-8 GEMVs with 1/s on sampled channels."""
    w, W, X, m_ref = up7b
    s_ref = O.candidate_scales(m_ref, np.array([10 / 19]))[0]
    q, sc, z = awq.awq_quantize_pack(gpu(W), gpu(torch.from_numpy(s_ref)))
    torch.cuda.synchronize()
    r = O.quantize_layer(f32(W), s_ref)
    words = O.pack_codes(r["q"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), r["step"].view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), r["z"])
    assert np.array_equal(q.cpu().numpy(), words)
    inv = (np.float32(1) / s_ref).astype(np.float32)
    rows = _sample_rows(w.N, 37, 1)
    for M in (1, 8):
        x = WL.decode_input(w, M)
        y = awq.awq_w4a16_gemm(gpu(x), q, sc, z, gpu(torch.from_numpy(inv)))
        torch.cuda.synchronize()
        ref = O.w4a16_matmul_rows(f32(x), words, r["step"], r["z"], rows, inv)
        err = rel_max_err(f32(y)[:, rows], ref, torch.float16)
        print(f"decode M={M}: rel max err {err:.3e} on {len(rows)} channels")
        assert err <= GEMM_TOL


def test_full_search_row_slice_and_properties(up7b):
    """Row slice of the layer with all 65536 tokens against the oracle
    (operand-precision scoring); the full layer on the GPU: the choice is the
    minimal loss, no worse than plain round-to-nearest, its s is the oracle's
    candidate for that index, and two runs are bit-identical."""
    w, W, X, m_ref = up7b
    alphas = WL.alpha_grid(20)
    al = gpu(torch.from_numpy(alphas))
    m = gpu(torch.from_numpy(m_ref))
    Wg, Xg = gpu(W), gpu(X)
    # slice: 64 rows, every token
    s, inv, L, best = awq.awq_search_scales(Wg[:64].contiguous(), Xg, m, al)
    torch.cuda.synchronize()
    i_mod, s_mod, _, L_mod = O.search_scales(f32(W[:64]), f32(X), m_ref, alphas,
                                             operand_model="fp16")
    L = L.cpu().numpy()
    assert np.all(np.abs(L - L_mod) <= 1e-5 * L_mod)
    order = np.argsort(L_mod)
    if (L_mod[order[1]] - L_mod[order[0]]) / L_mod[order[0]] > 2e-5:
        assert int(best.cpu()[0]) == i_mod
        assert np.array_equal(s.cpu().numpy().view(np.uint32), s_mod.view(np.uint32))
    # full layer
    outs = []
    for _ in range(2):
        s, inv, L, best = awq.awq_search_scales(Wg, Xg, m, al)
        torch.cuda.synchronize()
        outs.append((s.cpu().clone(), inv.cpu().clone(), L.cpu().clone(), int(best.cpu()[0])))
    (s, inv, L, b), (s2, inv2, L2, b2) = outs
    assert b == b2 and torch.equal(s, s2) and torch.equal(L, L2) and torch.equal(inv, inv2)
    L = L.numpy()
    assert L[b] == np.min(L) and np.all(L[:b] > L[b]) and L[b] <= L[0]
    S_ref = O.candidate_scales(m_ref, alphas)
    assert np.array_equal(s.numpy().view(np.uint32), S_ref[b].view(np.uint32))
    assert np.array_equal(inv.numpy().view(np.uint32),
                          (np.float32(1) / S_ref[b]).astype(np.float32).view(np.uint32))
    print(f"full search: alpha index {b}, loss {L[b]:.4e} vs round-to-nearest {L[0]:.4e}")


def test_full_prefill_gemm_sampled_channels():
    """M = 2048 bf16 prefill through the 8192 -> 28672 layer, bf16 output as in
    the benchmark, with 1/s; random packed codes, steps and zero points."""
    w = WL.workload(4, "up")
    g = np.random.Generator(np.random.PCG64(4242))
    N, K = w.N, w.K
    words = g.integers(-2 ** 31, 2 ** 31, (N, K // 8), dtype=np.int64).astype(np.int32)
    step = g.uniform(5e-4, 5e-3, (N, K // 128)).astype(np.float16)
    z = g.integers(0, 16, (N, K // 128)).astype(np.uint8)
    inv = (1.0 / np.exp(g.uniform(-1, 1, K))).astype(np.float32)
    x = WL.prefill_input(w, 2048)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), gpu(torch.from_numpy(inv)))
    torch.cuda.synchronize()
    rows = _sample_rows(N, 97, 2)
    ref = O.w4a16_matmul_rows(f32(x), words, step, z, rows, inv)
    err = rel_max_err(f32(y)[:, rows], ref, torch.bfloat16)
    print(f"prefill: rel max err {err:.3e} on {len(rows)} channels x 2048 tokens")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("group", [64, 256])
def test_full_groups_quantize_and_decode(up7b, group):
    """The full 7B layer quantized with groups of 64 and 256 (bit-exact codes,
    steps, zero points), then batch-1 and batch-8 products on sampled
    channels, in the launch configuration of the benchmark."""
    w, W, X, m_ref = up7b
    s_ref = O.candidate_scales(m_ref, np.array([6 / 19]))[0]
    q, sc, z = awq.awq_quantize_pack(gpu(W), gpu(torch.from_numpy(s_ref)), group)
    torch.cuda.synchronize()
    r = O.quantize_layer(f32(W), s_ref, group)
    words = O.pack_codes(r["q"])
    assert np.array_equal(sc.cpu().numpy().view(np.uint16), r["step"].view(np.uint16))
    assert np.array_equal(z.cpu().numpy(), r["z"])
    assert np.array_equal(q.cpu().numpy(), words)
    inv = (np.float32(1) / s_ref).astype(np.float32)
    rows = _sample_rows(w.N, 53, 3)
    for M in (1, 8):
        x = WL.decode_input(w, M)
        y = awq.awq_w4a16_gemm(gpu(x), q, sc, z, gpu(torch.from_numpy(inv)), group_size=group)
        torch.cuda.synchronize()
        ref = O.w4a16_matmul_rows(f32(x), words, r["step"], r["z"], rows, inv, group)
        err = rel_max_err(f32(y)[:, rows], ref, torch.float16)
        print(f"group {group} decode M={M}: rel max err {err:.3e}")
        assert err <= GEMM_TOL


@pytest.mark.parametrize("group", [64, 256])
def test_full_prefill_gemm_groups(group):
    """M = 2048 bf16 prefill through the 8192 -> 28672 layer with groups of 64
    and 256, sampled channels."""
    w = WL.workload(4, "up")
    g = np.random.Generator(np.random.PCG64(4343 + group))
    N, K = w.N, w.K
    words = g.integers(-2 ** 31, 2 ** 31, (N, K // 8), dtype=np.int64).astype(np.int32)
    step = g.uniform(5e-4, 5e-3, (N, K // group)).astype(np.float16)
    z = g.integers(0, 16, (N, K // group)).astype(np.uint8)
    x = WL.prefill_input(w, 2048)
    y = awq.awq_w4a16_gemm(gpu(x), gpu(torch.from_numpy(words)), gpu(torch.from_numpy(step)),
                           gpu(torch.from_numpy(z)), group_size=group)
    torch.cuda.synchronize()
    rows = _sample_rows(N, 211, 5)
    ref = O.w4a16_matmul_rows(f32(x), words, step, z, rows, None, group)
    err = rel_max_err(f32(y)[:, rows], ref, torch.bfloat16)
    print(f"group {group} prefill: rel max err {err:.3e} on {len(rows)} channels")
    assert err <= GEMM_TOL


@pytest.mark.parametrize("group,bits,sym,keep", [(64, 4, False, False), (128, 3, True, False),
                                                 (128, 4, False, True)])
def test_full_search_variants_row_slice(up7b, group, bits, sym, keep):
    """Quantizer variants and the mixed-precision baseline at the full token
    count (65536) on a 64-row slice, against the oracle scored in the
    operand precision."""
    w, W, X, m_ref = up7b
    alphas = WL.alpha_grid(20)[::4].copy()
    m = gpu(torch.from_numpy(m_ref))
    kept = O.salient_channels(m_ref, w.K // 100) if keep else None
    s, inv, L, best = awq.awq_search_scales(
        gpu(W[:64].contiguous()), gpu(X), m, gpu(torch.from_numpy(alphas)), group, bits=bits,
        symmetric=sym, kept=None if kept is None else gpu(torch.from_numpy(kept.astype(np.uint8))))
    torch.cuda.synchronize()
    i_mod, s_mod, _, L_mod = O.search_scales(f32(W[:64]), f32(X), m_ref, alphas, group,
                                             operand_model="fp16", bits=bits, symmetric=sym,
                                             keep=kept)
    L = L.cpu().numpy()
    print(f"variant g={group} bits={bits} sym={sym} keep={keep}: "
          f"max rel loss diff {np.max(np.abs(L - L_mod) / L_mod):.2e}")
    assert np.all(np.abs(L - L_mod) <= 1e-5 * L_mod)
    order = np.argsort(L_mod)
    if (L_mod[order[1]] - L_mod[order[0]]) / L_mod[order[0]] > 2e-5:
        assert int(best.cpu()[0]) == i_mod
        assert np.array_equal(s.cpu().numpy().view(np.uint32), s_mod.view(np.uint32))
