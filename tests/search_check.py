"""The search's outputs against the oracle: the losses against the exact
fp64 losses of the definition ("AWQ Math", "Searching the scale -- no
backprop required": the mean squared error of W x against
Q(W diag(s)) diag(s)^-1 x over the calibration tokens), the chosen index
against their argmin, s and 1/s bit-exact; the oracle scored in the
matrix-core operand precision as a second check.

Tolerance of a loss against the exact one: 8 standard deviations of the
change that the fp16 rounding of the error values causes (gpu_util.
loss_rounding_sigma; on every search input of these tests the operand-
precision oracle, which is exactly that rounding, stays within 2.1 of them),
plus 1e-5 of the loss for the fp32 accumulation on the matrix cores (and the
Gram form's fp32 chunks of X^T X).  The GPU losses within that tolerance of
the exact ones fix the GPU's argmin to the exact argmin whenever the exact
losses' best and runner-up lie more than twice the tolerance apart; a seed
whose gap is smaller cannot decide the index and fails as ill-posed.
The rigorous worst-case bound (gpu_util.loss_error_bound) is checked too; it
is about sqrt(K) looser and cannot decide the index on its own.
"""
import numpy as np

import oracle as O
from tests.gpu_util import FP16_U, loss_error_bound, loss_rounding_sigma

MODEL_RTOL = 1e-5       # GPU loss vs the operand-precision oracle (only the fp32 sums differ)
ACCUM_RTOL = 1e-5       # fp32 accumulation part of the tolerance against the exact loss
N_SIGMA = 8.0


def exact_tolerances(W64, X64, S, group, bits, sym, keep, L_ex):
    """Per candidate: (tolerance against the exact loss, rigorous bound)."""
    N, K = W64.shape
    T = X64.shape[0]
    G = X64.T @ X64
    tol, rig = [], []
    for i in range(S.shape[0]):
        r = O.quantize_layer(W64.astype(np.float32), S[i], group, bits, sym, keep)
        grid = O.dequantize(r["q"].reshape(N, K // group, group), r["D"],
                            r["z"].astype(np.float32)).reshape(N, K)
        Wh = O.unscale_activation(grid, S[i])
        if keep is not None:
            Wh = np.where(keep[None, :], W64, Wh)
        tol.append(N_SIGMA * loss_rounding_sigma(W64 - Wh, G, T, N) + ACCUM_RTOL * L_ex[i])
        rig.append(loss_error_bound(W64, X64, Wh, FP16_U)[0] + 1e-6 * L_ex[i])
    return np.array(tol), np.array(rig)


def check_search_outputs(L, best, s, inv, W, X, m_ref, alphas, x_is_fp16, group=128, bits=4,
                         sym=False, keep=None, label=""):
    """L float64 [n], best int, s / inv float32 [K] from the GPU; W, X float32
    host arrays holding the 16-bit inputs; m_ref the oracle's statistic.
    Returns the exact losses."""
    W64, X64 = W.astype(np.float64), X.astype(np.float64)
    S = O.candidate_scales(m_ref, alphas)
    L_ex = O.search_losses(W, X, S, group, bits=bits, symmetric=sym, keep=keep)
    L_mod = O.search_losses_operand_model(W, X, S, x_is_fp16, group, bits=bits, symmetric=sym,
                                          keep=keep)
    tol, rig = exact_tolerances(W64, X64, S, group, bits, sym, keep, L_ex)
    dev = np.abs(L - L_ex)
    assert np.all(dev <= tol), ("loss vs exact", dev / L_ex, tol / L_ex)
    assert np.all(dev <= rig), ("loss vs rigorous bound", dev, rig)
    assert np.all(np.abs(L - L_mod) <= MODEL_RTOL * L_mod), ("loss vs operand model", (L - L_mod) / L_mod)
    n = len(alphas)
    if n == 1:
        assert best == 0
        return L_ex
    i_ex = O.choose_candidate(L_ex)
    order = np.argsort(L_ex)
    gap = (L_ex[order[1]] - L_ex[order[0]]) / L_ex[order[0]]
    need = 2.0 * float(np.max(tol / L_ex))
    print(f"search {label} N={W.shape[0]} K={W.shape[1]} T={X.shape[0]} g={group} bits={bits} "
          f"sym={sym}: exact argmin {i_ex}, gap {gap:.2e} (decidable above {need:.2e}), "
          f"max |L - L_exact| / L_exact {np.max(dev / L_ex):.2e}")
    if gap <= need:
        raise AssertionError(f"ill-posed seed: the exact losses' best two are {gap:.2e} apart, "
                             f"within twice the tolerance {need:.2e}; choose another seed")
    assert best == i_ex
    assert np.array_equal(s.view(np.uint32), S[i_ex].view(np.uint32))
    assert np.array_equal(inv.view(np.uint32), (np.float32(1) / S[i_ex]).astype(np.float32).view(np.uint32))
    # second check: the operand-precision oracle decides the same index
    assert O.choose_candidate(L_mod) == i_ex
    return L_ex
