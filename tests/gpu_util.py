"""Helpers for the GPU parity tests: tensor conversion and tolerances derived
from the arithmetic of the HIP path.  No method arithmetic lives here."""
import numpy as np
import torch

FP16_U = 2.0 ** -11      # unit roundoff of fp16 (11 significant bits)
BF16_U = 2.0 ** -8       # unit roundoff of bf16 (8 significant bits)
F32_U = 2.0 ** -24
GEMM_TOL = 2e-3          # max|y_gpu - y_ref| / max|y_ref|, the stated bar


def f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of an fp16/bf16/f32 tensor on the host."""
    return t.detach().float().cpu().numpy()


def gpu(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda")


def half_ulp(ref: np.ndarray, out_dtype: torch.dtype) -> np.ndarray:
    """Half a unit in the last place of the output type at |ref| (0 for f32):
    the rounding of the stored output itself, which no kernel can avoid."""
    if out_dtype == torch.float32:
        return np.zeros_like(ref)
    bits = 11 if out_dtype == torch.float16 else 8
    a = np.maximum(np.abs(ref), 2.0 ** -24 if bits == 11 else 2.0 ** -126)
    e = np.floor(np.log2(a))
    return 2.0 ** (e - bits)


def rel_max_err(got: np.ndarray, ref: np.ndarray, out_dtype: torch.dtype = torch.float32) -> float:
    """max(|got - ref| - output rounding) / max|ref|."""
    den = float(np.max(np.abs(ref)))
    ex = np.abs(got.astype(np.float64) - ref) - half_ulp(ref, out_dtype)
    return max(0.0, float(np.max(ex))) / (den if den > 0 else 1.0)


def loss_error_bound(W, X, Wq_over_s, u_op):
    """Rigorous bound on |L_gpu - L_ref| for one candidate.

    The HIP path rounds E = W - W_hat once to the operand type (relative u_op,
    after an exact power-of-two row scale), computes E itself in float (a few
    roundings, below 2^-22 (|W| + |W_hat|) per element), and accumulates the
    K-long products in float (|error| <= K 2^-24 sum |e x|).  With
    P = E X^T and B the elementwise bound on |delta P|:
        |delta L| <= sum(2 |P| B + B^2) / (T N)
    """
    E = W - Wq_over_s
    A = np.abs(E) @ np.abs(X).T                     # [N, T]
    C = (np.abs(W) + np.abs(Wq_over_s)) @ np.abs(X).T
    K = W.shape[1]
    B = (u_op + K * F32_U) * A + 2.0 ** -22 * C
    P = E @ X.T
    T, N = X.shape[0], W.shape[0]
    return float(np.sum(2 * np.abs(P) * B + B * B)) / (T * N), float(np.sum(P * P)) / (T * N)


def loss_rounding_sigma(E, G, T, N):
    """Standard deviation of the change in one search loss caused by rounding
    each error value E[n, k] once to fp16, under the probabilistic model of
    rounding errors (Higham and Mary, "A new approach to probabilistic
    rounding error analysis", SIAM J. Sci. Comput. 2019): the rounding errors
    eta[n, k] are independent, zero-mean and |eta| <= 2^-11 |E| (half an fp16
    ulp; each row is first scaled by an exact power of two that keeps it in
    the normal range, so a subnormal error is at most 2^-38 of the row's
    largest value).  To first order
        L(E + eta) - L(E) = (2 / (T N)) sum_nk eta_nk c_nk,   c = E (X^T X),
    so Var <= (2 / (T N))^2 sum_nk Var(eta_nk) c_nk^2 with Var(eta) <= bound^2 / 3.
    E is [N, K] float64 (the exact W - W_hat), G = X^T X [K, K] float64."""
    c = E @ G
    rowmax = np.max(np.abs(E), axis=1, keepdims=True)
    var = (2.0 ** -11 * np.abs(E)) ** 2 / 3.0 + (rowmax * 2.0 ** -38) ** 2
    return 2.0 * float(np.sqrt(np.sum(var * c * c))) / (float(T) * float(N))
