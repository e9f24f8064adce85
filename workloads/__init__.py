"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module draws random numbers and casts them to the storage dtypes; it holds
none of the quantization method's arithmetic, so both the HIP path and the CPU
oracle can be fed from it without sharing any of the method.

Recipe (every tensor is reproducible from its configuration and role):

* weights      W[n, k]  = cast(N(0, sigma_w))
* activations  X[t, j]  = cast(Z[t, j] * b[j]),  Z ~ N(0, 1)
* outlier channels: the first round(p * K) entries of a seeded permutation of
  0..K-1 get a boost b[j] > 1 (a constant, or log-normal draws); every other
  channel has b[j] = 1.  The outlier set and boosts are fixed per activation
  tensor family, so decode / prefill activations reuse the calibration set's
  channels with fresh Z.  This mirrors the pages' observation that roughly
  0.1-1 % of input channels carry outsized activation ("AWQ Math", section
  "Saliency is an activation property, not a weight property").

Random streams come from NumPy's PCG64 seeded with a SeedSequence built from
(config id, role, layer, linear), so each tensor is independent of the order in
which others are drawn.  Values are drawn in float32 and cast with
round-to-nearest-even (NumPy for float16, torch for bfloat16).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

ROLE_W, ROLE_XCAL, ROLE_PERM, ROLE_BOOST, ROLE_XDEC, ROLE_XPRE = 1, 2, 3, 4, 5, 6

LINEARS_7B = {  # name -> (N = C_out, K = C_in), Llama-7B decoder layer
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}
LINEARS_70B = {  # Llama-70B-shaped decoder layer (GQA: k/v project 8192 -> 1024)
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672),
}
LINEAR_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "single": 0}


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    N: int
    K: int
    T: int                 # calibration tokens
    dtype: torch.dtype     # storage dtype of W and X
    sigma_w: float
    outlier_frac: float
    boost: str             # "const20" | "lognormal15"
    Ms: tuple              # activation rows at inference
    linear: str = "single"
    layer: int = 0


def _rng(cfg: int, role: int, layer: int = 0, linear: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, role, layer, linear])))


def workload(cfg: int, linear: str = "single", layer: int = 0) -> Workload:
    """The five synthetic workloads (Llama-shaped layers)."""
    if cfg == 1:
        return Workload(1, "linear 512x512 fp16", 512, 512, 64, torch.float16, 0.02, 0.01,
                        "const20", (1,))
    if cfg == 2:
        return Workload(2, "llama7b mlp up 4096->11008 fp16", 11008, 4096, 128 * 512,
                        torch.float16, 0.02, 0.005, "lognormal15", (1, 8), "up")
    if cfg == 3:
        N, K = LINEARS_7B[linear]
        return Workload(3, f"llama7b layer {linear} {K}->{N} fp16", N, K, 64, torch.float16, 0.02,
                        0.01, "const20", (1, 8, 32), linear, layer)
    if cfg == 4:
        if linear in ("single", "up", "gate"):
            N, K, lin = 28672, 8192, ("up" if linear == "single" else linear)
        elif linear == "down":
            N, K, lin = 8192, 28672, "down"
        else:
            raise ValueError(linear)
        return Workload(4, f"llama70b mlp {lin} {K}->{N} bf16 prefill", N, K, 2048, torch.bfloat16,
                        0.01, 0.01, "const20", (2048,), lin, layer)
    if cfg == 5:
        N, K = LINEARS_70B[linear]
        return Workload(5, f"llama70b layer {layer} {linear} {K}->{N} fp16", N, K, 256 * 512,
                        torch.float16, 0.01, 0.01, "const20", (1,), linear, layer)
    raise ValueError(f"unknown config {cfg}")


def _cast(a32: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    if dtype == torch.float16:
        return torch.from_numpy(a32.astype(np.float16))
    if dtype == torch.bfloat16:
        return torch.from_numpy(a32).to(torch.bfloat16)
    if dtype == torch.float32:
        return torch.from_numpy(a32)
    raise ValueError(dtype)


def weight(w: Workload) -> torch.Tensor:
    """W [N, K] in the workload's dtype, CPU."""
    g = _rng(w.cfg, ROLE_W, w.layer, LINEAR_IDS[w.linear])
    a = g.standard_normal((w.N, w.K), dtype=np.float32)
    a *= np.float32(w.sigma_w)
    return _cast(a, w.dtype)


def channel_boosts(w: Workload) -> tuple[np.ndarray, np.ndarray]:
    """(outlier channel indices, per-channel boost b[K] float32).

    Linears that read the same input in a decoder layer share the same
    activation statistics (q/k/v read one tensor, gate/up another); the
    boost stream is keyed by the input tensor, not by the linear."""
    group = {"q": 0, "k": 0, "v": 0, "o": 3, "gate": 4, "up": 4, "down": 6, "single": 0}[w.linear]
    n_out = int(round(w.outlier_frac * w.K))
    perm = _rng(w.cfg, ROLE_PERM, w.layer, group).permutation(w.K)
    idx = np.sort(perm[:n_out])
    b = np.ones(w.K, dtype=np.float32)
    if w.boost == "const20":
        b[idx] = 20.0
    elif w.boost == "lognormal15":
        gb = _rng(w.cfg, ROLE_BOOST, w.layer, group)
        b[idx] = gb.lognormal(mean=math.log(15.0), sigma=0.5, size=n_out).astype(np.float32)
    else:
        raise ValueError(w.boost)
    return idx, b


def activations(w: Workload, rows: int, role: int = ROLE_XCAL, seed_extra: int = 0) -> torch.Tensor:
    """X [rows, K] with the workload's outlier channels, CPU."""
    _, b = channel_boosts(w)
    group = {"q": 0, "k": 0, "v": 0, "o": 3, "gate": 4, "up": 4, "down": 6, "single": 0}[w.linear]
    g = _rng(w.cfg, role, w.layer, 16 * group + seed_extra)
    out = np.empty((rows, w.K), dtype=np.float32)
    chunk = max(1, (1 << 24) // max(1, w.K))
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        z = g.standard_normal((r1 - r0, w.K), dtype=np.float32)
        np.multiply(z, b[None, :], out=out[r0:r1])
    return _cast(out, w.dtype)


def calibration(w: Workload) -> torch.Tensor:
    return activations(w, w.T, ROLE_XCAL)


def decode_input(w: Workload, M: int = 1) -> torch.Tensor:
    return activations(w, M, ROLE_XDEC)


def prefill_input(w: Workload, M: int) -> torch.Tensor:
    return activations(w, M, ROLE_XPRE)


def alpha_grid(n: int = 20) -> np.ndarray:
    """Candidate exponents alpha_i = i / (n - 1), i = 0..n-1 (both ends of [0, 1])."""
    return np.arange(n, dtype=np.float64) / np.float64(n - 1)


def random_matrix(shape, dtype: torch.dtype, seed: int, scale: float = 1.0) -> torch.Tensor:
    """Plain seeded N(0, scale) tensor for edge-case tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9999, seed])))
    a = g.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return _cast(a, dtype)


# --------------------------------------------------------------------------
# Device-side generators for the 80-layer 70B-shaped stack (about 140 GB of
# fp16 weights, too large to draw on the host).  torch's device generator
# (Philox) seeded from the same (config, role, layer, linear) key; the outlier
# channels and boosts still come from channel_boosts.
# --------------------------------------------------------------------------
def _device_gen(device, cfg: int, role: int, layer: int = 0, linear: int = 0) -> torch.Generator:
    seed = int(np.random.SeedSequence([cfg, role, layer, linear]).generate_state(1, np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def device_weight(w: Workload, device, out: torch.Tensor | None = None) -> torch.Tensor:
    """W [N, K] in the workload's dtype, drawn on the device (into ``out`` if
    given) in pieces of at most 256 MB of float32."""
    g = _device_gen(device, w.cfg, ROLE_W, w.layer, LINEAR_IDS[w.linear])
    if out is None:
        out = torch.empty((w.N, w.K), dtype=w.dtype, device=device)
    rows = max(1, (1 << 26) // w.K)
    for r0 in range(0, w.N, rows):
        r1 = min(w.N, r0 + rows)
        piece = torch.empty((r1 - r0, w.K), dtype=torch.float32, device=device)
        piece.normal_(0.0, w.sigma_w, generator=g)
        out[r0:r1].copy_(piece)
    return out


def device_activations(w: Workload, rows: int, device, role: int = ROLE_XCAL) -> torch.Tensor:
    """X [rows, K] with the workload's outlier channels, drawn on the device."""
    _, b = channel_boosts(w)
    group = {"q": 0, "k": 0, "v": 0, "o": 3, "gate": 4, "up": 4, "down": 6, "single": 0}[w.linear]
    g = _device_gen(device, w.cfg, role, w.layer, 16 * group)
    bd = torch.from_numpy(b).to(device)
    out = torch.empty((rows, w.K), dtype=w.dtype, device=device)
    chunk = max(1, (1 << 26) // w.K)
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        z = torch.empty((r1 - r0, w.K), dtype=torch.float32, device=device)
        z.normal_(0.0, 1.0, generator=g)
        out[r0:r1].copy_(z * bd[None, :])
    return out


def device_packed(N: int, K: int, device, seed: int, group: int = 128,
                  step_range=(5e-4, 5e-3)) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Seeded random packed codes (any 32-bit word), fp16 steps and uint8 zero
    points in the layout of the quantizer's output, drawn on the device: the
    decode products do the same work on any values, so layers whose values do
    not matter for a measurement carry these."""
    g = _device_gen(device, 90, seed)
    q = torch.randint(-2 ** 31, 2 ** 31, (N, K // 8), dtype=torch.int64, device=device,
                      generator=g).to(torch.int32)
    sc = torch.empty((N, K // group), dtype=torch.float32, device=device)
    sc.uniform_(step_range[0], step_range[1], generator=g)
    z = torch.randint(0, 16, (N, K // group), dtype=torch.uint8, device=device, generator=g)
    return q, sc.to(torch.float16), z
