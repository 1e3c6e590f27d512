"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws random numbers and arranges them into the shapes the
STQ1_0 workloads use.  It holds none of the STQ1_0 arithmetic (no codebook,
no packing, no encoder, no matmul): the oracle under ``oracle/`` and the HIP
library under ``sparse_ternary_bit_amd/`` both receive exactly the arrays made
here and nothing else is shared between them.

Workload shapes follow the STQ1_0 descriptions on the pages (blocks of 256
weights; MoE layers with 256 routed experts and top-8 routing, per the
traictory.com article "Tencent's 200GB Hy4-preview ...", section "The claim,
stated precisely").  The pages measure on real Hy4 weights and calibration
data that are not available; Gaussian stand-ins of the stated shapes are used
instead (weights N(0, 0.02), activations N(0, 1)).

Host draws use NumPy's PCG64 (``numpy.random.default_rng``).  Full-size
tables (256 experts x 4096 x 7168 weights) are drawn on the GPU with torch's
seeded Philox generator, one expert at a time, because a host draw of 7.5e9
normals would take minutes; tests that check those against the oracle copy
the sampled rows of the same fp32 draw back to the host.
"""
from __future__ import annotations

import numpy as np

QK = 256  # weights per STQ1_0 block (shape constant only)
WEIGHT_STD = 0.02


# ----------------------------------------------------------------------------
# bf16 activations: the workloads feed bf16 inputs; both sides get the same bits
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even) and return the uint16 bits."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to the fp32 value they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_normal(rng: np.random.Generator, shape) -> tuple[np.ndarray, np.ndarray]:
    """N(0,1) activations rounded to bf16: returns (uint16 bits, fp32 values)."""
    bits = f32_to_bf16_bits(rng.normal(0.0, 1.0, size=shape).astype(np.float32))
    return bits, bf16_bits_to_f32(bits)


# ----------------------------------------------------------------------------
# weights and calibration statistics
# ----------------------------------------------------------------------------
def gaussian_weights(seed: int, n_rows: int, k: int, std: float = WEIGHT_STD) -> np.ndarray:
    """iid N(0, std) fp32 weight matrix [n_rows, k] (row-major, rows x K)."""
    return np.random.default_rng(seed).normal(0.0, std, size=(n_rows, k)).astype(np.float32)


def imatrix_from_calibration(calib: np.ndarray) -> np.ndarray:
    """Diagonal importance per input column: mean over calibration vectors of x_k^2.

    The pages contrast the diagonal-only imatrix with the full Hessian XX^T
    (lemmy post 66506, paragraph "Full-Hessian scoring"); its diagonal,
    normalised by the number of vectors, is this statistic.  Computed in fp64,
    handed over as fp32.
    """
    c = np.asarray(calib, dtype=np.float64)
    return (c * c).mean(axis=0).astype(np.float32)


def calibration_imatrix(seed: int, n_vec: int, k: int) -> np.ndarray:
    return imatrix_from_calibration(np.random.default_rng(seed).normal(0.0, 1.0, size=(n_vec, k)))


def heavy_tailed_imatrix(seed: int, n_vec: int, k: int, frac: float = 0.02, scale: float = 30.0) -> np.ndarray:
    """Importance from calibration vectors with outlier channels: a random
    `frac` of the k input channels have activations `scale` times larger
    (N(0, scale^2) instead of N(0, 1)), as in the activation outliers that
    make some input columns dominate the weighted error."""
    rng = np.random.default_rng(seed)
    sigma = np.ones(k)
    sigma[rng.choice(k, max(1, int(round(frac * k))), replace=False)] = scale
    return imatrix_from_calibration(rng.normal(0.0, 1.0, size=(n_vec, k)) * sigma)


def paired_channel_layer(seed: int, n_rows: int, k: int, n_vec: int, sign: float, coupling: float,
                         std: float = WEIGHT_STD):
    """One synthetic layer whose Hessian has strong off-diagonal terms.

    Within every 256-column block, column j+128 is paired with column j: its
    calibration activation is `coupling` * x_j plus independent noise of the
    remaining variance, and its weight is `sign` * w_j.  Paired columns sit
    in different groups of four, so a sign-symmetric quantizer makes their
    weight errors equal up to `sign`; the off-diagonal Hessian terms then
    scale the expected error by about 1 + sign * coupling against the
    diagonal-only estimate.  Returns (w fp32 [n_rows, k], x fp32 [n_vec, k])."""
    if k % 256:
        raise ValueError("k must be a multiple of 256")
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, size=(n_vec, k // 256, 2, 128))
    x[:, :, 1] = coupling * x[:, :, 0] + np.sqrt(max(0.0, 1.0 - coupling * coupling)) * x[:, :, 1]
    w = rng.normal(0.0, std, size=(n_rows, k // 256, 2, 128))
    w[:, :, 1] = sign * w[:, :, 0]
    return w.reshape(n_rows, k).astype(np.float32), x.reshape(n_vec, k).astype(np.float32)


# ----------------------------------------------------------------------------
# named workloads
# ----------------------------------------------------------------------------
def single_gemv_case():
    """Small GEMV case: W 256x1024 ~ N(0,0.02) (seed 0), imatrix from 64 N(0,1)
    calibration vectors (seed 1), x 1x1024 fp32 N(0,1) (seed 2)."""
    w = gaussian_weights(0, 256, 1024)
    q = calibration_imatrix(1, 64, 1024)
    x = np.random.default_rng(2).normal(0.0, 1.0, size=1024).astype(np.float32)
    return w, q, x


def uniform_topk_pairs(seed: int, n_tokens: int, n_experts: int = 256, top_k: int = 8):
    """Decode routing: per token, top_k distinct experts drawn uniformly.

    Returns (pair_expert, pair_token) int32 arrays of length n_tokens*top_k,
    token-major (token t's experts are pairs t*top_k ... t*top_k+top_k-1).
    """
    rng = np.random.default_rng(seed)
    experts = np.stack([rng.choice(n_experts, top_k, replace=False) for _ in range(n_tokens)])
    pair_expert = experts.reshape(-1).astype(np.int32)
    pair_token = np.repeat(np.arange(n_tokens, dtype=np.int32), top_k)
    return pair_expert, pair_token


def routing_weights(seed: int, n_tokens: int, top_k: int = 8) -> np.ndarray:
    """Decode routing weights, fp32 [n_tokens*top_k] token-major: per token the
    softmax of top_k N(0,1) draws (positive, summing to 1)."""
    z = np.random.default_rng(seed).normal(0.0, 1.0, size=(n_tokens, top_k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32).reshape(-1)


def prefill_routing(seed: int, n_tokens: int, n_experts: int = 256, top_k: int = 8):
    """Prefill routing: router logits N(0,1); softmax top-k (= top-k of the logits).

    Returns (row_token, offsets): the (token, expert) pairs counting-sorted by
    expert, stable in token order, as the token index of every sorted row
    (int64 [n_tokens*top_k]) and the expert prefix sums (int32 [n_experts+1]).
    """
    logits = np.random.default_rng(seed).normal(0.0, 1.0, size=(n_tokens, n_experts))
    top = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]
    counts = np.bincount(top.reshape(-1), minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].astype(np.int64).copy()
    row_token = np.empty(n_tokens * top_k, dtype=np.int64)
    for t in range(n_tokens):           # token order => stable within each expert
        for e in top[t]:
            row_token[fill[e]] = t
            fill[e] += 1
    return row_token, offsets


# ----------------------------------------------------------------------------
# GPU-side draws for full-size tables (torch is used as a seeded RNG only)
# ----------------------------------------------------------------------------
def torch_expert_weights(seed: int, expert: int, n_rows: int, k: int, device="cuda", std: float = WEIGHT_STD):
    """fp32 [n_rows, k] ~ N(0, std) for one expert, drawn on `device` with a
    Philox generator seeded by (seed, expert).  Deterministic for a given torch build."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 100003 + int(expert))
    w = torch.randn((n_rows, k), generator=g, device=device, dtype=torch.float32)
    return w.mul_(std)


def torch_bf16_normal(seed: int, shape, device="cuda"):
    """bf16 N(0,1) activations drawn on `device` (fp32 draw, RNE to bf16)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
