"""GPU-resident STQ1_0 workloads for the benchmark and the GPU tests.

Builds the expert tables and routed activations the workloads need, from the
seeded draws in ``synth_inputs`` and the library's own encoder.  Nothing here
is used by the oracle; tests that compare against the oracle copy the raw
fp32 weight rows they sample back to the host and let the oracle encode them.
"""
from __future__ import annotations

import numpy as np
import torch

import sparse_ternary_bit_amd as stq
import synth_inputs as S

N_EXPERTS = 256
N_ROWS = 4096      # gate + up rows of one expert (2 x 2048)
K = 7168
D_FF = N_ROWS // 2  # down projection: [K, D_FF] per expert
DOWN_SEED = 3000
TOP_K = 8
TABLE_SEED = 2000
IMATRIX_SEED = 3


def expert_stride(n: int = N_ROWS, k: int = K) -> int:
    """Bytes between experts: n rows rounded up to 16 bytes (4,816,896 at 4096 x 7168)."""
    b = n * stq.row_bytes(k)
    return (b + 15) // 16 * 16


def table_imatrix(k: int = K, device="cuda") -> torch.Tensor:
    return torch.from_numpy(S.calibration_imatrix(IMATRIX_SEED, 64, k)).to(device)


def encode_table(n_experts: int = N_EXPERTS, n: int = N_ROWS, k: int = K, seed: int = TABLE_SEED,
                 encoder: int = stq.ENC_WLS, rounds: int = 3, imatrix: torch.Tensor | None = None,
                 device="cuda") -> tuple[torch.Tensor, int]:
    """Draw each expert's fp32 weights on the GPU and encode them with the library.

    Returns (table uint8 [n_experts * stride], stride)."""
    stride = expert_stride(n, k)
    table = torch.zeros(n_experts * stride, dtype=torch.uint8, device=device)
    rb = stq.row_bytes(k)
    for e in range(n_experts):
        w = S.torch_expert_weights(seed, e, n, k, device=device)
        out = table[e * stride: e * stride + n * rb]
        stq.quantize_rows(w, imatrix, encoder=encoder, rounds=rounds, out=out)
        del w
    return table, stride


def encode_down_table(n_experts: int = N_EXPERTS, d_model: int = K, d_ff: int = D_FF, seed: int = DOWN_SEED,
                      device="cuda") -> tuple[torch.Tensor, int]:
    """Down projections [d_model, d_ff] of every expert, drawn like the gate/up table
    (N(0, 0.02), no imatrix), encoded by the library with 3 WLS rounds."""
    return encode_table(n_experts, d_model, d_ff, seed=seed, imatrix=None, device=device)


def expert_weight_rows(seed: int, expert: int, rows, n: int = N_ROWS, k: int = K, device="cuda") -> np.ndarray:
    """The same fp32 draw as encode_table, rows `rows` of expert `expert`, on the host."""
    w = S.torch_expert_weights(seed, expert, n, k, device=device)
    idx = torch.as_tensor(np.asarray(rows, dtype=np.int64), device=device)
    return w.index_select(0, idx).cpu().numpy()


def decode_pairs(seed: int, n_tokens: int, n_experts: int = N_EXPERTS, top_k: int = TOP_K, device="cuda"):
    pe, pt = S.uniform_topk_pairs(seed, n_tokens, n_experts, top_k)
    return (torch.from_numpy(pe).to(device), torch.from_numpy(pt).to(device), pe, pt)


def prefill_batch(n_tokens: int = 2048, k: int = K, n_experts: int = N_EXPERTS, top_k: int = TOP_K,
                  routing_seed: int = 7, x_seed: int = 8, device="cuda"):
    """Routed prefill activations grouped by expert.

    Returns (x_sorted bf16 [n_tokens*top_k, k] on device, offsets int32 [n_experts+1]
    on device, row_token int64 numpy, offsets numpy)."""
    row_token, offsets = S.prefill_routing(routing_seed, n_tokens, n_experts, top_k)
    x = S.torch_bf16_normal(x_seed, (n_tokens, k), device=device)
    x_sorted = x.index_select(0, torch.from_numpy(row_token).to(device)).contiguous()
    return x_sorted, torch.from_numpy(offsets).to(device), row_token, offsets
