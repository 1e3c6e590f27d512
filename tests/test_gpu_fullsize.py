"""Full-size parity on the benchmark's shapes: the 256-expert table of
4096 x 7168 gate+up matrices, the single-expert decode GEMV, the 16-token MoE
decode step, the batch-64 sweep point and the 2048-token prefill grouped
GEMM.  Sampled outputs are recomputed one by one by the oracle from the raw
fp32 weights (the oracle encodes the sampled rows itself)."""
import numpy as np
import pytest
import torch

from oracle import stq_oracle as O
import synth_inputs as S

pytestmark = pytest.mark.gpu

K, N = 7168, 4096
GEMV_TOL, GEMM_TOL = 1e-3, 2e-3


@pytest.fixture(scope="module")
def W():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import stq_workloads
    return stq_workloads


@pytest.fixture(scope="module")
def table(W):
    q = W.table_imatrix()
    t, stride = W.encode_table(imatrix=q)
    torch.cuda.synchronize()
    return t, stride, q.cpu().numpy()


def _packed_rows(t, stride, e, rows):
    """Blocks [len(rows), nb, 42] of rows `rows` of expert e, read from the GPU table."""
    blob = t[e * stride: e * stride + N * O.row_bytes(K)].cpu().numpy()
    return O.unpack_matrix(blob, N, K // 256)[np.asarray(rows)]


def _oracle_rows(W, e, rows, q):
    """The oracle's own encoding of rows `rows` of expert e (from the raw fp32
    draw), as a packed matrix of len(rows) rows."""
    w = W.expert_weight_rows(W.TABLE_SEED, e, rows)
    return O.quantize_rows(w, q)


def _oracle_blocks(W, e, rows, q):
    return O.unpack_matrix(_oracle_rows(W, e, rows, q), len(rows), K // 256)


def test_table_bytes_match_oracle(W, table):
    t, stride, q = table
    rng = np.random.default_rng(0)
    for e in (0, 1, 137, 255):
        rows = np.unique(np.concatenate([[0, 1, 2047, 2048, 4095], rng.integers(0, N, 11)]))
        assert np.array_equal(_packed_rows(t, stride, e, rows), _oracle_blocks(W, e, rows, q)), e


def test_amax_table_bytes_match_oracle(W):
    q = W.table_imatrix()
    t, stride = W.encode_table(n_experts=3, imatrix=q, encoder=1)
    rows = np.array([0, 5, 4095])
    w = W.expert_weight_rows(W.TABLE_SEED, 2, rows)
    assert np.array_equal(_packed_rows(t, stride, 2, rows),
                          O.unpack_matrix(O.quantize_rows(w, None, encoder="amax"), len(rows), K // 256))


def _check_pairs(W, table, y, pe, pt, xf, pairs, rows):
    t, stride, q = table
    for i in pairs:
        e, tok = int(pe[i]), int(pt[i])
        raw = _oracle_rows(W, e, rows, q)
        y_ref = O.gemv(raw, len(rows), K, xf[tok])
        A = O.tolerance_scale(raw, len(rows), K, xf[tok])[0]
        err = np.abs(y[i, rows].astype(np.float64) - y_ref)
        assert np.all(err <= GEMV_TOL * A), (i, e, tok, float(np.max(err / A)))


def test_single_expert_gemv(W, table):
    import sparse_ternary_bit_amd as stq
    t, stride, q = table
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 4095], rng.integers(0, N, 30)]))
    for draw in (0, 57, 99):
        x = S.torch_bf16_normal(4000 + draw, (1, K))
        pe = torch.tensor([draw], dtype=torch.int32, device="cuda")
        y = stq.gemv(t, stride, W.N_EXPERTS, N, K, x, pe).cpu().numpy()
        xf = x.float().cpu().numpy()
        _check_pairs(W, table, y, [draw], [0], xf, [0], rows)


@pytest.mark.parametrize("n_tokens,seed", [(16, 6), (64, 5064), (1, 5001)])
def test_moe_decode_step(W, table, n_tokens, seed):
    import sparse_ternary_bit_amd as stq
    t, stride, q = table
    pe_t, pt_t, pe, pt = W.decode_pairs(seed, n_tokens)
    x = S.torch_bf16_normal(seed + 1, (n_tokens, K))
    y = stq.gemv(t, stride, W.N_EXPERTS, N, K, x, pe_t, pt_t).cpu().numpy()
    assert y.shape == (n_tokens * 8, N) and np.all(np.isfinite(y))
    xf = x.float().cpu().numpy()
    rng = np.random.default_rng(seed)
    pairs = rng.choice(len(pe), size=min(8, len(pe)), replace=False)
    rows = np.unique(np.concatenate([[0, 4095], rng.integers(0, N, 14)]))
    _check_pairs(W, table, y, pe, pt, xf, pairs, rows)


def test_prefill_grouped_gemm(W, table):
    """The 2048-token prefill: six experts' outputs (every row routed to each,
    14 sampled columns) against the oracle.  The oracle's activation rows are
    the unsorted draw indexed by the routing (host side), not the permuted
    copy the kernel read, so a wrong permutation fails here; each expert is
    checked elementwise and normwise on its own."""
    import sparse_ternary_bit_amd as stq
    t, stride, q = table
    x_sorted, offsets_t, row_token, offsets = W.prefill_batch()
    assert offsets[-1] == 16384 and int(np.max(np.diff(offsets))) > 64
    y = stq.grouped_gemm(t, stride, W.N_EXPERTS, N, K, x_sorted, offsets_t)
    torch.cuda.synchronize()
    x = S.torch_bf16_normal(8, (2048, K)).float().cpu().numpy()   # the draw prefill_batch routes
    rng = np.random.default_rng(2)
    cols = np.unique(np.concatenate([[0, 4095], rng.integers(0, N, 12)]))
    experts = np.unique(np.concatenate([[0, 255, int(np.argmax(np.diff(offsets)))], rng.integers(1, 255, 3)]))
    for e in experts:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        xs = x[row_token[lo:hi]]
        ys = y[lo:hi].cpu().numpy()[:, cols].astype(np.float64)
        raw = _oracle_rows(W, int(e), cols, q)
        y_ref = O.gemv_tokens(raw, len(cols), K, xs)
        A = O.tolerance_scale(raw, len(cols), K, xs)
        err = np.abs(ys - y_ref)
        assert np.all(err <= GEMM_TOL * A), (int(e), float(np.max(err / A)))
        assert np.max(err) <= GEMM_TOL * np.max(np.abs(y_ref)), int(e)
