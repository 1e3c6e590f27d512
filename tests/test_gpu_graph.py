"""The decode and prefill entry points under HIP graph capture: a call
captured into a graph with a workspace the test owns, and replayed several
times with eager work and synchronisation between replays (new inputs, and
a larger eager call of the same entry point with its own workspace), gives
on every replay exactly the eager result for the inputs present at that
replay.  No memset is recorded: the kernels write every output element they
own, and the library allocates nothing, so nothing a replay touches can be
freed or moved by the calls between replays."""
import numpy as np
import pytest
import torch

from oracle import stq_oracle as O
import synth_inputs as S

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def stq():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import sparse_ternary_bit_amd as m
    return m


def _table(seed, n_experts, n, k):
    rb = O.row_bytes(k)
    stride = (n * rb + 15) // 16 * 16
    t = np.zeros(n_experts * stride, dtype=np.uint8)
    for e in range(n_experts):
        t[e * stride: e * stride + n * rb] = O.quantize_rows(S.gaussian_weights(seed + e, n, k), None)
    return torch.from_numpy(t).cuda(), stride


def _replay_matches_eager(capture_fn, eager_fn, refresh, out, larger=None, reps=4):
    capture_fn()                                  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            capture_fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(reps):
        refresh(r)                                # new inputs, written eagerly
        if larger is not None:
            larger()                              # a bigger eager call between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        want = eager_fn()
        torch.cuda.synchronize()
        assert torch.equal(got, want), r


def test_gemv_split_k_under_graph(stq):
    # one expert, one token: the k split and its ordered reduction both run in the graph
    n, k = 1024, 2048
    table, stride = _table(70, 3, n, k)
    x = S.torch_bf16_normal(71, (1, k))
    pe = torch.tensor([1], dtype=torch.int32, device="cuda")
    y = torch.empty((1, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(stq.gemv_plan(3, n, k, 1)[2], dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0                                 # the call splits k
    cap = lambda: stq.gemv(table, stride, 3, n, k, x, pe, out=y, workspace=ws)
    eager = lambda: stq.gemv(table, stride, 3, n, k, x, pe)
    xl = S.torch_bf16_normal(79, (6, k))
    pel = torch.tensor([0, 1, 2, 2, 1, 0], dtype=torch.int32, device="cuda")
    larger = lambda: stq.gemv(table, stride, 3, n, k, xl, pel)

    def refresh(r):
        x.copy_(S.torch_bf16_normal(72 + r, (1, k)))
        pe.fill_(r % 3)
    _replay_matches_eager(cap, eager, refresh, y, larger)


def test_gemv_batch_under_graph(stq):
    n, k, E, T = 768, 1024, 6, 5
    table, stride = _table(80, E, n, k)
    x = S.torch_bf16_normal(81, (T, k))
    pe_np, pt_np = S.uniform_topk_pairs(82, T, E, 3)
    pe = torch.from_numpy(pe_np).cuda()
    pt = torch.from_numpy(pt_np).cuda()
    y = torch.empty((T * 3, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, stq.gemv_plan(E, n, k, T * 3)[2]), dtype=torch.uint8, device="cuda")
    cap = lambda: stq.gemv(table, stride, E, n, k, x, pe, pt, out=y, workspace=ws)
    eager = lambda: stq.gemv(table, stride, E, n, k, x, pe, pt)

    def refresh(r):
        x.copy_(S.torch_bf16_normal(83 + r, (T, k)))
        pe.copy_(torch.from_numpy(S.uniform_topk_pairs(90 + r, T, E, 3)[0]).cuda())
    _replay_matches_eager(cap, eager, refresh, y)


def test_grouped_gemm_under_graph(stq):
    n, k = 256, 512
    offsets = torch.tensor([0, 20, 20, 101, 130], dtype=torch.int32, device="cuda")
    table, stride = _table(100, 4, n, k)
    x = S.torch_bf16_normal(101, (130, k))
    y = torch.empty((130, n), dtype=torch.float32, device="cuda")
    cap = lambda: stq.grouped_gemm(table, stride, 4, n, k, x, offsets, out=y)
    eager = lambda: stq.grouped_gemm(table, stride, 4, n, k, x, offsets)
    _replay_matches_eager(cap, eager, lambda r: x.copy_(S.torch_bf16_normal(102 + r, (130, k))), y)


def test_moe_ffn_under_graph(stq):
    d_model, d_ff, E, T, top_k = 512, 256, 4, 3, 2
    tg, sg = _table(110, E, 2 * d_ff, d_model)
    td, sd = _table(120, E, d_model, d_ff)
    x = S.torch_bf16_normal(111, (T, d_model))
    pe = torch.tensor([0, 1, 2, 1, 3, 0], dtype=torch.int32, device="cuda")
    pw = torch.from_numpy(S.routing_weights(112, T, top_k)).cuda()
    y = torch.empty((T, d_model), dtype=torch.float32, device="cuda")
    ws = torch.empty(stq.moe_ffn_workspace(E, d_model, d_ff, T, top_k), dtype=torch.uint8, device="cuda")
    cap = lambda: stq.moe_ffn_decode(tg, sg, td, sd, E, d_model, d_ff, x, pe, pw, top_k, out=y, workspace=ws)
    eager = lambda: stq.moe_ffn_decode(tg, sg, td, sd, E, d_model, d_ff, x, pe, pw, top_k)
    xl = S.torch_bf16_normal(119, (8, d_model))
    pel = torch.from_numpy(np.tile(np.arange(E, dtype=np.int32), 4)).cuda()
    pwl = torch.from_numpy(S.routing_weights(118, 8, top_k)).cuda()
    larger = lambda: stq.moe_ffn_decode(tg, sg, td, sd, E, d_model, d_ff, xl, pel, pwl, top_k)

    def refresh(r):
        x.copy_(S.torch_bf16_normal(113 + r, (T, d_model)))
        pw.copy_(torch.from_numpy(S.routing_weights(114 + r, T, top_k)).cuda())
    _replay_matches_eager(cap, eager, refresh, y, larger)


def test_layer_errors_under_graph(stq):
    # the H diagonal and per-tile partial sums live in the caller's workspace
    n, k, n_cal = 130, 512, 70
    w = S.torch_expert_weights(130, 0, n, k)
    x = S.torch_expert_weights(131, 0, n_cal, k, std=1.0)
    w_hat = stq.q2_roundtrip(w)
    ef = torch.empty(n, dtype=torch.float64, device="cuda")
    ed = torch.empty(n, dtype=torch.float64, device="cuda")
    both = torch.empty(2 * n, dtype=torch.float64, device="cuda")
    ws = torch.empty(stq.layer_errors_workspace(n, k, n_cal), dtype=torch.uint8, device="cuda")
    cap = lambda: (stq.layer_errors(w, w_hat, x, ef, ed, workspace=ws), both[:n].copy_(ef), both[n:].copy_(ed))
    wl = S.torch_expert_weights(133, 0, 2 * n, k)
    larger = lambda: stq.layer_errors(wl, stq.q2_roundtrip(wl), x)

    def eager():
        f, d = stq.layer_errors(w, w_hat, x)
        return torch.cat([f, d])

    def refresh(r):
        x.copy_(S.torch_expert_weights(132 + r, 0, n_cal, k, std=1.0))
    _replay_matches_eager(cap, eager, refresh, both, larger)
