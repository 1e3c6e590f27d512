"""CPU checks of the prefill routing harness (top-k routing, then a stable
counting sort of the (token, expert) pairs by expert), which lays out the
grouped GEMM's input.  The pages' MoE routes each token to the top 8 of its
256 routed experts (traictory.com, "Tencent's 200GB Hy4-preview: a 7x
compression claim that needs a second look", section "The claim, stated
precisely").  Each check uses a property that defines the result, not the
harness's own steps."""
import numpy as np
import pytest

import synth_inputs as S


def _check_routing(seed, n_tokens, n_experts, top_k):
    row_token, offsets = S.prefill_routing(seed, n_tokens, n_experts, top_k)
    logits = np.random.default_rng(seed).normal(0.0, 1.0, size=(n_tokens, n_experts))
    assert row_token.shape == (n_tokens * top_k,) and offsets.shape == (n_experts + 1,)
    assert offsets[0] == 0 and offsets[-1] == n_tokens * top_k and np.all(np.diff(offsets) >= 0)
    # every token appears exactly top_k times
    np.testing.assert_array_equal(np.bincount(row_token, minlength=n_tokens), np.full(n_tokens, top_k))
    chosen = np.zeros((n_tokens, n_experts), dtype=bool)
    for e in range(n_experts):
        toks = row_token[offsets[e]:offsets[e + 1]]
        # rows of one expert are distinct tokens in increasing order (stable in token order)
        assert np.all(np.diff(toks) > 0), e
        chosen[toks, e] = True
    # the experts a token reaches are its top_k logits: each chosen logit beats every other one
    assert np.all(chosen.sum(axis=1) == top_k)
    lo_chosen = np.where(chosen, logits, np.inf).min(axis=1)
    hi_other = np.where(chosen, -np.inf, logits).max(axis=1)
    assert np.all(lo_chosen > hi_other)
    # offsets are the prefix sums of the per-expert counts
    np.testing.assert_array_equal(np.diff(offsets), chosen.sum(axis=0))
    return row_token, offsets


@pytest.mark.parametrize("seed,n_tokens,n_experts,top_k", [(0, 1, 4, 1), (1, 37, 16, 4), (2, 200, 64, 8)])
def test_prefill_routing_small(seed, n_tokens, n_experts, top_k):
    _check_routing(seed, n_tokens, n_experts, top_k)


def test_prefill_routing_full_size():
    # 2048 tokens, top-8 of 256: 16384 rows, per-expert counts ~ Binomial(2048, 1/32)
    row_token, offsets = _check_routing(7, 2048, 256, 8)
    counts = np.diff(offsets)
    assert counts.sum() == 16384 and abs(counts.mean() - 64.0) < 1e-12
    assert 4.0 < counts.std() < 12.0 and counts.min() > 0


def test_gathered_rows_are_the_routed_tokens():
    # x_sorted = x[row_token]: row offsets[e] + j is the j-th token (in token order) routed to e
    row_token, offsets = S.prefill_routing(3, 50, 8, 2)
    x = np.arange(50 * 3, dtype=np.float64).reshape(50, 3)
    xs = x[row_token]
    for e in range(8):
        for j, r in enumerate(range(offsets[e], offsets[e + 1])):
            t = int(xs[r, 0]) // 3
            assert row_token[r] == t
            assert j == int(np.sum(row_token[offsets[e]:r] < t))
