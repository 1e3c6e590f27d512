"""The encoder's alternating rounds against the amax baseline on synthetic
rows, with near-uniform importance and with outlier-channel importance.

The pages' point (lemmy.durstig.online post 66506, "Scale and zero position
are fit together"): the zero should go where zeroing adds the least
importance-weighted error, which is not always the smallest weight; rounds of
refitting d and re-choosing zeros therefore matter most when a few input
channels dominate the importance.  These checks run the oracle only."""
import numpy as np
import pytest

from oracle import stq_oracle as O
import synth_inputs as S

N, K = 256, 1024


def _reductions(q):
    w = S.gaussian_weights(0, N, K)
    err = lambda packed: O.weighted_error(w, O.dequantize_rows(packed, N, K), q)
    e_amax = err(O.quantize_rows(w, q, encoder="amax"))
    return {r: 1.0 - err(O.quantize_rows(w, q, rounds=r)) / e_amax for r in (0, 1, 2, 3, 5)}


@pytest.fixture(scope="module")
def study():
    return {"uniform": _reductions(S.calibration_imatrix(1, 64, K)),
            "outliers": _reductions(S.heavy_tailed_imatrix(1, 64, K))}


def test_rounds_never_lose(study):
    for name, red in study.items():
        rs = sorted(red)
        assert all(red[a] <= red[b] + 1e-12 for a, b in zip(rs, rs[1:])), name


def test_well_below_amax(study):
    for name, red in study.items():
        assert red[3] >= 0.85, (name, red[3])


def test_rounds_matter_more_with_outlier_channels(study):
    gain_u = study["uniform"][3] - study["uniform"][0]
    gain_o = study["outliers"][3] - study["outliers"][0]
    assert gain_o > 10 * gain_u and gain_o > 0.01, (gain_u, gain_o)
    # the rounds remove over a quarter of the error left by the first fit
    left0, left3 = 1 - study["outliers"][0], 1 - study["outliers"][3]
    assert left3 < 0.75 * left0


def test_zeros_move_off_the_smallest_weight_more_often_with_outliers():
    w = S.gaussian_weights(0, N, K)
    moved = {}
    for name, q in (("uniform", S.calibration_imatrix(1, 64, K)), ("outliers", S.heavy_tailed_imatrix(1, 64, K))):
        tr = O.encode_trace(w, q, rounds=3)
        moved[name] = float(np.mean(tr["z"][0] != tr["z"][-1]))
    assert moved["outliers"] > moved["uniform"] > 0.0
