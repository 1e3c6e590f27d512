"""Oracle encodings of many full-size matrices at once (test infrastructure:
the full-size GPU tests hand the oracle raw fp32 weights, and one 4096 x 7168
WLS encoding takes several seconds on one core).  The encoder's array
operations release the interpreter lock, so a thread pool spreads them over
the cores; each matrix is encoded by the unchanged oracle."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

from oracle import stq_oracle as O


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def encode_all(mats, imatrix=None) -> list:
    """O.quantize_rows(w, imatrix) (WLS, 3 rounds) of every fp32 matrix in `mats`, in order."""
    mats = list(mats)
    with ThreadPoolExecutor(max_workers=min(workers(), max(1, len(mats)))) as ex:
        return list(ex.map(lambda w: O.quantize_rows(w, imatrix), mats))
