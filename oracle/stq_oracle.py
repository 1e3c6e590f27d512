"""STQ1_0 CPU oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct NumPy implementation of what the STQ1_0
sparse-ternary quantized matmul computes.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP library (no kernels, headers,
tables or helpers); the only thing both sides see is the seeded inputs from
``synth_inputs``.

Sources ("the pages"), cited by title/address and section:
  [LEMMY]  lemmy.durstig.online post 66506 (a relayed Reddit post), with run-in
           paragraphs "Four weights, five bits", "Scale and zero position are
           fit together", "Full-Hessian scoring", "Runtime".
  [AGI]    "Tencent compresses 770B Hunyuan Hy4 Preview into 214 GiB at ~2.38
           bits per weight" (agihunt.info), sections "Four weights, five bits",
           "Fitting and runtime".
  [TRAIC]  "Tencent's 200GB Hy4-preview: a 7x compression claim that needs a
           second look" (traictory.com), section "MIX-STQ1_0: where the bits go".
  [ALPHA]  "AngelSlim Shrinks Tencent's 1.5TB Hy4-Preview to 214 GiB at 6x
           Compression" (alphasignal.ai), summary bullets and section
           "How STQ1_0 works".

What the pages fix: each group of four weights takes values in {-d, 0, +d}
with exactly one zero lane; 4 zero positions x 8 sign choices = 32 patterns,
5 bits per group ([LEMMY] "Four weights, five bits"); the 5 bits are a 4-bit
code plus a 1-bit table select into a 32-entry codebook, and one fp16 scale is
shared by 256 weights, 42 bytes per block ([ALPHA] "How STQ1_0 works").  The
encoder alternates a weighted-least-squares fit of d with an
imatrix-weighted choice of the zero lane, for three rounds, and is compared
against an amax-scaled original encoder ([LEMMY] "Scale and zero position are
fit together"; [AGI] "Fitting and runtime"; [ALPHA] bullets).

Where the pages are silent the readings below are build decisions (bit order,
reduction order, rounding of d, the starting pattern); each is stated at the
function that makes it.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(format, encoder, GEMV), ``tests/test_oracle_ffn.py`` (routed-expert FFN) and
``tests/test_oracle_sensitivity.py`` (layer error, the 2-bit stand-in,
greedy allocation) against enumeration, exact rational arithmetic, closed
forms, hand-built cases or brute force.
"""
from __future__ import annotations

import numpy as np

QK = 256                 # weights per block                 [LEMMY] "Four weights, five bits"
GROUP = 4                # weights per group                 [LEMMY] "Four weights, five bits"
NGROUPS = QK // GROUP    # 64 groups per block
BLOCK_BYTES = 42         # 2 (fp16 d) + 32 (4-bit codes) + 8 (select bits)   [ALPHA] "How STQ1_0 works"
FP16_MAX = 65504.0


# -----------------------------------------------------------------------------
# O1: the 32-entry codebook
# -----------------------------------------------------------------------------
def pattern_of_code(c: int) -> tuple[int, int, int, int]:
    """Ternary pattern (t0, t1, t2, t3) of code c in [0, 32).

    Reading (the pages give no order): c = 8*z + m.  z = c >> 3 is the zero
    lane; the three other lanes, taken in increasing lane order, get -1 when
    their bit of m is set (lowest lane -> bit 0) and +1 otherwise.  The
    "table select" bit (c >> 4) is therefore 1 exactly when the zero sits in
    lanes 2..3, and the 4-bit code is c & 15.
    """
    if not 0 <= c < 32:
        raise ValueError("code out of range")
    z, m = c >> 3, c & 7
    out, r = [], 0
    for j in range(GROUP):
        if j == z:
            out.append(0)
        else:
            out.append(-1 if (m >> r) & 1 else 1)
            r += 1
    return tuple(out)


CODEBOOK = np.array([pattern_of_code(c) for c in range(32)], dtype=np.int8)  # [32, 4]


def codes_from_pattern(z: np.ndarray, neg: np.ndarray) -> np.ndarray:
    """Inverse of the codebook for arrays: z [...] zero lane, neg [..., 4] sign flags.

    The sign flag of the zero lane is ignored.
    """
    z = np.asarray(z, dtype=np.int64)
    neg = np.asarray(neg, dtype=bool)
    m = np.zeros(z.shape, dtype=np.int64)
    for j in range(GROUP):
        rank = j - (j > z).astype(np.int64)            # rank of lane j among the nonzero lanes
        bit = neg[..., j] & (z != j)
        m |= bit.astype(np.int64) << np.where(z != j, rank, 0)
    return (8 * z + m).astype(np.uint8)


# -----------------------------------------------------------------------------
# O2: block byte layout
# -----------------------------------------------------------------------------
def qs_position(g: int) -> tuple[int, int]:
    """(byte offset inside the block, bit shift) of the 4-bit code of group g.

    Reading (the pages fix only the 42-byte total): bytes 2..33 hold the 64
    four-bit codes.  Group g sits in byte 2 + 4*(g >> 3) + (g & 3), low nibble
    when bit 2 of g is clear, high nibble otherwise.  So the 32-bit word w of
    this field carries groups 8w..8w+7 and groups with equal g & 3 share a byte
    lane.
    """
    return 2 + 4 * (g >> 3) + (g & 3), 4 * ((g >> 2) & 1)


def qh_position(g: int) -> tuple[int, int]:
    """(byte offset inside the block, bit index) of the select bit of group g.

    Reading: bytes 34..41 hold the 64 select bits.  Group g's bit is bit
    ((g >> 2) & 7) of byte 34 + 4*(g >> 5) + (g & 3): the same byte lane as its
    code nibble, so the eight select bits for code word w sit at bits 2*(w&3)
    and 2*(w&3)+1 of the four bytes of select word w >> 2.
    """
    return 34 + 4 * (g >> 5) + (g & 3), (g >> 2) & 7


def pack_blocks(d16_bits: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Pack fp16 scale bits [nb] and 5-bit codes [nb, 64] into blocks [nb, 42].

    Bytes 0..1 hold d as IEEE binary16, little-endian.
    """
    d16_bits = np.asarray(d16_bits, dtype=np.uint16).reshape(-1)
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1, NGROUPS)
    nb = codes.shape[0]
    if d16_bits.shape[0] != nb:
        raise ValueError("one scale per block")
    if np.any(codes >= 32):
        raise ValueError("codes are 5-bit")
    out = np.zeros((nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, 0] = (d16_bits & 0xFF).astype(np.uint8)
    out[:, 1] = (d16_bits >> 8).astype(np.uint8)
    for g in range(NGROUPS):
        byte, shift = qs_position(g)
        out[:, byte] |= ((codes[:, g] & 15) << shift).astype(np.uint8)
        byte, bit = qh_position(g)
        out[:, byte] |= ((codes[:, g] >> 4) << bit).astype(np.uint8)
    return out


def unpack_blocks(raw: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Inverse of pack_blocks: blocks [nb, 42] -> (d16 bits [nb], codes [nb, 64])."""
    raw = np.asarray(raw, dtype=np.uint8).reshape(-1, BLOCK_BYTES)
    d16 = raw[:, 0].astype(np.uint16) | (raw[:, 1].astype(np.uint16) << 8)
    codes = np.zeros((raw.shape[0], NGROUPS), dtype=np.uint8)
    for g in range(NGROUPS):
        byte, shift = qs_position(g)
        nib = (raw[:, byte] >> shift) & 15
        byte, bit = qh_position(g)
        sel = (raw[:, byte] >> bit) & 1
        codes[:, g] = nib | (sel << 4)
    return d16, codes


def row_bytes(k: int) -> int:
    """Bytes of one packed row of k weights (k must be a multiple of 256)."""
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    return k // QK * BLOCK_BYTES


TILE_ROWS = 64


def block_offset(r: int, b: int, n_rows: int, nb: int) -> int:
    """Byte offset of block b (columns 256b..256b+255) of row r in a packed matrix.

    Reading (the pages fix only the 42-byte block): a matrix of n_rows rows is
    stored in row tiles of 64 consecutive rows (the last tile holds the
    n_rows % 64 leftover rows, if any); a tile stores block 0 of each of its
    rows in row order, then block 1 of each, and so on.
    """
    t0 = (r // TILE_ROWS) * TILE_ROWS
    rows_in_tile = min(TILE_ROWS, n_rows - t0)
    return (t0 * nb + b * rows_in_tile + (r - t0)) * BLOCK_BYTES


def _matrix_offsets(n_rows: int, nb: int) -> np.ndarray:
    """block_offset for every (row, block), as an array [n_rows, nb]."""
    r = np.arange(n_rows, dtype=np.int64)[:, None]
    b = np.arange(nb, dtype=np.int64)[None, :]
    t0 = (r // TILE_ROWS) * TILE_ROWS
    rows_in_tile = np.minimum(TILE_ROWS, n_rows - t0)
    return (t0 * nb + b * rows_in_tile + (r - t0)) * BLOCK_BYTES


def pack_matrix(blocks: np.ndarray) -> np.ndarray:
    """Blocks [n_rows, nb, 42] (row r, block b) -> the packed matrix as flat bytes."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    n_rows, nb = blocks.shape[0], blocks.shape[1]
    out = np.empty(n_rows * nb * BLOCK_BYTES, dtype=np.uint8)
    off = _matrix_offsets(n_rows, nb)
    idx = off[..., None] + np.arange(BLOCK_BYTES)
    out[idx.reshape(-1)] = blocks.reshape(-1)
    return out


def unpack_matrix(q: np.ndarray, n_rows: int, nb: int) -> np.ndarray:
    """Packed matrix (flat bytes) -> blocks [n_rows, nb, 42]."""
    q = np.asarray(q, dtype=np.uint8).reshape(-1)
    if q.shape[0] != n_rows * nb * BLOCK_BYTES:
        raise ValueError("matrix size does not match n_rows x nb blocks")
    idx = _matrix_offsets(n_rows, nb)[..., None] + np.arange(BLOCK_BYTES)
    return q[idx]


# -----------------------------------------------------------------------------
# O3: decode
# -----------------------------------------------------------------------------
def fp16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def dequantize_rows(q: np.ndarray, n_rows: int, k: int) -> np.ndarray:
    """Packed matrix of n_rows rows (flat, n_rows*k/256*42 bytes) -> fp32 weights [n_rows, k].

    Each weight is its block's fp16 scale widened to fp32 times the pattern
    value: +d, -d, or +0.0 in the zero lane ([LEMMY] "Four weights, five
    bits").  The sign is applied by negation, so it is exact for every d.
    """
    blocks = unpack_matrix(q, n_rows, k // QK) if k % QK == 0 else None
    if blocks is None:
        raise ValueError("k must be a multiple of 256")
    d16, codes = unpack_blocks(blocks.reshape(-1, BLOCK_BYTES))
    d = fp16_bits_to_f32(d16)[:, None, None]                    # [nb, 1, 1]
    t = CODEBOOK[codes.astype(np.int64)]                         # [nb, 64, 4]
    w = np.where(t > 0, d, np.negative(d))
    w = np.where(t == 0, np.float32(0.0), w).astype(np.float32)
    return w.reshape(n_rows, k)


# -----------------------------------------------------------------------------
# encoders (O4 amax baseline, O5 alternating WLS / zero choice)
# -----------------------------------------------------------------------------
def fp16_scale_bits(d: np.ndarray) -> np.ndarray:
    """Round a non-negative fp64 scale to the stored fp16 bits.

    Reading ([LEMMY] says only "FP16 scale"): fp64 -> fp32 with
    round-to-nearest-even, clamp to the largest finite fp16 (65504), then
    fp32 -> fp16 with round-to-nearest-even.  fp16 subnormals are kept.
    """
    f = np.asarray(d, dtype=np.float64).astype(np.float32)
    f = np.minimum(f, np.float32(FP16_MAX))
    return f.astype(np.float16).view(np.uint16)


def _group_partial(v: np.ndarray) -> np.ndarray:
    """Per-group sum of the 4 lanes, strictly in lane order: ((v0+v1)+v2)+v3."""
    return ((v[..., 0] + v[..., 1]) + v[..., 2]) + v[..., 3]


def _tree_sum(v: np.ndarray) -> np.ndarray:
    """Sum of the last axis (length a power of two) as a balanced tree of
    adjacent pairs: level 1 adds (0,1),(2,3),..., level 2 adds those pairs, ...

    Reading: the pages do not fix a summation order; this fixed order makes
    the encoder's result unique (it is the order of a 64-lane xor butterfly).
    """
    while v.shape[-1] > 1:
        v = v[..., 0::2] + v[..., 1::2]
    return v[..., 0]


def wls_scale(absw: np.ndarray, q: np.ndarray, z: np.ndarray) -> np.ndarray:
    """Weighted-least-squares d for fixed zero lanes (signs follow w).

    absw, q: fp64 [..., 64, 4]; z: int [..., 64].  With the zero lanes and the
    signs fixed, the weighted error sum q_i (|w_i| - d)^2 over the nonzero
    lanes is a quadratic in d whose minimiser is sum(q|w|) / sum(q)
    ([LEMMY] "Scale and zero position are fit together": d is fit by weighted
    least squares).  Reading: d = 0 when every nonzero lane has q = 0.
    """
    lane = np.arange(GROUP)
    keep = lane != z[..., None]
    num = _tree_sum(_group_partial(np.where(keep, q * absw, 0.0)))
    den = _tree_sum(_group_partial(np.where(keep, q, 0.0)))
    safe = np.where(den > 0.0, den, 1.0)
    return np.where(den > 0.0, num / safe, 0.0)


def choose_zero(absw: np.ndarray, q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Zero lane per group for a fixed scale d >= 0.

    Zeroing lane j instead of keeping it at sign(w_j)*d raises the weighted
    error by q_j*d*(2|w_j| - d); the lane with the least extra error is zeroed,
    which need not be the smallest |w_j| ([LEMMY] "Scale and zero position are
    fit together").  The common factor d >= 0 is dropped, ties go to the lowest
    lane, cost = q_j * (2|w_j| - d) evaluated in fp64 in that operation order.
    """
    cost = q * (2.0 * absw - d[..., None, None])
    return np.argmin(cost, axis=-1)


def _blocks_view(w: np.ndarray, imatrix) -> tuple[np.ndarray, np.ndarray]:
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % QK:
        raise ValueError("w must be [n_rows, k] with k % 256 == 0")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weights are outside the contract")
    n, k = w.shape
    wb = w.reshape(n, k // QK, NGROUPS, GROUP)
    if imatrix is None:
        qb = np.ones_like(wb)
    else:
        qv = np.asarray(imatrix, dtype=np.float32).reshape(-1)
        if qv.shape[0] != k or not np.all(np.isfinite(qv)) or np.any(qv < 0):
            raise ValueError("imatrix must be k finite non-negative values")
        qb = np.broadcast_to(qv.reshape(1, k // QK, NGROUPS, GROUP), wb.shape)
    return wb, qb


def encode_trace(w: np.ndarray, imatrix=None, rounds: int = 3) -> dict:
    """Run the WLS encoder and keep every intermediate (for the round tests).

    Order (reading of "alternates ... three alternating rounds", [LEMMY]):
      p0 = amax pattern (zero the smallest |w| of each group, signs of w);
      repeat `rounds` times: d <- WLS(p), p <- choose(d);
      finally d <- WLS(p) so the stored d fits the stored pattern.
    Returns fp64 arrays: 'absw','q' [n,nb,64,4], 'neg' bool, and lists
    'z' (rounds+1 patterns) and 'd' (rounds+1 scales, d[r] = WLS(z[r])).
    """
    wb, qb = _blocks_view(w, imatrix)
    absw = np.abs(wb.astype(np.float64))
    q = qb.astype(np.float64)
    neg = wb < 0                                   # -0.0 counts as positive
    z = np.argmin(absw, axis=-1)                   # p0: first smallest |w|
    zs, ds = [z], []
    for _ in range(rounds):
        d = wls_scale(absw, q, z)
        ds.append(d)
        z = choose_zero(absw, q, d)
        zs.append(z)
    ds.append(wls_scale(absw, q, z))
    return {"absw": absw, "q": q, "neg": neg, "z": zs, "d": ds}


def quantize_rows(w: np.ndarray, imatrix=None, encoder: str = "wls", rounds: int = 3) -> np.ndarray:
    """Encode fp32 rows [n, k] into a packed STQ1_0 matrix (flat uint8, n*k/256*42 bytes).

    encoder='wls'  : alternating WLS scale / weighted zero choice (O5), `rounds` rounds.
    encoder='amax' : the original ternary encoder ([ALPHA] bullets: it used
                     amax scaling): d = max|w| of the block, zero the smallest
                     |w| of each group (first on ties), signs of w.  `rounds`
                     is ignored.
    A missing imatrix means q = 1 for every column.
    """
    wb, _ = _blocks_view(w, imatrix)
    n, nb = wb.shape[0], wb.shape[1]
    neg = wb < 0
    if encoder == "amax":
        absw = np.abs(wb.astype(np.float64))
        z = np.argmin(absw, axis=-1)
        d = absw.reshape(n, nb, QK).max(axis=-1)
    elif encoder == "wls":
        if rounds < 0:
            raise ValueError("rounds must be >= 0")
        tr = encode_trace(w, imatrix, rounds)
        z, d = tr["z"][-1], tr["d"][-1]
    else:
        raise ValueError("encoder must be 'wls' or 'amax'")
    codes = codes_from_pattern(z, neg)
    packed = pack_blocks(fp16_scale_bits(d).reshape(-1), codes.reshape(-1, NGROUPS))
    return pack_matrix(packed.reshape(n, nb, BLOCK_BYTES))


# -----------------------------------------------------------------------------
# O6: weighted reconstruction error
# -----------------------------------------------------------------------------
def weighted_error(w: np.ndarray, w_hat: np.ndarray, imatrix=None, axis=None):
    """E = sum_i q_i (w_i - w_hat_i)^2 in fp64 (q = 1 when imatrix is None)."""
    w = np.asarray(w, dtype=np.float64)
    diff = w - np.asarray(w_hat, dtype=np.float64)
    q = np.ones(w.shape[-1]) if imatrix is None else np.asarray(imatrix, dtype=np.float64)
    return np.sum(q * diff * diff, axis=axis)


def pattern_error(absw, q, z, d) -> np.ndarray:
    """Per-block weighted error of pattern z (signs of w) with scale d (fp64)."""
    lane = np.arange(GROUP)
    zero = lane == z[..., None]
    err = np.where(zero, absw, absw - d[..., None, None])
    return np.sum(q * err * err, axis=(-1, -2))


# -----------------------------------------------------------------------------
# O7 / O8: products
# -----------------------------------------------------------------------------
def gemv(q: np.ndarray, n_rows: int, k: int, x: np.ndarray) -> np.ndarray:
    """y = W_hat x in fp64.  Each product fp32 x (bf16 or fp32) is exact in
    fp64; the fp64 dot adds relative error ~1e-16, far inside any tolerance."""
    w_hat = dequantize_rows(q, n_rows, k).astype(np.float64)
    return w_hat @ np.asarray(x, dtype=np.float64).reshape(k)


def gemv_tokens(q: np.ndarray, n_rows: int, k: int, x: np.ndarray) -> np.ndarray:
    """Y[t, n] = sum_k W_hat[n, k] x[t, k] for several tokens x [T, k] (fp64)."""
    w_hat = dequantize_rows(q, n_rows, k).astype(np.float64)
    return np.asarray(x, dtype=np.float64).reshape(-1, k) @ w_hat.T


def grouped_gemm(table: np.ndarray, expert_stride: int, n_rows: int, k: int,
                 x_sorted: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Per expert e: Y[off[e]:off[e+1]] = X[off[e]:off[e+1]] @ W_hat_e^T (fp64)."""
    table = np.asarray(table, dtype=np.uint8).reshape(-1)
    offsets = np.asarray(offsets, dtype=np.int64)
    x = np.asarray(x_sorted, dtype=np.float64).reshape(-1, k)
    y = np.zeros((x.shape[0], n_rows), dtype=np.float64)
    rb = row_bytes(k)
    for e in range(offsets.shape[0] - 1):
        lo, hi = offsets[e], offsets[e + 1]
        if hi <= lo:
            continue
        raw = table[e * expert_stride: e * expert_stride + n_rows * rb]
        y[lo:hi] = x[lo:hi] @ dequantize_rows(raw, n_rows, k).astype(np.float64).T
    return y


def tolerance_scale(q: np.ndarray, n_rows: int, k: int, x: np.ndarray) -> np.ndarray:
    """A[t, n] = sum_b d_{n,b} * sum_{k in block b} |x[t, k]| (fp64), the scale
    of the per-element error bound for row n and token t."""
    blocks = unpack_matrix(q, n_rows, k // QK)
    d16, _ = unpack_blocks(blocks.reshape(-1, BLOCK_BYTES))
    d = np.abs(fp16_bits_to_f32(d16).astype(np.float64)).reshape(n_rows, k // QK)
    ax = np.abs(np.asarray(x, dtype=np.float64).reshape(-1, k // QK, QK)).sum(axis=-1)
    return ax @ d.T


# -----------------------------------------------------------------------------
# Routed-expert FFN for decode (gate/up GEMV, SiLU gate times up, down GEMV,
# routing-weighted combine).  The pages run the routed experts' projections
# through STQ1_0 kernels ([LEMMY] "Runtime") in a MoE with top-8 of 256
# routed experts ([TRAIC] "The claim, stated precisely").  Readings (the pages
# give no layer code): the gate/up matrix holds the gate rows first, then the
# up rows; the activation is SiLU(gate) * up; the down projection is STQ1_0
# too; a token's output is the routing-weighted sum of its experts' outputs.
# -----------------------------------------------------------------------------
SILU_LIPSCHITZ = 1.1     # max |silu'(v)| is 1.0998...; used by the error bound


def silu(v: np.ndarray) -> np.ndarray:
    """silu(v) = v / (1 + exp(-v)) in fp64, evaluated as v * exp(v) / (1 + exp(v))
    for v < 0 so that exp never overflows."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = v[pos] / (1.0 + np.exp(-v[pos]))
    e = np.exp(v[~pos])
    out[~pos] = v[~pos] * e / (1.0 + e)
    return out


def _ffn_pair(gate_up: np.ndarray, down: np.ndarray, d_model: int, d_ff: int, x: np.ndarray, n_out: int):
    """g, u, h, z of one (token, expert) pair, all fp64 (z: the n_out rows `down` holds)."""
    gu = gemv(gate_up, 2 * d_ff, d_model, x)
    g, u = gu[:d_ff], gu[d_ff:]
    h = silu(g) * u
    z = gemv(down, n_out, d_ff, h)
    return g, u, h, z


def moe_ffn_decode(gate_up: dict, down: dict, d_model: int, d_ff: int, x: np.ndarray,
                   pair_expert: np.ndarray, pair_weight: np.ndarray, top_k: int, n_out: int | None = None) -> np.ndarray:
    """y[t] = sum_k w[t*top_k + k] * W_down_e (silu(W_gate_e x_t) * (W_up_e x_t)), fp64.

    gate_up[e] / down[e]: packed matrices of expert e ([2*d_ff, d_model] and
    [n_out, d_ff]: n_out rows of the down projection, all d_model of them by
    default; rows of a matrix-vector product are independent, so a subset of
    rows gives the same outputs for those rows); a pair whose expert is not
    among them makes its token's row NaN."""
    n_out = d_model if n_out is None else int(n_out)
    x = np.asarray(x, dtype=np.float64).reshape(-1, d_model)
    pe = np.asarray(pair_expert).reshape(-1)
    pw = np.asarray(pair_weight, dtype=np.float64).reshape(-1)
    y = np.zeros((x.shape[0], n_out), dtype=np.float64)
    for t in range(x.shape[0]):
        for k in range(top_k):
            p = t * top_k + k
            e = int(pe[p])
            if e not in gate_up or e not in down:
                y[t] = np.nan
                continue
            y[t] = y[t] + pw[p] * _ffn_pair(gate_up[e], down[e], d_model, d_ff, x[t], n_out)[3]
    return y


def moe_ffn_tolerance(gate_up: dict, down: dict, d_model: int, d_ff: int, x: np.ndarray,
                      pair_expert: np.ndarray, pair_weight: np.ndarray, top_k: int,
                      tol: float = 1e-3, eps_act: float = 1e-6, eps_sum: float = 2.0 ** -23,
                      n_out: int | None = None) -> np.ndarray:
    """Per-element bound on |y_gpu - y| derived from the GEMV bound |err| <= tol * A.

    For a pair with exact g, u, h (fp64) and GEMV bounds dg = tol*A_g, du = tol*A_u:
      |dh| <= L*dg*(|u| + du) + |silu(g)|*du + eps_act*(|h| + ...)      (L = max|silu'|)
      |dz| <= |W_down| dh + tol * A_down(|h| + dh)
    and the fp32 combine adds at most top_k*eps_sum*sum_k |w_k| (|z_k| + dz_k):
      bound[t] = sum_k |w_k| dz_k + top_k*eps_sum*sum_k |w_k| (|z_k| + dz_k).
    n_out: rows held by each down matrix, as in moe_ffn_decode."""
    n_out = d_model if n_out is None else int(n_out)
    x = np.asarray(x, dtype=np.float64).reshape(-1, d_model)
    pe = np.asarray(pair_expert).reshape(-1)
    pw = np.abs(np.asarray(pair_weight, dtype=np.float64).reshape(-1))
    bound = np.zeros((x.shape[0], n_out), dtype=np.float64)
    for t in range(x.shape[0]):
        acc_dz = np.zeros(n_out)
        acc_mag = np.zeros(n_out)
        for k in range(top_k):
            p = t * top_k + k
            e = int(pe[p])
            if e not in gate_up or e not in down:
                bound[t] = np.nan
                break
            g, u, h, z = _ffn_pair(gate_up[e], down[e], d_model, d_ff, x[t], n_out)
            a_gu = tolerance_scale(gate_up[e], 2 * d_ff, d_model, x[t])[0]
            dg, du = tol * a_gu[:d_ff], tol * a_gu[d_ff:]
            dh = SILU_LIPSCHITZ * dg * (np.abs(u) + du) + np.abs(silu(g)) * du
            dh = dh + eps_act * (np.abs(h) + dh)
            w_abs = np.abs(dequantize_rows(down[e], n_out, d_ff).astype(np.float64))
            dz = w_abs @ dh + tol * tolerance_scale(down[e], n_out, d_ff, np.abs(h) + dh)[0]
            acc_dz += pw[p] * dz
            acc_mag += pw[p] * (np.abs(z) + dz)
        else:
            bound[t] = acc_dz + top_k * eps_sum * acc_mag
    return bound


# -----------------------------------------------------------------------------
# Layer sensitivity and mixed-precision allocation ([LEMMY] "Full-Hessian
# scoring"; [AGI] "Four weights, five bits" on the per-layer mix).  The pages:
# sensitivity is measured with the full Hessian H = X X^T of the layer's
# calibration activations, whose off-diagonal terms the diagonal imatrix
# misses; layers are chosen greedily by error reduction per added byte, the
# alternative to STQ1_0 being a ~2-bit format (IQ2_XXS, not described on the
# pages).  Readings: the error of a quantized layer is ||(W - W_hat) X^T||_F^2
# over calibration rows X [N, k] (full) or sum_k (sum_i x_ik^2) (W - W_hat)_k^2
# (diagonal); the stand-in ~2-bit format is Q2 below.
# -----------------------------------------------------------------------------
Q2_BLOCK_BYTES = 66      # fp16 scale + 256 x 2-bit levels: 2.0625 bits per weight


def q2_roundtrip(w: np.ndarray) -> np.ndarray:
    """Stand-in 2-bit format: per 256 weights one scale s = rms/2 (rms = root
    mean square of the block, fp64; stored as fp16 via fp32, nearest-even,
    clamped to 65504) and levels {-3,-1,+1,+3}*s, each weight taking the
    nearest level (ties to the larger magnitude; the sign is the sign bit of w,
    so -0.0 maps to -s).  For Gaussian
    weights the levels sit near the minimum-error 4-level points (about
    +-0.45 and +-1.5 standard deviations).  Returns the reconstruction (fp32)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    b = w.reshape(n, k // QK, QK // GROUP, GROUP).astype(np.float64)
    # sum of squares in the encoder's fixed order (lanes of a group, then the
    # balanced tree of adjacent groups), so the stored scale is unique
    ss = _tree_sum(_group_partial(b * b))
    rms = np.sqrt(ss / QK)
    s16 = np.minimum(rms / 2.0, FP16_MAX).astype(np.float32).astype(np.float16).astype(np.float64)
    s = s16[..., None, None]
    a = np.abs(b)
    mag = np.where(a < 2.0 * s, s, 3.0 * s)           # nearest of s, 3s (2s exact in fp64)
    rec = np.where(np.signbit(b), -mag, mag)          # -0.0 counts as negative, like the sign bit
    return rec.reshape(n, k).astype(np.float32)


def layer_errors(w: np.ndarray, w_hat: np.ndarray, x_calib: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row reconstruction error of W_hat against W under the calibration
    rows x_calib [N, k]: full e[r] = sum_i (sum_k d_rk x_ik)^2 and diagonal
    e[r] = sum_k (sum_i x_ik^2) d_rk^2, d = W - W_hat, all in fp64."""
    d = np.asarray(w, dtype=np.float64) - np.asarray(w_hat, dtype=np.float64)
    x = np.asarray(x_calib, dtype=np.float64)
    full = ((d @ x.T) ** 2).sum(axis=1)
    diag = (d * d) @ (x * x).sum(axis=0)
    return full, diag


def layer_errors_tolerance(w: np.ndarray, w_hat: np.ndarray, x_calib: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row bounds on |err - err_ref| for two fp64 evaluations of
    layer_errors that differ only in summation order (the pages fix no
    precision; this is the standard fp64 bound, u = 2^-53, g(m) = m u/(1-m u)).

    Each p_ri = D_r . x_i sums k products, one rounding each for the
    difference, the product and every addition, so two evaluations differ by
    at most delta_ri = 2 g(k+2) A_ri with A_ri = sum_c |D_rc x_ic|; squaring
    moves p^2 by at most delta (2|p| + delta); the N nonnegative squares add
    with relative error g(N+1) on either side.  The diagonal sum has only
    nonnegative terms of k + N + 4 roundings each side."""
    d = np.asarray(w, dtype=np.float64) - np.asarray(w_hat, dtype=np.float64)
    x = np.asarray(x_calib, dtype=np.float64)
    u = 2.0 ** -53
    g = lambda m: m * u / (1.0 - m * u)
    k, n_cal = d.shape[1], x.shape[0]
    p = d @ x.T
    a = np.abs(d) @ np.abs(x).T
    delta = 2.0 * g(k + 2) * a
    sq = (delta * (2.0 * np.abs(p) + delta)).sum(axis=1)
    full = (p * p).sum(axis=1)
    b_full = sq + 2.0 * g(n_cal + 1) * (full + sq)
    diag = (d * d) @ (x * x).sum(axis=0)
    b_diag = 2.0 * g(k + n_cal + 4) * diag
    return b_full, b_diag


def greedy_allocation(gain: np.ndarray, extra_bytes: np.ndarray, budget: float) -> np.ndarray:
    """Layers to move to the larger format: repeatedly take the layer with the
    largest error reduction per added byte (lowest index on ties) while the
    added bytes stay within `budget`; layers that no longer fit are skipped.
    Returns a bool mask."""
    gain = np.asarray(gain, dtype=np.float64)
    extra = np.asarray(extra_bytes, dtype=np.float64)
    order = sorted(range(len(gain)), key=lambda i: (-(gain[i] / extra[i]), i))
    chosen = np.zeros(len(gain), dtype=bool)
    used = 0.0
    for i in order:
        if gain[i] > 0 and used + extra[i] <= budget:
            chosen[i] = True
            used += extra[i]
    return chosen


def spearman(a: np.ndarray, b: np.ndarray) -> float:
    """Spearman rank correlation (average ranks for ties)."""
    def ranks(v):
        v = np.asarray(v, dtype=np.float64)
        order = np.argsort(v, kind="stable")
        r = np.empty(len(v))
        r[order] = np.arange(len(v), dtype=np.float64)
        for val in np.unique(v):
            m = v == val
            if m.sum() > 1:
                r[m] = r[m].mean()
        return r
    ra, rb = ranks(a), ranks(b)
    ra -= ra.mean()
    rb -= rb.mean()
    return float((ra * rb).sum() / np.sqrt((ra * ra).sum() * (rb * rb).sum()))
