"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching the GPU.  No kernel runs."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "stq.h")


@pytest.fixture(scope="module")
def L():
    import sparse_ternary_bit_amd as stq
    if not os.path.exists(stq.lib_path()):
        from sparse_ternary_bit_amd import build
        build.build(verbose=False)
    return stq.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(stq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for want in ("stq_quantize_rows", "stq_gemv", "stq_grouped_gemm", "stq_dequantize_rows",
                 "stq_moe_ffn_decode", "stq_layer_errors", "stq_q2_roundtrip", "stq_greedy_allocation",
                 "stq_gemv_plan", "stq_row_bytes", "stq_status_string", "stq_last_error"):
        assert want in names


def test_every_declared_symbol_is_exported(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_row_bytes(L):
    assert L.stq_row_bytes(256) == 42
    assert L.stq_row_bytes(1024) == 168
    assert L.stq_row_bytes(7168) == 1176
    for bad in (0, -256, 100, 257):
        assert L.stq_row_bytes(bad) == -1


def test_status_strings(L):
    for s in range(5):
        assert L.stq_status_string(s)
    assert L.stq_status_string(99) == b"unknown status"


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _err(L):
    return L.stq_last_error().decode()


def test_quantize_rejects_bad_arguments(L):
    assert L.stq_quantize_rows(FAKE, None, 4, 100, 0, 3, FAKE, None) == 2
    assert "multiple of 256" in _err(L)
    assert L.stq_quantize_rows(FAKE, None, 4, 256, 7, 3, FAKE, None) == 1
    assert L.stq_quantize_rows(FAKE, None, 4, 256, 0, -1, FAKE, None) == 1
    assert L.stq_quantize_rows(None, None, 4, 256, 0, 3, FAKE, None) == 1
    assert L.stq_quantize_rows(FAKE + 2, None, 4, 256, 0, 3, FAKE, None) == 3
    assert L.stq_quantize_rows(FAKE, None, 4, 256, 0, 3, FAKE + 1, None) == 3
    assert L.stq_quantize_rows(FAKE, None, -1, 256, 0, 3, FAKE, None) == 1


def test_dequantize_rejects_bad_arguments(L):
    assert L.stq_dequantize_rows(FAKE, 2, 300, FAKE, None) == 2
    assert L.stq_dequantize_rows(FAKE + 1, 2, 256, FAKE, None) == 3
    assert L.stq_dequantize_rows(FAKE, 2, 256, FAKE + 2, None) == 3
    assert L.stq_dequantize_rows(None, 2, 256, FAKE, None) == 1


def _gemv(L, **kw):
    a = dict(w=FAKE, stride=4096 * 1176, ne=4, n=4096, k=7168, x=FAKE, xd=1, xs=7168, nt=4,
             pe=None, pt=None, np_=4, y=FAKE, ws=None, wsb=0)
    a.update(kw)
    return L.stq_gemv(a["w"], a["stride"], a["ne"], a["n"], a["k"], a["x"], a["xd"], a["xs"], a["nt"],
                      a["pe"], a["pt"], a["np_"], a["y"], a["ws"], a["wsb"], None)


def test_gemv_rejects_bad_arguments(L):
    assert _gemv(L, k=1000) == 2
    assert _gemv(L, ne=0) == 1
    assert _gemv(L, xd=5) == 1
    assert _gemv(L, stride=100) == 2
    assert "expert stride" in _err(L)
    assert _gemv(L, xs=100) == 2
    assert _gemv(L, np_=70000) == 2
    assert _gemv(L, w=FAKE + 8) == 3
    assert _gemv(L, stride=4096 * 1176 + 8) == 3
    assert _gemv(L, xs=7169) == 3
    assert _gemv(L, y=None) == 1
    assert _gemv(L, np_=-1) == 1


def test_gemv_refuses_missing_or_small_workspace(L, monkeypatch):
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    st, (sp, mp, need) = _plan(L, ne=4, np_=4)
    assert st == 0 and need > 0                       # four single-token experts: k is split
    assert _gemv(L) == 1 and "workspace" in _err(L)
    assert _gemv(L, ws=FAKE, wsb=need - 1) == 1 and str(need) in _err(L)
    assert _gemv(L, ws=FAKE + 16, wsb=need) == 3
    assert _gemv(L, ws=FAKE, wsb=-1) == 1
    monkeypatch.setenv("STQ_GEMV_PLAN", "1,1")       # no split: no workspace needed, none checked
    assert _plan(L, ne=4, np_=4)[1][2] == 0


def test_gemv_empty_work_is_ok_without_gpu(L):
    assert _gemv(L, np_=0, w=None, x=None, y=None) == 0
    assert _gemv(L, n=0, w=None, x=None, y=None) == 0


def _plan(L, ne=256, n=4096, k=7168, np_=8, cus=256):
    sp, mp, sb = ctypes.c_int32(-7), ctypes.c_int32(-7), ctypes.c_int64(-7)
    st = L.stq_gemv_plan(ne, n, k, np_, cus, ctypes.byref(sp), ctypes.byref(mp), ctypes.byref(sb))
    return st, (sp.value, mp.value, sb.value)


def _scratch(splits, parts, n_pairs, n):
    """Bytes of split outputs: fp32 partial sums per (slot, pair, row) padded
    to 256 bytes, then one int per pair (its part count) when experts are
    parted; nothing when no output is split."""
    if splits * parts == 1:
        return 0
    return (splits * parts * n_pairs * n * 4 + 255) // 256 * 256 + (4 * n_pairs if parts > 1 else 0)


def test_gemv_plan_for_the_decode_sweep(L, monkeypatch):
    """The 256-expert 4096 x 7168 layer, top-8, on 256 CUs: the plans the
    decode sweep runs under, and the scratch each needs.  At 64 tokens (512
    pairs, at least one per expert) the kernel variant with the matrix-core
    form runs, whose 3- and 4-token passes cost little more than a one-token
    pass, so experts are no longer parted by token count (measured: 315-324
    us at (1, 1) against 339-347 us at (1, 2))."""
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    for tokens, want in ((1, (7, 1)), (4, (2, 2)), (16, (1, 3)), (64, (1, 1))):
        st, (sp, mp, sb) = _plan(L, np_=8 * tokens)
        assert st == 0 and (sp, mp) == want, tokens
        assert sb == _scratch(sp, mp, 8 * tokens, 4096)
    assert _plan(L, np_=1) == (0, (28, 1, _scratch(28, 1, 1, 4096)))  # one pair: a block per workgroup
    st, plan0 = _plan(L, cus=0)  # the current device's CUs, 256 when no device answers
    assert st == 0
    import torch
    if not torch.cuda.is_available():
        assert plan0 == _plan(L, cus=256)[1]


def test_gemv_plan_fills_more_compute_units_with_more_splits(L, monkeypatch):
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    splits = [_plan(L, np_=8, cus=c)[1][0] for c in (8, 64, 128, 256, 304, 512, 1024)]
    assert splits == sorted(splits) and splits[0] < splits[-1]
    for c in (8, 64, 128, 256, 304, 512, 1024):
        for tokens in (1, 4, 16, 64):
            st, (sp, mp, sb) = _plan(L, np_=8 * tokens, cus=c)
            assert st == 0 and 1 <= sp <= 28 and 1 <= mp <= 8 and sb == _scratch(sp, mp, 8 * tokens, 4096)


def test_gemv_plan_partial_sums_cap(L, monkeypatch):
    """No plan writes more than 1 GiB of partial sums: from 4097 tokens of
    top-8 on 4096 rows every output goes straight to y."""
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    assert _plan(L, np_=8 * 4097) == (0, (1, 1, 0))
    assert _plan(L, np_=65535) == (0, (1, 1, 0))
    for np_ in (8, 100, 1000, 4000, 16384, 32768, 32776):
        st, (sp, mp, sb) = _plan(L, np_=np_)
        assert st == 0
        assert (sp, mp) == (1, 1) or sp * mp * np_ * 4096 * 4 <= 2 ** 30


@pytest.mark.parametrize("env,want", [("3,4", (3, 4)), ("5,8", (5, 8)), ("10,1", (10, 1)), ("27,1", (14, 1)),
                                      ("28,2", (28, 2))])
def test_gemv_plan_override(L, monkeypatch, env, want):
    """STQ_GEMV_PLAN="s,p" replaces the estimate; s splits are rounded to the
    split of ceil(28 / s) blocks each (27 -> 2 blocks -> 14 splits)."""
    monkeypatch.setenv("STQ_GEMV_PLAN", env)
    st, (sp, mp, sb) = _plan(L, np_=64)
    assert st == 0 and (sp, mp) == want and sb == _scratch(sp, mp, 64, 4096)


@pytest.mark.parametrize("env", ["0,1", "29,1", "3,9", "3,0", "x", "4", "-1,2"])
def test_gemv_plan_ignores_malformed_overrides(L, monkeypatch, env):
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    auto = _plan(L, np_=64)
    monkeypatch.setenv("STQ_GEMV_PLAN", env)
    assert _plan(L, np_=64) == auto


def test_gemv_plan_parts_need_the_leader_table(L, monkeypatch):
    """Experts are parted only while the workgroup's table space can rank
    them (8708 experts: two 34832-byte table buffers of int pairs); beyond,
    each expert is one unit even when forced."""
    monkeypatch.setenv("STQ_GEMV_PLAN", "1,3")
    assert _plan(L, ne=8708, np_=64)[1][:2] == (1, 3)
    assert _plan(L, ne=8709, np_=64) == (0, (1, 1, 0))
    monkeypatch.setenv("STQ_GEMV_PLAN", "4,3")
    assert _plan(L, ne=9000, np_=64) == (0, (4, 1, _scratch(4, 1, 64, 4096)))


def test_gemv_plan_rejects_bad_arguments(L):
    assert _plan(L, k=1000)[0] == 2
    assert _plan(L, ne=0)[0] == 1
    assert _plan(L, np_=70000)[0] == 2
    assert _plan(L, np_=-1)[0] == 1
    assert _plan(L, n=-1)[0] == 1
    assert _plan(L, cus=-1)[0] == 1
    sp, mp = ctypes.c_int32(), ctypes.c_int32()
    assert L.stq_gemv_plan(256, 4096, 7168, 8, 256, ctypes.byref(sp), ctypes.byref(mp), None) == 1
    assert "null" in _err(L)
    # nothing to launch: no split, no scratch
    assert _plan(L, np_=0) == (0, (1, 1, 0))
    assert _plan(L, n=0) == (0, (1, 1, 0))


def test_gemv_plan_binding(monkeypatch):
    import sparse_ternary_bit_amd as stq
    monkeypatch.delenv("STQ_GEMV_PLAN", raising=False)
    assert stq.gemv_plan(256, 4096, 7168, 128, n_cus=256) == (1, 3, _scratch(1, 3, 128, 4096))
    with pytest.raises(stq.StqError):
        stq.gemv_plan(256, 4096, 1000, 8)


def test_grouped_gemm_rejects_bad_arguments(L):
    def g(**kw):
        a = dict(w=FAKE, stride=4096 * 1176, ne=256, n=4096, k=7168, x=FAKE, off=FAKE, m=16, y=FAKE)
        a.update(kw)
        return L.stq_grouped_gemm(a["w"], a["stride"], a["ne"], a["n"], a["k"], a["x"], a["off"], a["m"],
                                  a["y"], None)
    assert g(k=300) == 2
    assert g(off=None) == 1
    assert g(x=FAKE + 8) == 3
    assert g(ne=70000) == 2
    assert g(stride=10) == 2
    assert g(m=-1) == 1
    assert g(m=0, w=None, x=None, y=None) == 0


def test_moe_ffn_rejects_bad_arguments(L):
    gu_stride, dn_stride = 4096 * 1176, 7168 * 336

    def f(**kw):
        a = dict(wg=FAKE, gs=gu_stride, wd=FAKE, ds=dn_stride, ne=256, dm=7168, ff=2048, x=FAKE, t=4,
                 pe=FAKE, pw=FAKE, k=8, y=FAKE)
        a.update(kw)
        return L.stq_moe_ffn_decode(a["wg"], a["gs"], a["wd"], a["ds"], a["ne"], a["dm"], a["ff"], a["x"], a["t"],
                                    a["pe"], a["pw"], a["k"], a["y"], a.get("ws"), a.get("wsb", 0), None)
    assert f(dm=7000) == 2
    assert f(ff=100) == 2
    assert f(k=0) == 1
    assert f(ne=0) == 1
    assert f(gs=10) == 2
    assert f(ds=dn_stride - 16) == 2
    assert f(t=10000) == 2            # more than 65535 pairs
    assert f(pw=None) == 1
    assert f(wd=FAKE + 4) == 3
    assert f(gs=gu_stride + 8) == 3
    assert f(x=FAKE + 2) == 3
    assert f(t=0, wg=None, wd=None, x=None, pe=None, pw=None, y=None) == 0
    assert f(wsb=-1) == 1


def _ffn_ws(L, ne=256, dm=7168, ff=2048, t=4, k=8, cus=256):
    wb = ctypes.c_int64(-7)
    st = L.stq_moe_ffn_workspace(ne, dm, ff, t, k, cus, ctypes.byref(wb))
    return st, wb.value


def test_moe_ffn_workspace_query(L):
    st, wb = _ffn_ws(L)
    P = 4 * 8
    # at least the pairs' gate/up rows, activations and down rows in fp32, on 256-byte boundaries
    assert st == 0 and wb >= P * (2 * 2048 + 2048 + 7168) * 4 and wb % 256 == 0
    st2, wb2 = _ffn_ws(L, t=64)
    assert st2 == 0 and wb2 > wb
    assert _ffn_ws(L, t=0) == (0, 0)
    assert _ffn_ws(L, dm=7000)[0] == 2
    assert _ffn_ws(L, t=10000)[0] == 2
    assert _ffn_ws(L, cus=-1)[0] == 1
    assert L.stq_moe_ffn_workspace(256, 7168, 2048, 4, 8, 256, None) == 1


def test_moe_ffn_refuses_missing_or_small_workspace(L):
    gs, ds = 4096 * 1176, 7168 * 336
    _, need = _ffn_ws(L)

    def f(ws, wsb):
        return L.stq_moe_ffn_decode(FAKE, gs, FAKE, ds, 256, 7168, 2048, FAKE, 4, FAKE, FAKE, 8, FAKE, ws, wsb, None)
    assert f(None, 0) == 1 and "workspace" in _err(L)
    assert f(FAKE, need - 1) == 1 and str(need) in _err(L)
    assert f(FAKE + 16, need) == 3


def test_layer_errors_rejects_bad_arguments(L):
    le = L.stq_layer_errors
    assert le(FAKE, FAKE, 4, 300, FAKE, 8, FAKE, FAKE, None, 0, None) == 2
    assert le(FAKE, FAKE, 4, 256, FAKE, 0, FAKE, FAKE, None, 0, None) == 1
    assert "n_calib" in _err(L)
    assert le(FAKE, FAKE, -1, 256, FAKE, 8, FAKE, FAKE, None, 0, None) == 1
    assert le(FAKE, None, 4, 256, FAKE, 8, FAKE, FAKE, None, 0, None) == 1
    assert le(FAKE + 4, FAKE, 4, 256, FAKE, 8, FAKE, FAKE, None, 0, None) == 3
    assert le(FAKE, FAKE, 4, 256, FAKE + 8, 8, FAKE, FAKE, None, 0, None) == 3
    assert le(FAKE, FAKE, 4, 256, FAKE, 8, FAKE + 4, FAKE, None, 0, None) == 3
    assert le(FAKE, FAKE, 4, 256, FAKE, 65536 * 64, FAKE, FAKE, None, 0, None) == 2
    assert le(None, None, 0, 256, None, 8, None, None, None, 0, None) == 0   # nothing to do


def test_layer_errors_workspace_query_and_refusal(L):
    wb = ctypes.c_int64(-7)
    assert L.stq_layer_errors_workspace(4096, 7168, 512, ctypes.byref(wb)) == 0
    assert wb.value == 8 * (7168 + 2 * 8 * 4096)        # H diagonal, then 2 partials per (row, 64-row tile)
    assert L.stq_layer_errors_workspace(0, 7168, 512, ctypes.byref(wb)) == 0 and wb.value == 0
    assert L.stq_layer_errors_workspace(4, 300, 8, ctypes.byref(wb)) == 2
    assert L.stq_layer_errors_workspace(4, 256, 0, ctypes.byref(wb)) == 1
    assert L.stq_layer_errors_workspace(4, 256, 8, None) == 1
    L.stq_layer_errors_workspace(4, 256, 8, ctypes.byref(wb))
    need = wb.value
    le = L.stq_layer_errors
    assert le(FAKE, FAKE, 4, 256, FAKE, 8, FAKE, FAKE, None, 0, None) == 1 and "workspace" in _err(L)
    assert le(FAKE, FAKE, 4, 256, FAKE, 8, FAKE, FAKE, FAKE, need - 8, None) == 1
    assert le(FAKE, FAKE, 4, 256, FAKE, 8, FAKE, FAKE, FAKE + 8, need, None) == 3


def test_library_allocates_no_device_memory(L):
    """No entry point allocates or frees device memory: the library does not
    even import HIP's allocators (workspaces are the caller's)."""
    import shutil
    import subprocess
    import sparse_ternary_bit_amd as stq
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not installed")
    out = subprocess.run([nm, "-D", "--undefined-only", stq.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    assert "hipLaunchKernel" in imported or any(n.startswith("hip") for n in imported)
    banned = {n for n in imported if re.match(r"^hip(Ext)?(Malloc|Free|HostMalloc|HostAlloc|MallocManaged|"
                                              r"MallocAsync|FreeAsync|MallocFromPool|MemPool)", n)}
    assert not banned, banned


def test_q2_roundtrip_rejects_bad_arguments(L):
    q2 = L.stq_q2_roundtrip
    assert q2(FAKE, 4, 128, FAKE, None) == 2
    assert q2(FAKE, -2, 256, FAKE, None) == 1
    assert q2(None, 4, 256, FAKE, None) == 1
    assert q2(FAKE + 4, 4, 256, FAKE, None) == 3
    assert q2(FAKE, 4, 256, FAKE + 8, None) == 3
    assert q2(None, 0, 256, None, None) == 0


def test_greedy_allocation_rejects_bad_arguments(L):
    import numpy as np
    g = np.ones(3)
    e = np.array([1.0, 0.0, 2.0])
    c = np.zeros(3, dtype=np.uint8)
    assert L.stq_greedy_allocation(g.ctypes.data, e.ctypes.data, 3, 10.0, c.ctypes.data) == 1
    assert "extra_bytes[1]" in _err(L)
    assert L.stq_greedy_allocation(None, e.ctypes.data, 3, 10.0, c.ctypes.data) == 1
    assert L.stq_greedy_allocation(g.ctypes.data, e.ctypes.data, -1, 10.0, c.ctypes.data) == 1


def test_greedy_allocation_matches_the_oracle(L):
    """A host function: its choice equals the oracle's on random layer sets,
    ties in the ratio included."""
    import numpy as np
    import sparse_ternary_bit_amd as stq
    from oracle import stq_oracle as O
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        gain = rng.normal(1.0, 1.0, n)
        gain[rng.random(n) < 0.2] = 2.0          # equal gains with equal sizes: ties
        extra = rng.choice([1.0, 2.0, 3.0], n)
        budget = float(rng.uniform(0, extra.sum()))
        got = stq.greedy_allocation(gain, extra, budget)
        want = O.greedy_allocation(gain, extra, budget)
        assert np.array_equal(got, want), trial


def test_stream_read_probe_rejects_bad_arguments(L):
    assert L.stq_stream_read_probe(FAKE, 100, FAKE, None) == 1
    assert L.stq_stream_read_probe(FAKE, -16, FAKE, None) == 1
    assert L.stq_stream_read_probe(None, 64, FAKE, None) == 1
    assert L.stq_stream_read_probe(FAKE + 8, 64, FAKE, None) == 3
    assert L.stq_stream_read_probe(None, 0, None, None) == 0


def test_mfma_and_lds_probes_reject_bad_arguments(L):
    import sparse_ternary_bit_amd as stq
    mfma = L.stq_mfma_loop_probe
    assert mfma(-1, FAKE, None) == 1
    assert mfma(4, None, None) == 1
    assert mfma(4, FAKE + 2, None) == 3
    assert mfma(0, None, None) == 0  # nothing to launch
    lds = L.stq_lds_read_probe
    assert lds(2, 4, FAKE, None) == 1
    assert lds(-1, 4, FAKE, None) == 1
    assert lds(0, -1, FAKE, None) == 1
    assert lds(1, 4, None, None) == 1
    assert lds(0, 4, FAKE + 1, None) == 3
    assert lds(1, 0, None, None) == 0
    # the binding's work counts are the header's
    hdr = open(os.path.join(os.path.dirname(stq.lib_path()), "..", "include", "stq.h")).read()
    assert f"#define STQ_MFMA_PROBE_FLOP_PER_ROUND {stq.MFMA_PROBE_FLOP_PER_ROUND!r}" in hdr
    assert f"#define STQ_LDS_PROBE_READS_PER_ROUND {stq.LDS_PROBE_READS_PER_ROUND}" in hdr
    assert stq.MFMA_PROBE_FLOP_PER_ROUND == 4096 * 4 * 8 * (2 * 16 * 16 * 32)
    assert stq.LDS_PROBE_READS_PER_ROUND == 4096 * 4 * 8


def test_gemv_noalloc_checks_and_refuses_shapes_beyond_its_scratch(L, monkeypatch):
    """stq_gemv_noalloc checks its arguments like stq_gemv and refuses, before
    touching the GPU, shapes whose plan needs more than its fixed scratch."""
    f = L.stq_gemv_noalloc
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    n, k, E, P = 4096, 7168, 2, 4096
    args = lambda **kw: [kw.get("w", FAKE), n * 1176, E, n, kw.get("k", k), FAKE, 1, k, P, None, None,
                         kw.get("np_", P), kw.get("y", FAKE), None]
    assert f(*args(k=1000)) == 2
    assert f(*args(y=None)) == 1
    assert f(*args(w=FAKE + 8)) == 3
    assert f(*args(np_=0, w=None, y=None)) == 0
    monkeypatch.setenv("STQ_GEMV_PLAN", "16,8")          # 128 slots of 4096 x 4096 fp32 partial sums
    assert _plan(L, ne=E, np_=P)[1][2] > 32 << 20
    assert f(*args()) == 2 and "scratch" in _err(L)
