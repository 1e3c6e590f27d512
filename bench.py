#!/usr/bin/env python3
"""Benchmark of the STQ1_0 sparse-ternary matmul on one MI355X.

One step is one pass of the hot path over one batch of synthetic input:
  * decode: the gathered GEMV of a 256-expert MoE layer (gate+up, 4096 x 7168
    per expert, 1.23 GB packed) at batch 1, 4, 16 and 64 tokens with fresh
    uniform top-8 routing, on the WLS-encoded table and on an amax-encoded
    table of the same weights (kernel speed must not depend on the encoder);
  * prefill: the grouped GEMM of 2048 tokens routed top-8 (16384 rows grouped
    by expert) against the same table;
  * the routed-expert FFN of the layer for decode (gate/up GEMV, SiLU(gate) *
    up, down GEMV against a 256 x 7168 x 2048 down table, routing combine) at
    batch 1, 16, 64, reported beside the headline as `moe_ffn_decode`;
  * the encoder as a layer-scale workload (`encode_layer`): both encoders on
    8 experts' fp32 gate/up weights drawn beforehand, extrapolated to the
    256-expert layer;
  * layer-sensitivity scoring (`layer_sensitivity`): full-Hessian and
    diagonal error of one expert's STQ1_0 gate/up matrix (4096 x 7168) under
    512 calibration rows, a dense fp64 contraction on the matrix cores, and
    the 2-bit stand-in's quantize-and-reconstruct pass.
Inputs are resident in HBM before timing starts.  `value` is the GEMV's
effective bandwidth over the sweep: algorithmic bytes (each touched expert's
packed bytes once, plus activations and outputs) divided by GEMV time.
Kernel durations come from HIP events recorded on the launch stream.

After the timed steps, reported beside the headline (not part of `value`):
  * `single_expert_gemv`: one expert's gate+up GEMV at batch 1 over 100
    resident experts, 1000 launches (median / p10 / p90), and the same 100
    calls replayed from a HIP graph;
  * `roofline_gemm.dense_bf16_gemm_TFLOP/s`: a dense bf16 GEMM of the
    prefill's total shape through the vendor library (torch.matmul), the
    matrix-core rate this GPU reaches on a plain contraction;
  * `stream_read_GB/s`: the library's plain streaming read of 2 GiB;
  * `roofline_gemm.mfma_loop_TFLOP/s`: a loop of independent bf16 MFMAs with
    no memory traffic, the matrix-core rate this GPU sustains;
  * `lds_probe`: LDS reads per ns per compute unit in the two forms the
    grouped GEMM issues (16-byte activation reads, pattern-table read pairs);
  * `cpu_baseline`: the oracle, single-threaded, on bounded samples (GEMV,
    MoE decode step, encoder, grouped GEMM).

  python bench.py [--steps K] [--warmup W] [--no-cpu] [--no-single-expert] [--no-dense-ref]
                  [--no-ffn] [--no-encode] [--no-sensitivity] [--copy-calibration]
  python bench.py --counters FETCH_DIR WRITE_DIR   (summarise rocprofv3 counter runs)
  python bench.py --source-hashes                  (hashes that stamp the profile summaries)
  python bench.py --trace-summary TRACE_DIR --steps K --warmup W
                                                   (per-kernel times of the timed steps from a
                                                    rocprofv3 --kernel-trace run of the same K, W)

HBM traffic: two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
WRITE_SIZE, with --copy-calibration so each run also holds plain copies of a
known size) are summarised by --counters into profiles/hbm_counters.json,
keyed by a hash of the kernel sources; `traffic` is reported only while that
hash matches the current sources.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP64_PEAK_TFLOPS = 78.6      # MI355X fp64 (matrix and vector)
SENS_CALIB = 512             # calibration rows of the sensitivity workload
BATCHES = (1, 4, 16, 64)
FFN_BATCHES = (1, 16, 64)
ENCODE_EXPERTS = 8
PREFILL_TOKENS = 2048
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")
COPY_MIB = 512               # plain copy used to calibrate the byte counters
COPY_REPS = 3


def kernel_source_hash(name: str) -> str:
    p = os.path.join(ROOT, "sparse_ternary_bit_amd", "csrc", name)
    h = hashlib.sha256()
    for f in (p, os.path.join(ROOT, "sparse_ternary_bit_amd", "csrc", "stq_device.hpp")):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_file: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source; otherwise None."""
    try:
        with open(PROFILE_COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_file)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel_file):
        return None
    return ent.get("bytes_per_launch")


def _read_counter_csvs(root: str, counter: str):
    """[(kernel_name, value)] per dispatch from rocprofv3 counter_collection.csv files."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                key = (f, r.get("Dispatch_Id"))
                name = r.get("Kernel_Name", "")
                per[key] = (name, per.get(key, (name, 0.0))[1] + float(r["Counter_Value"]))
    return list(per.values())


def summarise_counters(fetch_dir: str, write_dir: str) -> int:
    """Per-call HBM bytes of the GEMV (gemv_kernel plus its split reduction)
    and of the grouped GEMM, from FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each scaled by the factor that makes the plain copies in the
    same run read and write exactly their size."""
    out = {}
    lines = []
    factors = {}
    sums = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_counter_csvs(d, counter)
        copies = [v for (n, v) in rows if "copyBuffer" in n or "copy_kernel" in n]
        if not copies:
            print(f"no copy kernel dispatches in {d}", file=sys.stderr)
            return 1
        copy_kib = COPY_MIB * 1024.0
        big = [v for v in copies if v > 0.25 * copy_kib]
        f = copy_kib / (sum(big) / len(big))
        factors[counter] = f
        sums[counter] = {
            "gemv": (sum(v for (n, v) in rows if "gemv_kernel" in n), sum(1 for (n, _) in rows if "gemv_kernel" in n)),
            "reduce": (sum(v for (n, v) in rows if "reduce_splits_kernel" in n),
                       sum(1 for (n, _) in rows if "reduce_splits_kernel" in n)),
            "gemm": (sum(v for (n, v) in rows if "grouped_gemm_kernel" in n),
                     sum(1 for (n, _) in rows if "grouped_gemm_kernel" in n)),
        }
        lines.append(f"{counter}: plain copy of {COPY_MIB} MiB read as {sum(big) / len(big):.0f} KiB "
                     f"(mean of {len(big)}), scale factor {f:.4f}")
    calls = sums["FETCH_SIZE"]["gemv"][1]
    if calls == 0 or calls != sums["WRITE_SIZE"]["gemv"][1]:
        print("GEMV dispatch counts differ between the runs", file=sys.stderr)
        return 1
    gemv_fetch = (sums["FETCH_SIZE"]["gemv"][0] + sums["FETCH_SIZE"]["reduce"][0]) * 1024 * factors["FETCH_SIZE"] / calls
    gemv_write = (sums["WRITE_SIZE"]["gemv"][0] + sums["WRITE_SIZE"]["reduce"][0]) * 1024 * factors["WRITE_SIZE"] / calls
    out["k_gemv.hip"] = {"source_hash": kernel_source_hash("k_gemv.hip"), "calls": calls,
                         "fetch_bytes_per_call": round(gemv_fetch), "write_bytes_per_call": round(gemv_write),
                         "bytes_per_launch": round(gemv_fetch + gemv_write),
                         "scale_factors": {k: round(v, 5) for k, v in factors.items()}}
    lines.append(f"stq_gemv (gemv_kernel + reduce_splits_kernel), {calls} calls: "
                 f"fetch {gemv_fetch / 1e6:.2f} MB, write {gemv_write / 1e6:.2f} MB per call")
    g = sums["FETCH_SIZE"]["gemm"][1]
    if g and g == sums["WRITE_SIZE"]["gemm"][1]:
        gf = sums["FETCH_SIZE"]["gemm"][0] * 1024 * factors["FETCH_SIZE"] / g
        gw = sums["WRITE_SIZE"]["gemm"][0] * 1024 * factors["WRITE_SIZE"] / g
        out["k_gemm.hip"] = {"source_hash": kernel_source_hash("k_gemm.hip"), "calls": g,
                             "fetch_bytes_per_call": round(gf), "write_bytes_per_call": round(gw),
                             "bytes_per_launch": round(gf + gw),
                             "scale_factors": {k: round(v, 5) for k, v in factors.items()}}
        lines.append(f"grouped_gemm_kernel, {g} calls: fetch {gf / 1e6:.2f} MB, write {gw / 1e6:.2f} MB per call")
    with open(PROFILE_COUNTERS, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("\n".join(lines))
    return 0


def summarise_trace(trace_dir: str, warmup: int, steps: int) -> int:
    """Per-kernel durations from a rocprofv3 --kernel-trace run of this script:
    for every kernel called a multiple of (warmup + steps) times, the mean,
    min and max over the dispatches of the timed steps (the first warmup
    shares, by start time, are left out), beside the mean over all calls."""
    import csv
    import glob
    rows = {}
    for f in sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name", "")
                rows.setdefault(name, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    if not rows:
        print(f"no kernel_trace.csv under {trace_dir}", file=sys.stderr)
        return 1
    total = warmup + steps
    print("| Kernel | Calls | Timed calls | Mean timed us | Min us | Max us | Mean all us |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    out = []
    for name, ds in rows.items():
        ds.sort()
        dur = [(e - b) / 1e3 for b, e in ds]
        timed = dur[warmup * len(dur) // total:] if len(dur) % total == 0 else []
        out.append((sum(dur), name, len(dur), timed, dur))
    for _, name, n, timed, dur in sorted(out, reverse=True):
        short = name if len(name) <= 70 else name[:70] + "..."
        if timed:
            print(f"| {short} | {n} | {len(timed)} | {sum(timed) / len(timed):.1f} | {min(timed):.1f} | "
                  f"{max(timed):.1f} | {sum(dur) / n:.1f} |")
        else:
            print(f"| {short} | {n} | - | - | {min(dur):.1f} | {max(dur):.1f} | {sum(dur) / n:.1f} |")
    return 0


def cpu_baseline():
    """The oracle as it stands, timed on this host on bounded samples of the
    workloads (single-threaded: BLAS limited to one thread; the oracle's other
    array work is single-threaded NumPy):
      * GEMV: one 4096 x 7168 expert (the oracle's own WLS encoding of expert
        0's draw), one bf16 token: decode + fp64 dot, in the GPU's
        algorithmic-byte unit (`value`);
      * MoE decode step (16 tokens x top-8): 16 of its 128 pairs, each a full
        expert decode + dot as the oracle does it, scaled to the step;
      * encoder: WLS (3 rounds) rows/s on the 256 x 1024 case and on 1024
        rows of the 4096 x 7168 expert;
      * grouped GEMM: two experts' 64-token slices (decode + fp64 matmul), in
        useful TFLOP/s."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import stq_workloads as W
    import synth_inputs as S
    from oracle import stq_oracle as O

    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
           if k in os.environ}
    host_cores = len(os.sched_getaffinity(0))
    N, K = W.N_ROWS, W.K
    q = S.calibration_imatrix(W.IMATRIX_SEED, 64, K)
    w = W.expert_weight_rows(W.TABLE_SEED, 0, np.arange(N))
    out = {}
    with threadpool_limits(limits=1):
        # encoder: the small case, then 1024 rows of the expert; the whole expert is
        # encoded (untimed past its first 1024 rows) for the GEMV items below
        w1, q1, _ = S.single_gemv_case()
        t0 = time.perf_counter()
        O.quantize_rows(w1, q1)
        t_small = time.perf_counter() - t0
        t0 = time.perf_counter()
        parts = [O.quantize_rows(w[:1024], q)]
        t_big = time.perf_counter() - t0
        for r in range(1024, N, 1024):
            parts.append(O.quantize_rows(w[r:r + 1024], q))
        # row tiles of 64 rows are whole inside each 1024-row part, so the parts concatenate
        packed = np.concatenate([p.reshape(-1) for p in parts])
        del w
        xb, xf = S.bf16_normal(np.random.default_rng(4000), (16, K))
        expert_bytes = packed.nbytes
        # GEMV, one expert, one token
        O.gemv(packed, N, K, xf[0])                           # warm
        t0 = time.perf_counter()
        reps = 3
        for i in range(reps):
            O.gemv(packed, N, K, xf[i])
        t_gemv = (time.perf_counter() - t0) / reps
        gemv_gbs = (expert_bytes + K * 2 + N * 4) / t_gemv / 1e9
        # MoE decode step sample: 16 pairs (each decodes its expert), scaled to 128 pairs
        t0 = time.perf_counter()
        for i in range(16):
            O.gemv(packed, N, K, xf[i])
        t16 = time.perf_counter() - t0
        step_bytes = 101.96 * expert_bytes + 16 * K * 2 + 128 * N * 4
        step_s = t16 * 128 / 16
        # grouped GEMM sample: two experts x 64 tokens
        table = np.concatenate([packed, packed])
        xg = xf[np.arange(128) % 16]
        offs = np.array([0, 64, 128], dtype=np.int32)
        t0 = time.perf_counter()
        O.grouped_gemm(table, expert_bytes, N, K, xg, offs)
        t_gemm = time.perf_counter() - t0
    out = {"value": round(gemv_gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": (f"oracle GEMV of one 4096x7168 expert (decode + fp64 dot), one bf16 token, "
                      f"{reps} calls of {t_gemv:.2f} s; same algorithmic-byte count as the GPU figure. "
                      f"Single-threaded (BLAS limited to 1 thread); host has {host_cores} cores"),
           "host_cores": host_cores, "blas_threads": 1, "thread_env": env,
           "moe_decode_step_16x8": {"s_per_step": round(step_s, 2), "GB/s": round(step_bytes / step_s / 1e9, 4),
                                    "sample": "16 of the 128 pairs, scaled"},
           "encode_rows_per_s": {"256x1024": round(256 / t_small, 1), "4096x7168_expert": round(1024 / t_big, 1),
                                 "sample": "WLS, 3 rounds; 1024 rows of the expert"},
           "grouped_gemm": {"TFLOP/s": round(2.0 * 128 * N * K / t_gemm / 1e12, 6), "s": round(t_gemm, 2),
                            "sample": "2 experts x 64 tokens of the 2048-token prefill shape"}}
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-single-expert", action="store_true",
                    help="skip the single-expert GEMV over 100 resident experts (1000 launches)")
    ap.add_argument("--no-dense-ref", action="store_true",
                    help="skip the dense bf16 GEMM reference (hipBLASLt through torch) beside the grouped GEMM")
    ap.add_argument("--no-encode", action="store_true",
                    help="skip the timed layer-scale encode (8 experts, both encoders)")
    ap.add_argument("--no-sensitivity", action="store_true",
                    help="skip the layer-sensitivity scoring workload")
    ap.add_argument("--no-ffn", action="store_true",
                    help="skip the routed-expert FFN lines (profiling runs of the GEMV and GEMM alone)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"after timing, copy {COPY_MIB} MiB device to device {COPY_REPS} times (counter calibration)")
    ap.add_argument("--counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/hbm_counters.json")
    ap.add_argument("--source-hashes", action="store_true",
                    help="print the kernel-source hashes that stamp the profile summaries")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace run of this script made with the same --steps/--warmup")
    args = ap.parse_args()
    if args.counters:
        return summarise_counters(*args.counters)
    if args.trace_summary:
        return summarise_trace(args.trace_summary, args.warmup, args.steps)
    if args.source_hashes:
        for name in ("k_gemv.hip", "k_gemm.hip", "k_moe.hip", "k_codec.hip", "k_sens.hip", "k_probe.hip"):
            print(f"{name} {kernel_source_hash(name)}")
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the STQ1_0 path here has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import sparse_ternary_bit_amd as stq
    import stq_workloads as W
    import synth_inputs as S

    if not os.path.exists(stq.lib_path()):
        from sparse_ternary_bit_amd import build as _b
        _b.build(verbose=False)
    stq.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N, K, E = W.N_ROWS, W.K, W.N_EXPERTS
    rb = stq.row_bytes(K)
    expert_bytes = N * rb

    # ---------------- setup (untimed) ----------------
    q = W.table_imatrix(device=dev)
    t_wls, stride = W.encode_table(imatrix=q, encoder=stq.ENC_WLS, device=dev)
    t_amax, _ = W.encode_table(imatrix=q, encoder=stq.ENC_AMAX, device=dev)
    tables = {"wls": t_wls, "amax": t_amax}
    t_down, down_stride = W.encode_down_table(device=dev)
    down_bytes = W.K * stq.row_bytes(W.D_FF)

    total_steps = args.warmup + args.steps
    sweep = []   # per step: list of (batch, pe, pt, x, y, algorithmic bytes)
    for s in range(total_steps):
        items = []
        for B in BATCHES:
            pe_t, pt_t, pe, pt = W.decode_pairs(50000 + 1000 * s + B, B, device=dev)
            x = S.torch_bf16_normal(90000 + 1000 * s + B, (B, K), device=dev)
            y = torch.empty((B * W.TOP_K, N), dtype=torch.float32, device=dev)
            uniq = len(np.unique(pe))
            nbytes = uniq * expert_bytes + B * K * 2 + B * W.TOP_K * N * 4
            items.append((B, pe_t, pt_t, x, y, nbytes, uniq))
        ffn = []
        for B in FFN_BATCHES:
            pe_t, _, pe, _ = W.decode_pairs(70000 + 1000 * s + B, B, device=dev)
            pw = torch.from_numpy(S.routing_weights(80000 + 1000 * s + B, B, W.TOP_K)).to(dev)
            x = S.torch_bf16_normal(60000 + 1000 * s + B, (B, K), device=dev)
            y = torch.empty((B, K), dtype=torch.float32, device=dev)
            uniq = len(np.unique(pe))
            nbytes = uniq * (expert_bytes + down_bytes) + B * K * 2 + B * K * 4
            ffn.append((B, pe_t, pw, x, y, nbytes))
        items = (items, ffn)
        sweep.append(items)
    x_sorted, offsets_t, _, offsets = W.prefill_batch(PREFILL_TOKENS, K, device=dev)
    total_m = int(offsets[-1])
    y_pre = torch.empty((total_m, N), dtype=torch.float32, device=dev)
    gemm_flop = 2.0 * total_m * N * K

    # workspaces for the timed calls, sized once (the library allocates nothing)
    ws_gemv = torch.empty(max(stq.gemv_plan(E, N, K, B * W.TOP_K)[2] for B in BATCHES + (1,)) + 256,
                          dtype=torch.uint8, device=dev)
    ws_ffn = torch.empty(max(stq.moe_ffn_workspace(E, K, W.D_FF, B, W.TOP_K) for B in FFN_BATCHES) + 256,
                         dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def run_step(s, rec):
        # the prefill GEMM first: while it runs, the host queues the decode
        # sweep behind it, so the short GEMV calls run back to back instead of
        # waiting on the host between calls
        a, b = ev(), ev()
        a.record(stream)
        stq.grouped_gemm(t_wls, stride, E, N, K, x_sorted, offsets_t, out=y_pre)
        b.record(stream)
        rec["gemm"].append((a, b))
        # the two encodings of each batch back to back, first one then the
        # other on alternate steps, so both see the same neighbouring work
        # (the amax copy checks that speed does not depend on the encoder)
        order = ("wls", "amax") if s % 2 == 0 else ("amax", "wls")
        for (B, pe_t, pt_t, x, y, nbytes, uniq) in sweep[s][0]:
            for enc in order:
                a, b = ev(), ev()
                a.record(stream)
                stq.gemv(tables[enc], stride, E, N, K, x, pe_t, pt_t, out=y, workspace=ws_gemv)
                b.record(stream)
                rec["gemv"].append((enc, B, nbytes, uniq, a, b))
        for (B, pe_t, pw, x, y, nbytes) in ([] if args.no_ffn else sweep[s][1]):
            a, b = ev(), ev()
            a.record(stream)
            stq.moe_ffn_decode(t_wls, stride, t_down, down_stride, E, K, W.D_FF, x, pe_t, pw, W.TOP_K, out=y,
                               workspace=ws_ffn)
            b.record(stream)
            rec["ffn"].append((B, nbytes, a, b))

    # Python's cyclic garbage collector is off while the GPU is timed (as timeit
    # does): a full collection in this process takes up to tens of ms, and one
    # that lands while the launch queue runs dry leaves the GPU idle between the
    # two events of a call, which then counts as that call's time
    gc.collect()
    gc.disable()
    for s in range(args.warmup):
        run_step(s, {"gemv": [], "gemm": [], "ffn": []})
    torch.cuda.synchronize()

    rec = {"gemv": [], "gemm": [], "ffn": []}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.warmup, total_steps):
        run_step(s, rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if args.copy_calibration:
        src = torch.ones(COPY_MIB << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # streaming-read reference for the GEMV roofline: the library's plain
    # read kernel over 2 GiB gives the read rate this GPU sustains, reported
    # beside the published peak
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    big.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stq.stream_read_probe(big, sink)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record(stream)
    for _ in range(5):
        stq.stream_read_probe(big, sink)
    b.record(stream)
    torch.cuda.synchronize()
    stream_read_gbs = 5 * big.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
    del big, sink

    # matrix-core and LDS references beside the grouped GEMM: a loop of
    # independent bf16 MFMAs (no memory traffic), and LDS reads of the two
    # forms the GEMM issues (16-byte activation reads, pattern-table read pairs)
    n_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    fsink = torch.zeros(1, dtype=torch.float32, device=dev)
    isink = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps
    MFMA_ROUNDS, LDS_ROUNDS = 512, 1024
    t_mfma = timed(lambda: stq.mfma_loop_probe(MFMA_ROUNDS, fsink))
    mfma_loop_tflops = stq.MFMA_PROBE_FLOP_PER_ROUND * MFMA_ROUNDS / t_mfma / 1e12
    lds = {"cus": n_cus}
    for mode, name, nbytes in ((0, "b128", 1024), (1, "read2_b32", 512)):
        t = timed(lambda: stq.lds_read_probe(mode, LDS_ROUNDS, isink))
        per_ns = stq.LDS_PROBE_READS_PER_ROUND * LDS_ROUNDS / (t * 1e9) / n_cus
        lds[f"{name}_reads_per_ns_per_CU"] = round(per_ns, 3)
        lds[f"{name}_bytes_per_ns_per_CU"] = round(per_ns * nbytes, 1)
    del fsink, isink

    enc_out = None
    if not args.no_encode:
        # encoder as a layer-scale workload: 8 experts' fp32 gate/up weights drawn
        # beforehand, then only the quantize launches are timed
        ws = [S.torch_expert_weights(W.TABLE_SEED, e, N, K, device=dev) for e in range(ENCODE_EXPERTS)]
        outq = torch.empty(N * rb, dtype=torch.uint8, device=dev)
        enc_out = {}
        for name, enc in (("wls", stq.ENC_WLS), ("amax", stq.ENC_AMAX)):
            stq.quantize_rows(ws[0], q if enc == stq.ENC_WLS else None, encoder=enc, out=outq)  # warm
            a, b = ev(), ev()
            a.record(stream)
            for w_e in ws:
                stq.quantize_rows(w_e, q if enc == stq.ENC_WLS else None, encoder=enc, rounds=3, out=outq)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / len(ws)
            enc_out[name] = {"ms_per_expert": round(ms, 4),
                             "layer_ms": round(ms * E, 1),
                             "Gweights_per_s": round(N * K / (ms * 1e-3) / 1e9, 1),
                             "fp32_read_GB/s": round(N * K * 4 / (ms * 1e-3) / 1e9, 1)}
        del ws, outq

    sens_out = None
    if not args.no_sensitivity:
        # full-Hessian vs diagonal scoring of one expert's gate/up matrix: the
        # weights, their STQ1_0 reconstruction and the calibration rows are
        # resident before timing; only stq_layer_errors (and separately the
        # 2-bit stand-in pass) is timed
        w0 = S.torch_expert_weights(W.TABLE_SEED, 0, N, K, device=dev)
        gx = torch.Generator(device=dev)
        gx.manual_seed(4242)
        xc = torch.randn((SENS_CALIB, K), generator=gx, device=dev, dtype=torch.float32)
        xc.mul_(torch.rand((1, K), generator=gx, device=dev, dtype=torch.float32).mul_(9.9).add_(0.1))
        w0_hat = stq.dequantize_rows(stq.quantize_rows(w0, (xc * xc).mean(dim=0)), N, K)
        ef = torch.empty(N, dtype=torch.float64, device=dev)
        ed = torch.empty(N, dtype=torch.float64, device=dev)
        q2o = torch.empty_like(w0)
        lws = torch.empty(stq.layer_errors_workspace(N, K, SENS_CALIB), dtype=torch.uint8, device=dev)
        stq.layer_errors(w0, w0_hat, xc, ef, ed, workspace=lws)  # warm
        stq.q2_roundtrip(w0, q2o)
        reps = 20
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            stq.layer_errors(w0, w0_hat, xc, ef, ed, workspace=lws)
        b.record(stream)
        c, d_ = ev(), ev()
        c.record(stream)
        for _ in range(reps):
            stq.q2_roundtrip(w0, q2o)
        d_.record(stream)
        torch.cuda.synchronize()
        le_ms = a.elapsed_time(b) / reps
        q2_ms = c.elapsed_time(d_) / reps
        flop = 2.0 * N * K * SENS_CALIB
        tf = flop / (le_ms * 1e-3) / 1e12
        sens_out = {"rows": N, "k": K, "calibration_rows": SENS_CALIB,
                    "layer_errors_us": round(1e3 * le_ms, 1),
                    "roofline": {"bound": "mfma", "dtype": "f64", "achieved": round(tf, 2),
                                 "peak": FP64_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tf / FP64_PEAK_TFLOPS, 4),
                                 "flop_per_call": flop,
                                 "kernels": "hdiag_kernel + layer_errors_kernel + sum_partials_kernel"},
                    "q2_roundtrip_us": round(1e3 * q2_ms, 1),
                    "q2_roundtrip_GB/s": round(2 * N * K * 4 / (q2_ms * 1e-3) / 1e9, 1),
                    "full_over_diag": round(float(ef.sum() / ed.sum()), 4)}
        del w0, xc, w0_hat, ef, ed, q2o

    single_out = None
    if not args.no_single_expert:
        # one expert's gate+up GEMV at batch 1 over 100 resident experts
        # (481.7 MB, beyond the 256 MB last-level cache), one launch per expert in
        # rotation, 1000 launches in all; a short spin on the GPU before each
        # rotation lets the host queue the rotation ahead of the GPU, so each
        # launch's events bracket the kernels alone
        xs1 = [S.torch_bf16_normal(4000 + i, (1, K), device=dev) for i in range(100)]
        pes1 = [torch.tensor([i], dtype=torch.int32, device=dev) for i in range(100)]
        ys1 = torch.empty((1, N), dtype=torch.float32, device=dev)
        ws1 = torch.empty(max(1, stq.gemv_plan(E, N, K, 1)[2]), dtype=torch.uint8, device=dev)
        for i in range(100):
            stq.gemv(t_wls, stride, E, N, K, xs1[i], pes1[i], out=ys1, workspace=ws1)
        torch.cuda.synchronize()
        evs = []
        for rot in range(10):
            torch.cuda._sleep(20_000_000)
            for i in range(100):
                a, b = ev(), ev()
                a.record(stream)
                stq.gemv(t_wls, stride, E, N, K, xs1[i], pes1[i], out=ys1, workspace=ws1)
                b.record(stream)
                evs.append((a, b))
            torch.cuda.synchronize()
        sm = [a.elapsed_time(b) for (a, b) in evs]
        sb = expert_bytes + K * 2 + N * 4
        single_out = {"launches": len(sm), "experts_resident": 100, "bytes_per_call": sb,
                      "us_median": round(1e3 * float(np.median(sm)), 2),
                      "us_p10": round(1e3 * float(np.percentile(sm, 10)), 2),
                      "us_p90": round(1e3 * float(np.percentile(sm, 90)), 2),
                      "GB/s_median": round(sb / (float(np.median(sm)) * 1e-3) / 1e9, 1)}
        # the same 100 calls captured once into a HIP graph and replayed: a
        # decode loop's per-call cost without host launch gaps
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for i in range(100):
                    stq.gemv(t_wls, stride, E, N, K, xs1[i], pes1[i], out=ys1, workspace=ws1)
        torch.cuda.current_stream().wait_stream(cs)
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(5):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        per = a.elapsed_time(b) / 500
        single_out["graph_us_per_call"] = round(1e3 * per, 2)
        single_out["graph_GB/s"] = round(sb / (per * 1e-3) / 1e9, 1)
        del g, xs1, pes1, ys1, ws1

    dense_out = None
    if not args.no_dense_ref:
        # the MFMA rate a dense bf16 GEMM of the prefill's total shape reaches on
        # this GPU through the vendor library (hipBLASLt via torch.matmul):
        # [16384 x 7168] x [7168 x 4096], fp32 accumulation, bf16 out
        xa = torch.randn((total_m, K), device=dev, dtype=torch.float32).to(torch.bfloat16)
        wb = torch.randn((K, N), device=dev, dtype=torch.float32).to(torch.bfloat16)
        for _ in range(3):
            yd = xa @ wb
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(10):
            yd = xa @ wb
        b.record(stream)
        torch.cuda.synchronize()
        dms = a.elapsed_time(b) / 10
        dense_out = {"dense_bf16_gemm_TFLOP/s": round(gemm_flop / (dms * 1e-3) / 1e12, 1),
                     "dense_bf16_gemm_us": round(1e3 * dms, 1)}
        del xa, wb, yd

    # ---------------- results ----------------
    gemv_ms = [a.elapsed_time(b) for (_, _, _, _, a, b) in rec["gemv"]]
    gemv_bytes = [nb for (_, _, nb, _, _, _) in rec["gemv"]]
    tot_b, tot_ms = float(sum(gemv_bytes)), float(sum(gemv_ms))
    gemv_gbs = tot_b / (tot_ms * 1e-3) / 1e9
    per_batch = {}
    for enc in ("wls", "amax"):
        for B in BATCHES:
            sel = [(nb, ms, u) for (e_, b_, nb, u, _, _), ms in zip(rec["gemv"], gemv_ms) if e_ == enc and b_ == B]
            bb = sum(x[0] for x in sel)
            mm = sum(x[1] for x in sel)
            per_batch[f"{enc}_b{B}"] = {"GB/s": round(bb / (mm * 1e-3) / 1e9, 1),
                                        "us": round(1e3 * mm / len(sel), 2),
                                        "experts": round(sum(x[2] for x in sel) / len(sel), 1)}
    gemm_ms = [a.elapsed_time(b) for (a, b) in rec["gemm"]]
    gemm_avg = float(np.mean(gemm_ms))
    gemm_tflops = gemm_flop / (gemm_avg * 1e-3) / 1e12

    n_launch = len(gemv_ms)
    traffic = measured_traffic("k_gemv.hip")
    traffic_gemm = measured_traffic("k_gemm.hip")
    out = {
        "metric": "STQ1_0 expert GEMV HBM GB/s (% peak); prefill grouped-GEMM TFLOP/s (% peak)",
        "value": round(gemv_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * wall / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "moe_layer_sweep_and_prefill", "experts": E, "n": N, "k": K,
                   "top_k": W.TOP_K, "decode_batches": list(BATCHES), "decode_tables": ["wls", "amax"],
                   "prefill_tokens": PREFILL_TOKENS, "prefill_rows": total_m,
                   "weights": "iid N(0,0.02) fp32 encoded to STQ1_0 (42 B / 256)",
                   "activations": "bf16 N(0,1)"},
        "roofline": {"bound": "hbm", "achieved": round(tot_b / n_launch / (tot_ms / n_launch * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "gemv_kernel (stq_gemv)",
                     "stream_read_GB/s": round(stream_read_gbs, 1),
                     "frac_of_stream_read": round(gemv_gbs / stream_read_gbs, 4),
                     "algorithmic_bytes_per_launch": round(tot_b / n_launch),
                     "avg_launch_us": round(1e3 * tot_ms / n_launch, 2)},
        "roofline_gemm": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(gemm_tflops / BF16_PEAK_TFLOPS, 4),
                          "traffic": traffic_gemm, "kernel": "grouped_gemm_kernel (stq_grouped_gemm)",
                          "flop_per_launch": gemm_flop, "avg_launch_us": round(1e3 * gemm_avg, 1),
                          "launch_us_min_max": [round(1e3 * min(gemm_ms), 1), round(1e3 * max(gemm_ms), 1)],
                          "mfma_loop_TFLOP/s": round(mfma_loop_tflops, 1),
                          "frac_of_mfma_loop": round(gemm_tflops / mfma_loop_tflops, 4)},
        "lds_probe": lds,
        "gemv_sweep": per_batch,
    }
    ffn = {}
    for B in ([] if args.no_ffn else FFN_BATCHES):
        sel = [(nb, a.elapsed_time(b)) for (b_, nb, a, b) in rec["ffn"] if b_ == B]
        ms = sum(t for _, t in sel)
        ffn[f"b{B}"] = {"us": round(1e3 * ms / len(sel), 2),
                        "GB/s": round(sum(nb for nb, _ in sel) / (ms * 1e-3) / 1e9, 1)}
    if enc_out:
        out["encode_layer"] = {"experts_timed": ENCODE_EXPERTS,
                               "weights_per_expert": N * K,
                               "rounds": 3, **enc_out}
    if sens_out:
        out["layer_sensitivity"] = sens_out
    if ffn:
        out["moe_ffn_decode"] = {"layer": "256 experts, top-8, gate/up 4096x7168 + down 7168x2048, STQ1_0",
                                 "bytes": "touched experts' packed gate/up and down matrices, x and y", **ffn}
    if single_out:
        out["single_expert_gemv"] = single_out
    if dense_out:
        out["roofline_gemm"].update(dense_out)
        out["roofline_gemm"]["frac_of_dense_bf16_gemm"] = round(gemm_tflops / dense_out["dense_bf16_gemm_TFLOP/s"], 4)
    gc.enable()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
