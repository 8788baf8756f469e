#!/usr/bin/env python3
"""TwELL FFN forward throughput on one MI355X.

One step = one pass of the inference hot path over one batch: twell_pack
(gate GEMM + ReLU + TwELL epilogue, one dispatch) then twell_ffn_fwd (fused
up + down: one kernel, dispatched once per generation of resident workgroups,
two at this shape), on synthetic Llama-2B-shaped FFN inputs already
resident in HBM (T=16384 tokens, d_model=2048, d_ff=8192, bf16, T_n=128,
C=16, ~0.5% gate density).  Prints one JSON line.

Also timed in the same run, the same way: the library's dense MFMA FFN
(speed-up), per-kernel averages from HIP events on the launch stream (the
roofline object), and the CPU oracle on a bounded token sample
(cpu_baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, help="workload id (default: the 2B-class inference shape)")
    ap.add_argument("--rho", type=float, default=None, help="override the gate density (sweep workload)")
    ap.add_argument("--T", type=int, default=None, help="override the token count")
    ap.add_argument("--d-model", type=int, default=None,
                    help="override d_model (e.g. 4096 with --d-ff 11008: a Llama-7B-shaped layer)")
    ap.add_argument("--d-ff", type=int, default=None,
                    help="override d_ff (e.g. 1024: one GPU's share of the 2B-class FFN split 8 ways over neurons)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense comparator")
    ap.add_argument("--no-classic", action="store_true", help="skip the classic two-kernel ELL baseline")
    ap.add_argument("--no-train", action="store_true", help="skip the training-step measurement")
    ap.add_argument("--train-config", type=int, default=4, help="workload of the training-step measurement")
    ap.add_argument("--max-dense-rows", type=int, default=1024)
    ap.add_argument("--cold-iters", type=int, default=20,
                    help="iterations of the cold-cache timing (a 1 GiB write before each; 0 = skip)")
    ap.add_argument("--no-hipblaslt", action="store_true", help="skip the torch.matmul dense sanity point")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the step line: the density sweep of the 2B-class shape (0.1..5%% and a "
                         "16-token batch), TwELL (plain and hybrid) against the dense FFN; prints one JSON line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before timing, run one plain fp32 negation of this many MiB (reads and writes "
                         "exactly that much): the reference dispatch that scales rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE to bytes")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                    help="no GPU work: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --calib-copy-mib run into profiles/traffic_<kernel>.json")
    ap.add_argument("--traffic-command", default="", help="command line recorded with --traffic-summary")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of the step line: the MFMA-ceiling probe alone (the gate kernel's occupancy and "
                         "MFMA instruction with register operands, plus the shader clock during it); prints one JSON line")
    ap.add_argument("--gather-ceiling", action="store_true",
                    help="instead of the step line: the gather-ceiling probe alone (rows of the 2B-class "
                         "W_up^T / W_down, random and XCD-shared, two and eight rows in flight per wave); "
                         "prints one JSON line")
    return ap.parse_args()


# sources whose change invalidates a kernel's measured counters
KERNEL_SOURCES = {
    "gate_pack": ["k_gate_pack.hip", "gemm256.hpp", "gemm_core.hpp", "common.hpp"],
    "fused_updown": ["k_fused_updown.hip", "balance.hpp", "common.hpp"],
}
# substrings of the dispatch names of each kernel
KERNEL_NAMES = {"gate_pack": "gate_pack", "fused_updown": "fused_updown", "calib_copy": "neg_kernel"}


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "activation_sparse_feedforward_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, src_hash: str, per_launch_units: float):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summaries, only if they were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(p):
        return None
    with open(p) as fh:
        t = json.load(fh)
    if t.get("source_hash") != src_hash:
        return None
    return t.get("bytes_per_launch")


def _pmc_per_dispatch(path: str, counter: str):
    """{kernel key: mean counter value per dispatch} from a counter_collection.csv."""
    import csv
    vals = {}
    with open(path, newline="") as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            for key, pat in KERNEL_NAMES.items():
                if pat in row["Kernel_Name"]:
                    vals.setdefault(key, {}).setdefault(row["Dispatch_Id"], 0.0)
                    vals[key][row["Dispatch_Id"]] += float(row["Counter_Value"])
    return {k: (sum(d.values()) / len(d), len(d)) for k, d in vals.items()}


def traffic_summary(fetch_csv: str, write_csv: str, calib_mib: int, command: str, out_dir: str | None = None):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same counters
    read for the calibration copy of known size, and store bytes per launch
    (as traffic_<kernel>.json in out_dir, by default profiles/)."""
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    fetch = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_csv, "WRITE_SIZE")
    if "calib_copy" not in fetch or "calib_copy" not in write:
        raise SystemExit("no calibration copy dispatch in the counter files (run bench.py with --calib-copy-mib)")
    known = calib_mib * 1024 * 1024
    f_fac = known / (fetch["calib_copy"][0] * 1024)
    w_fac = known / (write["calib_copy"][0] * 1024)
    # one step calls twell_pack (one gate dispatch) and twell_ffn_fwd (one dispatch per generation of
    # lockstep workgroups), so the bytes of a call are a kernel's total over the gate dispatch count
    calls = fetch["gate_pack"][1] if "gate_pack" in fetch else None
    out = {}
    for key in KERNEL_SOURCES:
        if key not in fetch or key not in write:
            continue
        n_call = calls or fetch[key][1]
        rb = fetch[key][0] * fetch[key][1] / n_call * 1024 * f_fac
        wb = write[key][0] * write[key][1] / n_call * 1024 * w_fac
        rec = {"kernel": key, "source_hash": kernel_source_hash(KERNEL_SOURCES[key]),
               "fetch_kib_per_dispatch": round(fetch[key][0], 1), "write_kib_per_dispatch": round(write[key][0], 1),
               "dispatches": [fetch[key][1], write[key][1]], "calls": n_call,
               "calib_copy_bytes": known, "calib_fetch_kib": round(fetch["calib_copy"][0], 1),
               "calib_write_kib": round(write["calib_copy"][0], 1),
               "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
               "read_bytes_per_launch": int(rb), "write_bytes_per_launch": int(wb),
               "bytes_per_launch": int(rb + wb), "command": command}
        with open(os.path.join(out_dir, f"traffic_{key}.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        out[key] = rec
    print(json.dumps(out, indent=1))


def cpu_baseline(inp, budget_s: float, tile_n: int, slots: int, dtype: str):
    """Time the CPU oracle on bounded token samples of the timed workload: its
    dense float64 forward, and its sparse path (float64 gate, ReLU rounded to
    the storage dtype, TwELL pack, TwELL forward), each for about half the
    budget."""
    import numpy as np
    from oracle import twell_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    x = inp["x"]
    chunk = 256

    def run(fn, budget):
        done, t0 = 0, time.perf_counter()
        while done < x.shape[0]:
            fn(x[done:done + chunk])
            done += chunk
            if time.perf_counter() - t0 >= budget:
                break
        return done, time.perf_counter() - t0

    def sparse(xs):
        _, a = O.gate_forward(xs, inp["w_gate_t"])
        c, i, v = O.twell_pack(O.round_to_storage(a, dtype), tile_n, slots)
        return O.twell_forward(xs, c, i, v, tile_n, inp["w_up_t"], inp["w_down"])

    nd, td = run(lambda xs: O.ffn_forward(xs, inp["w_gate_t"], inp["w_up_t"], inp["w_down"]), budget_s / 2)
    ns, ts = run(sparse, budget_s / 2)
    return {"value": nd / td, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"dense: first {nd} tokens of the timed workload, oracle float64 forward (NumPy matmul), "
                      f"{td:.1f} s; sparse path: first {ns} tokens, oracle gate + TwELL pack + TwELL forward, "
                      f"{ts:.1f} s",
            "sparse_path_value": ns / ts}


def gather_ceiling(wu, wd, stream, steps=256, reps=5):
    """Rate at which the memory system serves the fused kernel's access pattern
    (one workgroup per CU of 16 waves, 8 for rows wider than 4 KB; whole weight
    rows, two rows per step) with no arithmetic: random rows (mostly past L2)
    and rows shared by every wave of an XCD (mostly from L2), each with two and
    with eight rows in flight per wave (four for rows wider than 4 KB).
    Returns GB/s per case and the ceilings (best of the two depths)."""
    import ctypes
    import numpy as np
    import torch
    path = os.path.join(ROOT, "activation_sparse_feedforward_amd", "libtwell_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the library first")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.twell_probe_gather.restype = ctypes.c_int
    lib.twell_probe_gather.argtypes = [P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, P, P]
    rows, row_bytes = wu.shape[0], wu.shape[1] * wu.element_size()
    waves, deep = (16, 8) if row_bytes <= 4096 else (8, 4)  # per workgroup; rows in flight per wave
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 16, dtype=torch.int32, device="cuda")
    st = stream.cuda_stream

    def run(shared, depth):
        rc = lib.twell_probe_gather(wu.data_ptr(), wd.data_ptr(), rows, row_bytes, steps, shared, depth, blocks,
                                    out.data_ptr(), st)
        if rc != 0:
            raise RuntimeError(f"twell_probe_gather returned {rc}")

    res = {}
    for shared, name in ((0, "random"), (1, "xcd_shared")):
        for depth in (1, 4):
            run(shared, depth)
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(shared, depth)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            nbytes = blocks * waves * steps * 2 * row_bytes
            res[f"{name}_rows_{2 if depth == 1 else deep}_in_flight_gbs"] = round(
                nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)
    res["random_ceiling_gbs"] = max(res["random_rows_2_in_flight_gbs"], res[f"random_rows_{deep}_in_flight_gbs"])
    res["xcd_shared_ceiling_gbs"] = max(res["xcd_shared_rows_2_in_flight_gbs"],
                                        res[f"xcd_shared_rows_{deep}_in_flight_gbs"])
    res["bytes_per_launch"] = blocks * waves * steps * 2 * row_bytes
    return res


def mfma_ceiling(stream, iters=20000, reps=5, random_operands=True):
    """Rate of the matrix cores under the gate kernel's MFMA load with nothing
    else: one workgroup of four waves per CU, each wave issuing
    v_mfma_f32_32x32x16_bf16 on 16 independent accumulators from registers,
    with operands of random bf16 values (eight A and eight B fragments cycled
    through, as a GEMM's change every k-step) or one constant fragment pair.
    Also the shader clock during the loop (shader-clock cycles over 100 MHz
    ticks, median over the waves) and the cycles one MFMA took at that clock.
    Returns TFLOP/s (median of `reps` launches) and those figures."""
    import ctypes
    import numpy as np
    import torch
    path = os.path.join(ROOT, "activation_sparse_feedforward_amd", "libtwell_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build the library first")
    lib = ctypes.CDLL(path)
    lib.twell_probe_mfma.restype = ctypes.c_int
    lib.twell_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(blocks * 8, dtype=torch.int64, device="cuda")
    # 16 x 64 pieces of 8 bf16 values, N(0, 1) (finite), seeded
    g = torch.Generator().manual_seed(5)
    frags = torch.randn(16 * 64 * 8, generator=g).to(torch.bfloat16).cuda() if random_operands else None

    def run():
        rc = lib.twell_probe_mfma(iters, blocks, frags.data_ptr() if frags is not None else None, out.data_ptr(),
                                  clocks.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"twell_probe_mfma returned {rc}")

    run()
    torch.cuda.synchronize()
    ts, ghz = [], []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz.append(float(np.median(c[:, 0] / (c[:, 1] / 100e6))) / 1e9)
    flop = blocks * 4 * iters * 16 * 32768.0
    ms = float(np.median(ts))
    clock = float(np.median(ghz))
    cyc = (float(np.median(clocks.view(-1, 2)[:, 0].cpu().numpy().astype(np.float64)))) / (iters * 16)
    return {"operands": "random" if random_operands else "constant",
            "tflops": round(flop / (ms * 1e-3) / 1e12, 1), "clock_ghz": round(clock, 3),
            "cycles_per_mfma": round(cyc, 2), "peak_at_clock_tflops": round(blocks * 4 * 32768 / 32 * clock * 1e9 / 1e12, 1),
            "flop_per_launch": flop, "ms_per_launch": round(ms, 4)}


def _pct(v):
    import numpy as np
    return {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
            "p90": round(float(np.percentile(v, 90)), 4)}


def cold_timing(phases, iters, stream):
    """Per-phase times with L2 and MALL flushed before every iteration: a 1 GiB
    buffer is written (and the write completed) before each timed pass.
    phases: list of (name, callable)."""
    import torch
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    out = {n: [] for n, _ in phases}
    out["total"] = []
    for k in range(iters):
        flush.fill_(float(k))
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(phases):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for i, (n, _) in enumerate(phases):
            out[n].append(ev[i].elapsed_time(ev[i + 1]))
        out["total"].append(ev[0].elapsed_time(ev[-1]))
    del flush
    return {n: _pct(v) for n, v in out.items()}


def hipblaslt_dense(x, wg, wu, wd, steps, warmup, stream):
    """The dense FFN through torch.matmul (hipBLASLt GEMMs, torch elementwise),
    as a sanity point for the library's own dense path."""
    import torch

    def run():
        g = torch.matmul(x, wg.t())
        u = torch.matmul(x, wu.t())
        return torch.matmul(torch.relu(g) * u, wd)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def step_bounds(w, density):
    """Lower bounds in microseconds on one MI355X (8 TB/s HBM, 2.5 PFLOP/s bf16
    MFMA) for the gate+pack kernel (read x and W_gate once, or its MFMA work),
    the fused kernel (its strictly required bytes: x, TwELL, every touched
    weight row once, y) and the dense FFN (read x and the three weights, write
    and read h, write y; or its MFMA work)."""
    eb = 2 if w.dtype == "bf16" else 4
    n_t = w.d_ff // w.tile_n
    xb = w.T * w.d_model * eb
    wb = w.d_ff * w.d_model * eb
    twell = w.T * n_t * (4 + w.slots * (1 + eb))
    touched = 1.0 - (1.0 - density) ** w.T
    gate = max((xb + wb + twell) / (PEAK_HBM_GBS * 1e3), 2.0 * w.T * w.d_model * w.d_ff / (PEAK_BF16_TFLOPS * 1e6))
    fused = (2 * xb + twell + 2 * touched * wb) / (PEAK_HBM_GBS * 1e3)
    dense = max((2 * xb + 3 * wb + 2 * w.T * w.d_ff * eb) / (PEAK_HBM_GBS * 1e3),
                6.0 * w.T * w.d_model * w.d_ff / (PEAK_BF16_TFLOPS * 1e6))
    return {"gate_pack": round(gate, 2), "fused": round(fused, 2), "twell_step": round(gate + fused, 2),
            "dense": round(dense, 2)}


def density_sweep(T, W, args):
    """TwELL forward (pack + fused, and pack + hybrid) against the library's
    dense FFN over the sweep densities at the 2B-class shape, plus a 16-token
    batch at 0.5%: per point the measured density, overflowing tiles, dense
    rows of the hybrid route, times, speed-ups and the fused kernel's gathered
    rate."""
    import numpy as np
    import torch
    stream = torch.cuda.current_stream()
    points = [(rho, None) for rho in W.SWEEP_RHOS] + [(0.005, 16)]
    out = []
    for rho, t_over in points:
        w = W.workload(5, rho=rho, T=t_over)
        inp = W.make_inputs(w)

        def dev(raw):
            return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()

        x, wg, wu, wd = (dev(inp[k + "_raw"]) for k in ("x", "w_gate_t", "w_up_t", "w_down"))
        desc = T.Desc(w.T, w.d_model, w.d_ff, w.tile_n, w.slots, w.dtype)
        cap = min(w.T, args.max_dense_rows)
        act = T.alloc_act(desc)
        route = T.alloc_route(desc, cap)
        sz = T.sizes(desc, cap)
        wsh = torch.empty(sz["ws_hybrid"], dtype=torch.uint8, device="cuda")
        wsd = torch.empty(sz["ws_dense_fwd"], dtype=torch.uint8, device="cuda")
        y = torch.empty((w.T, w.d_model), dtype=torch.bfloat16, device="cuda")
        stats = torch.zeros(2, dtype=torch.int64, device="cuda")
        T.twell_pack(desc, x, wg, act, stats=stats, stream=stream)
        T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y, route, wsh, stream=stream)
        torch.cuda.synchronize()
        nnz, ovf = int(stats[1]), int(stats[0])
        n_rows = route.n_rows.cpu().tolist()

        def timed(fn, k=args.steps, warm=args.warmup):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(k):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / k

        pack_ms = timed(lambda: T.twell_pack(desc, x, wg, act, stream=stream))
        fused_ms = timed(lambda: T.twell_ffn_fwd(desc, x, act, wu, wd, y, stream=stream))
        hyb_ms = timed(lambda: T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y, route, wsh, stream=stream))
        dense_ms = timed(lambda: T.twell_dense_ffn_fwd(desc, x, wg, wu, wd, y, wsd, stream=stream))
        gathered = nnz * 2 * w.d_model * 2
        bnd = step_bounds(w, nnz / (w.T * w.d_ff))
        extra = {"bounds_us": bnd,
                 "gate_pack_frac_of_bound": round(bnd["gate_pack"] / (pack_ms * 1e3), 4),
                 "fused_frac_of_bound": round(bnd["fused"] / (fused_ms * 1e3), 4),
                 "dense_frac_of_bound": round(bnd["dense"] / (dense_ms * 1e3), 4),
                 "speedup_plain_vs_dense_bound": round(bnd["dense"] / ((pack_ms + fused_ms) * 1e3), 3)}
        if w.T <= 64 and not args.no_hipblaslt:
            tm = hipblaslt_dense(x, wg, wu, wd, args.steps, args.warmup, stream)
            extra["dense_torch_matmul_ms"] = round(tm, 4)
            extra["speedup_plain_vs_torch_matmul"] = round(tm / (pack_ms + fused_ms), 3)
        out.append({"rho_target": rho, "T": w.T, "measured_density": round(nnz / (w.T * w.d_ff), 6),
                    "overflow_tiles": ovf, "dense_rows": n_rows[1], "dense_over_cap": n_rows[2],
                    "pack_ms": round(pack_ms, 4), "fused_ms": round(fused_ms, 4),
                    "hybrid_fwd_ms": round(hyb_ms, 4), "dense_ms": round(dense_ms, 4),
                    "speedup_plain": round(dense_ms / (pack_ms + fused_ms), 3),
                    "speedup_hybrid": round(dense_ms / (pack_ms + hyb_ms), 3),
                    "fused_gathered_gbs": round(gathered / (fused_ms * 1e-3) / 1e9, 1),
                    "gate_pack_tflops": round(2.0 * w.T * w.d_model * w.d_ff / (pack_ms * 1e-3) / 1e12, 1),
                    **extra})
        print(json.dumps({"sweep_point": out[-1]}), file=sys.stderr, flush=True)
        del x, wg, wu, wd, act, route, wsh, wsd, y
        torch.cuda.empty_cache()
    return out


def train_step(T, W, args, steps, warmup):
    """Time one training step of the FFN layer on the training workload:
    twell_pack + twell_ffn_fwd_hybrid + twell_ffn_bwd (HIP events per phase)."""
    import numpy as np
    import torch
    w = W.workload(args.train_config)
    inp = W.make_inputs(w, with_dy=True)

    def dev(raw):
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()

    x, wg, wu, wd, dy = (dev(inp[k + "_raw"]) for k in ("x", "w_gate_t", "w_up_t", "w_down", "dy"))
    desc = T.Desc(w.T, w.d_model, w.d_ff, w.tile_n, w.slots, w.dtype)
    cap = args.max_dense_rows
    act = T.alloc_act(desc)
    route = T.alloc_route(desc, cap)
    sz = T.sizes(desc, cap)
    wsf = torch.empty(sz["ws_hybrid"], dtype=torch.uint8, device="cuda")
    wsb = torch.empty(sz["ws_bwd"], dtype=torch.uint8, device="cuda")
    y = torch.empty((w.T, w.d_model), dtype=torch.bfloat16, device="cuda")
    dx = torch.empty_like(y)
    dws = [torch.empty((w.d_ff, w.d_model), dtype=torch.float32, device="cuda") for _ in range(3)]
    stream = torch.cuda.current_stream()

    def run(ev=None):
        if ev: ev[0].record(stream)
        T.twell_pack(desc, x, wg, act, stream=stream)
        if ev: ev[1].record(stream)
        T.twell_ffn_fwd_hybrid(desc, x, wg, act, wu, wd, y, route, wsf, stream=stream)
        if ev: ev[2].record(stream)
        T.twell_ffn_bwd(desc, x, act, route, wg, wu, wd, dy, w.l1_coef, dx, *dws, wsb, stream=stream)
        if ev: ev[3].record(stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for k in range(steps):
        run(evs[k])
    torch.cuda.synchronize()
    ph = [float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i in range(3)]
    n_rows = route.n_rows.cpu().tolist()
    tot = sum(ph)
    # peak device memory of one step above what is resident before it (inputs, weights, outputs)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    run()
    torch.cuda.synchronize()
    twell_peak = torch.cuda.max_memory_allocated() - base
    # what the forward keeps for the backward: the TwELL planes and the route (x is an input)
    saved = sz["count"] + sz["idx"] + sz["val"] + 4 * (max(w.T, 1) + cap + 3) + max(w.T, 1)
    ws_bytes = sz["ws_hybrid"] + sz["ws_bwd"]
    out = {"workload": w.name, "ms_per_step": round(tot, 4), "tokens_per_s": round(w.T / tot * 1e3, 1),
           "phases_ms": {"pack": round(ph[0], 4), "hybrid_fwd": round(ph[1], 4), "bwd": round(ph[2], 4)},
           "n_ell": n_rows[0], "n_dense": n_rows[1], "dense_over_cap": n_rows[2],
           "saved_activation_bytes": int(saved), "workspace_bytes": int(ws_bytes),
           "step_peak_extra_bytes": int(twell_peak)}
    if not args.no_dense:
        dn = dense_train_torch(x, wg, wu, wd, dy, w.l1_coef, steps, warmup, stream)
        out["dense_torch_matmul"] = dn
        out["speedup_vs_dense_train"] = round(dn["ms_per_step"] / tot, 3)
        out["saved_activation_ratio"] = round(saved / dn["saved_activation_bytes"], 4)
        # device memory a step needs beyond its inputs, weights and outputs, on both sides: TwELL keeps
        # the planes and the route from forward to backward and uses caller workspaces sized for
        # max_dense_rows (plus whatever it allocates during the step); the dense step's peak
        # allocation minus the outputs it allocates itself (y, dx and three bf16 dW)
        outputs = 2 * w.T * w.d_model * 2 + 3 * w.d_ff * w.d_model * 2
        twell_mem = saved + ws_bytes + twell_peak
        dense_mem = dn["step_peak_extra_bytes"] - outputs
        out["step_memory"] = {"twell_bytes": int(twell_mem), "dense_bytes": int(dense_mem),
                              "ratio": round(twell_mem / dense_mem, 4),
                              "twell_parts": {"saved": int(saved), "workspaces": int(ws_bytes),
                                              "allocated_in_step": int(twell_peak)},
                              "dense_outputs_excluded": int(outputs), "max_dense_rows": cap}
    return out


def dense_train_torch(x, wg, wu, wd, dy, l1, steps, warmup, stream):
    """Dense FFN layer training step (forward keeping g and u, backward of the
    same loss sum(y*dy) + l1*sum|h|) through torch.matmul, i.e. hipBLASLt GEMMs
    with their native transposed-operand modes: the comparator of the TwELL
    training step.  bf16 operands, fp32 accumulation, bf16 outputs (dW too)."""
    import numpy as np
    import torch

    def fwd():
        g = torch.matmul(x, wg.t())
        u = torch.matmul(x, wu.t())
        a = torch.relu(g)
        h = a * u
        return g, u, torch.matmul(h, wd)

    def bwd(g, u):
        a = torch.relu(g)
        h = a * u
        dh = torch.matmul(dy, wd.t()) + l1 * torch.sign(h)
        du = dh * a
        dg = dh * u * (g > 0)
        dx = torch.matmul(dg, wg) + torch.matmul(du, wu)
        return dx, torch.matmul(dg.t(), x), torch.matmul(du.t(), x), torch.matmul(h.t(), dy)

    def run():
        g, u, _ = fwd()
        return bwd(g, u)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        g, u, _ = fwd()
        ev[k][1].record(stream)
        bwd(g, u)
        ev[k][2].record(stream)
        del g, u
    torch.cuda.synchronize()
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    r = run()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    del r
    T_, F_ = x.shape[0], wg.shape[0]
    flops = 2.0 * T_ * x.shape[1] * F_ * 3 * 3  # 3 GEMMs forward, 6 backward, each 2*T*d*F
    return {"ms_per_step": round(f_ms + b_ms, 4), "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
            "tflops": round(flops / (f_ms + b_ms) / 1e9, 1),
            "saved_activation_bytes": int(2 * T_ * F_ * x.element_size()), "step_peak_extra_bytes": int(peak)}


def main():
    args = parse()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, args.calib_copy_mib, args.traffic_command)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from activation_sparse_feedforward_amd import twell as T
    from activation_sparse_feedforward_amd import workloads as W

    T.library()  # fail loudly if the HIP library is missing
    if args.sweep:
        print(json.dumps({"sweep": "llama2B_ffn_sweep_T16384_d2048_F8192", "steps": args.steps,
                          "warmup": args.warmup, "points": density_sweep(T, W, args)}), flush=True)
        return
    w = W.workload(args.config, T=args.T, rho=args.rho, d_model=args.d_model, d_ff=args.d_ff)
    overridden = args.T is not None or args.rho is not None or args.d_ff is not None or args.d_model is not None
    if args.mfma_ceiling:
        st = torch.cuda.current_stream()
        print(json.dumps({"mfma_ceiling": mfma_ceiling(st),
                          "mfma_constant_operands": mfma_ceiling(st, random_operands=False),
                          "kernel": "4 waves per CU, v_mfma_f32_32x32x16_bf16 on 16 accumulators, register operands"}),
              flush=True)
        return
    if args.gather_ceiling:
        wp = W.make_inputs(w)
        wu_p, wd_p = (torch.from_numpy(np.ascontiguousarray(wp[k + "_raw"]).view(np.int16)).view(torch.bfloat16).cuda()
                      for k in ("w_up_t", "w_down"))
        print(json.dumps({"gather_ceiling": gather_ceiling(wu_p, wd_p, torch.cuda.current_stream()),
                          "rows": "W_up^T and W_down of " + w.name}), flush=True)
        return
    wname = w.name if not overridden else f"{w.name}@T{w.T}_d{w.d_model}_F{w.d_ff}_rho{w.rho}"
    inp = W.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev(raw):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(raw)).cuda()

    x, wg, wu, wd = (dev(inp[k + "_raw"]) for k in ("x", "w_gate_t", "w_up_t", "w_down"))
    desc = T.Desc(w.T, w.d_model, w.d_ff, w.tile_n, w.slots, w.dtype)
    act = T.alloc_act(desc)
    y = torch.empty((w.T, w.d_model), dtype=dt, device="cuda")
    stats = torch.zeros(2, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        T.twell_pack(desc, x, wg, act, stream=stream)
        T.twell_ffn_fwd(desc, x, act, wu, wd, y, stream=stream)

    # one checked pass (stats) before timing
    T.twell_pack(desc, x, wg, act, stats=stats, stream=stream)
    T.twell_ffn_fwd(desc, x, act, wu, wd, y, stream=stream)
    torch.cuda.synchronize()
    nnz, ovf = int(stats[1]), int(stats[0])
    density = nnz / (w.T * w.d_ff)
    if not torch.isfinite(y.float()).all():
        raise RuntimeError("non-finite output")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calib_copy_mib > 0:
        src_c = torch.ones(args.calib_copy_mib * (1 << 18), dtype=torch.float32, device="cuda")
        dst_c = torch.empty_like(src_c)
        torch.cuda.synchronize()
        torch.neg(src_c, out=dst_c)
        torch.cuda.synchronize()
        del src_c, dst_c

    K = args.steps
    # per-kernel HIP events on the launch stream, inside the timed region: on
    # every step at large batches; below 2048 tokens on every 8th step, since
    # three event records (~3 us of host time each) would otherwise set the
    # pace of a ~20 us step
    ev_every = 1 if w.T >= 2048 else 8
    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for k in range(0, K, ev_every)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        e = ev.get(k)
        if e:
            e[0].record(stream)
        T.twell_pack(desc, x, wg, act, stream=stream)
        if e:
            e[1].record(stream)
        T.twell_ffn_fwd(desc, x, act, wu, wd, y, stream=stream)
        if e:
            e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pack_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev.values()]))
    fused_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev.values()]))
    ms_per_step = wall / K * 1e3
    value = w.T * K / wall

    # dense comparator, timed the same way
    dense = None
    if not args.no_dense:
        ws = torch.empty(T.sizes(desc)["ws_dense_fwd"], dtype=torch.uint8, device="cuda")
        yd = torch.empty_like(y)
        for _ in range(args.warmup):
            T.twell_dense_ffn_fwd(desc, x, wg, wu, wd, yd, ws, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            T.twell_dense_ffn_fwd(desc, x, wg, wu, wd, yd, ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / K
        flops = 6.0 * w.T * w.d_model * w.d_ff
        dense = {"ms_per_step": round(dense_ms, 4), "tokens_per_s": round(w.T / dense_ms * 1e3, 1),
                 "tflops": round(flops / dense_ms / 1e9, 1)}
        if args.cold_iters > 0:
            dense["cold_ms"] = cold_timing(
                [("dense", lambda: T.twell_dense_ffn_fwd(desc, x, wg, wu, wd, yd, ws, stream=stream))],
                args.cold_iters, stream)["dense"]
        del ws, yd
        if not args.no_hipblaslt and w.dtype == "bf16":
            hb = hipblaslt_dense(x, wg, wu, wd, K, args.warmup, stream)
            dense["torch_matmul_sanity"] = {"ms_per_step": round(hb, 4), "tflops": round(flops / hb / 1e9, 1)}
            torch.cuda.empty_cache()

    # classic ELL construction (dense gate write-back + conversion kernel), same fused kernel after it
    classic = None
    if not args.no_classic:
        wsc = torch.empty(T.sizes(desc)["ws_pack_classic"], dtype=torch.uint8, device="cuda")
        act_c = T.alloc_act(desc)
        for _ in range(args.warmup):
            T.twell_pack_classic(desc, x, wg, act_c, wsc, stream=stream)
        torch.cuda.synchronize()
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        for k in range(K):
            evc[k][0].record(stream)
            T.twell_pack_classic(desc, x, wg, act_c, wsc, stream=stream)
            evc[k][1].record(stream)
            T.twell_ffn_fwd(desc, x, act_c, wu, wd, y, stream=stream)
            evc[k][2].record(stream)
        torch.cuda.synchronize()
        cpk = float(np.mean([e[0].elapsed_time(e[1]) for e in evc]))
        cfu = float(np.mean([e[1].elapsed_time(e[2]) for e in evc]))
        classic = {"pack_classic_ms": round(cpk, 4), "fused_ms": round(cfu, 4), "ms_per_step": round(cpk + cfu, 4),
                   "dense_relu_bytes_written_and_read": 2 * w.T * w.d_ff * (2 if w.dtype == "bf16" else 4),
                   "epilogue_pack_speedup": round(cpk / pack_ms, 3),
                   "step_speedup_of_epilogue_packing": round((cpk + cfu) / (pack_ms + fused_ms), 3)}
        del wsc, act_c
        torch.cuda.empty_cache()

    cold = None
    if args.cold_iters > 0:
        cold = cold_timing([("gate_pack", lambda: T.twell_pack(desc, x, wg, act, stream=stream)),
                            ("fused_updown", lambda: T.twell_ffn_fwd(desc, x, act, wu, wd, y, stream=stream))],
                           args.cold_iters, stream)

    # roofline of the dominant kernel
    peak_mm = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    gate_flop = 2.0 * w.T * w.d_model * w.d_ff
    eb = 2 if w.dtype == "bf16" else 4
    # strictly required HBM bytes of the fused kernel: x, TwELL, every weight row touched once, y
    twell_bytes = w.T * desc.n_t * (4 + w.slots * (1 + eb))
    touched = 1.0 - (1.0 - density) ** w.T
    fused_bytes = 2 * w.T * w.d_model * eb + twell_bytes + 2 * touched * w.d_ff * w.d_model * eb
    gathered_bytes = nnz * 2 * w.d_model * eb
    src = {k: kernel_source_hash(f) for k, f in KERNEL_SOURCES.items()}
    if pack_ms >= fused_ms:
        ach = gate_flop / (pack_ms * 1e-3) / 1e12
        roof = {"kernel": "gate_pack", "bound": "mfma", "achieved": round(ach, 1), "peak": peak_mm,
                "unit": "TFLOP/s", "frac": round(ach / peak_mm, 4),
                "traffic": None if overridden or args.config != 3 else measured_traffic("gate_pack", src["gate_pack"], 1)}
    else:
        ach = fused_bytes / (fused_ms * 1e-3) / 1e9
        roof = {"kernel": "fused_updown", "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": None if overridden or args.config != 3 else measured_traffic("fused_updown", src["fused_updown"], 1)}

    # the gate kernel against what the matrix cores sustain under its MFMA load alone (bf16 only: the
    # probe issues the bf16 instruction)
    gate_vs_mfma = None
    if w.dtype == "bf16":
        mc = mfma_ceiling(stream)
        gate_vs_mfma = {"mfma_ceiling": mc, "achieved_tflops": round(gate_flop / (pack_ms * 1e-3) / 1e12, 1),
                        "frac_of_ceiling": round(gate_flop / (pack_ms * 1e-3) / 1e12 / mc["tflops"], 4)}

    # gather phase against the HBM peak: strictly required bytes, and the bytes the kernel moved past
    # L2 (rocprofv3 FETCH_SIZE + WRITE_SIZE of the current source, committed under profiles/)
    fused_req_gbs = fused_bytes / (fused_ms * 1e-3) / 1e9
    fused_info = {"required_hbm_gbs": round(fused_req_gbs, 1), "required_frac_of_hbm_peak": round(fused_req_gbs / PEAK_HBM_GBS, 4),
                  "gathered_gbs": round(gathered_bytes / (fused_ms * 1e-3) / 1e9, 1),
                  "gathered_bytes": int(gathered_bytes), "required_bytes": int(fused_bytes)}
    past_l2 = None if overridden or args.config != 3 else measured_traffic("fused_updown", src["fused_updown"], 1)
    if past_l2:
        fused_past_gbs = past_l2 / (fused_ms * 1e-3) / 1e9
        fused_info.update({"past_l2_bytes": int(past_l2), "past_l2_gbs": round(fused_past_gbs, 1),
                           "past_l2_frac_of_hbm_peak": round(fused_past_gbs / PEAK_HBM_GBS, 4)})
    # the same rows gathered by the probe: cache-served and past-L2 ceilings of this access pattern
    if w.dtype == "bf16":
        ceil = gather_ceiling(wu, wd, stream)
        fused_info["gather_ceiling"] = ceil
        fused_info["gathered_frac_of_ceiling"] = round(fused_info["gathered_gbs"] / ceil["xcd_shared_ceiling_gbs"], 4)
        if past_l2:
            fused_info["past_l2_frac_of_ceiling"] = round(fused_info["past_l2_gbs"] / ceil["random_ceiling_gbs"], 4)

    out = {
        "metric": "TwELL FFN tokens/sec at 99.5% act. sparsity; speedup vs dense; % roofline",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded PCG64; gate density set by a column-0 offset)",
        "config": {"workload": wname, "T": w.T, "d_model": w.d_model, "d_ff": w.d_ff, "tile_n": w.tile_n,
                   "slots": w.slots, "target_density": w.rho if w.density == "uniform" else w.density},
        "roofline": roof,
        "measured_density": round(density, 6),
        "overflow_tiles": ovf,
        "phases_ms": {"gate_pack": round(pack_ms, 4), "fused_updown": round(fused_ms, 4)},
        "phase_events_every": ev_every,
        "gate_pack_tflops": round(gate_flop / (pack_ms * 1e-3) / 1e12, 1),
        "gate_pack_vs_mfma_ceiling": gate_vs_mfma,
        "fused_updown": fused_info,
        "dense_ffn": dense,
        "classic_ell": classic,
        "speedup_vs_dense": round(dense["ms_per_step"] / ms_per_step, 3) if dense else None,
        "cold_ms": cold,
        "speedup_vs_dense_cold": (round(dense["cold_ms"]["median"] / cold["total"]["median"], 3)
                                  if dense and cold and "cold_ms" in dense else None),
    }
    if not args.no_train:
        del act, y
        torch.cuda.empty_cache()
        out["training"] = train_step(T, W, args, max(3, K // 2), 2)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, w.tile_n, w.slots, w.dtype)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
