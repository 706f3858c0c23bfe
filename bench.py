#!/usr/bin/env python3
"""Benchmark of the KDA core on one MI355X.

Metric: KDA prefill tokens/s at H = 96, d_k = d_v = 128, T = 32K (bf16 q/k/v,
fp32 g/beta/state), plus decode-step state HBM GB/s at 256 sequences x 96
heads with fp32 128 x 128 states.  Synthetic inputs (see synth.py) stand in
for K3 KDA-layer activations.

One "step" is one prefill of the dense workload (B = 1, T = 32768, H = 96):
every prefill row of the method (decay cumsum, scaled tiles, Gram tiles,
triangular solve, WY products, state pass, stores) runs once over the whole
batch.  The packed-varlen prefill (16 sequences, 32768 tokens), the
long-context prefill (one sequence of 1,048,576 tokens, 16 heads) and the
decode step (256 x 96 states, read once and written once per step, averaged
over 1000 steps) are timed in the same run and reported under
"prefill_varlen", "prefill_long_1m" and "decode"; "device_copy" gives the
bandwidth of a plain device copy as context for the HBM fractions.

Timing: inputs are resident in HBM before the timed region; untimed
warm-up steps (at least W, continued until 150 ms of back-to-back launches
have run, so that the device clocks have settled after the change of
workload; the counts are reported), then K timed steps bracketed by
torch.cuda.synchronize();
per-launch durations come from HIP events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes
to the C ABI).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published

# Algorithmic bytes per token-head of the bf16 prefill: q, k, v (3 x 256),
# g (512), beta (4), o (256).  The per-head state I/O (64 KiB) is excluded.
PREFILL_BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 256
# The fused entry reads bf16 decay logits z (256) instead of fp32 g.
FUSED_BYTES_PER_TOKEN_HEAD = 3 * 256 + 256 + 4 + 256
# Gated prefill: the gate logits (256) are read too; y (256) replaces o.
GATED_BYTES_PER_TOKEN_HEAD = PREFILL_BYTES_PER_TOKEN_HEAD + 256
# Backward: each input and output once -- q, k, v, g, beta and d_o read (1540),
# dq, dk, dv, dg and dbeta written (3 x 256 + 512 + 4).
BWD_IO_BYTES_PER_TOKEN_HEAD = 3 * 256 + 512 + 4 + 256 + 3 * 256 + 512 + 4
# Chunked flop count at the reference chunk C = 64, d = 128, causal tiles:
# A, P, W, U~ and P U at C^2 d each, plus W S, Q~ S and Kbar^T U at 2 C d^2
# each, per chunk of C tokens -> 5 C d + 6 d^2 per token-head.
PREFILL_FLOP_PER_TOKEN_HEAD = 5 * 64 * 128 + 6 * 128 * 128
# Decode: state read + write (2 x 64 KiB) + q, k, v (bf16) + g (fp32) + beta + o (bf16).
DECODE_BYTES_PER_UNIT = 2 * 128 * 128 * 4 + 3 * 128 * 2 + 128 * 4 + 4 + 128 * 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Sources each measured kernel is compiled from; a counter record is used only
# while these are unchanged: the kernel's headers and translation units, the
# C-ABI layer (it picks the kernel variant, slab width and segment plan),
# "flags:<file>" = the extra compiler flags build_lib.py gives that
# translation unit, and "build" = the flags every file is compiled with.
_PREFILL = ("kda_prefill_ws.h", "kda_device.h", "kda_internal.h", "kda_bounds.h", "kda_abi.cpp", "build")
KERNEL_SOURCES = {
    "kda_prefill_k3_dense_32k": _PREFILL + ("kda_prefill_ws_ilp.hip", "flags:kda_prefill_ws_ilp.hip"),
    "kda_prefill_k3_varlen_32k": _PREFILL + ("kda_prefill_bf16.hip", "flags:kda_prefill_bf16.hip"),
    "kda_prefill_gated_k3_varlen_32k": _PREFILL + ("kda_prefill_bf16.hip", "flags:kda_prefill_bf16.hip"),
    "kda_prefill_long_1m_h16": _PREFILL + ("kda_prefill_bf16.hip", "kda_segment.hip", "flags:kda_prefill_bf16.hip",
                                           "flags:kda_segment.hip"),
    "kda_decode_256x96": ("kda_decode.hip", "kda_device.h", "kda_internal.h", "kda_bounds.h", "kda_abi.cpp",
                          "build", "flags:kda_decode.hip"),
    "kda_prefill_fused_k3_dense_32k": _PREFILL + ("kda_prefill_ws_ilp.hip", "flags:kda_prefill_ws_ilp.hip"),
    "kda_prefill_fused_k3_varlen_32k": _PREFILL + ("kda_prefill_bf16.hip", "flags:kda_prefill_bf16.hip"),
    "kda_output_gate_32k_x96": ("kda_output_gate.hip", "kda_device.h", "kda_internal.h", "kda_bounds.h",
                                "kda_abi.cpp", "build"),
    "kda_backward_k3_dense_32k": _PREFILL + ("kda_backward.hip", "kda_backward.h", "kda_prefill_ws_ilp.hip",
                                             "kda_prefill_bf16.hip", "flags:kda_backward.hip",
                                             "flags:kda_prefill_ws_ilp.hip"),
}


def _flags_key(flags, root):
    """Compiler flags with absolute paths made relative to the repository, so
    that a digest does not depend on where the repository is checked out."""
    return [os.path.relpath(x, root) if os.path.isabs(x) else x for x in flags]


def kernel_source_digest(kernel):
    from linear_attention_recurrence_delta_amd import build_lib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_recurrence_delta_amd", "csrc")
    root = build_lib.ROOT
    for f in KERNEL_SOURCES[kernel]:
        if f == "build":
            h.update(repr((_flags_key(build_lib.COMMON, root), _flags_key(build_lib.DEVICE, root))).encode())
        elif f.startswith("flags:"):
            h.update(repr(_flags_key(build_lib.PER_FILE.get(f[len("flags:"):], []), root)).encode())
        else:
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


# The kernels of each counter record, as rocprofv3 names them (demangled),
# one entry per launch of the call: the record is the sum over the call's
# launches of each kernel's mean per dispatch.
RECORD_KERNELS = {
    "kda_prefill_k3_dense_32k": ["kda_prefill_ws_kernel<2, 2, 8, false, false, false, false>"],
    "kda_prefill_k3_varlen_32k": ["kda_prefill_ws_kernel<4, 2, 8, false, false, false, false>"],
    "kda_prefill_gated_k3_varlen_32k": ["kda_prefill_ws_kernel<4, 2, 8, false, false, false, true>"],
    "kda_prefill_fused_k3_dense_32k": ["kda_prefill_ws_kernel<2, 2, 8, true, false, false, false>"],
    "kda_prefill_fused_k3_varlen_32k": ["kda_prefill_ws_kernel<4, 2, 8, true, false, false, false>"],
    "kda_prefill_long_1m_h16": ["kda_prefill_ws_kernel<8, 2, 4, false, false, true, false>",
                                "kda_segment_combine_kernel",
                                "kda_prefill_ws_kernel<4, 2, 8, false, false, true, false>"],
    "kda_decode_256x96": ["kda_decode_kernel<kda::bf16_t, 128>"],
    "kda_output_gate_32k_x96": ["kda_output_gate_kernel<kda::bf16_t, 128>"],
    "kda_backward_k3_dense_32k": ["kda_prefill_ws_kernel<2, 2, 8, false, true, false, false>",
                                  "kda_backward_kernel", "kda_backward_sum_kernel"],
}
MFMA_RECORDS = ("kda_prefill_k3_dense_32k", "kda_prefill_k3_varlen_32k", "kda_prefill_gated_k3_varlen_32k",
                "kda_prefill_fused_k3_dense_32k", "kda_prefill_fused_k3_varlen_32k")


def _counter_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _kernel_means(rows, counter):
    """Mean counter value per dispatch for each kernel name of RECORD_KERNELS."""
    out = {}
    for names in RECORD_KERNELS.values():
        for name in names:
            v = [float(r["Counter_Value"]) for r in rows
                 if r["Counter_Name"] == counter and name in r["Kernel_Name"]]
            if v:
                out[name] = (sum(v) / len(v), len(v))
    return out


def _copy_factor(rows, counter, copy_bytes=1 << 30):
    """Bytes per counter unit, from the device copies that bench.py
    --calibrate-copy issues before any library launch (1 GiB each)."""
    first_kda = min((int(r["Dispatch_Id"]) for r in rows if "kda" in r["Kernel_Name"]), default=None)
    v = sorted((float(r["Counter_Value"]) for r in rows
                if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]
                and (first_kda is None or int(r["Dispatch_Id"]) < first_kda)), reverse=True)[:3]
    if not v:
        raise SystemExit("no calibration copies in the %s pass (run it with --calibrate-copy)" % counter)
    return copy_bytes / (sum(v) / len(v) * 1024.0), v


def record_counters(fetch_csv, write_csv, sq_csv=None, out_path=None):
    """Rebuild profiles/pmc_traffic.json from rocprofv3 --pmc passes (csv
    output) of bench.py: FETCH_SIZE and WRITE_SIZE (with --calibrate-copy)
    and optionally SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE.  Records are keyed by the current source digests."""
    fr, ww = _counter_rows(fetch_csv), _counter_rows(write_csv)
    f_fac, f_cal = _copy_factor(fr, "FETCH_SIZE")
    w_fac, w_cal = _copy_factor(ww, "WRITE_SIZE")
    fm, wm = _kernel_means(fr, "FETCH_SIZE"), _kernel_means(ww, "WRITE_SIZE")
    sq = None
    if sq_csv:
        sr = _counter_rows(sq_csv)
        sq = {c: _kernel_means(sr, c) for c in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
                                               "GRBM_GUI_ACTIVE")}
    rec = {"_note": (
        "HBM bytes per launch = 1024 (FETCH_SIZE * %.4f + WRITE_SIZE * %.4f) (counters in KiB), the factors from the 1 GiB "
        "device copies of the same passes (FETCH_SIZE %s KiB, WRITE_SIZE %s KiB per copy). A record lists "
        "the call's kernels; fetch_kib and write_kib are the sums over them of the mean per dispatch. "
        "source_digest = first 16 hex digits of the sha256 of the listed csrc/ files and, for flags:<file>, "
        "of the extra compiler flags build_lib.py gives that file, in order; a record is used only while it "
        "matches. mfma_counters: SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE "
        "(summed over the 8 XCDs) per launch. Written by bench.py --record-counters."
        % (f_fac, w_fac, ", ".join("%.1f" % x for x in f_cal),
           ", ".join("%.1f" % x for x in w_cal)))}
    for key, names in RECORD_KERNELS.items():
        if not all(n in fm and n in wm for n in names):
            log("no dispatches for %s: not recorded" % key)
            continue
        fk = sum(fm[n][0] for n in names)
        wk = sum(wm[n][0] for n in names)
        ent = {"source_digest": kernel_source_digest(key), "sources": list(KERNEL_SOURCES[key]),
               "kernels": {n: {"fetch_kib": round(fm[n][0], 1), "write_kib": round(wm[n][0], 1),
                               "dispatches": fm[n][1]} for n in names},
               "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
               "hbm_bytes_per_launch": int(round(1024.0 * (fk * f_fac + wk * w_fac)))}
        if sq and key in MFMA_RECORDS and all(names[0] in sq[c] for c in sq):
            ent["mfma_counters"] = {"mops_bf16": sq["SQ_INSTS_VALU_MFMA_MOPS_BF16"][names[0]][0],
                                    "busy_cycles": sq["SQ_VALU_MFMA_BUSY_CYCLES"][names[0]][0],
                                    "grbm_gui_active": sq["GRBM_GUI_ACTIVE"][names[0]][0],
                                    "xcds": 8, "simds": 1024}
        rec[key] = ent
    path = out_path or os.path.join(ROOT, "profiles", "pmc_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def measured_traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current sources of that kernel; else None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("source_digest") != kernel_source_digest(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


def measured_mfma(kernel):
    """MFMA counters of the committed rocprofv3 summary (same source-digest rule
    as measured_traffic): executed bf16 MFMA flops per launch (512 per
    SQ_INSTS_VALU_MFMA_MOPS_BF16) and SQ_VALU_MFMA_BUSY_CYCLES as a fraction of
    the SIMD-cycles of the launch (GRBM_GUI_ACTIVE is summed over the XCDs)."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path)).get(kernel)
    except ValueError:
        return None
    if not ent or ent.get("source_digest") != kernel_source_digest(kernel) or "mfma_counters" not in ent:
        return None
    c = ent["mfma_counters"]
    simd_cycles = c["grbm_gui_active"] / c["xcds"] * c["simds"]
    return {"executed_bf16_flop_per_launch": c["mops_bf16"] * 512.0,
            "busy_frac_of_simd_cycles": c["busy_cycles"] / simd_cycles}


def backward_entry(bw_ms, token_heads, T):
    """The backward call's timing (its three launches: the forward again with
    a bf16 state every 16 tokens, the reverse chunk kernel, the sum of the two
    value halves) and its HBM roofline over the whole call: the gradients'
    inputs and outputs are the algorithmic bytes (the states are the call's
    own intermediate data); traffic is what the three kernels move."""
    tot = sum(bw_ms) / len(bw_ms)
    io_bytes = BWD_IO_BYTES_PER_TOKEN_HEAD * token_heads
    return {
        "workload": "gradients of k3_dense_32k (dq, dk, dv, dg, dbeta) for a random bf16 d_o: the forward again "
                    "keeping the state every 16 tokens, then the reverse chunk kernel and the sum of its halves",
        "ms": tot, "tokens_per_s": T / (tot * 1e-3),
        "io_bytes_per_token_head": BWD_IO_BYTES_PER_TOKEN_HEAD,
        "roofline": {"bound": "hbm", "achieved": io_bytes / (tot * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": io_bytes / (tot * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic("kda_backward_k3_dense_32k"),
                     "kernel": "kda_prefill_backward (forward with 16-token states + reverse + sum)",
                     "bytes_per_launch": io_bytes},
    }


# Each timed workload gets its own warm-up right before it: `warmup` launches,
# continued until WARM_MS of back-to-back launches have run.  After a change
# of workload the device's clocks take about 45 ms of sustained work to settle
# (dense prefill, traced: first launches 2.0 ms, 1.58-1.60 ms from about the
# 25th on), so W launches alone would time part of that ramp.
WARM_MS = 150.0
WARMUP_LAUNCHES = {}


def time_launches(fn, reps, stream, warmup=0, name=None):
    """Warm up (see WARM_MS), then run fn reps times; return per-launch ms
    from events on `stream`.  The warm-up launch count goes to
    WARMUP_LAUNCHES[name]."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    n = 0
    t0 = time.perf_counter()
    while True:  # in groups of 4 launches, so the queue stays short and the device busy
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if n >= warmup and (time.perf_counter() - t0) * 1e3 >= WARM_MS:
                break
    if name:
        WARMUP_LAUNCHES[name] = n
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def host_description():
    """CPU model, logical CPUs of the host and CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(w, target_s):
    """The fp64 oracle, as it stands, on a bounded sample of the dense workload.

    The sample grows (tokens, then heads, then repeats of the same slice)
    until about target_s seconds of CPU work have run."""
    import oracle
    import torch

    oracle.build(force=False)
    threads = oracle.max_threads()
    H, T = w["H"], w["T"]
    nh, T_s = min(H, max(1, threads)), 1024
    while True:
        sl = lambda x: x[:T_s, :nh].detach().to("cpu").to(torch.float64).numpy()
        args = [sl(w[n]) for n in ("q", "k", "v", "g")]
        beta = w["beta"][:T_s, :nh].detach().cpu().double().numpy()
        t0 = time.perf_counter()
        oracle.prefill(*args, beta)
        dt = time.perf_counter() - t0
        if dt >= 0.25 * target_s or (T_s >= T and nh >= H):
            break
        grow = max(2.0, 0.5 * target_s / max(dt, 1e-3))
        if T_s < T:
            T_s = int(min(T, T_s * grow))
        else:
            nh = int(min(H, nh * grow))
    reps = max(1, int(round(target_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.prefill(*args, beta)
    total = time.perf_counter() - t0
    token_heads_per_s = reps * nh * T_s / total
    return {
        "value": token_heads_per_s / H,
        "unit": "tokens/s",
        "cores": min(nh, threads),
        "kind": "oracle",
        "host": host_description(),
        "sample": "%d run(s) of the first %d tokens x %d of the %d heads of the dense workload, %.1f s "
                  "of fp64 token-by-token recurrence on %d OpenMP threads; tokens/s = token-heads/s / %d heads"
                  % (reps, T_s, nh, H, total, min(nh, threads), H),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000, help="decode steps timed after the prefill steps")
    ap.add_argument("--long-steps", type=int, default=3,
                    help="timed runs of the 1M-token, 16-head prefill (0 skips it)")
    ap.add_argument("--chunk", type=int, default=0, help="prefill chunk size (0 = library default)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "long"], default="all")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward timing (counter runs of the prefill kernels alone; the backward's forward "
                         "launch is a variant of the same kernel)")
    ap.add_argument("--no-checkpoints", action="store_true",
                    help="skip the checkpointed prefill timing (counter runs per kernel launch)")
    ap.add_argument("--record-counters", nargs="+", metavar="CSV",
                    help="rebuild profiles/pmc_traffic.json from rocprofv3 --pmc csv files "
                         "(FETCH_SIZE, WRITE_SIZE[, SQ counters]) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.record_counters:
        if len(args.record_counters) not in (2, 3):
            raise SystemExit("--record-counters FETCH_CSV WRITE_CSV [SQ_CSV]")
        rec = record_counters(*args.record_counters)
        for k, v in rec.items():
            if not k.startswith("_"):
                log("%-34s %14d B per launch" % (k, v["hbm_bytes_per_launch"]))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each (sequence, head) "
              "recurrence is independent, so heads and sequences split across GPUs with no "
              "communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_recurrence_delta_amd as kda
    from linear_attention_recurrence_delta_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    result = {}
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x 1 GiB device-to-device")
        del src, dst

    # ---------------------------------------------------------------- prefill
    C = args.chunk or 0
    wd = None
    if args.only in ("all", "prefill"):
        log("generating k3_dense_32k / k3_varlen_32k inputs")
        wd = synth.workload_inputs("k3_dense_32k", dev)
        wv = synth.workload_inputs("k3_varlen_32k", dev)
        o_d = torch.empty_like(wd["v"])
        s_d = torch.empty((wd["N"], wd["H"], wd["d"], wd["d"]), dtype=torch.float32, device=dev)
        o_v = torch.empty_like(wv["v"])
        s_v = torch.empty((wv["N"], wv["H"], wv["d"], wv["d"]), dtype=torch.float32, device=dev)

    def run_dense():
        kda.kda_prefill(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"], None, None, chunk_size=C,
                        out=o_d, final_state=s_d)

    def run_varlen():
        kda.kda_prefill(wv["q"], wv["k"], wv["v"], wv["g"], wv["beta"], None, wv["cu"], chunk_size=C,
                        out=o_v, final_state=s_v)

    if args.only in ("all", "prefill"):
        token_heads = wd["T"] * wd["H"]
        t0 = time.perf_counter()
        dense_ms = time_launches(run_dense, args.steps, stream, args.warmup, "prefill_dense")
        wall_s = time.perf_counter() - t0
        varlen_ms = time_launches(run_varlen, args.steps, stream, args.warmup, "prefill_varlen")
        # the varlen pack through the gated entry: y = sigmoid(gate) * RMSNorm(o) * weight
        # fused into the o store (whole-head workgroups), and the same as two passes
        gen_g = torch.Generator(device=dev)
        gen_g.manual_seed(9)
        gv_gate = torch.randn(wv["v"].shape, generator=gen_g, device=dev).to(torch.bfloat16)
        gv_w = torch.ones(wv["d"], device=dev)
        y_v = torch.empty_like(wv["v"])

        def run_gated():
            kda.kda_prefill_output_gated(wv["q"], wv["k"], wv["v"], wv["g"], wv["beta"], gv_gate, gv_w, None, wv["cu"],
                                         chunk_size=C, out=y_v, final_state=s_v)

        def run_two_pass():
            run_varlen()
            kda.kda_output_gate(o_v, gv_gate, gv_w, eps=1e-6, out=y_v)

        gated_ms = time_launches(run_gated, args.steps, stream, args.warmup, "prefill_gated")
        two_pass_ms = time_launches(run_two_pass, args.steps, stream, args.warmup, "prefill_gated_two_pass")
        del gv_gate, y_v
        # the dense workload again with a state checkpoint every 1024 tokens
        ck_interval = 1024
        ck_buf = torch.empty((wd["T"] // ck_interval, wd["H"], wd["d"], wd["d"]), dtype=torch.float32, device=dev)

        def run_dense_ck():
            kda.kda_prefill_checkpointed(wd["q"], wd["k"], wd["v"], wd["g"], wd["beta"], None, None,
                                         checkpoint_interval=ck_interval, chunk_size=C, out=o_d,
                                         final_state=s_d, checkpoints=ck_buf)

        ck_ms = None
        if not args.no_checkpoints:
            ck_ms = time_launches(run_dense_ck, args.steps, stream, args.warmup, "prefill_checkpoints")
        # the dense workload through the fused entry (gate and q/k norm in the kernel)
        fu_ms = fu_v_ms = None
        if kda.kda_prefill_fused_supported(torch.bfloat16, wd["d"], wd["d"], C):
            fq, fk, fv, fz, fa, fb, _ = synth.fused_inputs(wd["T"], wd["H"], wd["d"], torch.bfloat16, 7, dev,
                                                           a_log_std=0.0)

            def run_fused():
                kda.kda_prefill_fused(fq, fk, fv, fz, fa, fb, None, None, chunk_size=C, out=o_d, final_state=s_d)

            fu_ms = time_launches(run_fused, args.steps, stream, args.warmup, "prefill_fused")

            # the varlen pack through the same entry (whole-head workgroups)
            def run_fused_varlen():
                kda.kda_prefill_fused(fq, fk, fv, fz, fa, fb, None, wv["cu"], chunk_size=C, out=o_v,
                                      final_state=s_v)

            fu_v_ms = time_launches(run_fused_varlen, args.steps, stream, args.warmup, "prefill_fused_varlen")
            del fq, fk, fv, fz, fa, fb
        # the output gate on the dense output (Sigmoid(gate) * RMSNorm(o) * weight)
        og_gate = torch.randn(o_d.shape, device=dev).to(o_d.dtype)
        og_w = torch.ones(wd["d"], device=dev)
        og_y = torch.empty_like(o_d)

        def run_gate():
            kda.kda_output_gate(o_d, og_gate, og_w, eps=1e-6, out=og_y)

        og_ms = time_launches(run_gate, args.steps, stream, args.warmup, "output_gate")
        del og_gate, og_y
        # the backward pass on the dense workload (forward again for its
        # 16-token states, then the reverse chunk kernel), preallocated buffers
        bw_ms = None
        if not args.no_backward and kda.kda_prefill_backward_supported(torch.bfloat16, wd["d"], wd["d"]):
            from linear_attention_recurrence_delta_amd._lib import lib as _kdalib
            gen = torch.Generator(device=dev)
            gen.manual_seed(8)
            b_do = torch.randn(wd["v"].shape, generator=gen, device=dev).to(torch.bfloat16)
            b_dq, b_dk, b_dv = (torch.empty_like(wd[x]) for x in ("q", "k", "v"))
            b_dg = torch.empty_like(wd["g"])
            b_db = torch.empty_like(wd["beta"])
            ws_b = int(_kdalib().kda_prefill_backward_workspace_bytes(wd["N"], wd["T"], wd["H"], wd["d"], wd["d"],
                                                                      kda.KDA_DTYPE_BF16))
            b_ws = torch.empty(ws_b, dtype=torch.uint8, device=dev)
            p_ = lambda t: t.data_ptr()

            def run_bwd():
                st = _kdalib().kda_prefill_backward(
                    wd["N"], wd["T"], wd["H"], wd["d"], wd["d"], kda.KDA_DTYPE_BF16, 1.0,
                    p_(wd["q"]), p_(wd["k"]), p_(wd["v"]), p_(wd["g"]), p_(wd["beta"]), None, None, p_(b_do), None,
                    p_(b_dq), p_(b_dk), p_(b_dv), p_(b_dg), p_(b_db), None, p_(b_ws), ws_b, stream.cuda_stream)
                if st != 0:
                    raise RuntimeError("kda_prefill_backward failed: %d" % st)

            bw_ms = time_launches(run_bwd, args.steps, stream, args.warmup, "prefill_backward")
            del b_do, b_dq, b_dk, b_dv, b_dg, b_db, b_ws
        d_avg = sum(dense_ms) / len(dense_ms)
        v_avg = sum(varlen_ms) / len(varlen_ms)
        log("dense prefill avg %.3f ms (min %.3f), varlen avg %.3f ms, wall %.3f s" %
            (d_avg, min(dense_ms), v_avg, wall_s))
        bytes_launch = PREFILL_BYTES_PER_TOKEN_HEAD * token_heads
        flop_launch = PREFILL_FLOP_PER_TOKEN_HEAD * token_heads
        achieved = bytes_launch / (d_avg * 1e-3) / 1e9
        result.update({
            "value": wd["T"] / (d_avg * 1e-3),
            "ms_per_step": d_avg,
            "roofline": {
                "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic("kda_prefill_k3_dense_32k"),
                "kernel": "kda_prefill_ws_kernel (bf16, d=128, chunk 16)", "bytes_per_launch": bytes_launch,
            },
            "mfma": {
                "flop_per_launch": flop_launch,
                "achieved_tflops": flop_launch / (d_avg * 1e-3) / 1e12,
                "peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                "frac": flop_launch / (d_avg * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
                "counters": measured_mfma("kda_prefill_k3_dense_32k"),
            },
            "prefill_checkpoints": None if ck_ms is None else {
                "workload": "k3_dense_32k with a state checkpoint every %d tokens (%d per head, %.0f MB)"
                            % (ck_interval, wd["T"] // ck_interval, ck_buf.numel() * 4 / 1e6),
                "ms": sum(ck_ms) / len(ck_ms),
                "overhead_vs_plain": (sum(ck_ms) / len(ck_ms)) / d_avg - 1.0,
            },
            "prefill_fused": None if fu_ms is None else {
                "workload": "k3_dense_32k through kda_prefill_fused: raw q/k normalised and g = -5 sigmoid(e^A z) "
                            "formed in the kernel from bf16 z (A = 0)",
                "ms": sum(fu_ms) / len(fu_ms),
                "tokens_per_s": wd["T"] / (sum(fu_ms) / len(fu_ms) * 1e-3),
                "hbm_gbs": FUSED_BYTES_PER_TOKEN_HEAD * token_heads / (sum(fu_ms) / len(fu_ms) * 1e-3) / 1e9,
                "bytes_per_token_head": FUSED_BYTES_PER_TOKEN_HEAD,
                "traffic": measured_traffic("kda_prefill_fused_k3_dense_32k"),
                "vs_plain": (sum(fu_ms) / len(fu_ms)) / d_avg,
                "varlen": None if fu_v_ms is None else {
                    "workload": "k3_varlen_32k through kda_prefill_fused (same raw inputs, cu_seqlens of the pack)",
                    "ms": sum(fu_v_ms) / len(fu_v_ms),
                    "vs_plain_varlen": (sum(fu_v_ms) / len(fu_v_ms)) / v_avg,
                    "hbm_gbs": FUSED_BYTES_PER_TOKEN_HEAD * wv["T"] * wv["H"] / (sum(fu_v_ms) / len(fu_v_ms) * 1e-3) / 1e9,
                    "traffic": measured_traffic("kda_prefill_fused_k3_varlen_32k"),
                },
            },
            "output_gate": {
                "workload": "Sigmoid(gate) * RMSNorm(o) * weight over 32768 x 96 rows of 128 bf16",
                "ms": sum(og_ms) / len(og_ms),
                "roofline": {"bound": "hbm", "achieved": 3 * o_d.numel() * 2 / (sum(og_ms) / len(og_ms) * 1e-3) / 1e9,
                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": 3 * o_d.numel() * 2 / (sum(og_ms) / len(og_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "traffic": measured_traffic("kda_output_gate_32k_x96"),
                             "kernel": "kda_output_gate_kernel<bf16, 128>",
                             "bytes_per_launch": 3 * o_d.numel() * 2},
            },
            "prefill_backward": None if bw_ms is None else backward_entry(bw_ms, token_heads, wd["T"]),
            "prefill_gated": {
                "workload": "k3_varlen_32k through kda_prefill_output_gated: y = sigmoid(gate) * RMSNorm(o) * weight "
                            "fused into the o store (whole-head workgroups); two_pass = kda_prefill then kda_output_gate",
                "ms": sum(gated_ms) / len(gated_ms),
                "vs_plain_varlen": (sum(gated_ms) / len(gated_ms)) / v_avg,
                "two_pass_ms": sum(two_pass_ms) / len(two_pass_ms),
                "bytes_per_token_head": GATED_BYTES_PER_TOKEN_HEAD,
                "hbm_gbs": GATED_BYTES_PER_TOKEN_HEAD * wv["T"] * wv["H"] / (sum(gated_ms) / len(gated_ms) * 1e-3) / 1e9,
                "traffic": measured_traffic("kda_prefill_gated_k3_varlen_32k"),
            },
            "prefill_varlen": {
                "tokens_per_s": wv["T"] / (v_avg * 1e-3), "ms": v_avg,
                "hbm_gbs": PREFILL_BYTES_PER_TOKEN_HEAD * wv["T"] * wv["H"] / (v_avg * 1e-3) / 1e9,
                "traffic": measured_traffic("kda_prefill_k3_varlen_32k"),
                "lengths": wv["lengths"],
            },
        })
        del o_v, s_v

    # ---------------------------------------------------- long-context prefill
    if args.only in ("all", "long") and args.long_steps > 0:
        log("generating long_1m_h16 inputs (T = 1048576, H = 16)")
        wl = synth.workload_inputs("long_1m_h16", dev)
        o_l = torch.empty_like(wl["v"])
        s_l = torch.empty((wl["N"], wl["H"], wl["d"], wl["d"]), dtype=torch.float32, device=dev)

        def run_long():
            kda.kda_prefill(wl["q"], wl["k"], wl["v"], wl["g"], wl["beta"], None, None, chunk_size=C,
                            out=o_l, final_state=s_l)

        long_ms = time_launches(run_long, args.long_steps, stream, 1, "prefill_long_1m")
        l_avg = sum(long_ms) / len(long_ms)
        l_bytes = PREFILL_BYTES_PER_TOKEN_HEAD * wl["T"] * wl["H"]
        log("long prefill avg %.3f ms" % l_avg)
        ws_l = kda.kda_prefill_ex_workspace_bytes(wl["N"], wl["T"], wl["H"], wl["d"], wl["d"], torch.bfloat16, C)
        units_l = wl["N"] * wl["H"]
        segs = ws_l // (units_l * 2 * wl["d"] * wl["d"] * 4) + 1 if ws_l else 1
        result["prefill_long_1m"] = {
            "workload": "long_1m_h16: B=1 T=1048576 H=16 d_k=d_v=128, bf16 q/k/v, fp32 g/beta/state",
            "tokens_per_s": wl["T"] / (l_avg * 1e-3), "ms": l_avg, "runs": args.long_steps,
            "hbm_gbs": l_bytes / (l_avg * 1e-3) / 1e9,
            "plan": {"segments_per_sequence": segs, "workspace_bytes": ws_l,
                     "launches": "segment map pairs, combine, all segments again" if segs > 1 else "direct"},
            "roofline": {"bound": "hbm", "achieved": l_bytes / (l_avg * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": l_bytes / (l_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("kda_prefill_long_1m_h16"),
                         "kernel": "kda_prefill_ws_kernel<8,2,4,...,SEG> (map pairs) + kda_segment_combine_kernel + kda_prefill_ws_kernel<4,2,8,...,SEG> (runs): whole call",
                         "bytes_per_launch": l_bytes},
        }
        del wl, o_l, s_l
        torch.cuda.empty_cache()

    # ---------------------------------------------------------------- decode
    if args.only in ("all", "decode"):
        N, H, d = 256, 96, 128
        ring = 16  # distinct input sets (about 500 MB, more than the 256 MB MALL)
        log("generating decode state and %d input sets" % ring)
        S = synth.decode_state(N, H, d, 0.05, 4, dev)
        sets = [synth.decode_inputs(N, H, d, torch.bfloat16, 1000 + i, dev) for i in range(ring)]
        o_dec = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
        it = [0]

        def run_decode():
            q, k, v, g, beta = sets[it[0] % ring]
            it[0] += 1
            kda.kda_decode_step(q, k, v, g, beta, S, out=o_dec)

        dec_ms = time_launches(run_decode, args.decode_steps, stream, 5, "decode")
        dec_avg = sum(dec_ms) / len(dec_ms)
        dec_bytes = DECODE_BYTES_PER_UNIT * N * H
        dec_gbs = dec_bytes / (dec_avg * 1e-3) / 1e9
        log("decode avg %.4f ms/step, %.1f GB/s" % (dec_avg, dec_gbs))
        result["decode"] = {
            "workload": "256 sequences x 96 heads, fp32 128x128 states, bf16 q/k/v, fp32 g/beta",
            "ms_per_step": dec_avg, "steps": args.decode_steps, "state_hbm_gbs": dec_gbs,
            "tokens_per_s": N / (dec_avg * 1e-3),
            "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dec_gbs / HBM_PEAK_GBS, "traffic": measured_traffic("kda_decode_256x96"),
                         "kernel": "kda_decode_kernel<bf16,128>", "bytes_per_launch": dec_bytes},
        }
        del S, sets

    line = {
        "metric": "KDA prefill tokens/s (H=96,d=128,T=32K) + decode state HBM GB/s",
        "value": result.get("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_note": "each timed workload: at least `warmup` launches, continued until %d ms of back-to-back "
                       "launches have run (the device clocks ramp for about 45 ms after a change of workload); "
                       "launches per workload in warmup_launches" % WARM_MS,
        "warmup_launches": WARMUP_LAUNCHES,
        "ms_per_step": result.get("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "k3_dense_32k: B=1 T=32768 H=96 d_k=d_v=128, bf16 q/k/v, fp32 g/beta/state",
                   "global_batch": 1, "seq_len": 32768, "heads": 96, "d_k": 128, "d_v": 128,
                   "chunk": C or 16, "parallelism": "none (1 GPU)"},
    }
    # Context: what a plain device-to-device copy reaches on this GPU.
    src = torch.ones(1 << 29, dtype=torch.float32, device=dev)  # 2 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_ms = time_launches(lambda: dst.copy_(src), 5, stream)
    result["device_copy"] = {"bytes_per_copy": 2 * src.numel() * 4,
                             "gbs": 2 * src.numel() * 4 / (min(copy_ms) * 1e-3) / 1e9,
                             "note": "best of 5 torch copy_ launches of 2 GiB (read + write bytes)"}
    del src, dst
    for key in ("roofline", "mfma", "prefill_varlen", "prefill_gated", "prefill_checkpoints", "prefill_fused",
                "output_gate",
                "prefill_backward",
                "prefill_long_1m", "decode", "device_copy"):
        if key in result:
            line[key] = result[key]

    if not args.no_cpu_baseline and args.only in ("all", "prefill"):
        log("timing the oracle (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(wd, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
