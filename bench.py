#!/usr/bin/env python3
"""Throughput of the MI355X LSTM forward in timestep-cells/s (B*T*H*L*D per second).

One "step" is one full forward pass (every layer: input projection GEMM and the
recurrence) over one batch of synthetic, seeded input already resident in HBM.
Default workload: 2 layers, unidirectional, input 256, hidden 512, T 128,
batch 64, fp32 -- the running example of the "Complete Trace: nn.LSTM" page
at a 64-sequence batch.

Prints one JSON line.  Besides throughput it reports
  roofline      the dominant kernel (the one with the larger share of device
                time) against its bound, timed live with HIP events recorded on
                the launch stream inside lstm_forward;
  cpu_baseline  the fp64 oracle on the host cores over a bounded sample of
                batch rows of the same workload (rows are independent).
"""
import argparse
import dataclasses
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LSTM fwd timestep-cells/sec (B·T·H·L·D) at 1 GPU; % of MFMA / LDS-BW roofline"
DEFAULT = "l2_in256_h512_t128_b64_f32"
# Published dense peaks of one MI355X.
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def rec_flops_per_launch(spec):
    """Algorithmic FLOPs of one layer's recurrence: 2*B*T*D*4H*H."""
    H = spec.hidden_size
    return 2.0 * spec.B * spec.T * spec.D * spec.gates * H * H


def proj_flops_per_launch(spec):
    """Average over layers of 2*T*B*D*4H*in_l (one GEMM launch per layer)."""
    H = spec.hidden_size
    tot = sum(2.0 * spec.T * spec.B * spec.D * spec.gates * H * spec.layer_input(l)
              for l in range(spec.num_layers))
    return tot / spec.num_layers


def run_oracle(sub, threads, lengths):
    import oracle
    spec = sub.spec
    if spec.mode != "lstm":
        return oracle.rnn_forward(spec.mode, sub.x, sub.params, spec.hidden_size, spec.num_layers,
                                  spec.bidirectional, h0=sub.h0, has_bias=spec.has_bias, bf16=sub.bf16,
                                  nthreads=threads)
    return oracle.lstm_forward(sub.x, sub.params, spec.hidden_size, spec.num_layers, spec.bidirectional,
                               h0=sub.h0, c0=sub.c0, has_bias=spec.has_bias, bf16=sub.bf16, nthreads=threads,
                               lengths=lengths)


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_threads():
    """The host threads this run may use: OMP_NUM_THREADS when set (a share of
    a larger machine), else every CPU the process sees."""
    try:
        n = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        n = 0
    return max(1, n if n > 0 else (os.cpu_count() or 1))


def cpu_baseline(inp, budget_s, lengths=None):
    """The fp64 oracle timed on the host cores, on a bounded sample of batch
    rows of the same workload (rows are independent): once on one thread and
    once on every thread this run may use, each sized from a one-row
    calibration to about budget_s / 2 seconds."""
    import numpy as np
    spec = inp.spec
    per_row_flops = spec.flops() / spec.B

    def timed(threads):
        t0 = time.perf_counter()
        run_oracle(inp.rows([0]), threads, None if lengths is None else lengths[[0]])
        one = time.perf_counter() - t0
        n = int(max(1, min(spec.B, (budget_s / 2) / max(one, 1e-6))))
        rows = sorted(set(int(r) for r in np.linspace(0, spec.B - 1, n).astype(int))) if n > 1 else [0]
        t0 = time.perf_counter()
        run_oracle(inp.rows(rows), threads, None if lengths is None else lengths[rows])
        wall = time.perf_counter() - t0
        steps = spec.T * len(rows) if lengths is None else int(np.sum(lengths[rows]))
        cells = steps * spec.hidden_size * spec.num_layers * spec.D
        return cells / wall, rows, wall

    threads = host_threads()
    v1, rows1, wall1 = timed(1)
    vn, rowsn, walln = timed(threads)
    what = f"full T={spec.T}" if lengths is None else "their valid steps (per-row lengths)"
    return {"value": vn, "unit": "timestep-cells/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rowsn)} of {spec.B} batch rows, {what}, all {spec.num_layers} layers, fp64, "
                      f"{walln:.1f} s wall on {threads} threads ({per_row_flops * len(rowsn) / walln / 1e9:.2f} "
                      f"GFLOP/s)",
            "single_thread": {"value": v1, "cores": 1,
                              "sample": f"{len(rows1)} of {spec.B} batch rows, {what}, {wall1:.1f} s wall "
                                        f"({per_row_flops * len(rows1) / wall1 / 1e9:.2f} GFLOP/s)"},
            "cpu_model": cpu_model(), "cpus_visible": os.cpu_count()}


def summarize_profile(path, command):
    """Per-kernel duration statistics from a rocprofv3 kernel trace (the
    rocpd SQLite database or a kernel_trace.csv), as a short text table."""
    import csv
    import sqlite3
    from collections import defaultdict
    durs = defaultdict(list)
    counters = defaultdict(lambda: defaultdict(list))
    if path.endswith(".db"):
        con = sqlite3.connect(path)
        for name, dur in con.execute("select name, duration from kernels"):
            durs[name].append(dur)
        try:
            for name, cname, val in con.execute(
                    "select k.name, p.counter_name, p.value from pmc_events p join kernels k "
                    "on p.dispatch_id = k.dispatch_id"):
                counters[name][cname].append(val)
        except sqlite3.Error:
            pass
    else:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name") or row.get("KernelName") or row.get("Name")
                if "Counter_Name" in row:
                    counters[name][row["Counter_Name"]].append(float(row["Counter_Value"]))
                    continue
                s, e = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
                durs[name].append(e - s)
    total = sum(sum(v) for v in durs.values()) or 1
    lines = [f"# rocprofv3 kernel summary", f"# command: {command}", f"# source: {os.path.basename(path)}",
             f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_ms':>10} {'pct':>6}  kernel"]
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{len(v):6d} {sum(v) / len(v) / 1e3:10.2f} {min(v) / 1e3:10.2f} {max(v) / 1e3:10.2f} "
                     f"{sum(v) / 1e6:10.3f} {100.0 * sum(v) / total:6.1f}  {name[:140]}")
    for name, cs in counters.items():
        for cname, vals in sorted(cs.items()):
            lines.append(f"# counter {cname} per dispatch: avg {sum(vals) / len(vals):.1f} over {len(vals)} "
                         f"dispatches of {name[:100]}")
    return "\n".join(lines)


def kernel_source_hash(kernel):
    """sha256 of the sources of `kernel` (every source file that defines or
    instantiates it, and the shared device headers; "a+b": of each kernel's);
    a stored counter profile is valid only for the sources it was taken from."""
    import hashlib
    import re as _re
    csrc = os.path.join(ROOT, "layer_lstm_forward_amd", "csrc")
    sources = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")) and f not in ("device.h", "kernels.h"))
    files = set()
    for k in kernel.split("+"):
        pat = _re.compile(r"\b" + _re.escape(k.strip()) + r"\s*[(<]")
        for name in sources:
            with open(os.path.join(csrc, name)) as fh:
                if pat.search(fh.read()):
                    files.add(name)
    h = hashlib.sha256()
    for f in sorted(files) + ["device.h", "kernels.h"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, kernel, workload, command):
    """HBM traffic of `kernel` from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for a plain copy of
    known size."""
    import csv
    from collections import defaultdict

    def per_dispatch(path, want):
        vals = defaultdict(list)
        with open(path) as f:
            for row in csv.DictReader(f):
                vals[row["Kernel_Name"]].append(float(row["Counter_Value"]))
        for name, v in vals.items():
            if want in name:
                return sum(v) / len(v), len(v), name
        raise SystemExit(f"no dispatch of {want} in {path}")

    cf, _, _ = per_dispatch(copy_fetch_csv, "copyBuffer")
    cw, _, _ = per_dispatch(copy_write_csv, "copyBuffer")
    copy_kib = 256 * 1024  # the calibration copy reads and writes 256 MiB
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    # "a+b": one launch is a dispatch of each kernel named; their per-dispatch figures add
    kf = kw = 0.0
    nf, nw, names = [], [], []
    for k in kernel.split("+"):
        f_, n_, name = per_dispatch(fetch_csv, k)
        w_, m_, _ = per_dispatch(write_csv, k)
        kf, kw = kf + f_, kw + w_
        nf.append(str(n_))
        nw.append(str(m_))
        names.append(name[:120])
    name = " + ".join(names)
    nf, nw = "+".join(nf), "+".join(nw)
    fetch_b = kf * 1024 * f_scale
    write_b = kw * 1024 * w_scale
    lines = ["# rocprofv3 HBM counters, one dispatch = one launch",
             f"# command: {command}",
             f"# workload: {workload}",
             f"# kernel: {name}",
             f"kernel_source_sha256: {kernel_source_hash(kernel.replace('<', ''))}",
             f"copy_calibration: FETCH_SIZE {cf:.1f} KiB and WRITE_SIZE {cw:.1f} KiB for a 262144 KiB copy "
             f"-> scale fetch x{f_scale:.4f}, write x{w_scale:.4f}",
             f"FETCH_SIZE_KiB_per_dispatch: {kf:.1f} (over {nf} dispatches)",
             f"WRITE_SIZE_KiB_per_dispatch: {kw:.1f} (over {nw} dispatches)",
             f"fetch_bytes_per_launch: {fetch_b:.0f}",
             f"write_bytes_per_launch: {write_b:.0f}",
             f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}"]
    return "\n".join(lines)


def counter_summary(kernel, workload, csv_paths, command):
    """Per-dispatch averages of every counter in rocprofv3 counter_collection
    csv files for the dispatches of `kernel`, with the ratios read from them:
      mfma_busy         SQ_VALU_MFMA_BUSY_CYCLES / (dispatch cycles at
                        2.4 GHz x 1024 SIMDs): the matrix pipes' busy fraction
                        (the counter adds each MFMA instruction's issue cycles,
                        so this equals achieved / peak matrix flops)
      lds_conflict      SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
      wait_any          SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES"""
    import csv
    from collections import defaultdict
    vals = defaultdict(list)
    durs = {}
    name = None
    for path in csv_paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                if kernel not in row["Kernel_Name"]:
                    continue
                name = row["Kernel_Name"]
                vals[row["Counter_Name"]].append(float(row["Counter_Value"]))
                if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                    durs[(path, row["Dispatch_Id"])] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    if name is None:
        raise SystemExit(f"no dispatch of {kernel} in {csv_paths}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    lines = ["# rocprofv3 counters, averages per dispatch (one dispatch = one launch)",
             f"# command: {command}", f"# workload: {workload}", f"# kernel: {name[:160]}",
             f"kernel_source_sha256: {kernel_source_hash(kernel.rstrip('<'))}"]
    for k in sorted(avg):
        lines.append(f"{k}: {avg[k]:.1f} (over {len(vals[k])} dispatches)")
    dur_ns = sum(durs.values()) / len(durs) if durs else None
    if dur_ns:
        lines.append(f"dispatch_us_under_counters: {dur_ns / 1e3:.2f}")
    if dur_ns and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        lines.append(f"mfma_busy: {avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (dur_ns * 2.4 * 1024):.4f}")
    if avg.get("SQ_LDS_IDX_ACTIVE"):
        lines.append(f"lds_conflict: {avg.get('SQ_LDS_BANK_CONFLICT', 0.0) / avg['SQ_LDS_IDX_ACTIVE']:.4f}")
    if avg.get("SQ_WAVE_CYCLES") and "SQ_WAIT_INST_ANY" in avg:
        lines.append(f"wait_any: {avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.4f}")
    if dur_ns and "GRBM_GUI_ACTIVE" in avg:
        # GRBM_GUI_ACTIVE adds the 8 XCDs' active cycles; per XCD and nanosecond
        # of the dispatch it approximates the clock (short dispatches overstate it)
        lines.append(f"grbm_active_ghz_per_xcd: {avg['GRBM_GUI_ACTIVE'] / 8 / dur_ns:.2f}")
    return "\n".join(lines)


def stored_traffic(kernel, workload):
    """traffic_bytes_per_launch from profiles/<kernel>_<workload>_hbm_counters.txt
    if it was taken from the current kernel sources, else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash(kernel):
        return None
    return float(fields["traffic_bytes_per_launch"])


def copy_calibration(nbytes, steps):
    """A plain device-to-device copy of a known size, for scaling the HBM
    byte counters (the copy moves exactly 2*nbytes: one read, one write)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4, "launches": steps}))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-profile":
        print(summarize_profile(sys.argv[2], " ".join(sys.argv[3:])))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        print(pmc_summary(*sys.argv[2:8], " ".join(sys.argv[8:])))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--counter-summary":
        # --counter-summary <kernel> <workload> <csv>[,<csv>...] <command text>
        print(counter_summary(sys.argv[2], sys.argv[3], sys.argv[4].split(","), " ".join(sys.argv[5:])))
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--copy-calibration":
        copy_calibration(int(sys.argv[2]) if len(sys.argv) > 2 else 256 << 20, 5)
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT)
    ap.add_argument("--recurrence", choices=["auto", "step", "persistent"], default="auto")
    ap.add_argument("--rec-tile", type=int, default=0)
    ap.add_argument("--proj-tile", type=int, default=0, help="LSTM_OPT_PROJ_TILE (0 automatic)")
    ap.add_argument("--layer-pipe", type=int, choices=[0, 1, 2], default=None,
                    help="LSTM_OPT_LAYER_PIPE (default: the library's, the layer wavefront where it applies)")
    ap.add_argument("--small-batch", type=int, choices=[0, 1], default=None,
                    help="LSTM_OPT_SMALL_BATCH (default: the library's, one XCD per direction where it applies)")
    ap.add_argument("--resident", type=int, choices=[0, 1, 2], default=None,
                    help="LSTM_OPT_RESIDENT (default: the library's, W_hh held across the chip where a layer "
                         "would otherwise step)")
    ap.add_argument("--read-pace", type=int, default=-1, help="LSTM_OPT_READ_PACE in ns (-1: the default)")
    ap.add_argument("--partial-buffers", type=int, default=0)
    ap.add_argument("--poll-sleep", type=int, default=-1)
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="with --train: dropout probability between layers (seed 1234)")
    ap.add_argument("--lengths", choices=["none", "mix", "ragged"], default="none",
                    help="variable-length rows (lstm_forward_lengths); the value then counts valid cells only")
    ap.add_argument("--batch-first", action="store_true", help="x [B, T, I] and y [B, T, D*H]")
    ap.add_argument("--mode", choices=["lstm", "gru", "rnn_tanh", "rnn_relu"], default="lstm",
                    help="recurrent mode (the workload's shape with another cell; forward only)")
    ap.add_argument("--train", action="store_true",
                    help="time a training step instead: lstm_forward_train + lstm_backward")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on exactly one GPU (the forward pass has no cross-GPU "
              "component here); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import layer_lstm_forward_amd as pkg
    from layer_lstm_forward_amd.synth import WORKLOADS, make_inputs, make_lengths

    spec = WORKLOADS[args.workload]
    if args.mode != "lstm":
        if args.train or args.lengths != "none":
            raise SystemExit("--mode other than lstm: forward only, without --lengths")
        spec = dataclasses.replace(spec, mode=args.mode)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {args.workload}: generating inputs")
    inp = make_inputs(spec)
    lengths = None if args.lengths == "none" else make_lengths(spec, args.lengths)
    cells = spec.cells if lengths is None else int(np.sum(lengths)) * spec.hidden_size * spec.num_layers * spec.D
    bf = spec.dtype == "bf16"

    def to_dev(a):
        if a is None:
            return None
        if bf and a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    x = to_dev(np.ascontiguousarray(inp.x.transpose(1, 0, 2)) if args.batch_first else inp.x)
    w = [to_dev(p) for p in inp.params]
    h0 = to_dev(inp.h0)
    c0 = None if inp.c0 is None or spec.mode != "lstm" else torch.from_numpy(inp.c0).to(dev)
    rec = {"auto": pkg.LSTM_REC_AUTO, "step": pkg.LSTM_REC_STEP, "persistent": pkg.LSTM_REC_PERSISTENT}
    opts = {}
    if args.partial_buffers:
        opts[pkg.LSTM_OPT_PARTIAL_BUFFERS] = args.partial_buffers
    if args.poll_sleep >= 0:
        opts[pkg.LSTM_OPT_POLL_SLEEP] = args.poll_sleep
    if args.proj_tile:
        opts[pkg.LSTM_OPT_PROJ_TILE] = args.proj_tile
    if args.layer_pipe is not None:
        opts[pkg.LSTM_OPT_LAYER_PIPE] = args.layer_pipe
    if args.small_batch is not None:
        opts[pkg.LSTM_OPT_SMALL_BATCH] = args.small_batch
    if args.resident is not None:
        opts[pkg.LSTM_OPT_RESIDENT] = args.resident
    if args.read_pace >= 0:
        opts[pkg.LSTM_OPT_READ_PACE] = args.read_pace
    m = pkg.LSTM(spec.input_size, spec.hidden_size, spec.num_layers, spec.bidirectional, bias=spec.has_bias,
                 dtype=spec.dtype, recurrence=rec[args.recurrence], rec_tile=args.rec_tile, options=opts,
                 batch_first=args.batch_first, mode=spec.mode)
    desc = m.describe(spec.T, spec.B)
    log(f"schedule: {desc}")
    yshape = (spec.B, spec.T) if args.batch_first else (spec.T, spec.B)
    out = (torch.empty(*yshape, spec.D * spec.hidden_size, dtype=x.dtype, device=dev),
           torch.empty(spec.num_layers * spec.D, spec.B, spec.hidden_size, dtype=x.dtype, device=dev),
           torch.empty(spec.num_layers * spec.D, spec.B, spec.hidden_size, dtype=torch.float32, device=dev)
           if spec.mode == "lstm" else None)
    stream = torch.cuda.current_stream(dev)
    if args.train:
        if args.dropout:
            m.set_dropout(args.dropout, 1234, 0)
        return train_bench(args, spec, m, x, w, h0, c0, stream, desc, lengths)

    for _ in range(args.warmup):
        m.forward(x, w, h0, c0, out=out, lengths=lengths)
    torch.cuda.synchronize()
    rc, flags = m.device_status()
    if rc != 0:
        log(f"device status after warmup: {rc} flags {flags}")
        sys.exit(1)
    log(f"warmup done ({args.warmup} steps)")

    pkg.lstm_set_option(m.plan, pkg.LSTM_OPT_TIMING, 1)
    pkg.lstm_read_timing(m.plan, reset=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        m.forward(x, w, h0, c0, out=out, lengths=lengths)
    ev1.record(stream)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    tm = pkg.lstm_read_timing(m.plan, reset=True)
    rc, flags = m.device_status()
    if rc != 0:
        log(f"device status after timed steps: {rc} flags {flags}")
        sys.exit(1)
    ms = total_ms / args.steps
    value = cells * args.steps / (total_ms / 1e3)
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, {value / 1e9:.3f} G cells/s; phases {tm}")

    proj_avg = tm["proj_ms"] / max(1, tm["proj_launches"])
    rec_avg = tm["rec_ms"] / max(1, tm["rec_launches"])
    # kernel names as the library reports them: "proj=<name><dtype>; rec=<name><..."
    names = dict(re.findall(r"(proj|rec)=(k_[a-z_]+)<", desc))
    if tm["rec_ms"] >= tm["proj_ms"]:
        kname, flops, avg = names.get("rec", "k_rec"), rec_flops_per_launch(spec), rec_avg
        if kname == "k_rec_wave":  # one launch runs every layer with its input products
            flops = (rec_flops_per_launch(spec) + proj_flops_per_launch(spec)) * spec.num_layers
        elif tm["rec_launches"] > tm["calls"] * spec.num_layers:  # stepping: a "launch" is one step
            flops /= spec.T
        else:  # layers whose input projection runs inside the recurrent launch
            fused = (re.findall(r"xproj=([a-z,]+)", desc) or [""])[0].split(",")
            H = spec.hidden_size
            flops += sum(2.0 * spec.T * spec.B * spec.D * 4 * H * spec.layer_input(l)
                         for l in range(spec.num_layers) if l < len(fused) and fused[l] == "fused") / spec.num_layers
    else:
        kname, flops, avg = names.get("proj", "k_proj"), proj_flops_per_launch(spec), proj_avg
    stepping = tm["rec_launches"] > tm["calls"] * spec.num_layers
    nbytes = alg_bytes_per_launch(spec, kname, desc, stepping)
    tflops = flops / (avg / 1e3) / 1e12
    gbs = None if nbytes is None else nbytes / (avg / 1e3) / 1e9
    # the bound is the resource whose time at peak is the larger for this launch
    hbm_bound = gbs is not None and nbytes / PEAK_HBM_GBS > flops / (PEAK_TFLOPS[spec.dtype] * 1e3)
    if hbm_bound:
        bound, achieved, peak, unit = "hbm", gbs, PEAK_HBM_GBS, "GB/s"
    else:
        bound, achieved, peak, unit = "mfma", tflops, PEAK_TFLOPS[spec.dtype], "TFLOP/s"
    traffic = stored_traffic(kname, args.workload)
    roof = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "traffic_GB_per_s": None if traffic is None else round(traffic / (avg / 1e3) / 1e9, 1),
            "kernel": kname,
            "avg_launch_ms": round(avg, 4), "flops_per_launch": flops, "alg_bytes_per_launch": nbytes,
            "mfma_frac": round(tflops / PEAK_TFLOPS[spec.dtype], 4),
            "hbm_frac": None if gbs is None else round(gbs / PEAK_HBM_GBS, 4),
            "phase_ms_per_step": {"proj": round(tm["proj_ms"] / max(1, tm["calls"]), 4),
                                  "rec": round(tm["rec_ms"] / max(1, tm["calls"]), 4)}}

    recurrence = recurrence_roofline(spec, desc, tm, args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle on a row sample")
        cpu = cpu_baseline(inp, args.cpu_budget, lengths)
        log(f"cpu baseline: {cpu}")

    metric = METRIC if spec.mode == "lstm" else METRIC.replace("LSTM", spec.mode.upper(), 1)
    line = {"metric": metric, "value": value, "unit": "timestep-cells/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic (seeded; random-init weights)",
            "config": {"workload": args.workload, "input_size": spec.input_size, "hidden_size": spec.hidden_size,
                       "num_layers": spec.num_layers, "bidirectional": spec.bidirectional, "T": spec.T,
                       "B": spec.B, "cells_per_step": cells, "schedule": desc,
                       **({} if lengths is None else {"lengths": args.lengths,
                                                       "valid_steps": int(np.sum(lengths))}),
                       **({"layout": "batch_first"} if args.batch_first else {}),
                       **({"cell": spec.mode} if spec.mode != "lstm" else {})},
            "roofline": roof, "recurrence": recurrence, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)
    # release the plan while the runtime is fully up, not from a finaliser at exit
    del m
    torch.cuda.synchronize()


PEAK_LDS_GBS = 78643.2  # 128 B per clock per CU, 256 CUs, 2.4 GHz


def alg_bytes_per_launch(spec, kname, desc, stepping):
    """Algorithmic HBM bytes of one launch of the dominant kernel (the
    per-unit figures times the units one launch covers), or None where no
    such figure is kept (the layer pipeline).  Every array read or written
    once per launch:
      k_proj*      x [T*B, in_l] + W_ih [D*4H, in_l] read, G [T*B, D*4H] fp32
                   written (mean over layers)
      k_rec        per layer: W_hh [D*4H, H], y [T, B, D*H] written, h0/c0 and
      k_rec_xcd    h_n/c_n, and either G read (hoisted) or x and W_ih read
      k_rec_res    (fused) (mean over layers)
      k_rec_step   one step: W_hh, G [B, D*4H] fp32, h_{t-1} [B, D*H] read, c
                   read and written, y [B, D*H] written
      k_rec_wave   the whole stack: every layer's W_ih and W_hh, x, the top
                   layer's y, each layer's h0/c0 and h_n/c_n"""
    H, B, T, D, L = spec.hidden_size, spec.B, spec.T, spec.D, spec.num_layers
    s = 2 if spec.dtype == "bf16" else 4
    G4 = spec.gates * H
    fused = (re.findall(r"xproj=([a-z,]+)", desc) or [""])[0].split(",")
    if kname.startswith("k_proj"):
        return sum(T * B * spec.layer_input(l) * s + D * G4 * spec.layer_input(l) * s + T * B * D * G4 * 4
                   for l in range(L)) / L
    states = 2 * D * B * H * (s + 4)  # h0, c0 read; h_n, c_n written
    if kname == "k_rec_wave":  # every layer in one launch: all weights, x, the top layer's y, states
        return (sum(D * G4 * (H + spec.layer_input(l)) * s for l in range(L)) + T * B * spec.input_size * s
                + T * B * D * H * s + L * 2 * D * B * H * (s + 4))
    if kname == "k_rec_step" or (kname == "k_rec" and stepping):
        return D * G4 * H * s + B * D * G4 * 4 + B * D * H * s + 2 * B * D * H * 4 + B * D * H * s
    if kname in ("k_rec", "k_rec_xcd", "k_rec_res"):
        tot = 0.0
        for l in range(L):
            io = (T * B * spec.layer_input(l) * s + D * G4 * spec.layer_input(l) * s
                  if l < len(fused) and fused[l] == "fused" else T * B * D * G4 * 4)
            tot += D * G4 * H * s + T * B * D * H * s + states + io
        return tot / L
    return None


def recurrence_roofline(spec, desc, tm, workload):
    """The recurrent phase against its own roofline: the larger of (a) its
    matrix-core time at the dtype's peak (the recurrent products, plus the
    input products when they run inside the recurrent launch), (b) W_hh read
    once per step from where it lives (registers: no bound; LDS at the LDS
    peak; streamed from HBM by the per-step GEMM kernel), W_ih likewise for
    the layer wavefront (read from LDS), and (c) its HBM traffic (the hoisted
    G read and y written).  frac = roofline time /
    measured time; per_step_us = measured time / sequential step slots."""
    H, B, T, D, L = spec.hidden_size, spec.B, spec.T, spec.D, spec.num_layers
    s = 2 if spec.dtype == "bf16" else 4
    G4 = spec.gates * H
    fused = (re.findall(r"xproj=([a-z,]+)", desc) or [""])[0].split(",")
    is_fused = [l < len(fused) and fused[l] == "fused" for l in range(L)]
    flops = sum(2.0 * B * T * D * G4 * (H + (spec.layer_input(l) if is_fused[l] else 0)) for l in range(L))
    rec_ms = tm["rec_ms"] / max(1, tm["calls"])
    pipe = "k_rec_wave" in desc
    slots = T + L - 1 if pipe else T * L
    if "k_rec_step" in desc or "mode=gemm-step" in desc:
        w_level, w_bw = "hbm", PEAK_HBM_GBS
    elif "w_hh=lds" in desc:
        w_level, w_bw = "lds", PEAK_LDS_GBS
    else:
        w_level, w_bw = "registers", None
    w_bytes = T * L * D * G4 * H * s
    hbm_bytes = sum((0 if is_fused[l] else T * B * D * G4 * 4) + T * B * D * H * s for l in range(L))
    terms = {"mfma_us": flops / (PEAK_TFLOPS[spec.dtype] * 1e12) * 1e6,
             "w_hh_us": None if w_bw is None else w_bytes / (w_bw * 1e9) * 1e6,
             "hbm_us": hbm_bytes / (PEAK_HBM_GBS * 1e9) * 1e6}
    if pipe:  # the wavefront keeps W_hh in registers and reads W_ih from LDS every step
        terms["w_ih_lds_us"] = T * sum(D * G4 * spec.layer_input(l) * s for l in range(L)) / (PEAK_LDS_GBS * 1e9) * 1e6
    bound = max((k for k in terms if terms[k] is not None), key=lambda k: terms[k])
    t_roof = terms[bound]
    return {"per_step_us": round(rec_ms * 1e3 / slots, 3), "slots": slots, "ms": round(rec_ms, 4),
            "w_hh_from": w_level, "bound": bound.replace("_us", ""),
            "terms_us": {k: None if v is None else round(v, 2) for k, v in terms.items()},
            "frac": round(t_roof / (rec_ms * 1e3), 4)}


def train_bench(args, spec, m, x, w, h0, c0, stream, desc, lengths=None):
    """A training step = lstm_forward_train + lstm_backward on the workload
    (synthetic output gradients); the value counts timestep-cells per second
    of the whole step.  The forward alone is timed beside it."""
    import numpy as np
    import torch
    import layer_lstm_forward_amd as pkg
    rng = np.random.default_rng(spec.seed + 11)
    dy = torch.from_numpy(rng.standard_normal((spec.T, spec.B, spec.D * spec.hidden_size)).astype(np.float32))
    dy = dy.to(x.device).to(x.dtype)

    lens = None if lengths is None else [int(v) for v in lengths]

    def step():
        y, hn, cn, reserve = m.forward_train(x, w, h0, c0, lengths=lens)
        return m.backward(x, w, y, reserve, dy, h0=h0, c0=c0, lengths=lens)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1, ev2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    ev0.record(stream)
    for _ in range(args.steps):
        m.forward_train(x, w, h0, c0, lengths=lens)
    ev1.record(stream)
    for _ in range(args.steps):
        step()
    ev2.record(stream)
    torch.cuda.synchronize()
    fwd_ms = ev0.elapsed_time(ev1) / args.steps
    ms = ev1.elapsed_time(ev2) / args.steps
    cells = spec.cells if lengths is None else int(np.sum(lengths)) * spec.hidden_size * spec.num_layers * spec.D
    value = cells / (ms / 1e3)
    log(f"training step: {ms:.3f} ms (forward_train {fwd_ms:.3f} ms, backward {ms - fwd_ms:.3f} ms), "
        f"{value / 1e9:.3f} G cells/s")

    # The backward's dominant work is its recurrence: per step and layer one
    # k_bwd_step launch (the recurrent product and the next step's cell
    # update), timed by the library's own events around each layer's loop of
    # T steps, in separate timed steps.
    pkg.lstm_set_option(m.plan, pkg.LSTM_OPT_TIMING, 1)
    pkg.lstm_read_timing(m.plan, reset=True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    tm = pkg.lstm_read_timing(m.plan, reset=True)
    pkg.lstm_set_option(m.plan, pkg.LSTM_OPT_TIMING, 0)
    H = spec.hidden_size
    flops = 2.0 * spec.B * spec.D * 4 * H * H  # dz_t [B, 4H] x W_hh [4H, H] per direction and step
    # the product's MFMAs run in the gradient dtype: bf16 for bf16 parameters with an even H
    peak = PEAK_TFLOPS["bf16" if spec.dtype == "bf16" and H % 2 == 0 else "f32"]
    avg = tm["bwd_rec_ms"] / max(1, tm["bwd_rec_launches"])
    achieved = flops / (avg / 1e3) / 1e12
    traffic = stored_traffic("k_bwd_step", args.workload)
    roof = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "traffic_GB_per_s": None if traffic is None else round(traffic / (avg / 1e3) / 1e9, 1),
            "kernel": "k_bwd_step", "launch": "one backward step",
            "avg_launch_ms": round(avg, 5), "flops_per_launch": flops,
            "phase_ms_per_step": {"bwd_rec": round(tm["bwd_rec_ms"] / max(1, tm["bwd_calls"]), 4),
                                  "bwd_gemm": round(tm["bwd_gemm_ms"] / max(1, tm["bwd_calls"]), 4),
                                  "bwd_gemm_launches": tm["bwd_gemm_launches"] // max(1, tm["bwd_calls"])}}
    log(f"backward phases: {tm}")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle's forward + backward on a row sample")
        cpu = cpu_baseline_train(spec, args.cpu_budget, args.dropout, lengths)
        log(f"cpu baseline: {cpu}")
    line = {"metric": "LSTM training step (forward_train + backward) timestep-cells/sec", "value": value,
            "unit": "timestep-cells/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": spec.dtype,
            "data": "synthetic (seeded; random-init weights and output gradients)",
            "config": {"workload": args.workload, "T": spec.T, "B": spec.B, "forward_train_ms": fwd_ms,
                       "backward_ms": ms - fwd_ms, "dropout": args.dropout, "schedule": desc},
            "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def cpu_baseline_train(spec, budget_s, dropout=0.0, lengths=None):
    """The fp64 oracle's forward + backward on a sample of batch rows (rows are
    independent), sized to the time budget from a one-row calibration."""
    import numpy as np
    import oracle
    from layer_lstm_forward_amd.synth import make_inputs
    inp = make_inputs(spec)
    threads = 1  # the oracle's backward runs on one thread
    rng = np.random.default_rng(spec.seed + 11)
    dy_all = rng.standard_normal((spec.T, spec.B, spec.D * spec.hidden_size)).astype(np.float32)

    def run(rows):
        sub = inp.rows(rows)
        oracle.lstm_backward(sub.x, sub.params, spec.hidden_size, spec.num_layers, spec.bidirectional,
                             np.ascontiguousarray(dy_all[:, rows]), h0=sub.h0, c0=sub.c0, has_bias=spec.has_bias,
                             bf16=sub.bf16, dropout=(dropout, 1234, 0) if dropout else None,
                             lengths=None if lengths is None else lengths[rows])
    t0 = time.perf_counter()
    run([0])
    one = time.perf_counter() - t0
    n = int(max(1, min(spec.B, budget_s / max(one, 1e-6))))
    rows = sorted(set(int(r) for r in np.linspace(0, spec.B - 1, n).astype(int))) if n > 1 else [0]
    t0 = time.perf_counter()
    run(rows)
    wall = time.perf_counter() - t0
    steps = spec.T * len(rows) if lengths is None else int(np.sum(lengths[rows]))
    cells = steps * spec.hidden_size * spec.num_layers * spec.D
    return {"value": cells / wall, "unit": "timestep-cells/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {spec.B} batch rows, full T={spec.T}, all {spec.num_layers} layers, "
                      f"forward + backward in fp64 (the oracle's backward recomputes its forward), "
                      f"{wall:.1f} s wall"}


if __name__ == "__main__":
    main()
