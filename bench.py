"""Throughput of the fine-grained FP8 hot path on one MI355X.

One step runs every row of the path once, back to back on one stream, on
seeded synthetic inputs already resident in HBM:

  quantizer  1x128 online quantization of X 8192x7168 (outliers in 16 channels)
  fprop      1x128 quantization of X 4096x7168 + block-scaled GEMM
             Y = X W^T 4096x18432x7168 (W pre-quantized 128x128, codes in the
             GEMM's operand-tiled layout), BF16 out; also timed with
             row-major weight codes
  backward   dY 4096x18432 quantized in both orientations from one read
             (1x128 rows for Dgrad, 128x1 columns for Wgrad); Dgrad dX = dY W
             from the transposed weight codes W_q^T; 128x1 quantization of X +
             Wgrad dW = dY^T X (FP32 out).  Dgrad reads operand-tiled W_q^T
             and Wgrad operand-tiled X_q^T (both also timed row-major).  Also reported: Dgrad reading W_q
             as stored ("dgrad_lds") and the dY quantization as two separate
             passes ("dual_quant")
  grouped    1x128 quantization of X 16384x7168 + one grouped launch over 8
             experts (multinomial token counts), W_e 2048x7168
  payload    FP8 token messages for the dispatch of X 4096x7168 to top-2 of
             8 experts (8192 messages of 7392 bytes, gathered in expert
             order): pack, unpack into the GEMM operand layout, restore BF16
  granularity  1xT quantization of X 8192x7168 for T = 32..1024 (the scale
             metadata cost, 4/T bytes per value) and clipping at the 2nd
             largest |x| of 1x128 tiles
  weights    128x128 quantization of W 18432x7168 with the transposed copy,
             both written operand-tiled
  policy     one caller-scale (history policy) quantization of a 128x7168 tile
             with amax and saturation count, plus the history update
  copy       a plain 1 GiB device-to-device copy (torch's copy kernel): the
             measured HBM rate beside the 8 TB/s spec, and the known-size
             kernel that calibrates the HBM byte counters

`value` is the metric's headline: TFLOP/s of the fprop row including its
quantization, 2*M*N*K / t_region, where t_region is the back-to-back
quantize-then-GEMM region, from HIP events on the launch stream averaged over
the timed steps.  Other rows are reported under "rows".  Beside the dual
(both-orientation) quantizers the bench times torch's copy of the same BF16
tensor, which moves the same bytes (read 2, write 2 per value): the rate a
plain kernel reaches on that traffic mix at that size.

    python bench.py [--steps K (50)] [--warmup W (10)] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s incl. fused 1x128 quant; quantizer GB/s"
PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 MFMA
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=2048)
    ap.add_argument("--only", default="", help="comma list of rows to run (default all)")
    return ap.parse_args()


def to_dev(a, torch):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.cuda()


def pair_buffers(M, K, N, torch):
    """Codes [M][K], scales [K/128][round_up(M, 4)] and BF16 Y [M][N] on the
    device, for a quantize-then-GEMM pair that allocates nothing per call."""
    return (torch.empty((M, K), dtype=torch.uint8, device="cuda"),
            torch.empty((K // 128, (M + 3) // 4 * 4), dtype=torch.float32, device="cuda"),
            torch.empty((M, N), dtype=torch.bfloat16, device="cuda"))


class Timer:
    """HIP events on the current stream around named regions of each step."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.acc = {}
        self.count = {}
        self.samples = {}

    def region(self, name, fn):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        out = fn()
        ev1.record()
        self.pending.append((name, ev0, ev1))
        return out

    def chain(self, name, parts):
        """Back-to-back launches bracketed by one event between each pair of
        them: part i is timed between events i and i+1 and the whole region
        between the first and the last, so the parts add up to the region
        exactly."""
        evs = [self.torch.cuda.Event(enable_timing=True)]
        evs[0].record()
        outs = []
        for pname, fn in parts:
            outs.append(fn(*outs[-1:]) if outs else fn())
            ev = self.torch.cuda.Event(enable_timing=True)
            ev.record()
            self.pending.append((pname, evs[-1], ev))
            evs.append(ev)
        self.pending.append((name, evs[0], evs[-1]))
        return outs

    def collect(self):
        self.torch.cuda.synchronize()
        for name, a, b in self.pending:
            t = a.elapsed_time(b)
            self.acc[name] = self.acc.get(name, 0.0) + t
            self.samples.setdefault(name, []).append(t)
            self.count[name] = self.count.get(name, 0) + 1
        self.pending.clear()

    def mean_ms(self, name):
        return self.acc[name] / self.count[name]

    def spread_ms(self, name):
        """(median, p10, p90) of the region over the timed steps."""
        v = np.sort(np.asarray(self.samples[name]))
        return float(np.median(v)), float(np.quantile(v, 0.1)), float(np.quantile(v, 0.9))

    def reset(self):
        self.pending.clear()
        self.acc.clear()
        self.count.clear()
        self.samples.clear()


def traffic_from_profiles(record, kernel_src):
    """HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE) from a
    committed PMC summary under profiles/, if the kernel source it was taken
    from is unchanged; else None."""
    path = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        digest = hashlib.sha256(open(os.path.join(ROOT, kernel_src), "rb").read()).hexdigest()
        if rec.get("source_sha256") != digest:
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


def cpu_baseline(x_bits, w_bits, sample_rows):
    """Oracle (numpy, float64) on a bounded sample of the fprop workload:
    1x128 quantization of the first `sample_rows` rows of X and their block
    GEMM against the first 4096 rows of W (pre-quantized by the oracle,
    untimed)."""
    from oracle import gemm as og
    from oracle import quant
    K, Ns = 7168, 4096
    xb = x_bits[:sample_rows]
    Wq, sW = quant.quant_weight(w_bits[:Ns])
    t0 = time.perf_counter()
    Xq, sX = quant.quant_rows(xb)
    og.fprop(Xq, sX, Wq, sW)
    dt = time.perf_counter() - t0
    flop = 2.0 * sample_rows * Ns * K
    cores = len(os.sched_getaffinity(0))
    # the quantizer oracle alone on one core (numpy runs it single-threaded)
    qrows = min(1024, sample_rows)
    t1 = time.perf_counter()
    quant.quant_rows(xb[:qrows])
    dq = time.perf_counter() - t1
    qbytes = qrows * K * (3 + 4 / 128)
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = ""
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {}).get("name", "")
    except Exception:
        pass
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"1x128 quant of {sample_rows}x{K} X rows + float64 block GEMM against "
                      f"{Ns}x{K} pre-quantized W ({flop:.3e} FLOP, {dt:.1f} s)",
            "quantizer_oracle_GB/s_1core": qbytes / dq / 1e9,
            "quantizer_sample": f"{qrows}x{K} rows, {dq:.2f} s",
            "cpu_model": cpu_model, "blas": blas}


_X_SHARED = None   # the rows the pool workers quantize (inherited through fork)


def _quant_rows_chunk(bounds):
    from oracle import quant
    lo, hi = bounds
    t = time.perf_counter()
    quant.quant_rows(_X_SHARED[lo:hi])
    return time.perf_counter() - t


def quant_oracle_all_cores(x_bits):
    """The quantizer oracle over `x_bits` split into row chunks on a fork-based
    process pool, one process per core (at most 16); run before anything
    touches the GPU, so the forked workers inherit no device state."""
    import multiprocessing as mp
    global _X_SHARED
    _X_SHARED = x_bits
    procs = max(1, min(16, len(os.sched_getaffinity(0))))
    edges = np.linspace(0, x_bits.shape[0], 4 * procs + 1).astype(int)
    chunks = [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]
    with mp.get_context("fork").Pool(procs) as pool:
        pool.map(_quant_rows_chunk, [(0, 8)] * procs)   # workers import the oracle
        t0 = time.perf_counter()
        pool.map(_quant_rows_chunk, chunks)
        dt = time.perf_counter() - t0
    _X_SHARED = None
    nbytes = x_bits.size * (3 + 4 / 128)
    return {"quantizer_oracle_GB/s_all_cores": nbytes / dt / 1e9, "quantizer_all_cores_procs": procs,
            "quantizer_all_cores_sample": f"{x_bits.shape[0]}x{x_bits.shape[1]} rows, {dt:.2f} s"}


def device_info():
    """Engine-clock levels and power cap of the first GPU, read from sysfs
    (no helper process is started; empty where the files are missing)."""
    import glob
    info = {}
    try:
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            sclk = os.path.join(dev, "pp_dpm_sclk")
            if not os.path.exists(sclk):
                continue
            with open(sclk) as f:
                info["sclk_levels"] = [l.strip() for l in f if l.strip()]
            for cap in glob.glob(os.path.join(dev, "hwmon", "hwmon*", "power1_cap")):
                with open(cap) as f:
                    info["power_cap_W"] = int(f.read().strip()) / 1e6
            break
    except Exception:
        pass
    return info


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import synthetic as syn
    only = set(s for s in args.only.split(",") if s)
    want = (lambda r: not only or r in only)
    cpu_pool = None
    if not args.no_cpu_baseline and want("fprop"):
        # before the GPU is touched: the forked pool workers must not inherit it
        log("timing the quantizer oracle on all host cores ...")
        cpu_pool = quant_oracle_all_cores(syn.activation_with_outliers(4096, 7168, seed=0))

    import torch
    import fine_grained_fp8_amd as fp8

    fp8.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    # ---------------- inputs (seeded, synthetic, resident in HBM) ----------------
    t0 = time.time()
    d = {}
    if want("quantizer") or want("granularity"):
        d["x2"] = to_dev(syn.activation_with_outliers(8192, 7168, seed=0), torch)
    host = {}
    if want("toy"):
        xb1, wb1 = syn.toy_layer(0)
        d["x1"] = to_dev(xb1, torch)
        d["wq1_tl"], d["ws1"], _ = fp8.quant_weight_128x128(to_dev(wb1, torch), tiled=True)
    if want("fprop") or want("backward") or want("weights"):
        host["w3"] = syn.gaussian((18432, 7168), seed=1, std=0.02)
        d["w3"] = to_dev(host["w3"], torch)
    if want("fprop") or want("backward") or want("payload"):
        host["x3"] = syn.activation_with_outliers(4096, 7168, seed=0)
        d["x3"] = to_dev(host["x3"], torch)
    if want("fprop") or want("backward"):
        # untimed: the weight codes in the GEMM's operand-tiled layout (Fprop and
        # Dgrad from W_q^T), and row-major for the comparison rows
        d["wq3_tl"], d["ws3"], d["wq3t_tl"] = fp8.quant_weight_128x128(d["w3"], transposed=True, tiled=True)
        d["wq3"], _, d["wq3t"] = fp8.quant_weight_128x128(d["w3"], transposed=True)
    if want("payload"):
        d["src6"] = to_dev(syn.dispatch_rows(4096, 8, 2, seed=5), torch)
        d["msg6"] = fp8.pack_tokens(d["x3"], d["src6"])
    if want("backward"):
        d["dy4"] = to_dev(syn.gaussian((4096, 18432), seed=4, std=1e-3), torch)
        d["dy4_copy"] = torch.empty_like(d["dy4"])
        d["x3_copy"] = torch.empty_like(d["x3"])
    if want("grouped"):
        counts = syn.expert_counts(16384, 8, seed=0)
        d["off5"] = to_dev(syn.expert_offsets(counts).astype(np.int32), torch)
        d["x5"] = to_dev(syn.activation_with_outliers(16384, 7168, seed=0), torch)
        wq5, ws5, wt5 = [], [], []
        for e in range(8):
            we = to_dev(syn.gaussian((2048, 7168), seed=100 + e, std=0.02), torch)
            q, s, _ = fp8.quant_weight_128x128(we)
            qt, _, _ = fp8.quant_weight_128x128(we, tiled=True)
            wq5.append(q); ws5.append(s); wt5.append(qt)
        d["wq5"] = torch.stack(wq5).contiguous()
        d["wq5_tl"] = torch.stack(wt5).contiguous()
        d["ws5"] = torch.stack(ws5).contiguous()
        d["counts5"] = counts
    if want("policy"):
        steps = list(syn.drift_sequence(steps=2, M=128, K=7168, seed=0, spike_step=1))
        d["xp"] = to_dev(steps[1][2], torch)
        d["hist"] = torch.ones((56, 128), dtype=torch.float32, device="cuda")
        d["sp"] = torch.ones((56, 128), dtype=torch.float32, device="cuda")
        d["sat"] = torch.zeros(1, dtype=torch.int32, device="cuda")
    # caller buffers for the headline pair (codes, scales, Y) and the toy
    # layer, reused by every call: the timed regions hold kernels only
    if want("fprop"):
        d["fp_bufs"] = pair_buffers(4096, 7168, 18432, torch)
    if want("toy"):
        d["toy_bufs"] = pair_buffers(128, 128, 256, torch)
    if want("copy"):
        d["cp_src"] = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        d["cp_dst"] = torch.empty_like(d["cp_src"])
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s")

    tm = Timer(torch)

    def step():
        if want("quantizer"):
            tm.region("quantizer", lambda: fp8.quant_act_1x128(d["x2"], "row"))
        if want("toy"):
            tb = d["toy_bufs"]
            tm.chain("toy", [("toy.quant", lambda: fp8.quant_act_1x128(d["x1"], "row", out=tb[0],
                                                                       scales_out=tb[1])),
                             ("toy.gemm", lambda o: fp8.block_gemm("fprop_tiled", o[0], o[1], d["wq1_tl"],
                                                                   d["ws1"], out=tb[2]))])
        if want("fprop"):
            # the headline region: quantization of X, then the GEMM, with one
            # event between them
            fb = d["fp_bufs"]
            (q, s, _), _ = tm.chain("fprop", [
                ("fprop.quant", lambda: fp8.quant_act_1x128(d["x3"], "row", out=fb[0], scales_out=fb[1])),
                ("fprop.gemm", lambda o: fp8.block_gemm("fprop_tiled", o[0], o[1], d["wq3_tl"], d["ws3"],
                                                        out=fb[2]))])
            # the same GEMM reading row-major weight codes, for comparison
            tm.region("fprop_rowmajor.gemm", lambda: fp8.block_gemm("fprop", q, s, d["wq3"], d["ws3"]))
            # the same product with the 1x128 quantization fused into the GEMM
            tm.region("fprop_fused.gemm", lambda: fp8.block_gemm_fused_quant(d["x3"], d["wq3"], d["ws3"]))
        if want("backward"):
            ev0 = torch.cuda.Event(enable_timing=True); ev0.record()
            # dY in both orientations from one read (Dgrad rows, Wgrad columns)
            dq, ds, dqt, dst = tm.region("bwd.quant_dual", lambda: fp8.quant_act_dual(d["dy4"]))
            tm.region("dgrad.gemm", lambda: fp8.block_gemm("dgrad_t_tiled", dq, ds, d["wq3t_tl"], d["ws3"]))
            tm.region("dgrad_lds.gemm", lambda: fp8.block_gemm("dgrad", dq, ds, d["wq3"], d["ws3"]))
            xqt, xst, _ = tm.region("wgrad.quant_x", lambda: fp8.quant_act_1x128(d["x3"], "col_tiled"))
            tm.region("wgrad.gemm", lambda: fp8.block_gemm("wgrad_tiled", dqt, dst, xqt, xst,
                                                           out_dtype=torch.float32))
            ev1 = torch.cuda.Event(enable_timing=True); ev1.record()
            tm.pending.append(("backward", ev0, ev1))
            tm.region("dgrad_rowmajor.gemm", lambda: fp8.block_gemm("dgrad_t", dq, ds, d["wq3t"], d["ws3"]))
            xqr, xsr, _ = fp8.quant_act_1x128(d["x3"], "col")
            tm.region("wgrad_rowmajor.gemm", lambda: fp8.block_gemm("wgrad", dqt, dst, xqr, xsr,
                                                                    out_dtype=torch.float32))
            # the same two quantizations as separate passes, for comparison
            tm.region("bwd.quant_row", lambda: fp8.quant_act_1x128(d["dy4"], "row"))
            tm.region("bwd.quant_col", lambda: fp8.quant_act_1x128(d["dy4"], "col"))
            # X in both orientations from one read (Fprop rows, saved columns for Wgrad)
            tm.region("fwd.quant_dual_x", lambda: fp8.quant_act_dual(d["x3"], tiled=True))
            tm.region("fwd.quant_row_x", lambda: fp8.quant_act_1x128(d["x3"], "row"))
            # torch's copy kernel on the dual passes' read/write bytes
            tm.region("ref.copy_dy", lambda: d["dy4_copy"].copy_(d["dy4"]))
            tm.region("ref.copy_x", lambda: d["x3_copy"].copy_(d["x3"]))
        if want("grouped"):
            (q, s, _), _ = tm.chain("grouped", [
                ("grouped.quant", lambda: fp8.quant_act_1x128(d["x5"], "row")),
                ("grouped.gemm", lambda o: fp8.block_gemm_grouped(d["off5"], o[0], o[1], d["wq5_tl"], d["ws5"],
                                                                  tiled=True))])
            tm.region("grouped_rowmajor.gemm", lambda: fp8.block_gemm_grouped(d["off5"], q, s, d["wq5"], d["ws5"]))
        if want("granularity"):
            for T in (32, 64, 128, 256, 512, 1024):
                tm.region(f"tiles.{T}", lambda T=T: fp8.quant_act_tiles(d["x2"], T, 1))
            tm.region("tiles.128.rank2", lambda: fp8.quant_act_tiles(d["x2"], 128, 2))
        if want("payload"):
            tm.region("payload.pack", lambda: fp8.pack_tokens(d["x3"], d["src6"], out=d["msg6"]))
            tm.region("payload.unpack", lambda: fp8.unpack_tokens(d["msg6"], 7168))
            tm.region("payload.dequant", lambda: fp8.dequant_tokens(d["msg6"], 7168))
        if want("weights"):
            tm.region("weights", lambda: fp8.quant_weight_128x128(d["w3"], transposed=True, tiled=True))
        if want("policy"):
            def pol():
                fp8.quant_act_1x128(d["xp"], "row", scales_in=d["sp"], return_amax=True,
                                    sat_count=d["sat"])
            tm.region("policy", pol)
        if want("copy"):
            tm.region("copy", lambda: d["cp_dst"].copy_(d["cp_src"]))

    for _ in range(args.warmup):
        step()
        tm.collect()
    tm.reset()
    torch.cuda.synchronize()
    # A short spin on the stream lets the host queue the timed steps ahead of
    # the GPU, so each region's events bracket GPU work only (no host latency).
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(2_000_000)
    t_start = time.perf_counter()
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    ev_start.record()
    for i in range(args.steps):
        step()
    ev_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    steps_ms = ev_start.elapsed_time(ev_end)
    tm.collect()

    # Roofline kernels, timed as batches of back-to-back launches between one
    # event pair on the launch stream (per-launch events add a few us to a
    # 30 us kernel): the standalone quantizer and the Fprop GEMM.
    def batch_ms(fn, n):
        fn()
        torch.cuda.synchronize()
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(1_000_000)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    batch = {}
    if want("quantizer"):
        # rotate over 4 input copies (4 x 117 MB > the 256 MB MALL) so the
        # input streams from HBM as it does inside a training step
        xs = [d["x2"]] + [d["x2"].clone() for _ in range(3)]
        it = iter(range(1 << 30))
        batch["quantizer"] = batch_ms(lambda: fp8.quant_act_1x128(xs[next(it) & 3], "row"), 20)
        del xs
    probe = None

    def quant_then_gemm(x, w, sw, bufs):
        q, s, _ = fp8.quant_act_1x128(x, "row", out=bufs[0], scales_out=bufs[1])
        return fp8.block_gemm("fprop_tiled", q, s, w, sw, out=bufs[2])

    if want("toy"):
        batch["toy.pair"] = batch_ms(lambda: quant_then_gemm(d["x1"], d["wq1_tl"], d["ws1"], d["toy_bufs"]), 200)
    if want("fprop"):
        # the headline pair back to back with no event between the two launches
        batch["fprop.pair"] = batch_ms(lambda: quant_then_gemm(d["x3"], d["wq3_tl"], d["ws3"], d["fp_bufs"]), 10)
        q3, s3, _ = fp8.quant_act_1x128(d["x3"], "row")
        y3 = d["fp_bufs"][2]
        batch["fprop.gemm"] = batch_ms(lambda: fp8.block_gemm("fprop_tiled", q3, s3, d["wq3_tl"], d["ws3"],
                                                              out=y3), 5)
        # context for the roofline: the GEMM's MFMA alone in a loop, on the
        # bench's own operand bytes (2 KB of weight codes, 2 KB of X codes),
        # one workgroup of four waves per CU as in the GEMM
        codes = torch.cat([d["wq3_tl"].reshape(-1)[:2048], q3.reshape(-1)[:2048]]).contiguous()
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        iters = 20000
        probe = {"what": f"{n_cu} workgroups x 4 waves x 8 x {iters} FP8 16x16x128 MFMAs, no memory "
                         "traffic, operands from the bench's weight and X codes; plain = the GEMMs' "
                         "v_mfma_f32_16x16x128_f8f6f4, scaled = its block-scaled encoding, fold = plain "
                         "+ the 4 FP32 fold FMAs per MFMA (the GEMMs' per-block mix)"}
        for mode in ("plain", "scaled", "fold"):
            t_probe = batch_ms(lambda: fp8.probe_mfma(codes, n_cu, iters, mode), 5)
            probe[mode] = {"TFLOP/s": n_cu * 4 * 8 * iters * 65536.0 / t_probe / 1e9, "ms": t_probe}
        probe["TFLOP/s"] = probe["fold"]["TFLOP/s"]
    log("batches: " + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in batch.items()))
    log(f"timed {args.steps} steps: {steps_ms:.2f} ms on the GPU, {wall:.2f} s wall")

    rows = {}
    QB = 8192 * 7168 * (2 + 1) + (7168 // 128) * 8192 * 4
    if want("quantizer"):
        B = 8192 * 7168 * (2 + 1) + (7168 // 128) * 8192 * 4
        t = tm.mean_ms("quantizer")
        rows["quantizer"] = {"ms": t, "GB/s": B / t / 1e6, "bytes": B,
                             "hbm_frac": B / t / 1e6 / PEAK_HBM_GBPS}
    F3 = 2.0 * 4096 * 18432 * 7168
    value = None
    roofline = None
    if want("fprop"):
        tq, tg, tt = tm.mean_ms("fprop.quant"), tm.mean_ms("fprop.gemm"), tm.mean_ms("fprop")
        # the headline: 2MNK over the timed region (quantization + GEMM back
        # to back on one stream; its two parts add up to it exactly)
        value = F3 / tt / 1e9
        trm = tm.mean_ms("fprop_rowmajor.gemm")
        rows["fprop"] = {"ms_quant": tq, "ms_gemm": tg, "ms_region": tt,
                         "TFLOP/s_incl_quant": value, "TFLOP/s_gemm": F3 / tg / 1e9,
                         "what": "1x128 quantization kernel then the GEMM kernel, back to back on one stream "
                                 "(the unfused pair; the fused kernel is the row fprop_fused_quant)",
                         "ms_pair_back_to_back": batch["fprop.pair"],
                         "TFLOP/s_pair_back_to_back": F3 / batch["fprop.pair"] / 1e9,
                         "quant_GB/s": 4096 * 7168 * (3 + 4 / 128) / tq / 1e6,
                         "weights": "operand-tiled codes",
                         "ms_gemm_rowmajor_weights": trm, "TFLOP/s_gemm_rowmajor_weights": F3 / trm / 1e9,
                         "ms_gemm_median_p10_p90": tm.spread_ms("fprop.gemm"),
                         "ms_quant_plus_gemm_median_p10_p90": tm.spread_ms("fprop")}
        tf = tm.mean_ms("fprop_fused.gemm")
        rows["fprop_fused_quant"] = {
            "ms": tf, "TFLOP/s": F3 / tf / 1e9,
            "what": "BF16 X in, 1x128 quantization fused into a 128x128-tile GEMM (row-major weight codes)",
            "unfused_ms_quant_plus_gemm_rowmajor": tq + trm, "unfused_ms_quant_plus_gemm_tiled": tq + tg,
            "fused_over_unfused_tiled": tf / (tq + tg)}
        # the kernel's mean launch duration over the timed steps (HIP events
        # around each launch on its stream); the back-to-back batch after the
        # steps runs under sustained power and is reported beside it
        achieved = F3 / tg / 1e9
        traffic = traffic_from_profiles("fprop_gemm_traffic.json", "fine_grained_fp8_amd/csrc/gemm.hip")
        roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / PEAK_FP8_TFLOPS, "traffic": traffic,
                    "kernel": "block_gemm_direct_kernel<FPROP,bf16,tiled weights> 4096x18432x7168",
                    "algorithmic_flop_per_launch": F3, "ms_per_launch": tg,
                    "timing": f"mean over the {args.steps} timed steps, HIP events around each launch on the launch stream",
                    "ms_per_launch_back_to_back": batch["fprop.gemm"],
                    "TFLOP/s_back_to_back": F3 / batch["fprop.gemm"] / 1e9,
                    "mfma_loop": probe,
                    "frac_of_mfma_loop": achieved / probe["TFLOP/s"] if probe else None}
    if want("toy"):
        F1 = 2.0 * 128 * 256 * 128
        rows["toy"] = {"what": "toy layer y = W x: 1x128 quantization of X 128x128, then the GEMM against "
                               "W 256x128 (pre-quantized, operand-tiled codes), BF16 out",
                       "us_region": tm.mean_ms("toy") * 1e3, "us_quant": tm.mean_ms("toy.quant") * 1e3,
                       "us_gemm": tm.mean_ms("toy.gemm") * 1e3,
                       "us_pair_back_to_back": batch["toy.pair"] * 1e3,
                       "region_median_p10_p90_us": [v * 1e3 for v in tm.spread_ms("toy")],
                       "flop": F1}
    if want("backward"):
        tdual, tg1 = tm.mean_ms("bwd.quant_dual"), tm.mean_ms("dgrad.gemm")
        tq3, tg2 = tm.mean_ms("wgrad.quant_x"), tm.mean_ms("wgrad.gemm")
        trow, tcol = tm.mean_ms("bwd.quant_row"), tm.mean_ms("bwd.quant_col")
        EL = 4096 * 18432
        tcd = tm.mean_ms("ref.copy_dy")
        rows["dual_quant"] = {"ms": tdual, "GB/s": EL * (2 + 2 + 8 / 128) / tdual / 1e6,
                              "ms_separate_row_plus_col": trow + tcol,
                              "GB/s_separate": EL * 2 * (3 + 4 / 128) / (trow + tcol) / 1e6,
                              "speedup_vs_separate": (trow + tcol) / tdual,
                              "ms_same_traffic_copy": tcd, "frac_of_same_traffic_copy": tcd / tdual}
        tdx = tm.mean_ms("fwd.quant_dual_x")
        tsx = tm.mean_ms("fwd.quant_row_x") + tm.mean_ms("wgrad.quant_x")
        EX = 4096 * 7168
        tcx = tm.mean_ms("ref.copy_x")
        rows["dual_quant_x"] = {"ms": tdx, "GB/s": EX * (2 + 2 + 8 / 128) / tdx / 1e6,
                                "ms_separate_row_plus_col": tsx, "speedup_vs_separate": tsx / tdx,
                                "ms_same_traffic_copy": tcx, "frac_of_same_traffic_copy": tcx / tdx}
        # each GEMM is charged the share of the dual pass its operand costs
        tq1 = tq2 = tdual / 2
        tdr = tm.mean_ms("dgrad_rowmajor.gemm")
        rows["dgrad"] = {"ms_quant_share": tq1, "ms_gemm": tg1, "TFLOP/s_incl_quant": F3 / (tq1 + tg1) / 1e9,
                         "TFLOP/s_gemm": F3 / tg1 / 1e9, "layout": "dgrad_t_tiled (W_q^T, operand-tiled)",
                         "ms_gemm_rowmajor_weights": tdr, "TFLOP/s_gemm_rowmajor_weights": F3 / tdr / 1e9}
        tl = tm.mean_ms("dgrad_lds.gemm")
        rows["dgrad_lds"] = {"ms_gemm": tl, "TFLOP/s_gemm": F3 / tl / 1e9, "layout": "dgrad (W_q read transposed)"}
        twr = tm.mean_ms("wgrad_rowmajor.gemm")
        rows["wgrad"] = {"ms_quant_dy_share": tq2, "ms_quant_x_col": tq3, "ms_gemm": tg2,
                         "TFLOP/s_incl_quant": F3 / (tq2 + tq3 + tg2) / 1e9, "TFLOP/s_gemm": F3 / tg2 / 1e9,
                         "layout": "wgrad_tiled (X_q^T operand-tiled)",
                         "ms_gemm_rowmajor": twr, "TFLOP/s_gemm_rowmajor": F3 / twr / 1e9,
                         "col_quant_x_GB/s": 4096 * 7168 * (3 + 4 / 128) / tq3 / 1e6}
    if want("grouped"):
        F5 = 2.0 * 16384 * 2048 * 7168
        tq, tg = tm.mean_ms("grouped.quant"), tm.mean_ms("grouped.gemm")
        tgr = tm.mean_ms("grouped_rowmajor.gemm")
        rows["grouped"] = {"ms_quant": tq, "ms_gemm": tg, "ms_region": tm.mean_ms("grouped"),
                           "TFLOP/s_incl_quant": F5 / tm.mean_ms("grouped") / 1e9,
                           "TFLOP/s_gemm": F5 / tg / 1e9, "tokens_per_expert": [int(c) for c in d["counts5"]],
                           "weights": "operand-tiled codes",
                           "ms_gemm_rowmajor_weights": tgr, "TFLOP/s_gemm_rowmajor_weights": F5 / tgr / 1e9}
    if want("weights"):
        B = 18432 * 7168 * 4 + (18432 // 128) * (7168 // 128) * 4
        t = tm.mean_ms("weights")
        rows["weights"] = {"ms": t, "GB/s": B / t / 1e6}
    if want("granularity"):
        EL = 8192 * 7168
        g = {}
        for T in (32, 64, 128, 256, 512, 1024):
            t = tm.mean_ms(f"tiles.{T}")
            g[f"T{T}"] = {"ms": t, "GB/s": EL * (3 + 4 / T) / t / 1e6, "scale_bytes_per_value": 4 / T}
        t = tm.mean_ms("tiles.128.rank2")
        g["T128_rank2"] = {"ms": t, "GB/s": EL * (3 + 4 / 128) / t / 1e6}
        rows["granularity"] = g
    if want("payload"):
        n_msg, MB = 8192, 7392
        tp, tu, tdq = tm.mean_ms("payload.pack"), tm.mean_ms("payload.unpack"), tm.mean_ms("payload.dequant")
        rows["payload"] = {"messages": n_msg, "message_bytes": MB,
                           "ms_pack": tp, "GB/s_pack": n_msg * (2 * 7168 + MB) / tp / 1e6,
                           "ms_unpack": tu, "GB/s_unpack": n_msg * 2 * MB / tu / 1e6,
                           "ms_dequant": tdq, "GB/s_dequant": n_msg * (MB + 2 * 7168) / tdq / 1e6}
    if want("policy"):
        rows["policy"] = {"ms": tm.mean_ms("policy")}
    if want("copy"):
        t = tm.mean_ms("copy")
        rows["copy"] = {"ms": t, "GB/s": 2.0 * (1 << 30) / t / 1e6, "bytes": 2 * (1 << 30)}

    cpu = None
    if not args.no_cpu_baseline and want("fprop"):
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(host["x3"], host["w3"], args.cpu_sample_rows)
        if cpu_pool:
            cpu.update(cpu_pool)

    if value is None and "quantizer" in rows:
        value = rows["quantizer"]["GB/s"]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s" if want("fprop") else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": steps_ms / args.steps,
        "wall_s": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "fprop: 1x128 quant of X 4096x7168 + block-scaled FP8 GEMM "
                               "Y=X W^T 4096x18432x7168, BF16 out (W pre-quantized 128x128, "
                               "operand-tiled codes)",
                   "M": 4096, "N": 18432, "K": 7168},
        "roofline": roofline,
        "roofline_quantizer": ({"bound": "hbm", "achieved": QB / batch["quantizer"] / 1e6, "peak": PEAK_HBM_GBPS,
                                "unit": "GB/s", "frac": QB / batch["quantizer"] / 1e6 / PEAK_HBM_GBPS,
                                "ms_per_launch": batch["quantizer"],
                                "timing": "20 back-to-back launches over 4 rotated inputs, HIP events",
                                "algorithmic_bytes_per_launch": QB,
                                "traffic": traffic_from_profiles("quant_rows_traffic.json",
                                                                 "fine_grained_fp8_amd/csrc/quant.hip"),
                                "kernel": "quant_rows_kernel<online> 8192x7168"}
                               if "quantizer" in rows else None),
        "cpu_baseline": cpu,
        "device": device_info(),
        "rows": rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
