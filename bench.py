#!/usr/bin/env python3
"""Benchmark of the dense matrix-unit GEMM path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs all|headline|name,...]

Headline (the JSON line's `value`): gemm_bf16 at M = N = K = 4096, A row-major,
B stored N x K, BF16 output, inputs N(0,1) rounded to BF16, in TFLOP/s.  A
"step" is one launch of that GEMM; K back-to-back steps are timed between two
device synchronisations, with one pair of HIP events around them on the
stream they run on.  Before the timed region the headline kernel is timed
with the protocol of the vidyal.ai page, Step 2 (protocol_rounds): a warm-up,
three rounds of back-to-back launches, the median of the last three quarters
of each, the rounds' agreement, and clocks and power polled during those
launches; the roofline object's per-kernel rate comes from it, and the
timed region then runs at the GPU's steady clocks.  The FP8 E4M3 4096^3
kernel, the metric's other half, gets the same protocol in its leg.  The other workloads (B row-major, FP8 per-tensor E4M3/E5M2, the
block-scaled 8192x7168x7168 GEMM and its quantizers, the LLM-shaped sweep,
256^3) are timed the same way in the same process and reported under "legs",
with "mfma_ceiling": the sustained matrix-unit rate with no memory traffic,
for N(0,1) and for constant operands.  "bf16_4096_operand_data" (run only
when named in --legs) times the headline kernel itself on N(0,1), all-ones
and all-zero operands.

Operands are resident in HBM before timing starts.  The 4096^3 legs rotate
over several operand copies whose total exceeds the 256 MB Infinity Cache, so
successive launches do not find their operands in the last-level cache.

`cpu_baseline` times the CPU oracle (FP64, all host threads) on a bounded
sample of the headline workload: blocks of 256 output rows until 10 s have
passed or the whole product is done.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk x 2.4 GHz (published 2.5 PFLOP/s dense)
PEAK_FP8_TFLOPS = 5033.2   # 256 CU x 8192 FLOP/clk x 2.4 GHz (published 5.0 PFLOP/s dense)
PEAK_FP4_TFLOPS = 10066.3  # 256 CU x 16384 FLOP/clk x 2.4 GHz (published 10.1 PFLOP/s dense)
PEAK_HBM_GBS = 8000.0
METRIC = "GEMM TFLOP/s and % of MFMA peak, 4096³ BF16 and FP8 E4M3, 1×MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["dense_matrix_unit_amd/csrc/gemm.hip", "dense_matrix_unit_amd/csrc/gemm_common.h",
                  "dense_matrix_unit_amd/csrc/dmu_device.h"]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def time_launches(torch, launch, steps, warmup):
    """Run `launch(i)` warmup times, then time `steps` back-to-back launches
    between two synchronisations.  Returns the wall-clock time per launch and
    the GPU time per launch from one pair of HIP events around the timed
    launches (on their stream).  No event sits between two launches: each
    recorded event puts a gap of several microseconds between the kernels
    around it (4096^3 BF16: 110 us per launch with an event pair around each,
    102 us without)."""
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for i in range(steps):
        launch(i)
    b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return {"wall_ms": (t1 - t0) * 1e3 / steps, "event_mean_ms": a.elapsed_time(b) / steps}


class ClockSampler:
    """Shader clock and socket power polled every ~100 ms by a thread that
    runs amd-smi (a child process), for as long as the sampler is open.
    Samples carry their host time, so they can be matched to the rounds they
    fell in.  Inactive (no samples) when amd-smi is missing or the process
    runs under rocprofv3, whose preloaded library keeps amd-smi from
    starting."""

    def __init__(self):
        import shutil

        self.smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
        self.active = os.path.exists(self.smi) and not (
            "rocprof" in os.environ.get("LD_PRELOAD", "") or
            any(k.startswith("ROCPROF") for k in os.environ))
        self.samples = []
        self._stop = None
        self._th = None

    @staticmethod
    def _num(x):
        v = x.get("value") if isinstance(x, dict) else x
        return float(v) if isinstance(v, (int, float)) else None

    def _poll(self):
        import subprocess

        while not self._stop.is_set():
            try:
                r = subprocess.run([self.smi, "metric", "-g", "0", "-c", "-p", "--json"],
                                   capture_output=True, text=True, timeout=5)
                d = json.loads(r.stdout)["gpu_data"][0]
                clks = [self._num(v.get("clk")) for k, v in d["clock"].items()
                        if k.startswith("gfx_") and isinstance(v, dict)]
                clks = [c for c in clks if c]
                pw = self._num(d["power"]["socket_power"])
                if clks and pw:
                    # the clock is the median over the 8 XCDs of one sample
                    self.samples.append((time.perf_counter(), statistics.median(clks), pw))
            except Exception:  # a sample that fails to parse is skipped
                pass
            self._stop.wait(0.1)

    def __enter__(self):
        import threading

        if self.active:
            self._stop = threading.Event()
            self._th = threading.Thread(target=self._poll, daemon=True)
            self._th.start()
        return self

    def __exit__(self, *exc):
        if self._th is not None:
            self._stop.set()
            self._th.join(timeout=10)

    def between(self, t0, t1):
        return [(c, w) for ts, c, w in self.samples if t0 <= ts <= t1]


def protocol_rounds(torch, launch, flop, peak, rounds=3, seconds=1.0, warm_s=0.5, batch=10):
    """The timing protocol of the vidyal.ai page, Step 2: a warm-up of
    `warm_s` seconds of back-to-back launches, then `rounds` rounds of
    `seconds` each; each round keeps the median of the last three quarters of
    its timings, the rounds must agree within 2%, and clocks and power are
    polled every ~100 ms while the rounds run.  Throughput and clock come from
    the same launches.  The page brackets every launch with events; here one
    event pair brackets each batch of `batch` back-to-back launches, because
    on this runtime an event between two kernels adds a gap of several
    microseconds to the timeline (and ~2% to the bracketed kernel)."""
    i = 0
    with ClockSampler() as smp:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            for _ in range(20):
                launch(i)
                i += 1
            torch.cuda.synchronize()
        out = []
        for _ in range(rounds):
            marks = []
            torch.cuda.synchronize()
            ts = time.perf_counter()
            while time.perf_counter() - ts < seconds:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(batch):
                    launch(i)
                    i += 1
                b.record()
                marks.append((a, b))
            torch.cuda.synchronize()
            te = time.perf_counter()
            d = [x.elapsed_time(y) / batch for x, y in marks]
            med = statistics.median(d[len(d) // 4:])
            clk = smp.between(ts, te)
            out.append({"median_ms": round(med, 5), "TFLOP_per_s": round(flop / med / 1e9, 1),
                        "launches": len(d) * batch,
                        "sclk_mhz_median": statistics.median(c for c, _ in clk) if clk else None,
                        "socket_power_w_median": (statistics.median(w for _, w in clk)
                                                  if clk else None),
                        "clock_samples": len(clk)})
    meds = [r["median_ms"] for r in out]
    ms = statistics.median(meds)
    spread = (max(meds) - min(meds)) / ms
    clk_all = [r["sclk_mhz_median"] for r in out if r["sclk_mhz_median"]]
    sclk = statistics.median(clk_all) if clk_all else None
    tf = flop / ms / 1e9
    return {"ms": round(ms, 5), "TFLOP_per_s": round(tf, 1), "pct_peak": round(100 * tf / peak, 1),
            "rounds": out, "spread": round(spread, 4), "rounds_agree_within_2pct": spread <= 0.02,
            "sclk_mhz_median": sclk,
            "pct_peak_at_measured_sclk": (round(100 * tf / (peak * sclk / 2400.0), 1)
                                          if sclk else None),
            "statistic": "median over %d rounds of each round's median of the last 75%% of "
                         "per-launch times from HIP events around batches of %d back-to-back "
                         "launches; %.1f s warm-up, %.1f s rounds, clocks and power polled "
                         "during the rounds" % (rounds, batch, warm_s, seconds)}


class Bench:
    def __init__(self, args):
        import torch

        import dense_matrix_unit_amd as dmu
        from dense_matrix_unit_amd import workloads as wl

        self.torch, self.dmu, self.wl, self.args = torch, dmu, wl, args
        dmu.load_library()  # raises if the HIP library is not built
        self.dev = torch.device("cuda:0")

    # ---- input helpers (harness step: FP32 sources -> BF16, untimed)
    def normal_bf16(self, shape, seed):
        t = self.torch.from_numpy(self.wl.normal(shape, seed)).to(self.dev)
        return t.to(self.torch.bfloat16)

    def normal_f32(self, shape, seed):
        return self.torch.from_numpy(self.wl.normal(shape, seed)).to(self.dev)

    def copies(self, t, n):
        return [t] + [t.clone() for _ in range(n - 1)]

    # ---- legs
    def gemm_bf16_leg(self, M, N, K, layout, steps, warmup, copies=1, out_f32=False,
                      seed_dist="normal", B=None, protocol=False, protocol_seconds=1.0):
        torch, dmu = self.torch, self.dmu
        bshape = (N, K) if layout == dmu.B_COL_MAJOR else (K, N)
        if seed_dist == "uniform":
            A = torch.from_numpy(self.wl.uniform_pm1((M, K), 1)).to(self.dev).to(torch.bfloat16)
            B = torch.from_numpy(self.wl.uniform_pm1(bshape, 2)).to(self.dev).to(torch.bfloat16)
        else:
            A = self.normal_bf16((M, K), 1)
            if B is None:
                B = self.normal_bf16(bshape, 2)
        As, Bs = self.copies(A, copies), self.copies(B, copies)
        outs = [torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16,
                            device=self.dev) for _ in range(min(copies, 2))]

        def launch(i):
            dmu.gemm_bf16(As[i % copies], Bs[i % copies], outs[i % len(outs)], layout)

        t = time_launches(torch, launch, steps, warmup)
        flop = 2.0 * M * N * K
        bytes_ = 2.0 * (M * K + N * K) + (4.0 if out_f32 else 2.0) * M * N
        r = self.report(t, flop, bytes_, PEAK_BF16_TFLOPS, copies)
        if protocol:
            r["protocol"] = protocol_rounds(torch, launch, flop, PEAK_BF16_TFLOPS,
                                            seconds=protocol_seconds)
        return r

    def fp8_operands(self, M, N, K, fmt, block=None):
        torch, dmu = self.torch, self.dmu
        if block:
            Xa, _ = self.wl.normal_with_outlier_rows((M, K), 1)
            Xa = torch.from_numpy(Xa).to(self.dev)
        else:
            Xa = self.normal_f32((M, K), 1)
        Xb = self.normal_f32((N, K), 2)
        Qa = torch.empty((M, K), dtype=torch.uint8, device=self.dev)
        Qb = torch.empty((N, K), dtype=torch.uint8, device=self.dev)
        if block:
            sa = torch.empty((M, K // 128), dtype=torch.float32, device=self.dev)
            sb = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=self.dev)
            dmu.quantize_fp8(Xa, Qa, sa, fmt, (1, 128))
            dmu.quantize_fp8(Xb, Qb, sb, fmt, (128, 128))
        else:
            sa = torch.empty(1, dtype=torch.float32, device=self.dev)
            sb = torch.empty(1, dtype=torch.float32, device=self.dev)
            dmu.quantize_fp8(Xa, Qa, sa, fmt)
            dmu.quantize_fp8(Xb, Qb, sb, fmt)
        return Xa, Xb, Qa, Qb, sa, sb

    def gemm_fp8_leg(self, M, N, K, fmt, steps, warmup, copies=1, block=False, promoted=False,
                     protocol=False, protocol_seconds=1.0):
        """promoted: per-tensor operands run through the block-scaled path with
        every scale equal, i.e. partial sums promoted into FP32 every 128 K.
        protocol: also time the kernel with protocol_rounds."""
        torch, dmu = self.torch, self.dmu
        Xa, Xb, Qa, Qb, sa, sb = self.fp8_operands(M, N, K, fmt, block)
        del Xa, Xb
        if promoted:
            sa = sa.reshape(1, 1).expand(M, K // 128).contiguous()
            sb = sb.reshape(1, 1).expand((N + 127) // 128, K // 128).contiguous()
            block = True
        Qas, Qbs = self.copies(Qa, copies), self.copies(Qb, copies)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=self.dev)
        mode = dmu.SCALE_BLOCK if block else dmu.SCALE_TENSOR

        def launch(i):
            dmu.gemm_fp8_scaled(Qas[i % copies], Qbs[i % copies], sa, sb, out, fmt, fmt, mode)

        t = time_launches(torch, launch, steps, warmup)
        flop = 2.0 * M * N * K
        bytes_ = 1.0 * (M * K + N * K) + 2.0 * M * N + 4.0 * (sa.numel() + sb.numel())
        r = self.report(t, flop, bytes_, PEAK_FP8_TFLOPS, copies)
        if protocol:
            r["protocol"] = protocol_rounds(torch, launch, flop, PEAK_FP8_TFLOPS,
                                            seconds=protocol_seconds)
        return r

    def fused_leg(self, kind, steps, warmup, copies):
        """4096^3 with the fused epilogue: "bf16_gelu" (BF16 in, + bias, GELU,
        BF16 out) or "fp8_relu_fp8out" (per-tensor E4M3 in, + bias, ReLU, E4M3
        out with a static scale)."""
        torch, dmu = self.torch, self.dmu
        M = N = K = 4096
        bias = self.normal_f32((N,), 3)
        if kind == "bf16_gelu":
            As = self.copies(self.normal_bf16((M, K), 1), copies)
            Bs = self.copies(self.normal_bf16((N, K), 2), copies)
            out = torch.empty((M, N), dtype=torch.bfloat16, device=self.dev)

            def launch(i):
                dmu.gemm_bf16_fused(As[i % copies], Bs[i % copies], out, dmu.B_COL_MAJOR, bias,
                                    dmu.ACT_GELU)
            peak, ab = PEAK_BF16_TFLOPS, 2.0
        else:
            Xa, Xb, Qa, Qb, sa, sb = self.fp8_operands(M, N, K, dmu.E4M3)
            del Xa, Xb
            Qas, Qbs = self.copies(Qa, copies), self.copies(Qb, copies)
            out = torch.empty((M, N), dtype=torch.uint8, device=self.dev)
            ds = torch.full((1,), 0.25, dtype=torch.float32, device=self.dev)

            def launch(i):
                dmu.gemm_fp8_fused(Qas[i % copies], Qbs[i % copies], sa, sb, out, dmu.E4M3,
                                   dmu.E4M3, bias, dmu.ACT_RELU, dmu.E4M3, ds)
            peak, ab = PEAK_FP8_TFLOPS, 1.0
        t = time_launches(torch, launch, steps, warmup)
        flop = 2.0 * M * N * K
        bytes_ = ab * (M * K + N * K) + (2.0 if kind == "bf16_gelu" else 1.0) * M * N + 4.0 * N
        return self.report(t, flop, bytes_, peak, copies)

    def attention_leg(self, causal, steps, warmup):
        """The attention chain: 32 heads (batch 2 x 16), 4096 queries and keys,
        d = 128, N(0,1) BF16 Q, K, V, scale 1/sqrt(d), with and without the
        causal mask.  FLOP: the two products over the keys each row sees,
        4 d per (row, key) pair."""
        torch, dmu = self.torch, self.dmu
        w = self.wl.WORKLOADS["attention_bf16_32x4096x4096x128"]
        H, S, d = w["heads"], w["S"], w["d"]
        Q = self.normal_bf16((H * S, d), 1).view(H, S, d)
        K = self.normal_bf16((H * S, d), 2).view(H, S, d)
        V = self.normal_bf16((H * S, d), 3).view(H, S, d)
        O = torch.empty_like(Q)
        scale = d ** -0.5

        def launch(i):
            dmu.attention_bf16(Q, K, V, O, scale, causal)

        t = time_launches(torch, launch, steps, warmup)
        pairs = S * (S + 1) / 2 if causal else S * S
        flop = 4.0 * d * H * pairs
        bytes_ = 2.0 * 4 * H * S * d
        r = self.report(t, flop, bytes_, PEAK_BF16_TFLOPS, 1)
        r["heads"], r["seq"], r["head_dim"], r["causal"] = H, S, d, bool(causal)
        return r

    def grouped_leg(self, steps, warmup):
        """Mixture-of-experts grouped BF16 product: 32 experts, 16384 routed
        rows split by expert_rows (seed 4), N = 4096, K = 7168; the row offsets
        are a device array, as routing leaves them."""
        torch, dmu = self.torch, self.dmu
        w = self.wl.WORKLOADS["moe_bf16_32x16384x4096x7168"]
        G, N, K, T = w["G"], w["N"], w["K"], w["total_rows"]
        counts = self.wl.expert_rows(G, T, self.wl.SEED_ROUTING)
        offs = torch.zeros(G + 1, dtype=torch.int64, device=self.dev)
        offs[1:] = torch.cumsum(torch.from_numpy(counts).to(self.dev), 0)
        A = self.normal_bf16((T, K), 1)
        B = self.normal_bf16((G * N, K), 2).view(G, N, K)
        out = torch.empty((T, N), dtype=torch.bfloat16, device=self.dev)

        def launch(i):
            dmu.gemm_grouped_bf16(A, B, offs, out)

        t = time_launches(torch, launch, steps, warmup)
        flop = 2.0 * T * N * K
        bytes_ = 2.0 * (T * K + G * N * K + T * N)
        r = self.report(t, flop, bytes_, PEAK_BF16_TFLOPS, 1)
        r["experts"] = G
        r["rows_per_expert_min_max"] = [int(counts.min()), int(counts.max())]
        return r

    def gemm_mx_leg(self, M, N, K, fmt, steps, warmup, copies=1):
        """Microscaled FP8: operands quantized by quantize_mxfp8 (one E8M0
        scale per row and 32 K), product by gemm_mxfp8."""
        torch, dmu = self.torch, self.dmu
        Qa = torch.empty((M, K), dtype=torch.uint8, device=self.dev)
        Qb = torch.empty((N, K), dtype=torch.uint8, device=self.dev)
        Sa = torch.empty((M, K // 32), dtype=torch.uint8, device=self.dev)
        Sb = torch.empty((N, K // 32), dtype=torch.uint8, device=self.dev)
        dmu.quantize_mxfp8(self.normal_f32((M, K), 1), Qa, Sa, fmt)
        dmu.quantize_mxfp8(self.normal_f32((N, K), 2), Qb, Sb, fmt)
        Qas, Qbs = self.copies(Qa, copies), self.copies(Qb, copies)
        Sas, Sbs = self.copies(Sa, copies), self.copies(Sb, copies)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=self.dev)

        def launch(i):
            j = i % copies
            dmu.gemm_mxfp8(Qas[j], Qbs[j], Sas[j], Sbs[j], out, fmt, fmt)

        t = time_launches(torch, launch, steps, warmup)
        flop = 2.0 * M * N * K
        bytes_ = (1.0 + 1.0 / 32) * (M * K + N * K) + 2.0 * M * N
        return self.report(t, flop, bytes_, PEAK_FP8_TFLOPS, copies)

    def gemm_mxfp4_leg(self, M, N, K, steps, warmup, copies=1):
        """Microscaled FP4: operands quantized by quantize_mxfp4, product by
        gemm_mxfp4."""
        torch, dmu = self.torch, self.dmu
        Qa = torch.empty((M, K // 2), dtype=torch.uint8, device=self.dev)
        Qb = torch.empty((N, K // 2), dtype=torch.uint8, device=self.dev)
        Sa = torch.empty((M, K // 32), dtype=torch.uint8, device=self.dev)
        Sb = torch.empty((N, K // 32), dtype=torch.uint8, device=self.dev)
        dmu.quantize_mxfp4(self.normal_f32((M, K), 1), Qa, Sa)
        dmu.quantize_mxfp4(self.normal_f32((N, K), 2), Qb, Sb)
        Qas, Qbs = self.copies(Qa, copies), self.copies(Qb, copies)
        Sas, Sbs = self.copies(Sa, copies), self.copies(Sb, copies)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=self.dev)

        def launch(i):
            j = i % copies
            dmu.gemm_mxfp4(Qas[j], Qbs[j], Sas[j], Sbs[j], out)

        t = time_launches(torch, launch, steps, warmup)
        flop = 2.0 * M * N * K
        bytes_ = (0.5 + 1.0 / 32) * (M * K + N * K) + 2.0 * M * N
        return self.report(t, flop, bytes_, PEAK_FP4_TFLOPS, copies)

    def quantize_mx_leg(self, rows, cols, fmt, steps, warmup):
        torch, dmu = self.torch, self.dmu
        X = self.normal_f32((rows, cols), 1)
        fp4 = fmt == dmu.E2M1
        Q = torch.empty((rows, cols // 2 if fp4 else cols), dtype=torch.uint8, device=self.dev)
        S = torch.empty((rows, cols // 32), dtype=torch.uint8, device=self.dev)
        copies = max(1, -(-320 * 2 ** 20 // (4 * rows * cols)))  # beyond the Infinity Cache
        Xs = self.copies(X, copies)

        def launch(i):
            if fp4:
                dmu.quantize_mxfp4(Xs[i % copies], Q, S)
            else:
                dmu.quantize_mxfp8(Xs[i % copies], Q, S, fmt)

        t = time_launches(torch, launch, steps, warmup)
        bytes_ = ((4.5 if fp4 else 5.0) + 1.0 / 32) * rows * cols
        ms = t["event_mean_ms"]
        return {"ms": round(ms, 5), "GB_per_s": round(bytes_ / ms / 1e6, 1),
                "pct_hbm_peak": round(100 * bytes_ / ms / 1e6 / PEAK_HBM_GBS, 1),
                "algorithmic_MB": round(bytes_ / 1e6, 2), "wall_ms": round(t["wall_ms"], 5),
                "input_copies": copies}

    def quantize_leg(self, rows, cols, fmt, block, steps, warmup, outliers=False, noalloc=False):
        torch, dmu = self.torch, self.dmu
        quantize = dmu.quantize_fp8_noalloc if noalloc else dmu.quantize_fp8
        if outliers:
            X, _ = self.wl.normal_with_outlier_rows((rows, cols), 1)
            X = torch.from_numpy(X).to(self.dev)
        else:
            X = self.normal_f32((rows, cols), 1)
        Q = torch.empty((rows, cols), dtype=torch.uint8, device=self.dev)
        br, bc = (rows, cols) if block is None else block
        s = torch.empty(((rows // br) * (cols // bc),), dtype=torch.float32, device=self.dev)
        # rotate over input copies larger than the 256 MB Infinity Cache, so a
        # call does not find the previous calls' input there
        copies = max(1, -(-320 * 2 ** 20 // (4 * rows * cols)))
        Xs = self.copies(X, copies)

        def launch(i):
            quantize(Xs[i % copies], Q, s, fmt, block)

        t = time_launches(torch, launch, steps, warmup)
        bytes_ = 5.0 * rows * cols + 4.0 * s.numel()
        ms = t["event_mean_ms"]
        return {"ms": round(ms, 5), "GB_per_s": round(bytes_ / ms / 1e6, 1),
                "pct_hbm_peak": round(100 * bytes_ / ms / 1e6 / PEAK_HBM_GBS, 1),
                "algorithmic_MB": round(bytes_ / 1e6, 2), "wall_ms": round(t["wall_ms"], 5),
                "input_copies": copies}

    def mfma_ceiling_leg(self, steps, warmup):
        """Sustained MFMA rate with no memory traffic (dmu_probe_mfma_rate): the
        ceiling the GEMM K loops can reach, for N(0,1) operands and for constant
        ones (the power drawn depends on the operand bits)."""
        torch, dmu = self.torch, self.dmu
        res = {}
        grid = 1024
        for name, kind, iters, peak in (("bf16", dmu.PROBE_BF16_32X32X16, 2048, PEAK_BF16_TFLOPS),
                                        ("fp8_e4m3", dmu.PROBE_FP8_32X32X64, 1024,
                                         PEAK_FP8_TFLOPS),
                                        ("mxfp8_e4m3", dmu.PROBE_MXFP8_32X32X64, 1024,
                                         PEAK_FP8_TFLOPS),
                                        ("mxfp4_e2m1", dmu.PROBE_MXFP4_32X32X64, 2048,
                                         PEAK_FP4_TFLOPS)):
            fb = 16 if name == "bf16" else 32
            n = 8 * 64 * fb
            if name == "bf16":
                rnd = self.normal_bf16((n // 2,), 1).view(torch.uint8)
                ones = torch.full((n // 2,), 1.0, dtype=torch.bfloat16, device=self.dev)
                ones = ones.view(torch.uint8)
            else:
                q = torch.empty((n,), dtype=torch.uint8, device=self.dev)
                sc = torch.empty(1, dtype=torch.float32, device=self.dev)
                dmu.quantize_fp8(self.normal_f32((1, n), 1), q.view(1, n), sc, dmu.E4M3)
                one = 0x22 if name == "mxfp4_e2m1" else 0x38  # E2M1 1.0 twice / E4M3 1.0
                rnd, ones = q, torch.full((n,), one, dtype=torch.uint8, device=self.dev)
            out = torch.empty(grid * 256, dtype=torch.float32, device=self.dev)
            flop = 2.0 * grid * 4 * 16 * iters * (32 * 32 * (16 if name == "bf16" else 64))
            for dist, src in (("normal", rnd), ("ones", ones)):
                t = time_launches(torch, lambda i: dmu.probe_mfma_rate(kind, src, iters, grid, out),
                                  steps, warmup)
                tf = flop / t["event_mean_ms"] / 1e9
                res["%s_%s" % (name, dist)] = {"TFLOP_per_s": round(tf, 1),
                                               "pct_peak": round(100 * tf / peak, 1),
                                               "ms": round(t["event_mean_ms"], 4)}
        return res

    @staticmethod
    def report(t, flop, bytes_, peak, copies):
        ms = t["event_mean_ms"]
        tf = flop / ms / 1e9
        return {"ms": round(ms, 5), "wall_ms": round(t["wall_ms"], 5), "TFLOP_per_s": round(tf, 1),
                "pct_peak": round(100 * tf / peak, 1),
                "GB_per_s_algorithmic": round(bytes_ / ms / 1e6, 1),
                "operand_copies": copies}


def cpu_baseline(A_bf16, B_bf16, budget_s=10.0):
    """Time the CPU oracle on 256-row blocks of the headline GEMM."""
    import numpy as np

    import oracle

    import torch

    A = A_bf16.cpu().view(torch.int16).numpy().view(np.uint16)
    B = B_bf16.cpu().view(torch.int16).numpy().view(np.uint16)
    M, K = A.shape
    N = B.shape[0]
    done, t0 = 0, time.perf_counter()
    while done < M and time.perf_counter() - t0 < budget_s:
        oracle.gemm_bf16(A, B, oracle.B_COL_MAJOR, rows=np.arange(done, min(M, done + 256)))
        done = min(M, done + 256)
    dt = time.perf_counter() - t0
    return {"value": round(2.0 * done * N * K / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "rows 0..%d of the 4096^3 BF16 product (FP64 sums, exact decoding), %.1f s"
                      % (done - 1, dt)}


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def traffic_for(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json),
    valid only while the kernel source is unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--legs", default="all", help="all | headline | comma list of leg names")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--protocol-seconds", type=float, default=1.0,
                    help="length of each of the three timing-protocol rounds (0: no protocol; "
                         "the per-kernel rate then comes from the timed launches' HIP events)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="only run a device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: libdmu has no multi-GPU path. The GEMM "
              "would shard over N without communication, each GPU running this kernel on "
              "its column shard. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4}))
        return

    b = Bench(args)
    dmu = b.dmu
    names = None if args.legs == "all" else set(args.legs.split(","))
    # legs that run only when named: they launch the headline kernel on other
    # operands, which would mix into its kernel-trace statistics
    opt_in = {"bf16_4096_operand_data"}
    want = lambda name: (names is None and name not in opt_in) or (names is not None and
                                                                   name in names)
    S, W = args.steps, args.warmup
    S4, W4 = max(S // 4, 10), max(W // 4, 5)

    # ---- headline: exactly S timed launches of the 4096^3 BF16 GEMM
    log("headline gemm_bf16 4096^3 (B N x K, BF16 out): %d warmup + %d timed launches" % (W, S))
    A = b.normal_bf16((4096, 4096), 1)
    B = b.normal_bf16((4096, 4096), 2)
    As, Bs = b.copies(A, 6), b.copies(B, 6)
    out = torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")

    def launch(i):
        dmu.gemm_bf16(As[i % 6], Bs[i % 6], out, dmu.B_COL_MAJOR)

    flop = 2.0 * 4096 ** 3
    # the per-kernel rate of the roofline: the page's protocol.  It runs first:
    # after the host's input set-up the first launches run up to ~30% slow
    # while the GPU's clocks ramp, and the protocol's warm-up and rounds take
    # that ramp before the timed region, which stays exactly W + S launches.
    proto = None
    if args.protocol_seconds > 0:
        proto = protocol_rounds(torch, launch, flop, PEAK_BF16_TFLOPS,
                                seconds=args.protocol_seconds)
        log("headline per kernel: %.1f TFLOP/s (%.1f%% of peak), rounds %s, spread %.2f%%, "
            "sclk %s MHz" % (proto["TFLOP_per_s"], proto["pct_peak"],
                             [r["median_ms"] for r in proto["rounds"]], 100 * proto["spread"],
                             proto["sclk_mhz_median"]))
    t = time_launches(torch, launch, S, W)
    value = flop / (t["wall_ms"] * 1e-3) / 1e12
    log("headline: %.1f TFLOP/s wall over the %d timed launches (%.5f ms per launch by the "
        "events around them)" % (value, S, t["event_mean_ms"]))
    if proto is not None:
        achieved, kernel_ms = proto["TFLOP_per_s"], proto["ms"]
    else:
        kernel_ms = t["event_mean_ms"]
        achieved = flop / kernel_ms / 1e9
    del As, Bs, out

    legs = {}
    if want("bf16_4096_nn"):
        legs["bf16_4096_nn"] = b.gemm_bf16_leg(4096, 4096, 4096, dmu.B_ROW_MAJOR, S, W, copies=6)
        log("bf16 4096 B row-major: %s" % legs["bf16_4096_nn"])
    for name, fmt in (("fp8_e4m3_4096", dmu.E4M3), ("fp8_e5m2_4096", dmu.E5M2)):
        if want(name):
            legs[name] = b.gemm_fp8_leg(4096, 4096, 4096, fmt, S, W, copies=10,
                                        protocol=(name == "fp8_e4m3_4096" and
                                                  args.protocol_seconds > 0),
                                        protocol_seconds=args.protocol_seconds)
            log("%s: %s" % (name, legs[name]))
    if want("fp8_e4m3_4096_promoted"):
        legs["fp8_e4m3_4096_promoted"] = b.gemm_fp8_leg(4096, 4096, 4096, dmu.E4M3, S, W, copies=10,
                                                         promoted=True)
        log("fp8_e4m3_4096 promoted every 128 K: %s" % legs["fp8_e4m3_4096_promoted"])
    if want("mxfp8_e4m3_4096"):
        legs["mxfp8_e4m3_4096"] = b.gemm_mx_leg(4096, 4096, 4096, dmu.E4M3, S, W, copies=10)
        log("mxfp8 e4m3 4096: %s" % legs["mxfp8_e4m3_4096"])
    if want("bf16_4096_bias_gelu"):
        legs["bf16_4096_bias_gelu"] = b.fused_leg("bf16_gelu", S, W, 6)
        log("bf16 4096 + bias + GELU: %s" % legs["bf16_4096_bias_gelu"])
    if want("fp8_e4m3_4096_bias_relu_fp8out"):
        legs["fp8_e4m3_4096_bias_relu_fp8out"] = b.fused_leg("fp8_relu_fp8out", S, W, 10)
        log("fp8 4096 + bias + ReLU -> E4M3: %s" % legs["fp8_e4m3_4096_bias_relu_fp8out"])
    # the attention legs follow half a second of input generation on the host,
    # during which the idle GPU clocks down: they need a longer warmup
    SA, WA = max(S // 2, 20), max(W // 2, 20)
    if want("attention_bf16_32x4096x4096x128"):
        legs["attention_bf16_32x4096x4096x128"] = b.attention_leg(False, SA, WA)
        log("attention 32 x 4096 x 4096 x 128: %s" % legs["attention_bf16_32x4096x4096x128"])
    if want("attention_bf16_32x4096x4096x128_causal"):
        legs["attention_bf16_32x4096x4096x128_causal"] = b.attention_leg(True, SA, WA)
        log("attention causal: %s" % legs["attention_bf16_32x4096x4096x128_causal"])
    if want("moe_bf16_32x16384x4096x7168"):
        legs["moe_bf16_32x16384x4096x7168"] = b.grouped_leg(S4, W4)
        log("moe grouped: %s" % legs["moe_bf16_32x16384x4096x7168"])
    if want("mxfp4_4096"):
        legs["mxfp4_4096"] = b.gemm_mxfp4_leg(4096, 4096, 4096, S, W, copies=10)
        log("mxfp4 4096: %s" % legs["mxfp4_4096"])
    if want("quantize_mxfp4_4096"):
        legs["quantize_mxfp4_4096"] = b.quantize_mx_leg(4096, 4096, dmu.E2M1, S, W)
        log("quantize mxfp4 4096^2: %s" % legs["quantize_mxfp4_4096"])
    if want("quantize_mx_e4m3_4096"):
        legs["quantize_mx_e4m3_4096"] = b.quantize_mx_leg(4096, 4096, dmu.E4M3, S, W)
        log("quantize mx 4096^2: %s" % legs["quantize_mx_e4m3_4096"])
    if want("quantize_e4m3_4096_tensor"):
        legs["quantize_e4m3_4096_tensor"] = b.quantize_leg(4096, 4096, dmu.E4M3, None, S, W)
        log("quantize 4096^2: %s" % legs["quantize_e4m3_4096_tensor"])
        legs["quantize_e4m3_4096_tensor_noalloc"] = b.quantize_leg(4096, 4096, dmu.E4M3, None, S,
                                                                   W, noalloc=True)
        log("quantize 4096^2, allocation-free entry: %s"
            % legs["quantize_e4m3_4096_tensor_noalloc"])
    if want("fp8_block_8192x7168x7168"):
        legs["fp8_block_8192x7168x7168"] = b.gemm_fp8_leg(
            8192, 7168, 7168, dmu.E4M3, S4, W4, block=True, protocol=args.protocol_seconds > 0,
            protocol_seconds=args.protocol_seconds)
        log("block-scaled: %s" % legs["fp8_block_8192x7168x7168"])
    if want("quantize_block"):
        legs["quantize_e4m3_8192x7168_1x128"] = b.quantize_leg(8192, 7168, dmu.E4M3, (1, 128),
                                                                S4, W4, outliers=True)
        legs["quantize_e4m3_7168x7168_128x128"] = b.quantize_leg(7168, 7168, dmu.E4M3,
                                                                  (128, 128), S4, W4)
        log("block quantizers: %s %s" % (legs["quantize_e4m3_8192x7168_1x128"],
                                        legs["quantize_e4m3_7168x7168_128x128"]))
    if want("llm_28672x8192"):
        Bllm = b.normal_bf16((28672, 8192), 2)
        for M in (16, 128, 1024, 8192):
            legs["bf16_llm_M%d_N28672_K8192" % M] = b.gemm_bf16_leg(
                M, 28672, 8192, dmu.B_COL_MAJOR, S if M < 1024 else S4, W4, B=Bllm,
                protocol=M == 8192 and args.protocol_seconds > 0,
                protocol_seconds=args.protocol_seconds)
            log("llm M=%d: %s" % (M, legs["bf16_llm_M%d_N28672_K8192" % M]))
        del Bllm
    if want("bf16_4096_lds_layouts"):
        # the bank-conflict ablation of the vidyal.ai page, Step 3: the headline
        # kernel with its XOR-swizzled LDS rows, plain rows and padded rows
        A = b.normal_bf16((4096, 4096), 1)
        B = b.normal_bf16((4096, 4096), 2)
        As, Bs = b.copies(A, 6), b.copies(B, 6)
        o = torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")
        for lay, nm in ((dmu.LDS_SWIZZLED, "swizzled"), (dmu.LDS_PLAIN, "plain"),
                        (dmu.LDS_PADDED, "padded")):
            t_l = time_launches(torch, lambda i: dmu.probe_gemm_bf16_layout(lay, As[i % 6], Bs[i % 6],
                                                                              o), S, W)
            legs["bf16_4096_lds_" + nm] = b.report(t_l, 2.0 * 4096 ** 3, 2.0 * 3 * 4096 ** 2,
                                                   PEAK_BF16_TFLOPS, 6)
            log("bf16 4096 LDS layout %s: %s" % (nm, legs["bf16_4096_lds_" + nm]))
        del As, Bs, o
    if want("bf16_256"):
        legs["bf16_256_f32out"] = b.gemm_bf16_leg(256, 256, 256, dmu.B_ROW_MAJOR, S, W,
                                                  out_f32=True, seed_dist="uniform")
        log("256^3: %s" % legs["bf16_256_f32out"])

    if want("bf16_4096_operand_data"):
        # the headline kernel, unchanged, on operands that draw less power per
        # MFMA: the same instructions and memory traffic, a different clock
        for dist in ("normal", "ones", "zeros"):
            fill = {"normal": None, "ones": 1.0, "zeros": 0.0}[dist]
            if fill is None:
                Ad, Bd = b.normal_bf16((4096, 4096), 1), b.normal_bf16((4096, 4096), 2)
            else:
                Ad = torch.full((4096, 4096), fill, dtype=torch.bfloat16, device="cuda")
                Bd = Ad.clone()
            As, Bs = b.copies(Ad, 6), b.copies(Bd, 6)
            o = torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")
            t_d = time_launches(torch, lambda i: dmu.gemm_bf16(As[i % 6], Bs[i % 6], o,
                                                                dmu.B_COL_MAJOR), S, W)
            legs["bf16_4096_operands_" + dist] = b.report(t_d, 2.0 * 4096 ** 3,
                                                          2.0 * 3 * 4096 ** 2,
                                                          PEAK_BF16_TFLOPS, 6)
            log("bf16 4096 operands %s: %s" % (dist, legs["bf16_4096_operands_" + dist]))
            del As, Bs, o, Ad, Bd
    if want("mfma_ceiling"):
        legs["mfma_ceiling"] = b.mfma_ceiling_leg(S4, W4)
        log("mfma ceiling (no memory traffic): %s" % legs["mfma_ceiling"])

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(A, B)
        log("cpu baseline: %s" % cpu)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": round(t["wall_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) FP32 sources rounded to BF16 (PCG64 seeds 1, 2)",
        "config": {"workload": "gemm_bf16 M=N=K=4096, A row-major, B stored N x K, FP32 "
                               "accumulate, BF16 out", "M": 4096, "N": 4096, "K": 4096,
                   "operand_copies": 6},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 1),
        "fp8_e4m3_4096": legs.get("fp8_e4m3_4096"),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for("gemm_bf16_4096_tn"),
                     "kernel": "gemm_kernel<kBF16, B col-major, 256x256>",
                     "kernel_ms": round(kernel_ms, 5)},
        "protocol": proto,
        "cpu_baseline": cpu,
        "legs": legs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
