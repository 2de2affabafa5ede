"""Benchmark: fused per-layer DP clip+accumulate on one MI355X.

A step is one pass of the whole hot path over the seven linears of one
Llama-13B-shaped decoder layer (q, k, v, o: 5120x5120; gate, up: 5120->13824;
down: 13824->5120) at B = 8, T = 2048, bf16 inputs, fp32 accumulation, each
linear clipped on its own (C = 1) with Philox noise (sigma = 1, seed 0,
offset 0): per linear, the norm phase the library picks for the shape (at
these shapes the Gram identity: per-sample Gram blocks of X and G by MFMA,
no per-sample gradient stored), the ordered reduction to clip factors, and
the clipped sum as one scaled-accumulate GEMM with the noise epilogue.

Beside the headline the same line reports the staged form (each per-sample
gradient tile stored in device memory once, then combined) as a labelled
comparison with its extra device memory, and the other workloads: one fp32
linear, the GPT-2 MLP up-projection (with its inputs in and out of the
Infinity Cache), the ragged Llama-13B batch, and the RoBERTa-large projected
variant.

Inputs are seeded synthetic Gaussians (no dataset) generated on the host and
resident in HBM before timing starts.  Prints one JSON line.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "fused DP clip+accumulate TFLOP/s and samples/s per linear layer; % MFMA peak"

# Figures per launch of the dominant kernels on this workload (the automatic
# path: Gram on all seven linears), from rocprofv3 runs of this script
# (profiles/gram_accumulate_llama13b_layer_B8_T2048_*.md): HBM bytes from two
# --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch, averaged over
# the seven linears) scaled by what the same counters read for a plain 1 GiB
# device copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0); MfmaUtil (MFMA-busy cycles
# per SIMD cycle, percent); and the kernel-trace average duration.  Each
# kernel's figures hold only for the sources whose SHA-256 is stored with them
# and the default workload; they are reported as null otherwise.
KERNEL_SOURCES = {"accumulate": ("accum_big.hip", "common.hpp"),
                  "gram_norm": ("gram_big.hip", "common.hpp")}
KERNEL_COUNTERS = {
    "batch": 8, "seq": 2048, "linears": "q,k,v,o,gate,up,down",
    "fetch_scale": 2.0, "write_scale": 1.0,
    "kernels": {
        "accumulate": {"sources_sha256": "cfc2fa80dca168539b532d85f1c9cac808c9ce9461eb95419b504cb4245f4141",
                       "fetch_kib": 1129356.27, "write_kib": 279698.29, "mfma_busy_pct": 60.04,
                       "trace_avg_us": 1290.7},
        "gram_norm": {"sources_sha256": "51d8ce09f519858dcd13a5155fb6c9ea7f3f83ebdad8b08bc83deabd8e6bed25",
                      "fetch_kib": 413893.85, "write_kib": 163988.44, "mfma_busy_pct": 63.73,
                      "trace_avg_us": 430.3},
    },
    # --norm-path values that run these kernels on every linear of the workload
    "paths": ("0", "1"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--seq", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--linears", default="q,k,v,o,gate,up,down")
    ap.add_argument("--norm-path", type=int, default=0, choices=(0, 1, 2, 3),
                    help="0: the library's per-call choice (default); 1 Gram, 2 direct, 3 staged")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (to scale HBM byte counters)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workload configurations (fp32 single linear, GPT-2 MLP "
                         "up-projection, ragged Llama-13B layer, RoBERTa projected)")
    ap.add_argument("--no-staged", action="store_true",
                    help="skip the staged-path comparison of the headline step")
    ap.add_argument("--only", default="",
                    help="comma-separated subset of c1,c2,c4,c5: measure only those workload "
                         "configurations (no headline step) and print them as one JSON line; "
                         "for profiling one configuration")
    return ap.parse_args()


class ClockSampler:
    """Samples the GPU's shader clock from a helper thread while the timed
    steps run (the part is power-limited under MFMA load, so the clock
    explains part of the gap to the spec peak): the current level of the
    driver's pp_dpm_sclk file, read every 10 ms, else rocm-smi.  Reports None
    when neither is readable."""

    def __init__(self):
        import glob
        import threading
        self.mhz = []
        self.source = None
        self._files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read_sysfs(self):
        import re
        for f in self._files:
            try:
                with open(f) as fh:
                    for line in fh:
                        if "*" in line:
                            m = re.search(r"(\d+)\s*mhz", line, re.IGNORECASE)
                            if m:
                                return int(m.group(1))
            except OSError:
                continue
        return None

    def _read_smi(self):
        import re
        import subprocess
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10)
        m = re.search(r"sclk[^(]*\((\d+)\s*mhz\)", r.stdout, re.IGNORECASE)
        return int(m.group(1)) if m else None

    def _run(self):
        import subprocess
        while not self._stop.is_set():
            v = self._read_sysfs()
            if v is not None:
                self.source = "pp_dpm_sclk"
            else:
                try:
                    v = self._read_smi()
                    self.source = "rocm-smi"
                except (OSError, subprocess.SubprocessError):
                    return
            if v is not None:
                self.mhz.append(v)
            self._stop.wait(0.01)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join(timeout=15)

    def summary(self):
        if not self.mhz:
            return None
        return {"source": self.source, "samples": len(self.mhz), "min_mhz": min(self.mhz),
                "max_mhz": max(self.mhz), "mean_mhz": round(sum(self.mhz) / len(self.mhz))}


def time_calls(torch, fn, steps, warmup, min_ms=20.0, warm_ms=100.0):
    """Average milliseconds per call of fn() (events on the current stream).

    Warm-up: `warmup` calls, then more until about warm_ms of wall time has
    passed, so that a GPU idle before (clock down) has reached its working
    clock.  Timed: `steps` calls, or more for short calls, so that the timed
    region spans at least min_ms."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n_warm = 0
    while (time.perf_counter() - t0) * 1e3 < warm_ms:
        for _ in range(16):
            fn()
        n_warm += 16
        torch.cuda.synchronize()
    reps = steps
    if n_warm:
        per_call = (time.perf_counter() - t0) * 1e3 / n_warm
        reps = max(steps, int(min_ms / max(per_call, 1e-4)) + 1)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def call_memory(dp):
    """Resets the library's record of the most device memory one call took
    beyond its inputs and outputs; returns a reader of it."""
    dp.set_option("workspace_call_high", 0)
    return lambda: int(dp.get_option("workspace_call_high"))


def measure_configs(dp, torch, steps, warmup, only=None):
    """The other workloads, one fused call per linear, on the automatic path."""
    import workloads
    out = {}

    def to_device(a, dtype):
        if dtype == "bf16":
            return upload(a, torch)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def dense(makers, name, note, peak=PEAK_BF16_TFLOPS):
        dev, lins = [], []
        for make in makers:
            lin = make()
            lins.append(lin)
            print(f"# {name}: generated {lin.name}", file=sys.stderr, flush=True)
            X, G = to_device(lin.X, lin.dtype), to_device(lin.G, lin.dtype)
            mask = None if lin.mask is None else torch.from_numpy(np.ascontiguousarray(lin.mask)).cuda()
            o = torch.empty((lin.dout, lin.din), dtype=torch.float32, device=X.device)
            nrm = torch.empty((lin.B,), dtype=torch.float32, device=X.device)
            dev.append((lin, X, G, mask, o, nrm))

        def layer():
            for lin, X, G, mask, o, nrm in dev:
                dp.linear_clip_accumulate(X, G, mask, C=lin.C, sigma=lin.sigma, seed=lin.seed,
                                          offset=lin.offset, grad_out=o, norms_out=nrm)
        mem = call_memory(dp)
        ms = time_calls(torch, layer, steps, warmup)
        paths = [norm_path_of(dp, lambda d=d: dp.linear_clip_accumulate(
            d[1], d[2], d[3], C=d[0].C, sigma=d[0].sigma, seed=d[0].seed, offset=d[0].offset,
            grad_out=d[4], norms_out=d[5])) for d in dev]
        useful = sum(2.0 * l.active_tokens() * l.din * l.dout for l in lins)
        B = lins[0].B
        tf = useful / (ms * 1e-3) / 1e12
        out[name] = {"note": note,
                     "norm_path": ", ".join(f"{l.name} {p}" for l, p in zip(lins, paths)),
                     "linears": len(lins), "ms": round(ms, 4),
                     "useful_tflops": round(tf, 3), "peak_tflops": peak,
                     "frac_of_peak": round(tf / peak, 5),
                     "samples_per_s": round(B / (ms * 1e-3), 1),
                     "tokens_per_s": round(sum(l.active_tokens() for l in lins) / len(lins)
                                           / (ms * 1e-3), 1),
                     "extra_device_bytes_per_call_max": mem()}
        print(f"# {name}: {out[name]}", file=sys.stderr, flush=True)
        del dev
        torch.cuda.empty_cache()

    want = (lambda k: True) if only is None else (lambda k: k in only)

    if want("c1"):
        dense([lambda: workloads.config_c1(sigma=1.0).linears[0]], "c1_fp32_B4_T16_64to32",
              "one fp32 linear, sigma 1; launch-latency bound; peak = fp32 vector 157.3 TFLOP/s",
              peak=PEAK_FP32_TFLOPS)
        dense([lambda: workloads.config_c1(sigma=0.0).linears[0]], "c1_fp32_B4_T16_64to32_sigma0",
              "as above, sigma 0", peak=PEAK_FP32_TFLOPS)
    if want("c2"):
        dense([lambda: workloads.config_c2().linears[0]], "c2_gpt2_up_B32_T512_768to3072",
              "bf16, sigma 0.8; inputs (126 MB) resident in the Infinity Cache across calls")
        # the GPT-2 layer on each norm path, one after another on the same inputs:
        # Gram, direct, the single pass (each per-sample gradient once, on chip)
        # and the opt-in staged form
        lin = workloads.config_c2().linears[0]
        X, G = upload(lin.X, torch), upload(lin.G, torch)
        o = torch.empty((lin.dout, lin.din), dtype=torch.float32, device=X.device)
        nrm = torch.empty((lin.B,), dtype=torch.float32, device=X.device)
        f = 2.0 * lin.B * lin.T * lin.din * lin.dout
        by_path = {}
        for path, name in ((1, "gram"), (2, "direct"), (4, "one pass"), (3, "staged")):
            dp.set_option("norm_path", path)
            try:
                call = lambda: dp.linear_clip_accumulate(X, G, None, C=lin.C, sigma=lin.sigma,
                                                         grad_out=o, norms_out=nrm)
                mem = call_memory(dp)
                ms = time_calls(torch, call, steps, warmup)
                taken = norm_path_of(dp, call)
                by_path[name] = {"ms": round(ms, 4), "useful_tflops": round(f / (ms * 1e-3) / 1e12, 2),
                                 "norm_path_taken": taken, "extra_device_bytes_per_call_max": mem()}
            finally:
                dp.set_option("norm_path", 0)
        out["c2_gpt2_up_by_norm_path"] = {
            "note": "as c2, each norm path forced in turn (the automatic choice is listed above)",
            **by_path}
        del X, G, o, nrm

        # the same layer with its bias (weight and bias clipped together)
        lin = workloads.config_c2().linears[0]
        X, G = upload(lin.X, torch), upload(lin.G, torch)

        # c2's inputs (126 MB) fit in the 256 MB Infinity Cache: also time calls
        # that each follow a 512 MB write, which evicts them
        flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=X.device)
        o = torch.empty((lin.dout, lin.din), dtype=torch.float32, device=X.device)
        nrm = torch.empty((lin.B,), dtype=torch.float32, device=X.device)
        times = []
        for i in range(steps + warmup):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dp.linear_clip_accumulate(X, G, None, C=lin.C, sigma=lin.sigma, grad_out=o, norms_out=nrm)
            e1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
        ms = sum(times) / len(times)
        f = 2.0 * lin.B * lin.T * lin.din * lin.dout
        out["c2_gpt2_up_B32_T512_768to3072_flushed"] = {
            "note": "as c2, each call after a 512 MB write that evicts the inputs from the cache",
            "linears": 1, "ms": round(ms, 4), "useful_tflops": round(f / (ms * 1e-3) / 1e12, 2),
            "frac_of_peak": round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
            "samples_per_s": round(lin.B / (ms * 1e-3), 1)}
        del flush
        o = torch.empty((lin.dout, lin.din), dtype=torch.float32, device=X.device)
        ob = torch.empty((lin.dout,), dtype=torch.float32, device=X.device)
        nrm = torch.empty((lin.B,), dtype=torch.float32, device=X.device)
        ms = time_calls(torch, lambda: dp.linear_clip_accumulate_bias(
            X, G, None, C=lin.C, sigma=lin.sigma, grad_out=o, bias_grad_out=ob, norms_out=nrm),
            steps, warmup)
        f = 2.0 * lin.B * lin.T * lin.din * lin.dout
        out["c2_gpt2_up_with_bias"] = {
            "note": "as c2, plus the bias gradient (column sums of G) in the clipping norm and sum",
            "linears": 1, "ms": round(ms, 4), "useful_tflops": round(f / (ms * 1e-3) / 1e12, 2),
            "frac_of_peak": round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
            "samples_per_s": round(lin.B / (ms * 1e-3), 1)}
        del X, G, o, ob, nrm
        torch.cuda.empty_cache()
    if want("c4"):
        dense([lambda i=i: workloads.config_c4_linear(i) for i in range(len(workloads.C4_LINEARS))],
              "c4_llama13b_ragged_B16_T2048_7_linears",
              "bf16, prefix masks T_i ~ U[128, 2048], C 0.5, sigma 1.2; useful flops over active tokens")

    if want("c5"):
        # projected variant: Y = X P with P from gaussian_fill(seed 7, offset 0, 1/sqrt(r)), r = 256
        r = 256
        dev, Ps = [], {}
        lins = workloads.config_c5().linears
        for lin in lins:
            if lin.din not in Ps:
                Ps[lin.din] = dp.gaussian_fill(7, 0, lin.din * r, 1.0 / 16.0,
                                               dtype=torch.bfloat16).view(lin.din, r)
            X, G = upload(lin.X, torch), upload(lin.G, torch)
            o = torch.empty((lin.dout, r), dtype=torch.float32, device=X.device)
            nrm = torch.empty((lin.B,), dtype=torch.float32, device=X.device)
            dev.append((lin, X, G, o, nrm))

        def proj_layer():
            for lin, X, G, o, nrm in dev:
                dp.linear_clip_accumulate_projected(X, G, Ps[lin.din], C=lin.C, sigma=lin.sigma,
                                                    grad_out=o, norms_out=nrm)
        ms = time_calls(torch, proj_layer, steps, warmup)
        paths = sorted({norm_path_of(dp, lambda d=d: dp.linear_clip_accumulate_projected(
            d[1], d[2], Ps[d[0].din], C=d[0].C, sigma=d[0].sigma, grad_out=d[3], norms_out=d[4]))
            for d in dev})
        useful = sum(2.0 * l.B * l.T * (l.din + l.dout) * r for l in lins)
        out["c5_roberta_large_projected_r256_6_linears"] = {
            "note": "bf16, projection then clip in r space; useful flops 2*B*T*(din+dout)*r",
            "norm_path": ",".join(paths),
            "linears": len(lins), "ms": round(ms, 4),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2),
            "frac_of_peak": round(useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
            "samples_per_s": round(lins[0].B / (ms * 1e-3), 1)}

        # the same six calls in one library call, queued on the library's streams so that
        # the linears' small launches overlap (each linear still clipped on its own; the
        # noise offsets are consecutive, as that call requires with sigma > 0)
        assert all(l.C == lins[0].C and l.sigma == lins[0].sigma for l in lins)
        mX, mG = [d[1] for d in dev], [d[2] for d in dev]
        mP, mo, mn = [Ps[d[0].din] for d in dev], [d[3] for d in dev], [d[4] for d in dev]

        def many_layer():
            dp.linear_clip_accumulate_projected_many(mX, mG, mP, None, C=lins[0].C,
                                                     sigma=lins[0].sigma, grad_outs=mo,
                                                     norms_outs=mn)
        ms = time_calls(torch, many_layer, steps, warmup)
        out["c5_roberta_large_projected_r256_6_linears_side_streams"] = {
            "note": "as c5 above, the six projected calls queued together "
                    "(linear_clip_accumulate_projected_many: the caller's stream and one library "
                    "stream, calls alternating; each output bitwise the single call's for the "
                    "same offsets)",
            "linears": len(lins), "ms": round(ms, 4),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2),
            "frac_of_peak": round(useful / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
            "samples_per_s": round(lins[0].B / (ms * 1e-3), 1)}

        # the same, with P drawn from its seed inside the projection (never stored)
        def seeded_layer():
            for lin, X, G, o, nrm in dev:
                dp.linear_clip_accumulate_projected_seeded(X, G, r, None, p_seed=7, p_offset=0,
                                                           C=lin.C, sigma=lin.sigma, grad_out=o,
                                                           norms_out=nrm)
        ms = time_calls(torch, seeded_layer, steps, warmup)
        out["c5_roberta_large_projected_seeded_r256_6_linears"] = {
            "note": "as above, P drawn from Philox seed 7 in each call (once into workspace), never kept",
            "linears": len(lins), "ms": round(ms, 4),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2),
            "samples_per_s": round(lins[0].B / (ms * 1e-3), 1)}
        dp.set_option("p_in_kernels", 1)
        try:
            ms = time_calls(torch, seeded_layer, steps, warmup)
        finally:
            dp.set_option("p_in_kernels", 0)
        out["c5_roberta_large_projected_seeded_in_kernel_r256_6_linears"] = {
            "note": "as above, P drawn inside the projection kernel in every token tile; no P tensor",
            "linears": len(lins), "ms": round(ms, 4),
            "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2),
            "samples_per_s": round(lins[0].B / (ms * 1e-3), 1)}

        # projected Adam step on the privatised projected gradients (moments in
        # r-space, weight update W -= lr U P^T with P drawn from its seed)
        states = []
        for lin, X, G, o, nrm in dev:
            states.append((o, torch.zeros_like(o), torch.zeros_like(o),
                           torch.zeros((lin.dout, lin.din), dtype=torch.float32, device=o.device)))
        seeded_layer()
        step_no = [0]

        def adam_layer():
            step_no[0] += 1
            for h, m, v, W in states:
                dp.projected_adam_step(h, m, v, W, step_no[0], 1e-4, P=None, p_seed=7, p_offset=0)
        ms = time_calls(torch, adam_layer, steps, warmup)
        flops = sum(2.0 * l.dout * l.din * r for l in lins)
        bytes_ = sum(4.0 * (6 * l.dout * r + 2 * l.dout * l.din) for l in lins)
        out["c5_roberta_large_projected_adam_step_6_linears"] = {
            "note": "moments + U P^T update (fp32 MFMA), P drawn from its seed; flops 2*dout*din*r, "
                    "bytes: h, m, v, U in r-space and W read+written",
            "linears": len(lins), "ms": round(ms, 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "gb_per_s": round(bytes_ / (ms * 1e-3) / 1e9, 1)}
    return out


def copy_calibration(steps):
    """A plain copy of known size: reads and writes exactly 1 GiB per launch."""
    import torch
    n = (1 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 1 << 30, "copy_calibration_bytes_written": 1 << 30,
                      "launches": steps}), flush=True)


def kernel_record(args, kernel):
    """The committed profile figures of `kernel`, or None when its sources or
    the workload differ from the profiled ones."""
    c = KERNEL_COUNTERS
    k = c["kernels"].get(kernel)
    if k is None or str(args.norm_path) not in c["paths"] or args.batch != c["batch"] \
            or args.seq != c["seq"] or args.linears != c["linears"]:
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sample_gradient_clipping_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return k if h.hexdigest() == k["sources_sha256"] else None


def kernel_traffic(args, kernel):
    """Counter-derived HBM bytes per launch of `kernel`, or None."""
    k = kernel_record(args, kernel)
    if k is None:
        return None
    c = KERNEL_COUNTERS
    return (k["fetch_kib"] * c["fetch_scale"] + k["write_kib"] * c["write_scale"]) * 1024.0


def kernel_counter(args, kernel, name):
    """A per-kernel figure (MFMA-busy %, trace average) from the committed profile, or None."""
    k = kernel_record(args, kernel)
    return None if k is None else k.get(name)


def norm_path_of(dp, call):
    """Which norm path the library took for one call (from its kernel timing)."""
    dp.timing_reset()
    dp.set_option("timing", 1)
    try:
        call()
        names = dp.timing_collect()
    finally:
        dp.set_option("timing", 0)
        dp.timing_reset()
    for key, path in (("staged_norm", "staged"), ("gram_norm", "gram"), ("direct_norm", "direct"),
                      ("onepass", "one pass"), ("tiny_layer", "one workgroup")):
        if key in names:
            return path
    return "unknown"


def staged_bytes(l):
    """Staged per-sample tiles of one linear (256 x 256 fp32 tiles, padded)."""
    tiles = -(-l.din // 256) * -(-l.dout // 256)
    return 4.0 * l.B * tiles * 65536


def upload(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def cpu_baseline(lins, budget_s):
    """The fp64 oracle (untuned) on a bounded sample of the step: whole
    linears (all samples) in the step's order until about budget_s of CPU
    work has been done."""
    from oracle import dp_linear
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    done, dt, flops = [], 0.0, 0.0
    for lin in lins:
        if done and dt >= budget_s:
            break
        t0 = time.perf_counter()
        dp_linear.oracle_linear(lin.X, lin.G, None, lin.C, lin.sigma, lin.seed, lin.offset, "bf16")
        dt += time.perf_counter() - t0
        flops += 2.0 * lin.B * lin.T * lin.din * lin.dout
        done.append(lin.name)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle (per-sample g_i materialised, clip, sum, Philox noise) on "
                   f"{len(done)} of the step's {len(lins)} linears ({', '.join(done)}), all "
                   f"{lins[0].B} samples each, T={lins[0].T}; {dt:.1f} s wall; host "
                   f"os.cpu_count()={os.cpu_count()}"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(multi-GPU data parallelism is a design note, not built)"}))
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.steps)
        return
    if args.only:
        only = {c.strip() for c in args.only.split(",") if c.strip()}
        bad = only - {"c1", "c2", "c4", "c5"}
        if bad:
            print(json.dumps({"error": f"unknown configuration(s) {sorted(bad)}"}))
            sys.exit(2)
        import torch
        import sample_gradient_clipping_amd as dp
        dp.load()
        print(json.dumps({"configs": measure_configs(dp, torch, args.steps, args.warmup, only)}))
        return
    import torch
    import sample_gradient_clipping_amd as dp
    import workloads

    dp.load()
    dp.set_option("norm_path", args.norm_path)
    dev = torch.device("cuda:0")
    names = [n.strip() for n in args.linears.split(",")]
    idx = [i for i, (n, _, _) in enumerate(workloads.C3_LINEARS) if n in names]
    t_gen = time.perf_counter()
    lins, dev_in = [], []
    for i in idx:
        lin = workloads.config_c3_linear(i, B=args.batch, T=args.seq)
        X, G = upload(lin.X, torch), upload(lin.G, torch)
        out = torch.empty((lin.dout, lin.din), dtype=torch.float32, device=dev)
        norms = torch.empty((lin.B,), dtype=torch.float32, device=dev)
        dev_in.append((X, G, out, norms))
        lins.append(lin)
        print(f"# generated+uploaded {lin.name} {lin.din}->{lin.dout}", file=sys.stderr, flush=True)
    gen_s = time.perf_counter() - t_gen

    def step():
        for lin, (X, G, out, norms) in zip(lins, dev_in):
            dp.linear_clip_accumulate(X, G, None, C=lin.C, sigma=lin.sigma, seed=lin.seed,
                                      offset=lin.offset, grad_out=out, norms_out=norms)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step wall time; the library's record of the device memory each
    # call takes beyond its inputs and outputs is reset first
    mem = call_memory(dp)
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        s0.record()
        for _ in range(args.steps):
            step()
        s1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = s0.elapsed_time(s1) / args.steps
    extra_bytes = mem()
    pool_high = int(dp.get_option("workspace_reserved_high"))

    # per-kernel durations: HIP events recorded by the library on the launch
    # stream around every kernel, over a second pass of the same K steps
    dp.timing_reset()
    dp.set_option("timing", 1)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = dp.timing_collect()
    dp.set_option("timing", 0)
    dp.timing_reset()

    # determinism: the outputs of two further steps must match bit for bit
    step()
    torch.cuda.synchronize()
    first = [o.clone() for (_, _, o, _) in dev_in]
    step()
    torch.cuda.synchronize()
    deterministic = all(torch.equal(a, o) for a, (_, _, o, _) in zip(first, dev_in))
    del first

    # per linear: the fused call alone, and a plain bf16 GEMM G^T X of the same
    # shape (no clipping, no noise) as the non-DP reference
    per_linear = []
    paths = []
    for lin, (X, G, out, norms) in zip(lins, dev_in):
        call = lambda: dp.linear_clip_accumulate(
            X, G, None, C=lin.C, sigma=lin.sigma, seed=lin.seed, offset=lin.offset,
            grad_out=out, norms_out=norms)
        paths.append(norm_path_of(dp, call))
        ms = time_calls(torch, call, args.steps, 2, warm_ms=0.0)
        Gt = G.reshape(-1, lin.dout).t().contiguous()
        X2 = X.reshape(-1, lin.din)
        ms_gemm = time_calls(torch, lambda: torch.matmul(Gt, X2), args.steps, 2, warm_ms=0.0)
        del Gt
        f = 2.0 * lin.B * lin.T * lin.din * lin.dout
        per_linear.append({"linear": lin.name, "din": lin.din, "dout": lin.dout,
                           "norm_path": paths[-1],
                           "useful_gflop": round(f / 1e9, 1), "ms": round(ms, 4),
                           "useful_tflops": round(f / (ms * 1e-3) / 1e12, 2),
                           "samples_per_s": round(lin.B / (ms * 1e-3), 1),
                           "tokens_per_s": round(lin.B * lin.T / (ms * 1e-3), 1),
                           "plain_bf16_gemm_ms": round(ms_gemm, 4),
                           "dp_over_plain_throughput": round(ms_gemm / ms, 3)})

    useful = sum(2.0 * l.B * l.T * l.din * l.dout for l in lins)
    contraction = lambda l: 2.0 * l.B * l.T * l.din * l.dout
    gram_flops = lambda l: float(l.B) * l.T * l.T * (l.din + l.dout)
    executed = sum(contraction(l) + (gram_flops(l) if p == "gram" else contraction(l) if p == "direct"
                                     else 0.0) for l, p in zip(lins, paths))
    tflops = useful / (ms_step * 1e-3) / 1e12
    samples_per_s = args.batch / (ms_step * 1e-3)   # a step is one layer over the batch

    # MFMA kernels and the flops each does per linear; the dominant one (most
    # time per step) is the roofline kernel.
    mfma_flops = {
        "onepass": lambda l, p: contraction(l) if p == "one pass" else 0.0,
        "staged_norm": lambda l, p: contraction(l) if p == "staged" else 0.0,
        "direct_norm": lambda l, p: contraction(l) if p == "direct" else 0.0,
        "gram_norm": lambda l, p: gram_flops(l) if p == "gram" else 0.0,
        "accumulate": lambda l, p: contraction(l) if p not in ("staged", "one pass") else 0.0,
    }
    kernel_desc = {
        "onepass": "onepass (per-sample gradient tiles once, cross-workgroup norm reduction, "
                   "clipped running sum in registers)",
        "staged_norm": "staged_norm (per-sample gradient tiles by MFMA, their sums of squares, "
                       "tiles stored once for the combine pass)",
        "direct_norm": "direct_norm (per-sample gradient tiles by MFMA, sums of squares)",
        "gram_norm": "gram_norm (per-sample Gram blocks by MFMA, weighted product sum)",
        "accumulate": "accumulate (scaled-accumulate GEMM + noise epilogue)",
    }

    def achieved_tflops(k):
        ms, n = ktimes.get(k, (0.0, 0))
        if n == 0:
            return None
        f = sum(mfma_flops[k](l, p) for l, p in zip(lins, paths)) * args.steps
        return f / (ms * 1e-3) / 1e12

    dom = max((k for k in mfma_flops if k in ktimes), key=lambda k: ktimes[k][0])
    dom_n = ktimes[dom][1]
    dom_flops = sum(mfma_flops[dom](l, p) for l, p in zip(lins, paths)) * args.steps / dom_n
    dom_avg_ms = ktimes[dom][0] / dom_n
    dom_achieved = dom_flops / (dom_avg_ms * 1e-3) / 1e12
    # algorithmic bytes per launch of the dominant kernel: X and G read once
    # (bf16), plus what it must write -- the staged tiles (staged_norm) or the
    # fp32 result (accumulate)
    users = [(l, p) for l, p in zip(lins, paths) if mfma_flops[dom](l, p) > 0]
    dom_algo_bytes = sum(2.0 * l.B * l.T * (l.din + l.dout)
                         + (staged_bytes(l) if dom == "staged_norm" else
                            4.0 * l.din * l.dout if dom == "accumulate" else 0.0)
                         for l, _ in users) / max(len(users), 1)
    traffic = kernel_traffic(args, dom)

    # the combine pass of the staged path is bound by HBM: staged tiles read
    # once, the fp32 result written once
    comb_ms, comb_n = ktimes.get("staged_combine", (0.0, 0))
    comb = None
    if comb_n:
        st = [l for l, p in zip(lins, paths) if p == "staged"]
        comb_bytes = sum(staged_bytes(l) + 4.0 * l.din * l.dout for l in st) / len(st)
        comb_gbs = comb_bytes / ((comb_ms / comb_n) * 1e-3) / 1e9
        comb = {"kernel": "staged_combine (sum_i c_i g_i + noise, / B, from the staged tiles)",
                "bound": "hbm", "achieved": round(comb_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(comb_gbs / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": round(comb_bytes),
                "traffic": None if kernel_traffic(args, "staged_combine") is None
                else round(kernel_traffic(args, "staged_combine"))}

    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian X, lognormal-scaled G; no dataset)",
        "config": {"workload": "llama13b_decoder_layer_7_linears_B8_T2048_bf16",
                   "batch": args.batch, "seq_len": args.seq, "linears": names,
                   "C": 1.0, "sigma": 1.0,
                   "norm_path": ("auto: " if args.norm_path == 0 else "forced: ")
                                + ", ".join(f"{l.name} {p}" for l, p in zip(lins, paths)),
                   "parallelism": "none (1 GPU)"},
        "samples_per_s": round(samples_per_s, 1),
        "samples_per_s_note": "batch / step time: one step clips the whole layer for B samples",
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "extra_device_bytes_per_call_max": extra_bytes,
        "workspace_pool_reserved_high_bytes": pool_high,
        "executed_tflops": round(executed / (ms_step * 1e-3) / 1e12, 2),
        "kernels_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in ktimes.items()},
        "roofline": {
            "kernel": kernel_desc[dom],
            "bound": "mfma",
            "achieved": round(dom_achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else round(traffic),
            "avg_launch_ms": round(dom_avg_ms, 4),
            "flops_per_launch": round(dom_flops),
            "mfma_busy_pct": kernel_counter(args, dom, "mfma_busy_pct"),
            "committed_trace_avg_ms": None if kernel_counter(args, dom, "trace_avg_us") is None
            else kernel_counter(args, dom, "trace_avg_us") / 1e3,
            "committed_trace_frac": None if kernel_counter(args, dom, "trace_avg_us") is None
            else round(dom_flops / (kernel_counter(args, dom, "trace_avg_us") * 1e-6) / 1e12
                       / PEAK_BF16_TFLOPS, 4),
            "note": "achieved from this run's HIP events on the launch stream; committed_trace_* "
                    "from the rocprofv3 kernel trace in profiles/ (boxes differ by ~5% in clock)",
        },
        "roofline_kernel_bytes_per_launch": {"algorithmic": round(dom_algo_bytes),
                                             "hbm_counters": None if traffic is None else round(traffic)},
        "combine_roofline": comb,
        "mfma_kernel_tflops": {k: round(achieved_tflops(k), 2) for k in mfma_flops
                               if achieved_tflops(k) is not None},
        "per_linear": per_linear,
        "bitwise_deterministic": bool(deterministic),
        "gpu_sclk_during_timed_steps": clock.summary(),
        "wall_s_timed": round(wall, 3),
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_staged and args.norm_path != 3:
        # The staged form, for comparison only: every per-sample gradient tile
        # computed once and stored in device memory (the explicit storage the
        # FlashDP abstract sets its method against), then combined.
        dp.set_option("norm_path", 3)
        try:
            smem = call_memory(dp)
            ms_staged = time_calls(torch, step, args.steps, 2, warm_ms=0.0)
            staged_extra = smem()
            spaths = [norm_path_of(dp, lambda l=l, d=d: dp.linear_clip_accumulate(
                d[0], d[1], None, C=l.C, sigma=l.sigma, seed=l.seed, offset=l.offset,
                grad_out=d[2], norms_out=d[3])) for l, d in zip(lins, dev_in)]
        finally:
            dp.set_option("norm_path", args.norm_path)
        res["staged_path_comparison"] = {
            "note": "opt-in staged form (norm_path 3): per-sample gradient tiles stored in device "
                    "memory once, then combined; not the method's form, which keeps no "
                    "per-sample gradient",
            "norm_path": ", ".join(f"{l.name} {p}" for l, p in zip(lins, spaths)),
            "ms_per_step": round(ms_staged, 4),
            "useful_tflops": round(useful / (ms_staged * 1e-3) / 1e12, 2),
            "frac_of_peak": round(useful / (ms_staged * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "samples_per_s": round(args.batch / (ms_staged * 1e-3), 1),
            "extra_device_bytes_per_call_max": staged_extra}
    # group clipping: one clip factor per sample over the seven linears
    Xs = [X for (X, _, _, _) in dev_in]
    Gs = [G for (_, G, _, _) in dev_in]
    outs = [o for (_, _, o, _) in dev_in]
    offs = dp.consecutive_offsets([(l.dout, l.din) for l in lins])
    gmem = call_memory(dp)
    ms_group = time_calls(torch, lambda: dp.group_clip_accumulate(
        Xs, Gs, None, C=1.0, sigma=1.0, offsets=offs, grad_outs=outs), args.steps, 2, warm_ms=0.0)
    res["group_clip_layer"] = {
        "note": "the same seven linears, clipped jointly (one c_i per sample over the layer)",
        "ms": round(ms_group, 4), "useful_tflops": round(useful / (ms_group * 1e-3) / 1e12, 2),
        "frac_of_peak": round(useful / (ms_group * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "samples_per_s": round(args.batch / (ms_group * 1e-3), 1),
        "extra_device_bytes_per_call_max": gmem()}
    del Xs, Gs, outs
    if not args.no_configs:
        del dev_in
        torch.cuda.empty_cache()
        res["configs"] = measure_configs(dp, torch, args.steps, 2)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(lins, args.cpu_budget_s)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
