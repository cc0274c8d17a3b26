"""Benchmark of the causal GQA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the forward (one kernel launch) over the whole
workload, inputs already resident in HBM.  Prints ONE JSON line with the
throughput (causal FLOP / s: 4*D per kept (query, key) pair and query head),
the roofline of the kernel (with the clock it ran at and the matrix-core and
exponential ceilings measured at that occupancy), an oracle-match check on sampled query tokens of
the benchmarked output, and the fp64 CPU oracle's own throughput on a bounded
sample of the same workload.  Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "causal GQA fwd TFLOP/s (bf16) at S=10231, % of MFMA peak; oracle-match"
# MI355X dense bf16 MFMA peak as AMD publishes it: 256 CU x 4096 flop/clk x 2.4 GHz.
PEAK_BF16_TFLOPS = 2516.6


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-seconds", type=float, default=1.2,
                    help="untimed launches of the same step, for at least this long, before "
                         "the warmup steps: the board ramps its clock over the first tens of ms "
                         "of load, and the clock readings refresh about once a second")
    ap.add_argument("--workload", default=workloads.PRIMARY,
                    choices=sorted(workloads.ALL_WORKLOADS))
    ap.add_argument("--path", default="fused",
                    choices=("fused", "splitkv", "prologue", "pool", "qpro"),
                    help="fused: one kernel per call (the default, the benchmarked path); "
                         "splitkv: per-split partials through a workspace, then a merge kernel; "
                         "prologue: the Q/K RMS norm + RoPE kernel alone (HBM-bound); "
                         "pool: reference-video token pooling of the workload's prompt length; "
                         "qpro: the Q/K prologue + causal forward, two passes vs Q fused")
    ap.add_argument("--splits", type=int, default=4, help="KV splits of the splitkv path")
    ap.add_argument("--head-major", action="store_true",
                    help="bidirectional workloads: write O as [Hq, S, D]")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target wall time of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true", help="skip the oracle-match sample")
    ap.add_argument("--no-calib", action="store_true",
                    help="skip the matrix-core and exponential calibration loops")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (calibrates the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


def copy_probe(mib: int) -> None:
    """One plain copy kernel of a known size, for scaling the HBM byte counters."""
    import torch

    n = mib * 1024 * 1024
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n}), flush=True)


# the benchmarked kernel's source: the head-dim-128 forward (its statements, its launch shape,
# its generated phases, and the shared parameter block / helpers it includes)
KERNEL_SOURCES = ("gqa_fwd_wide_kernel.hpp", "tile_phases.inc", "gqa_fwd_kernel.hpp")
KERNEL_NAME = "gqa_fwd_wide_kernel<WideConfig<128, 8>, false, true, false>"
# counter runs of that kernel on the benchmarked workload (trace, utilisation, HBM traffic)
PROFILE = "gqa_fwd_wide_s10231.txt"


def kernel_source_hash() -> str:
    """sha256 over the benchmarked kernel's source files, in KERNEL_SOURCES order."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "causal_grouped_query_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded(profile: str, key: str):
    """A figure recorded in profiles/<profile> for the current kernel source, or None.

    The file holds a line `<key>: VALUE source_sha256: H`; the figure applies only while the
    kernel's source (KERNEL_SOURCES, hashed in that order) is still H."""
    path = os.path.join(ROOT, "profiles", profile)
    want = kernel_source_hash()
    try:
        with open(path) as f:
            for line in f:
                if line.startswith(key + ":"):
                    parts = line.split()
                    if parts[3] == want:
                        return float(parts[1])
    except (OSError, IndexError, ValueError):
        pass
    return None


def _int_or_none(x):
    return None if x is None else int(x)


class ClockSampler:
    """Reads the shader (gfx) clock of every XCD and the socket power from amdsmi's
    gpu_metrics on a thread while the launches run.  The firmware refreshes that table about
    once a second (its system_clock_counter field changes then), so the reader polls every
    few ms from the warmup on and keeps each refresh published inside the timed region
    [begin, end] once.  Reports nothing (None) where amdsmi is missing or refuses."""

    def __init__(self, period_s: float = 0.005):
        self.period = period_s
        self.samples = []   # (time, table counter, mean current gfxclk over XCDs, XCD clocks, W)
        self.error = None
        self.thread = None
        self.stop_flag = False
        self.begin = self.end = self.window_begin = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            self._sample()          # fails here, not in the thread, if the call is refused
        except Exception as e:      # noqa: BLE001 -- any failure just disables the sampler
            self.amdsmi = None
            self.error = f"{type(e).__name__}: {e}"[:200]

    @staticmethod
    def _valid(x):
        return isinstance(x, int) and 0 < x < 100000

    def _sample(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if self._valid(c)]
        if not clks and self._valid(m.get("current_gfxclk")):
            clks = [m["current_gfxclk"]]
        pw = m.get("current_socket_power")
        self.samples.append((time.perf_counter(), m.get("system_clock_counter"),
                             sum(clks) / len(clks) if clks else None, clks,
                             pw if self._valid(pw) else None))

    def _run(self):
        while not self.stop_flag:
            try:
                self._sample()
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"[:200]
                return
            time.sleep(self.period)

    def start(self):
        if self.amdsmi is not None:
            import threading

            self.thread = threading.Thread(target=self._run, daemon=True)
            self.thread.start()

    def stop(self):
        self.stop_flag = True
        if self.thread is not None:
            self.thread.join()
        if self.amdsmi is not None:
            try:
                self.amdsmi.amdsmi_shut_down()
            except Exception:       # noqa: BLE001
                pass

    def refreshes(self):
        """The table refreshes first seen inside [window_begin, end], one sample each
        (window_begin defaults to the start of the timed region)."""
        lo = self.window_begin if self.window_begin is not None else self.begin
        if lo is None or self.end is None:
            return []
        before = [smp[1] for smp in self.samples if smp[0] < lo]
        seen = {before[-1]} if before else set()
        out = []
        for smp in self.samples:
            if lo <= smp[0] <= self.end and smp[1] not in seen and smp[2] is not None:
                seen.add(smp[1])
                out.append(smp)
        return out

    def summary(self):
        fresh = self.refreshes()
        if not fresh:
            return {"source": "amdsmi gpu_metrics", "mhz_mean": None,
                    "error": self.error or "the metrics table was not refreshed inside the "
                                           "sampled window"}
        c = np.array([smp[2] for smp in fresh])
        out = {"source": "amdsmi gpu_metrics current_gfxclks (mean over the 8 XCDs), each "
                         "firmware refresh (about 1/s) published from 0.25 s into the settle "
                         "launches to the end of the timed launches",
               "refreshes": int(len(c)), "mhz_mean": round(float(c.mean()), 1),
               "xcd_mhz_last": fresh[-1][3]}
        pw = [smp[4] for smp in fresh if smp[4] is not None]
        if pw:
            out["socket_power_w_mean"] = round(float(np.mean(pw)), 1)
        return out


def to_device(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def reference(oracle, inp, w, tokens):
    """The oracle's (O, LSE) for the sampled query tokens of workload w."""
    if not w.causal:
        return oracle.gqa_bidirectional(inp["q"], inp["k"], inp["v"], w.scale, tokens=tokens)
    return oracle.gqa_causal_varlen(inp["q"], inp["k"], inp["v"], w.cu_seqlens, w.scale,
                                    tokens=tokens)


def calibration_loops(stream, achieved_tflops: float, settle_s: float = 0.3,
                      launches: int = 60, iters: int = 4096) -> dict:
    """The matrix-core and exponential ceilings at the clock the GPU holds
    (h3attn_calib_loop, one wave per SIMD, the attention kernel's occupancy; and the MFMA
    loop once more with two waves per SIMD, to show whether issue or power sets it).  Each loop
    first runs untimed for settle_s so the clock settles to its own load, then `launches`
    launches are timed with events; the in-kernel stamps of the last one give the clock
    and each wave's own cycles per instruction."""
    import torch

    import causal_grouped_query_amd as h3

    ncu = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    stamps = torch.zeros((2 * ncu * 4, 4), dtype=torch.int64, device="cuda")
    sink = torch.empty(2 * ncu * 256, dtype=torch.float32, device="cuda")
    out = {}
    for kind, name, per_iter, wps in ((h3.CALIB_MFMA, "mfma_loop", 8, 1),
                                      (h3.CALIB_MFMA_ZERO, "mfma_loop_zero_operands", 8, 1),
                                      (h3.CALIB_EXP, "exp_loop", 16, 1),
                                      (h3.CALIB_MFMA_PAIRED, "mfma_loop_two_waves_per_simd", 8, 2)):
        nwg = ncu * wps

        def run():
            return h3.calib_loop(kind, nwg, iters, stream=stream, stamps=stamps, sink=sink)[1]

        t = time.perf_counter()
        while time.perf_counter() - t < settle_s:
            for _ in range(10):
                run()
            torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(launches):
            khz = run()
        b.record(stream)
        b.synchronize()
        seconds = a.elapsed_time(b) * 1e-3 / launches
        st = stamps[: nwg * 4].cpu().numpy().astype(np.float64)
        cycles, ticks = st[:, 1] - st[:, 0], st[:, 3] - st[:, 2]
        ghz = float(np.median(cycles / (ticks / (khz * 1e3)))) / 1e9 if khz > 0 else None
        waves = nwg * 4
        # per SIMD, from the event-timed launches at the stamped clock (launch overhead
        # included); and each wave's own loop, from its stamps
        per_simd = (ghz * 1e9 * seconds / (iters * per_iter * wps)) if ghz else None
        entry = {"cycles_per_instruction_per_simd": round(per_simd, 2) if per_simd else None,
                 "wave_loop_cycles_per_instruction":
                     round(float(np.median(cycles)) / (iters * per_iter), 2),
                 "clock_ghz": round(ghz, 3) if ghz else None,
                 "launch_ms": round(seconds * 1e3, 4), "waves_per_simd": wps,
                 "workgroups": nwg, "iterations": iters}
        if kind == h3.CALIB_MFMA_PAIRED:
            tflops = waves * iters * per_iter * 32768 / seconds / 1e12
            entry.update({"instruction": "v_mfma_f32_32x32x16_bf16, random bf16 operands, "
                                         "two waves per SIMD",
                          "tflops": round(tflops, 1),
                          "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)})
        elif kind == h3.CALIB_MFMA:
            tflops = waves * iters * per_iter * 32768 / seconds / 1e12
            entry.update({"instruction": "v_mfma_f32_32x32x16_bf16, random bf16 operands",
                          "tflops": round(tflops, 1),
                          "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                          "kernel_frac_of_loop": round(achieved_tflops / tflops, 4)})
        elif kind == h3.CALIB_MFMA_ZERO:
            tflops = waves * iters * per_iter * 32768 / seconds / 1e12
            entry.update({"instruction": "v_mfma_f32_32x32x16_bf16, all-zero operands "
                                         "(no datapath toggling; not a ceiling for real data)",
                          "tflops": round(tflops, 1),
                          "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4)})
        else:
            entry.update({"instruction": "v_exp_f32",
                          "g_exp_per_s": round(waves * 64 * iters * per_iter / seconds / 1e9, 1)})
        out[name] = entry
    return out


def host_cpu_model() -> str | None:
    """The host CPU's model name (first processor in /proc/cpuinfo), None where unknown."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, w, target_s: float):
    """fp64 oracle throughput on a bounded sample of query tokens (all heads)."""
    import oracle

    rng = np.random.Generator(np.random.PCG64(w.seed + 77))
    T = w.total_tokens
    starts = np.concatenate([[0], np.cumsum(w.seqlens)[:-1]])

    def pair_count(tokens):
        # visible keys of each packed token: its local position + 1 (all S keys without
        # the causal mask)
        if not w.causal:
            return int(len(tokens) * T)
        seq = np.searchsorted(np.cumsum(w.seqlens), tokens, side="right")
        return int(np.sum(tokens - starts[seq] + 1))

    def run(tokens):
        t0 = time.perf_counter()
        reference(oracle, inp, w, tokens)
        return time.perf_counter() - t0

    calib = rng.integers(0, T, size=16)
    dt = run(calib)
    rate = 4 * w.head_dim * w.n_q_heads * pair_count(calib) / max(dt, 1e-6)   # flop/s
    per_token = 4 * w.head_dim * w.n_q_heads * (T / len(w.seqlens)) / (2 if w.causal else 1)
    # batches of uniformly drawn tokens until about target_s of oracle time is spent (the
    # first estimate of the rate comes from a few tokens and can be off by a few times)
    n, dt, flop = 0, 0.0, 0
    while dt < 0.8 * target_s and n < T:
        m = int(np.clip((target_s - dt) * rate / per_token, 8, T - n))
        batch = np.sort(rng.integers(0, T, size=m))
        log(f"cpu baseline: {m} sampled query tokens x {w.n_q_heads} heads "
            f"(~{m * per_token / rate:.1f} s expected)")
        dt += run(batch)
        flop += 4 * w.head_dim * w.n_q_heads * pair_count(batch)
        n += m
        rate = flop / max(dt, 1e-6)
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": (f"{n} query tokens drawn uniformly from the {w.name} workload, all "
                   f"{w.n_q_heads} heads, full {'causal ' if w.causal else ''}rows; "
                   f"{flop:.3e} flop in {dt:.1f} s"),
    }


def bench_prologue(args, w, inp, torch, h3):
    """The Q/K prologue (RMS norm with synthetic weights + RoPE, theta 1e6) on the workload's
    Q and K: HBM-bound, reported in GB/s of algorithmic traffic against 8 TB/s."""
    HBM_PEAK_GBS = 8000.0
    D = w.head_dim
    rng = np.random.Generator(np.random.PCG64(w.seed + 900))
    wq_bits = workloads.f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    wk_bits = workloads.f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    q, k = to_device(inp["q"], torch), to_device(inp["k"], torch)
    wq, wk = to_device(wq_bits, torch), to_device(wk_bits, torch)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    stream = torch.cuda.current_stream()

    def step():
        h3.qk_norm_rope(q, k, wq, wk, eps=1e-6, rope=True, rope_theta=1e6, q_out=qo, k_out=ko,
                        stream=stream)

    for _ in range(args.warmup):
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    ms_per_step = starts[0].elapsed_time(ends[-1]) / args.steps
    T = w.total_tokens
    elems = T * (w.n_q_heads + w.n_kv_heads) * D
    nbytes = 2 * elems * 2 + 2 * 2 * D                     # read + write bf16, two weights
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (float(per_launch.mean()) * 1e-3) / 1e9
    result = {
        "metric": f"Q/K RMS norm + RoPE prologue GB/s (bf16), {w.name}",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": T, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": D, "path": "prologue",
                   "norm": "RMS, synthetic U(0.5,1.5) weights, eps 1e-6", "rope_theta": 1e6},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "qk_prologue_kernel",
                     "avg_launch_ms": round(float(per_launch.mean()), 5),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_check or not args.no_cpu_baseline:
        import oracle

        t0 = time.perf_counter()
        rq = oracle.qk_norm_rope(inp["q"], weight=wq_bits, eps=1e-6, rope=True, theta=1e6)
        rk = oracle.qk_norm_rope(inp["k"], weight=wk_bits, eps=1e-6, rope=True, theta=1e6)
        dt = time.perf_counter() - t0
        worst = 0.0
        for gpu, ref in ((qo, rq), (ko, rk)):
            g = gpu.float().cpu().double().numpy()
            rms = np.sqrt((ref ** 2).mean(axis=-1, keepdims=True))
            bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * rms
            worst = max(worst, float((np.abs(g - ref) / bound).max()))
        if not args.no_check:
            result["oracle_match"] = {"elements": int(elems), "worst_err_over_bound": worst,
                                      "bound": "2^-8 |exact| + 2^-16 row RMS",
                                      "pass": bool(worst <= 1.0)}
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {"value": nbytes / dt / 1e9, "unit": "GB/s",
                                      "cores": oracle.threads(),
                                      "cpu_model": host_cpu_model(), "kind": "oracle",
                                      "sample": f"the full Q and K of {w.name} ({elems} elements) "
                                                f"in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


def bench_qpro(args, w, inp, torch, h3):
    """The encoder's attention step with the Q/K prologue (RMS norm with synthetic weights +
    RoPE, theta 1e6), two ways on the same inputs: the prologue kernel over Q and K then the
    causal forward (two passes), and the K-only prologue then the causal forward that
    normalises and rotates Q as it loads it (fused).  value = causal flop / fused step time."""
    D = w.head_dim
    rng = np.random.Generator(np.random.PCG64(w.seed + 900))
    wq_bits = workloads.f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    wk_bits = workloads.f32_to_bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    q, k, v = to_device(inp["q"], torch), to_device(inp["k"], torch), to_device(inp["v"], torch)
    wq, wk = to_device(wq_bits, torch), to_device(wk_bits, torch)
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((w.n_q_heads, w.total_tokens), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def two_pass():
        h3.qk_norm_rope(q, k, wq, wk, q_out=qo, k_out=ko, stream=stream)
        h3.gqa_causal_fwd(qo, ko, v, softmax_scale=w.scale, out=o, lse=lse, stream=stream)

    def fused():
        h3.qk_norm_rope(None, k, None, wk, k_out=ko, stream=stream)
        h3.gqa_causal_qnorm_rope_fwd(q, ko, v, q_norm_weight=wq, softmax_scale=w.scale, out=o,
                                     lse=lse, stream=stream)

    def timed(step):
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    # alternate so both see the same clock; report the median of three rounds each
    t2, t1 = [], []
    for _ in range(3):
        t2.append(timed(two_pass))
        t1.append(timed(fused))
    ms_two, ms_fused = float(np.median(t2)), float(np.median(t1))
    flop = w.flop()
    result = {
        "metric": f"Q/K norm+RoPE + causal GQA fwd TFLOP/s (bf16), {w.name}",
        "value": round(flop / (ms_fused * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_fused, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": w.total_tokens, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": D, "path": "qpro",
                   "norm": "RMS, synthetic U(0.5,1.5) weights, eps 1e-6", "rope_theta": 1e6,
                   "ms_two_pass": round(ms_two, 5), "ms_fused": round(ms_fused, 5),
                   "fused_over_two_pass": round(ms_two / ms_fused, 4)},
    }
    if not args.no_check:
        import oracle

        fused()
        torch.cuda.synchronize()
        rq = workloads.f32_to_bf16_bits(oracle.qk_norm_rope(inp["q"], weight=wq_bits)
                                        .astype(np.float32))
        rk = workloads.f32_to_bf16_bits(oracle.qk_norm_rope(inp["k"], weight=wk_bits)
                                        .astype(np.float32))
        tokens = workloads.sample_tokens(w.seqlens, 8, seed=w.seed + 1000)
        o_ref, lse_ref = oracle.gqa_causal(rq, rk, inp["v"], w.scale, tokens=tokens)
        tok_t = torch.from_numpy(tokens).to("cuda")
        o_s = o.index_select(0, tok_t).double().cpu().numpy()
        l_s = lse.index_select(1, tok_t).double().cpu().numpy()
        rel = float(np.linalg.norm(o_s - o_ref) / np.linalg.norm(o_ref))
        mx = float(np.abs(o_s - o_ref).max())
        lmx = float(np.abs(l_s - lse_ref).max())
        result["oracle_match"] = {"tokens": int(len(tokens)), "rel_l2": rel, "max_abs": mx,
                                  "lse_abs": lmx,
                                  "pass": bool(rel <= 5e-3 and mx <= 2e-2 and lmx <= 1e-3)}
    print(json.dumps(result), flush=True)


def bench_pool(args, w, torch, h3):
    """Token pooling of a prompt of the workload's length: the issue's ~7500 reference-video
    tokens ([2300, 9800) of 10231) pooled by 4, C = 4096 synthetic embedding channels.
    HBM-bound, reported in GB/s of algorithmic traffic against 8 TB/s."""
    HBM_PEAK_GBS = 8000.0
    T, C = w.total_tokens, 4096
    begin, end, factor = min(2300, T), min(9800, T), 4
    rng = np.random.Generator(np.random.PCG64(w.seed + 950))
    x_bits = workloads.f32_to_bf16_bits(rng.standard_normal((T, C)).astype(np.float32))
    x = to_device(x_bits, torch)
    n = h3.pool_tokens_out_len(T, begin, end, factor)
    out = torch.empty((n, C), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        h3.pool_tokens(x, begin, end, factor, out=out, stream=stream)

    for _ in range(args.warmup):
        step()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    ms_per_step = starts[0].elapsed_time(ends[-1]) / args.steps
    nbytes = (T + n) * C * 2
    achieved = nbytes / (float(per_launch.mean()) * 1e-3) / 1e9
    result = {
        "metric": f"reference-video token pooling GB/s (bf16), {T} tokens",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": T, "channels": C, "span": [begin, end],
                   "factor": factor, "out_tokens": n, "path": "pool"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pool_tokens_kernel",
                     "avg_launch_ms": round(float(per_launch.mean()), 5),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    if not args.no_check or not args.no_cpu_baseline:
        import oracle

        t0 = time.perf_counter()
        ref = oracle.pool_tokens(x_bits, begin, end, factor)
        dt = time.perf_counter() - t0
        g = out.float().cpu().double().numpy()
        bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * np.abs(ref).max()
        worst = float((np.abs(g - ref) / bound).max())
        if not args.no_check:
            result["oracle_match"] = {"elements": int(n * C), "worst_err_over_bound": worst,
                                      "pass": bool(worst <= 1.0)}
        if not args.no_cpu_baseline:
            result["cpu_baseline"] = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1,
                                      "cpu_model": host_cpu_model(),
                                      "kind": "oracle", "sample": f"the full [{T}, {C}] prompt, "
                                      f"numpy float64 loops, in {dt:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by KV head or sequence with no communication, see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import causal_grouped_query_amd as h3

    w = workloads.ALL_WORKLOADS[args.workload]
    if args.path == "splitkv" and (w.varlen or not w.causal):
        print("bench.py: the split-KV path takes one causal sequence", file=sys.stderr)
        sys.exit(2)
    log(f"workload {w.name}: seqlens={w.seqlens} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
        f"D={w.head_dim}")
    if args.path == "pool":
        bench_pool(args, w, torch, h3)
        return
    inp = workloads.generate(w)
    if args.path == "prologue":
        bench_prologue(args, w, inp, torch, h3)
        return
    if args.path == "qpro":
        if w.varlen or not w.causal:
            print("bench.py: the qpro path takes one causal sequence", file=sys.stderr)
            sys.exit(2)
        bench_qpro(args, w, inp, torch, h3)
        return
    q, k, v = to_device(inp["q"], torch), to_device(inp["k"], torch), to_device(inp["v"], torch)
    o = (torch.empty((w.n_q_heads, w.total_tokens, w.head_dim), dtype=torch.bfloat16,
                     device="cuda") if args.head_major else torch.empty_like(q))
    lse = torch.empty((w.n_q_heads, w.total_tokens), dtype=torch.float32, device="cuda")
    cu = torch.tensor(w.cu_seqlens, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    workspace = None
    if args.path == "splitkv":
        need = h3.splitkv_workspace_bytes(w.total_tokens, w.n_q_heads, w.head_dim, args.splits)
        workspace = torch.empty(need, dtype=torch.uint8, device="cuda")

    def step():
        if args.path == "splitkv":
            h3.gqa_causal_splitkv_fwd(q, k, v, args.splits, softmax_scale=w.scale, out=o, lse=lse,
                                      workspace=workspace, stream=stream)
        elif not w.causal:
            h3.gqa_fwd(q, k, v, causal=False, head_major_out=args.head_major,
                       softmax_scale=w.scale, out=o, lse=lse, stream=stream)
        elif w.varlen:
            h3.gqa_causal_varlen_fwd(q, k, v, cu, max(w.seqlens), softmax_scale=w.scale, out=o,
                                     lse=lse, stream=stream)
        else:
            h3.gqa_causal_fwd(q, k, v, softmax_scale=w.scale, out=o, lse=lse, stream=stream)

    sampler = ClockSampler()
    sampler.start()
    settle_steps, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(20):
            step()
        settle_steps += 20
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_settle
    sampler.window_begin = t_settle + min(0.25, settle_s)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"settle {settle_steps} launches in {settle_s:.2f} s, warmup {args.warmup} done")

    # timed region: K steps; events on the launch stream around each launch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = sampler.begin = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    sampler.end = time.perf_counter()
    wall = sampler.end - t0
    sampler.stop()
    clock = sampler.summary()
    log(f"shader clock during the timed launches: {clock}")
    per_launch = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])  # ms
    total_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step (wall {wall * 1e3 / args.steps:.4f}"
        f" ms/step), launch median {np.median(per_launch):.4f} ms min {per_launch.min():.4f} ms")

    flop = w.flop()
    value = flop / (ms_per_step * 1e-3) / 1e12
    avg_launch_ms = float(per_launch.mean())
    achieved = flop / (avg_launch_ms * 1e-3) / 1e12

    calib = None
    if not args.no_calib:
        try:
            calib = calibration_loops(stream, achieved)
            log(f"calibration loops: {calib}")
        except Exception as e:  # reported in the line; the measurement above stands
            calib = {"error": f"{type(e).__name__}: {e}"}

    primary = w.name == workloads.PRIMARY and args.path == "fused"
    # MFMA peak at the clock the part actually ran: 256 CU x 4096 bf16 flop/clk x f
    f_ghz = clock["mhz_mean"] / 1e3 if clock.get("mhz_mean") else None
    clock["peak_at_clock_tflops"] = round(256 * 4096 * f_ghz / 1e3, 1) if f_ghz else None
    clock["frac_at_clock"] = (round(achieved / clock["peak_at_clock_tflops"], 4)
                              if f_ghz else None)
    counter_ghz = recorded(PROFILE, "clock_ghz") if primary else None
    clock["counter_clock_ghz"] = counter_ghz
    clock["counter_clock_note"] = ("GRBM_GUI_ACTIVE per XCD / kernel duration, recorded in "
                                   f"profiles/{PROFILE} for this source"
                                   if counter_ghz else "no counter run of this source recorded")

    metric = METRIC
    if not primary:
        metric = (f"{'causal' if w.causal else 'bidirectional'} GQA fwd TFLOP/s (bf16), "
                  f"{w.name}, {args.path} path; oracle-match")
    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {"launches": settle_steps, "seconds": round(settle_s, 3),
                   "note": "untimed launches of the same step before the warmup, so the timed "
                           "launches run at the board's steady clock"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "seq_lens": list(w.seqlens),
            "total_tokens": w.total_tokens,
            "n_q_heads": w.n_q_heads,
            "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim,
            "causal": w.causal,
            **({"o_layout": "[Hq,S,D]"} if args.head_major else {}),
            "path": args.path,
            **({"splits": args.splits} if args.path == "splitkv" else {}),
            "inputs": ("N(0,1) bf16, seeded" if w.kind == "normal" else
                       "stress: 4 N(0,1) Q/K, U(-1,1) V, 5% shared spike keys, seeded"),
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": _int_or_none(recorded(PROFILE, "traffic_bytes_per_launch")
                                    if primary else None),
            "kernel": (KERNEL_NAME if args.path == "fused" else
                       "gqa_causal_fwd_kernel<split> + merge_splits_kernel (one call, timed together)"),
            "avg_launch_ms": round(avg_launch_ms, 5),
            "algorithmic_flop_per_launch": flop,
            "shader_clock": clock,
            **({"calibration": calib} if calib is not None else {}),
        },
    }

    if not args.no_check:
        import oracle

        tokens = workloads.sample_tokens(w.seqlens, 16, seed=w.seed + 1000)
        o_ref, lse_ref = reference(oracle, inp, w, tokens)
        idx = torch.from_numpy(tokens).cuda()
        o_tok = o.transpose(0, 1) if args.head_major else o      # [T, Hq, D] view
        o_s = o_tok.index_select(0, idx).double().cpu().numpy()
        l_s = lse.index_select(1, idx).double().cpu().numpy()
        rel = float(np.linalg.norm(o_s - o_ref) / np.linalg.norm(o_ref))
        mx = float(np.abs(o_s - o_ref).max())
        lmx = float(np.abs(l_s - lse_ref).max())
        result["oracle_match"] = {
            "tokens": int(len(tokens)), "rel_l2": rel, "max_abs": mx, "lse_abs": lmx,
            "pass": bool(rel <= 5e-3 and mx <= 2e-2 and lmx <= 1e-3)}
        log(f"oracle match on {len(tokens)} tokens: rel_l2={rel:.2e} max_abs={mx:.2e} "
            f"lse_abs={lmx:.2e}")

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_seconds)
        log(f"cpu baseline {result['cpu_baseline']['value']:.4f} TFLOP/s on "
            f"{result['cpu_baseline']['cores']} threads")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
