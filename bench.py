"""Benchmark of the FP8 W8A8 linear-layer hot path on one MI355X.

Default workload: one Qwen3-8B-shaped decoder block at decode (M = 64 tokens, hidden 4096,
7 linears: q/o 4096x4096, k/v 1024x4096, gate/up 12288x4096, down 4096x12288). One step is the
whole hot path over that block:

  1. per-step re-quantization of all 7 bf16 weights to E4M3 with 128x128 FP32 block scales,
     in one batched launch,
  2. dynamic 1x128 per-token quantization of each linear's bf16 input activation,
  3. the blockwise-scaled FP8 GEMMs (bf16 output).

The weights are laid out as a serving engine keeps them: q/k/v concatenated along N (6144x4096)
and gate/up concatenated (24576x4096), so the block is 4 GEMMs over 4 activation quantizations
(one per distinct input), with the same bytes and FLOPs as the 7 separate linears.

Inputs are seeded synthetic tensors resident in HBM (weights N(0, 0.02) with 0.1 % x10 outliers,
activations N(0, 1) with 1 % x20 outlier channels), rotated over enough copies that every step
reads more than 1 GiB, so the 256 MiB Infinity Cache cannot hold a step's working set.

Prints one JSON line. `value` is the step's algorithmic HBM traffic (bytes each kernel must move
at least once) divided by the step time, in GB/s; per-part GB/s and the GEMMs' TFLOP/s are
reported beside it. `roofline` describes the dominant kernel (the weight re-quantization), timed
with HIP events around each of its launches inside the timed region. `cpu_baseline` times the
CPU oracle on a bounded sample of the same step.

Other workloads (`--workload`): qwen3-8b-prefill (M = 8192), llama31-8b-mlp (M in {256, 4096}),
llama31-8b-weight-sync (32 layers of weights), qwen3-30b-a3b-moe (grouped expert GEMMs),
qwen3-8b-kv-cache (per-tensor Q/K/V recalibration and FP8 KV-cache store over 36 layers),
qwen3-8b-backward (FP8 Dgrad and Wgrad of the decoder block's linears over 8192 tokens).
"""

from __future__ import annotations

import argparse
import json
import os
import queue
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
ROTATE_BYTES = 1 << 30
COPY_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-8b-decode",
                    choices=["qwen3-8b-decode", "qwen3-8b-prefill", "llama31-8b-mlp",
                             "llama31-8b-weight-sync", "qwen3-30b-a3b-moe", "qwen3-8b-kv-cache",
                             "qwen3-8b-backward", "qwen3-8b-decode-fused-act"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--scales", default="fp32", choices=["fp32", "pow2"],
                    help="block-scale format: fp32(amax/448) (default) or powers of two, whose "
                         "GEMMs apply the scales in the matrix cores (accum 'mx')")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (a known-size reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


class KernelTimer:
    """HIP events around launches of one kernel on the current stream, averaged at the end."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []
        self.bytes = 0

    def reset(self):
        self.pairs = []
        self.bytes = 0

    def launch(self, fn, nbytes):
        a = self.torch.cuda.Event(enable_timing=True)
        b = self.torch.cuda.Event(enable_timing=True)
        a.record()
        out = fn()
        b.record()
        self.pairs.append((a, b))
        self.bytes += nbytes
        return out

    def result(self):
        ms = sum(a.elapsed_time(b) for a, b in self.pairs)
        n = len(self.pairs)
        return dict(launches=n, avg_us=1e3 * ms / max(n, 1),
                    gbs=self.bytes / max(ms, 1e-12) / 1e6)


# --------------------------------------------------------------------------------- workloads


def w_bytes(N, K):
    """Algorithmic bytes of re-quantizing a bf16 [N][K] weight: read 2, write 1 per element,
    plus the float32 scale of each 128x128 block."""
    return 3 * N * K + 4 * (N // 128) * (K // 128)


def a_bytes(M, K):
    return 3 * M * K + 4 * M * (K // 128)


def g_bytes(M, N, K, out_bytes=2):
    return M * K + N * K + out_bytes * M * N + 4 * M * (K // 128) + 4 * (N // 128) * (K // 128)


#: Linears that read the same input, stored concatenated along N as a serving engine does
#: (per-128x128-block quantization of the concatenation equals that of the parts: every N is a
#: multiple of 128). Each group is one activation quantization and one GEMM.
FUSED_GROUPS = (("qkv_proj", ("q_proj", "k_proj", "v_proj")), ("gate_up_proj", ("gate_proj", "up_proj")))


def serving_layout(linears):
    """(name, N, K) groups of `linears` with the FUSED_GROUPS merged (consecutive, same K)."""
    out, i = [], 0
    while i < len(linears):
        for fused, parts in FUSED_GROUPS:
            names = tuple(l[0] for l in linears[i:i + len(parts)])
            if names == parts and len({l[2] for l in linears[i:i + len(parts)]}) == 1:
                out.append((fused, sum(l[1] for l in linears[i:i + len(parts)]), linears[i][2]))
                i += len(parts)
                break
        else:
            out.append(tuple(linears[i]))
            i += 1
    return tuple(out)


class DenseBlock:
    """The GEMMs of one decoder block at a given M: re-quantize, quantize, multiply.

    The per-step weight re-quantization of all linears is one batched launch (timed on its own
    with HIP events); the activation quantizations and GEMMs of the block are captured once
    per weight copy into a HIP graph and replayed, so host launch overhead does not pace the GPU.
    """

    def __init__(self, torch, fq, synth, linears, M, seed, requant=True, scales="fp32"):
        self.torch, self.fq = torch, fq
        self.scales = scales
        self.accum = "mx" if scales == "pow2" else None
        self.linears, self.M, self.requant = linears, M, requant
        dev = "cuda"
        wbytes = sum(2 * N * K for _, N, K in linears)
        self.copies = max(1, -(-ROTATE_BYTES // wbytes)) if requant else 1
        self.w = [[synth.weight_bf16(N, K, seed=seed + 100 * c + i, outlier_frac=0.001, device=dev)
                   for i, (_, N, K) in enumerate(linears)] for c in range(self.copies)]
        self.x = [synth.act_bf16(M, K, seed=seed + 7 + i, device=dev)
                  for i, (_, N, K) in enumerate(linears)]
        self.wq = [[torch.empty((N, K), dtype=torch.uint8, device=dev) for _, N, K in linears]
                   for _ in range(self.copies)]
        self.sw = [[torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
                    for _, N, K in linears] for _ in range(self.copies)]
        self.descs = [fq.weight_descs(self.w[c], self.wq[c], self.sw[c]) for c in range(self.copies)]
        self.xq = [torch.empty((M, K), dtype=torch.uint8, device=dev) for _, N, K in linears]
        self.sa = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _, N, K in linears]
        self.y = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _, N, K in linears]
        self.ws = []
        for _, N, K in linears:
            nb = fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, M, N, K)
            self.ws.append(fq.new_workspace(nb, dev))
        for c in range(self.copies):  # every copy holds valid codes before the first replay
            self.requant_step(c)
        self.it = 0
        self.bytes_w = sum(w_bytes(N, K) for _, N, K in linears) if requant else 0
        self.bytes_a = sum(a_bytes(M, K) for _, N, K in linears)
        self.bytes_g = sum(g_bytes(M, N, K) for _, N, K in linears)
        self.flops = sum(2 * M * N * K for _, N, K in linears)
        self.t_w = KernelTimer(torch)
        self.graphs = None

    def roofline_us(self):
        """Roofline time of the captured part: per GEMM max(flops / FP8 peak, bytes / HBM peak),
        plus the activation quantizations at HBM peak."""
        t = sum(max(2 * self.M * N * K / (FP8_PEAK_TFLOPS * 1e12), g_bytes(self.M, N, K) /
                    (HBM_PEAK_GBS * 1e9)) for _, N, K in self.linears)
        return 1e6 * (t + self.bytes_a / (HBM_PEAK_GBS * 1e9))

    def requant_step(self, c):
        self.fq.quant_weights(None, None, None, descs=self.descs[c], scale=self.scales)

    def linears_step(self, c):
        fq = self.fq
        for i in range(len(self.linears)):
            fq.quant_act(self.x[i], self.xq[i], self.sa[i], scale=self.scales)
            fq.gemm(self.xq[i], self.sa[i], self.wq[c][i], self.sw[c][i], y=self.y[i], accum=self.accum,
                    workspace=self.ws[i])

    def capture(self):
        torch = self.torch
        for c in range(self.copies):  # warm the launch paths (LDS attributes) before capture
            self.linears_step(c)
        torch.cuda.synchronize()
        self.graphs = []
        for c in range(self.copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.linears_step(c)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def step(self, timed=False):
        c = self.it % self.copies
        self.it += 1
        if self.requant:
            if timed:
                self.t_w.launch(lambda: self.requant_step(c), self.bytes_w)
            else:
                self.requant_step(c)
        self.graphs[c].replay()

    def time_gemm(self, i, reps):
        """HIP events around `reps` eager launches of GEMM i alone (its activation already
        quantized), on the current stream: the per-launch duration of that kernel."""
        fq, t = self.fq, KernelTimer(self.torch)
        c = 0
        g = lambda: fq.gemm(self.xq[i], self.sa[i], self.wq[c][i], self.sw[c][i], y=self.y[i],
                            accum=self.accum, workspace=self.ws[i])
        fq.quant_act(self.x[i], self.xq[i], self.sa[i], scale=self.scales)
        for _ in range(3):
            g()
        for _ in range(reps):
            t.launch(g, 0)
        self.torch.cuda.synchronize()
        return t.result()["avg_us"]

    def time_linears(self, reps):
        """Kernel time of the captured act-quant + GEMM part alone (graph replays)."""
        torch = self.torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(reps):
            self.graphs[r % self.copies].replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps


# ---------------------------------------------------------------------------- measured traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "quant_weight_blk128__qwen3-8b-decode-step.traffic.txt")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_big_kernel__qwen3-8b-prefill.traffic.txt")


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch of a kernel from committed FETCH_SIZE / WRITE_SIZE counter runs
    (scaled by a 1 GiB copy), or None if the kernel's sources have changed since the counters
    were taken."""
    import hashlib

    try:
        with open(path) as f:
            d = json.load(f)
        h = hashlib.sha256()
        for rel in d["source_files"]:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != d["source_sha256"]:
            return None
        return float(d["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# --------------------------------------------------------------------------------- gpu clocks

def gpu_clocks():
    """Engine and memory clock tables of the visible GPUs from the driver's sysfs files (MHz; the
    entry the driver marks current is reported as `*_now_mhz`), or None where they are not
    readable. The current entry is the driver's report, not a cycle count: under a vendor FP8
    GEMM it read a level at which that GEMM's throughput would exceed the matrix cores' peak, so
    it is printed as context and used for nothing else."""
    import glob

    def table(path):
        try:
            with open(path) as f:
                rows = [l.split() for l in f.read().strip().splitlines()]
        except OSError:
            return None, None
        mhz, now = [], None
        for r in rows:
            if len(r) >= 2 and r[1].lower().endswith("mhz"):
                v = int(r[1][:-3])
                mhz.append(v)
                if "*" in r[2:]:
                    now = v
        return mhz, now

    out = []
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        sclk, sclk_now = table(dev + "/pp_dpm_sclk")
        mclk, mclk_now = table(dev + "/pp_dpm_mclk")
        if sclk is None and mclk is None:
            continue
        out.append({"card": dev.split("/")[-2], "sclk_levels_mhz": sclk, "sclk_now_mhz": sclk_now,
                    "mclk_levels_mhz": mclk, "mclk_now_mhz": mclk_now})
    return out or None


def sample_clocks(done_event, period_s=0.002, max_samples=200):
    """Engine clock of the first GPU sampled every `period_s` until `done_event` has completed:
    min / median / max of the current level (MHz) and the number of samples, plus the tables."""
    import time

    first, now = None, []
    while len(now) < max_samples:
        c = gpu_clocks()
        if not c:
            return None
        first = first or c
        if c[0]["sclk_now_mhz"] is not None:
            now.append(c[0]["sclk_now_mhz"])
        if done_event.query():
            break
        time.sleep(period_s)
    now.sort()
    out = dict(first[0])
    out.pop("sclk_now_mhz", None)
    if now:
        out.update(sclk_samples=len(now), sclk_min_mhz=now[0], sclk_median_mhz=now[len(now) // 2],
                   sclk_max_mhz=now[-1])
    return out


# ------------------------------------------------------------------------------ cpu baseline


def cpu_baseline_dense(linears, M, seed, budget_linears, min_seconds=10.0, scales="fp32"):
    """Time the CPU oracle on the linears of the step, in order and cycling, for at least
    `budget_linears` linears and `min_seconds` of oracle time (full per-linear work: weight
    re-quantization, activation quantization, GEMM)."""
    import numpy as np
    import torch

    from oracle import gemm as og
    from oracle import quant as oq
    from workloads import synth

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    total_bytes = 0
    elapsed = 0.0
    done = []
    i = 0
    while i < budget_linears or elapsed < min_seconds:
        name, N, K = linears[i % len(linears)]
        w = bits(synth.weight_bf16(N, K, seed=seed + i, outlier_frac=0.001))
        x = bits(synth.act_bf16(M, K, seed=seed + 7 + i))
        t0 = time.perf_counter()
        wq, sw = oq.quant_weight_blk128(w, scale=scales)
        xq, sa = oq.quant_act_tok128(x, scale=scales)
        og.gemm_blockscaled(xq, sa, wq, sw, out="bf16")
        elapsed += time.perf_counter() - t0
        total_bytes += w_bytes(N, K) + a_bytes(M, K) + g_bytes(M, N, K)
        done.append(name)
        i += 1
    return dict(value=total_bytes / elapsed / 1e9, unit="GB/s", cores=int(blas_threads),
                quantizer_threads=1, gemm_blas_threads=int(blas_threads),
                host_cpus=os.cpu_count(), host_cpus_usable=len(os.sched_getaffinity(0)),
                kind="oracle", seconds=elapsed,
                sample=f"{len(done)} linears of the block at M={M} ({','.join(done)}): weight "
                       f"re-quant + activation quant + fp64 GEMM each; quantizers single-threaded "
                       f"numpy, GEMM fp64 BLAS; input generation not timed")


def _quant_inputs(tensors):
    """bf16 bit patterns (uint16 numpy) of the step's tensors, each ("w", name, N, K, seed, nbytes)
    or ("x", name, M, K, seed, nbytes)."""
    import numpy as np
    import torch

    from workloads import synth

    out = []
    for kind, _, R, K, seed, _ in tensors:
        t = (synth.weight_bf16(R, K, seed=seed, outlier_frac=0.001) if kind == "w"
             else synth.act_bf16(R, K, seed=seed))
        out.append(t.view(torch.int16).numpy().view(np.uint16))
    return out


def _quantize(tensors, inputs, scales):
    from oracle import quant as oq

    for (kind, *_), t in zip(tensors, inputs):
        if kind == "w":
            oq.quant_weight_blk128(t, scale=scales)
        else:
            oq.quant_act_tok128(t, scale=scales)


def _quant_worker(tensors, scales, barrier, results):
    """One process of the all-cores run: make its share of the inputs, wait for every process,
    quantize, report (start, end) on the system-wide monotonic clock."""
    inputs = _quant_inputs(tensors)
    barrier.wait(timeout=300)
    t0 = time.monotonic()
    _quantize(tensors, inputs, scales)
    results.put((t0, time.monotonic()))


def partition_by_bytes(tensors, procs):
    """Deal the tensors (tuples whose last field is their byte count) out to `procs` shares,
    largest first, each to the share with the fewest bytes so far. Returns (shares, bytes per
    share)."""
    shares, load = [[] for _ in range(procs)], [0] * procs
    for t in sorted(tensors, key=lambda t: -t[-1]):
        j = load.index(min(load))
        shares[j].append(t)
        load[j] += t[-1]
    return shares, load


def cpu_quantizers_all_cores(linears, M, seed, scales="fp32"):
    """The oracle's two quantizers over one step's tensors (each linear's bf16 weight and its
    [M][K] activations): first one tensor after another in this process, then the same tensors
    partitioned over one process per usable core (at most one process per tensor, larger
    tensors dealt out first to the least-loaded process). The processes are fresh interpreters
    (spawn), so this must run before this process touches the GPU. Input generation is not
    timed; the all-cores time runs from the first process's start to the last one's end."""
    import multiprocessing as mp

    tensors = []
    for i, (name, N, K) in enumerate(linears):
        tensors.append(("w", name, N, K, seed + i, w_bytes(N, K)))
        tensors.append(("x", name, M, K, seed + 7 + i, a_bytes(M, K)))
    total_bytes = sum(t[5] for t in tensors)

    inputs = _quant_inputs(tensors)
    t0 = time.perf_counter()
    _quantize(tensors, inputs, scales)
    t_one = time.perf_counter() - t0
    del inputs

    procs = max(1, min(len(os.sched_getaffinity(0)), len(tensors)))
    shares, load = partition_by_bytes(tensors, procs)
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(procs), ctx.Queue()
    ps = [ctx.Process(target=_quant_worker, args=(sh, scales, barrier, results)) for sh in shares]
    for p in ps:
        p.start()
    spans, deadline = [], time.monotonic() + 600
    try:
        while len(spans) < procs:
            try:
                spans.append(results.get(timeout=1.0))
            except queue.Empty:
                # a process that ended without a result (an error) fails the run at once
                if any(p.exitcode not in (None, 0) for p in ps) or time.monotonic() > deadline:
                    raise RuntimeError("a process of the all-cores oracle run failed")
    finally:
        for p in ps:
            if p.is_alive() and len(spans) < procs:
                p.terminate()
            p.join()
    t_all = max(e for _, e in spans) - min(s for s, _ in spans)
    return dict(one_thread={"value": total_bytes / t_one / 1e9, "unit": "GB/s", "cores": 1,
                            "seconds": t_one},
                all_cores={"value": total_bytes / t_all / 1e9, "unit": "GB/s", "cores": procs,
                           "seconds": t_all, "largest_share_bytes": max(load)},
                kind="oracle",
                sample=f"weight re-quantization and 1x128 activation quantization of the "
                       f"{len(linears)} linears of the block at M={M} ({len(tensors)} tensors, "
                       f"{total_bytes / 1e6:.0f} MB of algorithmic bytes), partitioned by tensor "
                       f"over {procs} processes")


# ------------------------------------------------------------------------------------- main


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from workloads import synth

    # the oracle's quantizers on every host core: worker processes are started here, before
    # anything in this process touches the GPU
    quant_cpu = None
    profiled = ("rocprof" in os.environ.get("LD_PRELOAD", "")
                or any(k.startswith("ROCPROF") for k in os.environ))
    if args.workload == "qwen3-8b-decode" and not args.no_cpu_baseline and profiled:
        # a profiler's preloaded library may already hold the GPU: start no processes
        quant_cpu = {"skipped": "running under a profiler"}
    elif args.workload == "qwen3-8b-decode" and not args.no_cpu_baseline:
        try:
            quant_cpu = cpu_quantizers_all_cores(synth.DENSE_LINEARS_QWEN3_8B, 64, seed=6000,
                                                 scales=args.scales)
        except Exception as e:  # reported in the line; the GPU measurement goes on
            quant_cpu = {"error": f"{type(e).__name__}: {e}"}

    import fp8_blockwise_quantization_amd as fq

    torch.cuda.set_device(0)
    fq.lib()
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    dev_name = torch.cuda.get_device_name(0)
    props = torch.cuda.get_device_properties(0)

    if args.workload == "qwen3-8b-decode":
        linears, M, requant = synth.DENSE_LINEARS_QWEN3_8B, 64, True
        cfg = {"workload": "Qwen3-8B decoder block, decode step", "tokens_M": 64, "hidden": 4096,
               "linears": [list(l) for l in linears], "weight_requant_per_step": True,
               "gemm_out": "bf16", "config_index": 1}
    elif args.workload == "qwen3-8b-prefill":
        linears, M, requant = synth.DENSE_LINEARS_QWEN3_8B, 8192, False
        cfg = {"workload": "Qwen3-8B decoder block, prefill", "tokens_M": 8192, "hidden": 4096,
               "linears": [list(l) for l in linears], "weight_requant_per_step": False,
               "gemm_out": "bf16", "config_index": 2}
    elif args.workload == "llama31-8b-mlp":
        return run_mlp(args, torch, fq, synth, dev_name)
    elif args.workload == "llama31-8b-weight-sync":
        return run_weight_sync(args, torch, fq, synth, dev_name)
    elif args.workload == "qwen3-8b-kv-cache":
        return run_kv_cache(args, torch, fq, synth, dev_name)
    elif args.workload == "qwen3-8b-backward":
        return run_backward(args, torch, fq, synth, dev_name)
    elif args.workload == "qwen3-8b-decode-fused-act":
        return run_fused_act(args, torch, fq, synth, dev_name)
    else:
        return run_moe(args, torch, fq, synth, dev_name)

    groups = serving_layout(linears)
    cfg["gemms"] = [list(g) for g in groups]
    cfg["layout"] = ("q/k/v and gate/up weights concatenated along N (one activation "
                     "quantization and one GEMM per shared input)")
    cfg["scales"] = args.scales
    blk = DenseBlock(torch, fq, synth, groups, M, seed=1000 + args.seed, requant=requant,
                     scales=args.scales)
    blk.capture()
    for _ in range(args.warmup):
        blk.step()
    torch.cuda.synchronize()
    # one event at every step boundary: the total gives ms_per_step, the differences the spread
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for i in range(args.steps):
        blk.step(timed=True)
        marks[i + 1].record()
    clocks = sample_clocks(marks[-1])  # the host is ahead of the GPU: the timed steps run
    torch.cuda.synchronize()
    ms = marks[0].elapsed_time(marks[-1]) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    step_bytes = blk.bytes_w + blk.bytes_a + blk.bytes_g
    value = step_bytes / (ms * 1e-3) / 1e9
    lin_ms = blk.time_linears(max(args.steps, 10))
    roof_us = blk.roofline_us()
    parts = {"act_quant_and_gemm_graph": {
        "us_per_step": 1e3 * lin_ms, "bytes": blk.bytes_a + blk.bytes_g, "flops": blk.flops,
        "gbs": (blk.bytes_a + blk.bytes_g) / (lin_ms * 1e-3) / 1e9,
        "gemm_tflops": blk.flops / (lin_ms * 1e-3) / 1e12,
        "roofline_us": roof_us, "frac_roofline": roof_us / (1e3 * lin_ms),
        "roofline_rule": "sum over the GEMMs of max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s) plus "
                         "activation-quant bytes / 8 TB/s"}}
    if requant:
        r = blk.t_w.result()
        parts["quant_weight_batched"] = dict(r, frac_hbm=r["gbs"] / HBM_PEAK_GBS)
        roof = {"kernel": "quant_weight_blk128_kernel", "bound": "hbm", "achieved": r["gbs"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": r["gbs"] / HBM_PEAK_GBS,
                "traffic": measured_traffic(), "avg_launch_us": r["avg_us"],
                "algorithmic_bytes_per_launch": blk.bytes_w,
                "per_unit": "3 B per weight element + 4 B per 128x128 block",
                "units_per_launch": "all weights of the block (192,937,984 elements, 11,776 "
                                    "blocks) in one launch"}
    else:
        # dominant kernel: the largest GEMM of the block, timed per launch
        gi = max(range(len(blk.linears)), key=lambda j: blk.linears[j][1] * blk.linears[j][2])
        gname, gN, gK = blk.linears[gi]
        g_us = blk.time_gemm(gi, max(args.steps, 10))
        tf = 2 * M * gN * gK / (g_us * 1e-6) / 1e12
        roof = {"kernel": "gemm_big_kernel", "bound": "mfma", "achieved": tf,
                "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / FP8_PEAK_TFLOPS,
                "traffic": measured_traffic(PREFILL_TRAFFIC_FILE)
                if (M, gN, gK) == (8192, 24576, 4096) and args.scales == "fp32" else None,
                "avg_launch_us": g_us,
                "algorithmic_flops_per_launch": 2 * M * gN * gK,
                "per_unit": "2 flops per multiply-add: 2*M*N*K per GEMM",
                "units_per_launch": f"{gname}: M={M}, N={gN}, K={gK}"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(linears, M, seed=5000, budget_linears=7 if M <= 256 else 1,
                                 scales=args.scales)
        cpu["gpu_over_oracle"] = value / cpu["value"]  # whole step, same algorithmic bytes
        if quant_cpu is not None:
            cpu["quantizers"] = quant_cpu
            if requant and "all_cores" in quant_cpu:
                # the GPU's weight re-quantization against the oracle's quantizers on every core
                quant_cpu["gpu_weight_requant_over_oracle_all_cores"] = (
                    parts["quant_weight_batched"]["gbs"] / quant_cpu["all_cores"]["value"])
    line = {
        "metric": "blockscaled FP8 GEMM TFLOP/s (% MFMA peak); block-quant GB/s (% HBM peak)",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "ms_per_step_p10_p50_p90": [per_step[len(per_step) // 10], per_step[len(per_step) // 2],
                                    per_step[(9 * len(per_step)) // 10]],
        "dtype": "fp8-e4m3 x fp8-e4m3 -> f32 accumulate, bf16 out", "data": "synthetic",
        "config": cfg,
        "step_bytes": step_bytes, "step_gemm_flops": blk.flops,
        "parts": parts, "roofline": roof, "cpu_baseline": cpu, "gpu": dev_name,
        "cus": props.multi_processor_count, "clocks_during_timed_steps": clocks,
    }
    print(json.dumps(line), flush=True)


def _timed(torch, fn, steps, warmup, timers=()):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for t in timers:  # only launches inside the timed region count
        t.reset()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def run_fused_act(args, torch, fq, synth, dev_name):
    """The decode GEMMs of one Qwen3-8B block (serving layout: q/k/v, o, gate/up, down) at small
    token counts, two ways: activation quantization and GEMM as two launches per GEMM, or the
    GEMM with the quantization fused in (one launch). Both are timed as the host launches them
    (where small batches are launch-bound) and replayed from a HIP graph (GPU time only)."""
    groups = serving_layout(synth.DENSE_LINEARS_QWEN3_8B)
    pow2 = args.scales == "pow2"
    accum = "mx" if pow2 else "fp8"
    g = torch.Generator(device="cuda").manual_seed(11 + args.seed)
    weights = []
    for i, (name, N, K) in enumerate(groups):
        w = synth.weight_bf16(N, K, seed=9100 + i, device="cuda")
        weights.append(fq.quant_weight(w, scale=args.scales))
        del w
    results = []
    for M in (1, 16, 64):
        xs = [synth.act_bf16(M, K, seed=9200 + M + i, device="cuda")
              for i, (_, _, K) in enumerate(groups)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, N, _ in groups]
        qs = [(torch.empty((M, K), dtype=torch.uint8, device="cuda"),
               torch.empty((M, K // 128), dtype=torch.float32, device="cuda")) for _, _, K in groups]
        ws = fq.new_workspace(max(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, M, N, K)
                                  for _, N, K in groups), "cuda")

        def unfused():
            for x, (wq, sw), y, (xq, sa) in zip(xs, weights, ys, qs):
                fq.quant_act(x, xq, sa, scale=args.scales)
                fq.gemm(xq, sa, wq, sw, y=y, workspace=ws, accum=accum)

        def fused():
            for x, (wq, sw), y in zip(xs, weights, ys):
                fq.gemm_fused_act(x, wq, sw, y=y, workspace=ws, accum=accum, scale=args.scales)

        row = {"M": M}
        for label, fn in (("unfused", unfused), ("fused", fused)):
            row[f"eager_{label}_us"] = 1e3 * _timed(torch, fn, max(args.steps, 20), max(args.warmup, 3))
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fn()
            row[f"graph_{label}_us"] = 1e3 * _timed(torch, graph.replay, max(args.steps, 20),
                                                    max(args.warmup, 3))
        row["graph_fused_over_unfused"] = row["graph_fused_us"] / row["graph_unfused_us"]
        row["eager_fused_over_unfused"] = row["eager_fused_us"] / row["eager_unfused_us"]
        results.append(row)
    print(json.dumps({
        "workload": "Qwen3-8B decode GEMMs (q/k/v, o, gate/up, down), activation quantization "
                    "fused into the GEMM vs a separate launch",
        "metric": "microseconds per block (4 GEMMs with their activation quantization)",
        "scales": args.scales, "launches_per_block": {"unfused": 2 * len(groups),
                                                      "fused": len(groups)},
        "gemms": [list(gr) for gr in groups], "results": results, "gpu": dev_name}), flush=True)


def run_mlp(args, torch, fq, synth, dev_name):
    out = []
    for M in (256, 4096):
        blk = DenseBlock(torch, fq, synth, serving_layout(synth.LLAMA31_8B_LAYER_LINEARS[4:]), M,
                         seed=2000 + M, requant=False, scales=args.scales)
        blk.capture()
        ms = blk.time_linears(max(args.steps, 10))
        out.append({"M": M, "us_per_step": 1e3 * ms, "gemm_tflops_incl_act_quant":
                    blk.flops / (ms * 1e-3) / 1e12,
                    "gbs": (blk.bytes_a + blk.bytes_g) / (ms * 1e-3) / 1e9})
    print(json.dumps({"workload": "Llama-3.1-8B MLP (gate/up/down) GEMMs + act quant",
                      "scales": args.scales, "results": out, "gpu": dev_name}), flush=True)


def run_weight_sync(args, torch, fq, synth, dev_name):
    """Re-quantize every linear weight of 32 Llama-3.1-8B layers (6.98e9 elements, 14 GB bf16)."""
    layers = 32
    shapes = [(N, K) for _ in range(layers) for _, N, K in synth.LLAMA31_8B_LAYER_LINEARS]
    ws, wqs, sws = [], [], []
    uniq = {}
    for li, (N, K) in enumerate(shapes):
        ws.append(synth.weight_bf16(N, K, seed=3000 + li, outlier_frac=0.001, device="cuda"))
        wqs.append(torch.empty((N, K), dtype=torch.uint8, device="cuda"))
        sws.append(torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda"))
    tot = sum(w_bytes(N, K) for N, K in shapes)
    timer = KernelTimer(torch)
    descs = fq.weight_descs(ws, wqs, sws)

    def step():  # 224 matrices -> 7 launches of 32
        timer.launch(lambda: fq.quant_weights(None, None, None, descs=descs), tot)

    ms = _timed(torch, step, max(1, args.steps // 4), max(1, args.warmup // 2), (timer,))
    r = timer.result()
    print(json.dumps({"workload": "Llama-3.1-8B weight sync, 32 layers", "elements":
                      sum(N * K for N, K in shapes), "bytes": tot, "ms_per_pass": ms,
                      "GB/s": tot / (ms * 1e-3) / 1e9, "frac_hbm": tot / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                      "events": r, "launches_per_pass": -(-len(shapes) // 32), "gpu": dev_name}),
          flush=True)


def run_kv_cache(args, torch, fq, synth, dev_name):
    """Per-tensor FP8 of Qwen3-8B's attention inputs over 36 layers: (1) recalibration -- the
    running amax of Q, K and V (column slices of each layer's fused [T][6144] QKV output) over a
    4096-token calibration batch in one batched call, then the 108 scales; (2) the KV-cache store
    of an 8192-token prefill chunk: each layer's K and V quantized with its scale into a
    65536-row FP8 cache at slot-mapped rows (one launch per layer for its K and V, replayed from a
    HIP graph)."""
    layers, hidden, kv, T_cal, T_new, cache_rows = 36, 4096, 1024, 4096, 8192, 65536
    qkv_cols = hidden + 2 * kv
    cal = [synth.act_bf16(T_cal, qkv_cols, seed=7000 + l, device="cuda") for l in range(layers)]
    xs = [c[:, lo:hi] for c in cal for lo, hi in ((0, hidden), (hidden, hidden + kv),
                                                  (hidden + kv, qkv_cols))]
    amax = torch.zeros(len(xs), dtype=torch.float32, device="cuda")
    scale = torch.empty_like(amax)
    amax_descs = fq.tensor_descs(xs, amax)
    cal_bytes = sum(2 * x.shape[0] * x.shape[1] for x in xs)
    t_cal = KernelTimer(torch)

    def recal():
        amax.zero_()
        t_cal.launch(lambda: fq.amax_batched(None, amax, descs=amax_descs), cal_bytes)
        fq.scale_from_amax(amax, scale)

    new = [synth.act_bf16(T_new, 2 * kv, seed=8000 + l, device="cuda") for l in range(layers)]
    g = torch.Generator(device="cuda").manual_seed(9)
    slots = torch.randperm(cache_rows, generator=g, device="cuda")[:T_new].contiguous()
    kc = [torch.empty((cache_rows, kv), dtype=torch.uint8, device="cuda") for _ in range(layers)]
    vc = [torch.empty((cache_rows, kv), dtype=torch.uint8, device="cuda") for _ in range(layers)]
    recal()
    torch.cuda.synchronize()

    # one launch per layer: its K and V rows, each with its own scale and cache
    kv_descs = [fq.quant_descs([new[l][:, :kv], new[l][:, kv:]],
                            [scale[3 * l + 1:3 * l + 2], scale[3 * l + 2:3 * l + 3]],
                            [kc[l], vc[l]], [slots, slots]) for l in range(layers)]

    def store():
        for l in range(layers):
            fq.quant_per_tensor_batched(descs=kv_descs[l])

    store()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        store()
    store_bytes = layers * 2 * (T_new * kv * 3 + T_new * 8)
    ms_cal = _timed(torch, recal, max(args.steps, 5), max(args.warmup, 2), (t_cal,))
    r_cal = t_cal.result()
    ms_store = _timed(torch, graph.replay, max(args.steps, 5), max(args.warmup, 2))
    amax_gbs = r_cal["gbs"]
    print(json.dumps({
        "workload": "Qwen3-8B per-tensor FP8 Q/K/V recalibration and KV-cache store, 36 layers",
        "metric": "per-tensor quantizer GB/s (% HBM peak)",
        "recalibration": {"tensors": len(xs), "calibration_tokens": T_cal, "bytes": cal_bytes,
                          "ms_per_pass_incl_scales": ms_cal, "amax_launch_us": r_cal["avg_us"],
                          "amax_gbs": amax_gbs, "amax_frac_hbm": amax_gbs / HBM_PEAK_GBS,
                          "per_unit": "2 B per element read"},
        "kv_store": {"launches": layers, "new_tokens": T_new, "cache_rows": cache_rows,
                     "bytes": store_bytes, "ms_per_pass": ms_store,
                     "gbs": store_bytes / (ms_store * 1e-3) / 1e9,
                     "frac_hbm": store_bytes / (ms_store * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "per_unit": "3 B per element + 8 B slot per row"},
        "gpu": dev_name}), flush=True)


def run_backward(args, torch, fq, synth, dev_name):
    """FP8 backward of the Qwen3-8B decoder block's linears (serving layout: q/k/v and gate/up
    fused) over T = 8192 tokens. Per linear: the output gradient dY quantized both ways from one
    read (1x128 rows for Dgrad, 128x1 token groups stored transposed for Wgrad), the input X in
    128x1 token groups, the weight's transposed block-quantized copy, then Dgrad = dYq WqT^T
    (blockwise-scaled GEMM) and Wgrad = dYqT XqT^T (row-scaled GEMM). Each part is captured in
    its own HIP graph and timed over replays; bf16 outputs, FP8 slice sums (the FP32-scale
    default) or, with --scales pow2, matrix-core scales."""
    T = 8192
    groups = serving_layout(synth.DENSE_LINEARS_QWEN3_8B)
    acc = "mx" if args.scales == "pow2" else None
    L = []
    for i, (name, N, K) in enumerate(groups):
        L.append(dict(name=name, N=N, K=K,
                      dy=synth.act_bf16(T, N, seed=9000 + i, device="cuda") * 0.01,
                      x=synth.act_bf16(T, K, seed=9100 + i, device="cuda"),
                      w=synth.weight_bf16(N, K, seed=9200 + i, outlier_frac=0.001, device="cuda")))

    def quant_part():
        for l in L:
            l["q_dy"] = fq.quant_colwise(l["dy"], rowwise=True, scale=args.scales, **l.get("o_dy", {}))
            l["q_x"] = fq.quant_colwise(l["x"], scale=args.scales, **l.get("o_x", {}))
            l["q_w"] = fq.quant_weight_t(l["w"], scale=args.scales, **l.get("o_w", {}))

    quant_part()  # allocate the outputs once, then reuse them in place
    for l in L:
        dyt, s_dyt, dyq, s_dy = l["q_dy"]
        l["o_dy"] = dict(xtq=dyt, sat=s_dyt, xq=dyq, sa=s_dy)
        xt, s_xt, _, _ = l["q_x"]
        l["o_x"] = dict(xtq=xt, sat=s_xt)
        wqt, swt, _, _ = l["q_w"]
        l["o_w"] = dict(wqt=wqt, swt=swt)
        l["dx"] = torch.empty((T, l["K"]), dtype=torch.bfloat16, device="cuda")
        l["dw"] = torch.empty((l["N"], l["K"]), dtype=torch.bfloat16, device="cuda")
        l["ws_dx"] = fq.new_workspace(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM, T, l["K"], l["N"]), "cuda")
        l["ws_dw"] = fq.new_workspace(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GEMM_ROWSCALED, l["N"], l["K"], T), "cuda")

    def dgrad_part():
        for l in L:
            _, _, dyq, s_dy = l["q_dy"]
            wqt, swt, _, _ = l["q_w"]
            fq.gemm(dyq, s_dy, wqt, swt, y=l["dx"], workspace=l["ws_dx"], accum=acc)

    def wgrad_part():
        for l in L:
            dyt, s_dyt, _, _ = l["q_dy"]
            xt, s_xt, _, _ = l["q_x"]
            fq.gemm_rowscaled(dyt, s_dyt, xt, s_xt, y=l["dw"], workspace=l["ws_dw"], accum=acc)

    res = {}
    flops = sum(2 * T * l["N"] * l["K"] for l in L)
    qbytes = sum(T * l["N"] * (2 + 2) + T * l["N"] // 128 * 8 + T * l["K"] * 3 + T * l["K"] // 128 * 4
                 + l["N"] * l["K"] * 3 for l in L)
    for name, fn in (("quantizers", quant_part), ("dgrad", dgrad_part), ("wgrad", wgrad_part)):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        res[name] = _timed(torch, g.replay, max(args.steps, 5), max(args.warmup, 2))
    print(json.dumps({
        "workload": "Qwen3-8B decoder block linears, FP8 backward (Dgrad + Wgrad), 8192 tokens",
        "metric": "blockscaled FP8 GEMM TFLOP/s (% MFMA peak); quantizer GB/s (% HBM peak)",
        "gemms": [[l["name"], l["N"], l["K"]] for l in L], "tokens": T, "scales": args.scales,
        "quantizers": {"ms": res["quantizers"], "bytes": qbytes,
                       "gbs": qbytes / (res["quantizers"] * 1e-3) / 1e9,
                       "frac_hbm": qbytes / (res["quantizers"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       "per_unit": "dY: 2 B read + 2 B of codes (both layouts) per element + both "
                                   "scale sets; X: 3 B per element + scales; W: 3 B per element"},
        "dgrad": {"ms": res["dgrad"], "tflops": flops / (res["dgrad"] * 1e-3) / 1e12,
                  "frac_mfma": flops / (res["dgrad"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS},
        "wgrad": {"ms": res["wgrad"], "tflops": flops / (res["wgrad"] * 1e-3) / 1e12,
                  "frac_mfma": flops / (res["wgrad"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS},
        "gpu": dev_name}), flush=True)


def run_moe(args, torch, fq, synth, dev_name):
    """Qwen3-30B-A3B MoE layer: act quant + grouped gate/up (2048->1536) and down (768->2048)."""
    T, H, I, E, topk = 4096, 2048, 768, 128, 8
    counts = synth.moe_routing_counts(T, E, topk, seed=synth.seed_of(5, 0))
    off = synth.offsets_from_counts(counts).cuda()
    M = int(counts.sum())
    x1 = synth.act_bf16(M, H, seed=41, device="cuda")
    x2 = synth.act_bf16(M, I, seed=42, device="cuda")
    w1 = synth.weight_bf16(2 * I, H, seed=43, batch=E, device="cuda")
    w2 = synth.weight_bf16(H, I, seed=44, batch=E, device="cuda")
    wq1 = torch.empty((E, 2 * I, H), dtype=torch.uint8, device="cuda")
    sw1 = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device="cuda")
    wq2 = torch.empty((E, H, I), dtype=torch.uint8, device="cuda")
    sw2 = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device="cuda")
    # per-step expert re-quantization: [E][N][K] is one [E*N][K] matrix whose 128x128 blocks never
    # straddle two experts (N % 128 == 0), so both expert tensors are one batched launch
    wdescs = fq.weight_descs([w1.view(E * 2 * I, H), w2.view(E * H, I)],
                             [wq1.view(E * 2 * I, H), wq2.view(E * H, I)],
                             [sw1.view(E * 2 * I // 128, H // 128), sw2.view(E * H // 128, I // 128)])
    wq_bytes = w_bytes(E * 2 * I, H) + w_bytes(E * H, I)
    fq.quant_weights(None, None, None, descs=wdescs, scale=args.scales)
    xq1, sa1 = fq.quant_act(x1, scale=args.scales)
    xq2, sa2 = fq.quant_act(x2, scale=args.scales)
    accum = "mx" if args.scales == "pow2" else None
    y1 = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    tg = KernelTimer(torch)
    b1 = g_bytes(M, 2 * I, H) + (E - 1) * 2 * I * H + 4 * (E - 1) * (2 * I // 128) * (H // 128)
    b2 = g_bytes(M, H, I) + (E - 1) * H * I + 4 * (E - 1) * (H // 128) * (I // 128)

    def step():
        fq.quant_act(x1, xq1, sa1, scale=args.scales)
        tg.launch(lambda: fq.grouped_gemm(xq1, sa1, wq1, sw1, off, y=y1, accum=accum), b1)
        fq.quant_act(x2, xq2, sa2, scale=args.scales)
        tg.launch(lambda: fq.grouped_gemm(xq2, sa2, wq2, sw2, off, y=y2, accum=accum), b2)

    ms = _timed(torch, step, args.steps, args.warmup, (tg,))
    r = tg.result()
    tq = KernelTimer(torch)
    _timed(torch, lambda: tq.launch(lambda: fq.quant_weights(None, None, None, descs=wdescs,
                                                             scale=args.scales), wq_bytes),
           args.steps, args.warmup, (tq,))
    rq = tq.result()
    flops = 2 * M * (2 * I) * H + 2 * M * H * I
    g_ms = r["avg_us"] * r["launches"] / 1e3 / max(1, args.steps)
    roof_us = 1e6 * (max(2 * M * (2 * I) * H / (FP8_PEAK_TFLOPS * 1e12), b1 / (HBM_PEAK_GBS * 1e9)) +
                     max(2 * M * H * I / (FP8_PEAK_TFLOPS * 1e12), b2 / (HBM_PEAK_GBS * 1e9)))
    print(json.dumps({"workload": "Qwen3-30B-A3B MoE layer (T=4096, E=128, top-8, Zipf 1.1)",
                      "scales": args.scales,
                      "rows": M, "max_expert_rows": int(counts.max()), "ms_per_step": ms,
                      "grouped_gemm": r, "grouped_tflops": flops / (g_ms * 1e-3) / 1e12,
                      "grouped_roofline_us": roof_us,
                      "grouped_frac_roofline": roof_us / (1e3 * g_ms),
                      "expert_requant": dict(rq, bytes=wq_bytes, frac_hbm=rq["gbs"] / HBM_PEAK_GBS,
                                             what="all 2 x 128 expert weights, one batched launch"),
                      "roofline_rule": "per GEMM max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s), every "
                                       "expert's weights read once",
                      "gpu": dev_name}), flush=True)


if __name__ == "__main__":
    main()
