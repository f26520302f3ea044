"""Benchmark of the FP8 W8A8 linear-layer hot path on one MI355X.

Default workload (`qwen3-8b-prefill`): one Qwen3-8B-shaped decoder block at prefill (M = 8192
tokens, hidden 4096, 7 linears: q/o 4096x4096, k/v 1024x4096, gate/up 12288x4096, down
4096x12288). One step is the dynamic 1x128 quantization of each distinct bf16 input activation
and the blockwise-scaled FP8 GEMMs (bf16 output), replayed from a HIP graph. `value` is the GEMM
TFLOP/s of the step (2MNK over the 7 linears / step time); `roofline` is the largest GEMM's kernel
(gate/up, 8192 x 24576 x 4096), its launches replayed from a HIP graph and timed with HIP events
on the stream they run on. Parts
of the same line: every GEMM's launch time, the 32-layer Llama-3.1-8B weight sync (20.94 GB of
algorithmic traffic per pass) and the decode step below.

Decode workload (`qwen3-8b-decode`, M = 64): per-step re-quantization of all 7 bf16 weights to
E4M3 with 128x128 FP32 block scales in one batched launch, then the activation quantizations and
GEMMs; `value` is the step's algorithmic HBM traffic / step time (GB/s), `roofline` the weight
re-quantization kernel. Its weights rotate over enough copies that every step reads more than
1 GiB, so the 256 MiB Infinity Cache cannot hold a step's working set.

The weights are laid out as a serving engine keeps them: q/k/v concatenated along N (6144x4096)
and gate/up concatenated (24576x4096), so the block is 4 GEMMs over 4 activation quantizations
(one per distinct input), with the same bytes and FLOPs as the 7 separate linears.

Inputs are seeded synthetic tensors resident in HBM (weights N(0, 0.02) with 0.1 % x10 outliers,
activations N(0, 1) with 1 % x20 outlier channels). Every workload prints one JSON line of the
same schema (`roofline` of its dominant kernel, `cpu_baseline` = the CPU oracle timed on a bounded
sample of the same workload on this host's cores).

Other workloads (`--workload`): llama31-8b-mlp (M in {256, 4096}), llama31-8b-weight-sync (32
layers of weights), qwen3-30b-a3b-moe (grouped expert GEMMs), qwen3-8b-kv-cache (per-tensor Q/K/V
recalibration and FP8 KV-cache store over 36 layers), qwen3-8b-backward (FP8 Dgrad and Wgrad of
the decoder block's linears over 8192 tokens), qwen3-8b-decode-fused-act (decode GEMMs on bf16
activations, the activation quantization fused in, against two calls per GEMM).
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
    ap.add_argument("--workload", default="qwen3-8b-prefill",
                    choices=["qwen3-8b-decode", "qwen3-8b-prefill", "llama31-8b-mlp",
                             "llama31-8b-weight-sync", "qwen3-30b-a3b-moe", "qwen3-8b-kv-cache",
                             "qwen3-8b-backward", "qwen3-8b-decode-fused-act",
                             "qwen3-30b-a3b-moe-fused-act"])
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


def graph_launch_us(torch, fn, reps, replays=3):
    """Average duration of one call of `fn` (a single kernel launch, or a fixed sequence): `reps`
    calls captured in a HIP graph, HIP events around `replays` replays on the current stream.
    Unlike events around eager launches this leaves out the host's launch cost, which is longer
    than a decode-sized GEMM."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(reps):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (replays * reps)


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
        """Per-launch duration of GEMM i alone (its activation already quantized): launches
        replayed from a HIP graph, timed with HIP events on the current stream. The launches
        cycle through at least 1 GiB of weight codes (the quantized copies, then clones of them),
        so that the memory-side cache never holds the next launch's weights."""
        fq, torch = self.fq, self.torch
        _, N, K = self.linears[i]
        n_pool = max(self.copies, -(-ROTATE_BYTES // (N * K)))
        pool = [(self.wq[c][i], self.sw[c][i]) for c in range(self.copies)]
        pool += [(self.wq[c % self.copies][i].clone(), self.sw[c % self.copies][i].clone())
                 for c in range(self.copies, n_pool)]
        n = [0]

        def g():
            wq, sw = pool[n[0] % n_pool]
            n[0] += 1
            fq.gemm(self.xq[i], self.sa[i], wq, sw, y=self.y[i], accum=self.accum,
                    workspace=self.ws[i])

        fq.quant_act(self.x[i], self.xq[i], self.sa[i], scale=self.scales)
        us = graph_launch_us(torch, g, max(reps, n_pool))
        del pool
        return us

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
WSYNC_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                                  "quant_weight_blk128__llama31-8b-weight-sync.traffic.txt")
MOE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_big_kernel__qwen3-30b-a3b-moe.traffic.txt")


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


def cpu_baseline_dense(linears, M, seed, budget_linears, min_seconds=10.0, scales="fp32",
                       unit="GB/s"):
    """Time the CPU oracle on the linears of the step, in order and cycling, for at least
    `budget_linears` linears and `min_seconds` of oracle time (full per-linear work: weight
    re-quantization, activation quantization, GEMM). `unit`: GB/s of algorithmic bytes or
    TFLOP/s of GEMM flops over the oracle's time."""
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
    total_flops = 0
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
        total_flops += 2 * M * N * K
        done.append(name)
        i += 1
    if unit == "TFLOP/s":
        value = total_flops / elapsed / 1e12
    else:
        value = total_bytes / elapsed / 1e9
    return dict(value=value, unit=unit, cores=int(blas_threads),
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
        if M > 0:  # M == 0: the weights alone (a weight-sync sample)
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
                sample=(f"weight re-quantization and 1x128 activation quantization of the "
                        f"{len(linears)} linears of the block at M={M}" if M > 0 else
                        f"weight re-quantization of {len(linears)} weight matrices") +
                       f" ({len(tensors)} tensors, {total_bytes / 1e6:.0f} MB of algorithmic "
                       f"bytes), partitioned by tensor over {procs} processes")


# ------------------------------------------------------------------------------------- main


METRIC = "blockscaled FP8 GEMM TFLOP/s (% MFMA peak); block-quant GB/s (% HBM peak)"
DTYPE = "fp8-e4m3 x fp8-e4m3 -> f32 accumulate, bf16 out"
GEMM_KERNEL = "gemm_big_kernel"  # the large-M blockscaled GEMM kernel (what rocprofv3 lists)
WQ_KERNEL = "quant_weight_blk128_kernel"


def roof_mfma(kernel, flops, us, units, traffic=None):
    """`roofline` of a matrix-core-bound kernel: algorithmic flops per launch over its average
    launch duration, against the FP8 dense peak."""
    tf = flops / (us * 1e-6) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": tf, "peak": FP8_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": tf / FP8_PEAK_TFLOPS, "traffic": traffic,
            "avg_launch_us": us, "algorithmic_flops_per_launch": flops,
            "per_unit": "2 flops per multiply-add: 2*M*N*K per GEMM", "units_per_launch": units}


def roof_hbm(kernel, nbytes, us, per_unit, units, traffic=None):
    """`roofline` of an HBM-bound kernel: algorithmic bytes per launch over its average launch
    duration, against the HBM peak."""
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "avg_launch_us": us,
            "algorithmic_bytes_per_launch": nbytes, "per_unit": per_unit,
            "units_per_launch": units}


def emit(args, value, unit, ms, cfg, roofline, cpu, **extra):
    """Print the one JSON line of a workload (the same schema for every workload)."""
    line = {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
            "config": cfg}
    line.update(extra)
    line["roofline"] = roofline
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


def timed_steps(torch, step, steps, warmup):
    """`warmup` untimed steps, then `steps` steps with an event at every step boundary: returns
    (ms per step, sorted per-step ms, the last event)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record()
    for i in range(steps):
        step()
        marks[i + 1].record()
    return marks


def finish_marks(torch, marks):
    torch.cuda.synchronize()
    n = len(marks) - 1
    ms = marks[0].elapsed_time(marks[-1]) / n
    per = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(n))
    return ms, [per[n // 10], per[n // 2], per[(9 * n) // 10]]


def dense_parts(blk, args, M):
    """Per-GEMM launch timings and the captured act-quant + GEMM part of a dense block."""
    lin_ms = blk.time_linears(max(args.steps, 10))
    roof_us = blk.roofline_us()
    gemms = []
    for i, (name, N, K) in enumerate(blk.linears):
        us = blk.time_gemm(i, max(args.steps, 10))
        fl = 2 * M * N * K
        gemms.append({"gemm": name, "M": M, "N": N, "K": K, "avg_launch_us": us,
                      "tflops": fl / (us * 1e-6) / 1e12,
                      "frac_fp8_peak": fl / (us * 1e-6) / 1e12 / FP8_PEAK_TFLOPS,
                      "gbs": g_bytes(M, N, K) / (us * 1e-6) / 1e9,
                      "frac_roofline": 1e6 * max(fl / (FP8_PEAK_TFLOPS * 1e12),
                                                 g_bytes(M, N, K) / (HBM_PEAK_GBS * 1e9)) / us})
    graph = {"us_per_step": 1e3 * lin_ms, "bytes": blk.bytes_a + blk.bytes_g, "flops": blk.flops,
             "gbs": (blk.bytes_a + blk.bytes_g) / (lin_ms * 1e-3) / 1e9,
             "gemm_tflops": blk.flops / (lin_ms * 1e-3) / 1e12,
             "roofline_us": roof_us, "frac_roofline": roof_us / (1e3 * lin_ms),
             "roofline_rule": "sum over the GEMMs of max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s) "
                              "plus activation-quant bytes / 8 TB/s"}
    return graph, gemms


class WeightSync:
    """Every linear weight of 32 Llama-3.1-8B layers (224 matrices, 6.98e9 elements, 20.94 GB of
    algorithmic traffic) re-quantized per pass in ceil(224 / 32) = 7 batched launches."""

    LAYERS = 32

    def __init__(self, torch, fq, synth, scales="fp32"):
        self.torch, self.fq, self.scales = torch, fq, scales
        self.shapes = [(N, K) for _ in range(self.LAYERS) for _, N, K in
                       synth.LLAMA31_8B_LAYER_LINEARS]
        ws, wqs, sws = [], [], []
        for li, (N, K) in enumerate(self.shapes):
            ws.append(synth.weight_bf16(N, K, seed=3000 + li, outlier_frac=0.001, device="cuda"))
            wqs.append(torch.empty((N, K), dtype=torch.uint8, device="cuda"))
            sws.append(torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda"))
        self.tensors = (ws, wqs, sws)
        self.descs = [fq.weight_descs(ws[i:i + 32], wqs[i:i + 32], sws[i:i + 32])
                      for i in range(0, len(ws), 32)]
        self.sizes = [sum(w_bytes(N, K) for N, K in self.shapes[i:i + 32])
                      for i in range(0, len(ws), 32)]
        self.bytes = sum(self.sizes)
        self.elements = sum(N * K for N, K in self.shapes)
        self.timer = KernelTimer(torch)

    def step(self):  # one launch per group of 32 matrices, each timed
        for d, nb in zip(self.descs, self.sizes):
            self.timer.launch(lambda: self.fq.quant_weights(None, None, None, descs=d,
                                                            scale=self.scales), nb)

    def measure(self, steps, warmup):
        ms = _timed(self.torch, self.step, steps, warmup, (self.timer,))
        r = self.timer.result()
        return ms, r

    def free(self):
        self.tensors = None
        self.descs = None


def weight_sync_part(torch, fq, synth, args):
    sync = WeightSync(torch, fq, synth, scales=args.scales)
    ms, r = sync.measure(max(3, args.steps // 4), 1)
    part = {"matrices": len(sync.shapes), "elements": sync.elements, "bytes": sync.bytes,
            "launches_per_pass": len(sync.descs), "ms_per_pass": ms,
            "gbs": sync.bytes / (ms * 1e-3) / 1e9,
            "frac_hbm": sync.bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_avg_launch_us": r["avg_us"], "kernel_gbs": r["gbs"],
            "kernel_frac_hbm": r["gbs"] / HBM_PEAK_GBS,
            "per_unit": "3 B per weight element + 4 B per 128x128 block"}
    sync.free()
    del sync
    torch.cuda.empty_cache()
    return part


def decode_part(torch, fq, synth, args):
    """The Qwen3-8B decode step (M = 64) with its per-step weight re-quantization: step time and
    its parts, for the line of another workload."""
    blk = DenseBlock(torch, fq, synth, serving_layout(synth.DENSE_LINEARS_QWEN3_8B), 64,
                     seed=1000 + args.seed, requant=True, scales=args.scales)
    blk.capture()
    marks = timed_steps(torch, lambda: blk.step(timed=True), max(args.steps, 10), args.warmup)
    ms, spread = finish_marks(torch, marks)
    step_bytes = blk.bytes_w + blk.bytes_a + blk.bytes_g
    graph, gemms = dense_parts(blk, args, 64)
    r = blk.t_w.result()
    out = {"tokens_M": 64, "ms_per_step": ms, "ms_per_step_p10_p50_p90": spread,
           "step_bytes": step_bytes, "gbs": step_bytes / (ms * 1e-3) / 1e9,
           "act_quant_and_gemm_graph": graph, "gemms": gemms,
           "quant_weight_batched": dict(r, frac_hbm=r["gbs"] / HBM_PEAK_GBS,
                                        bytes=blk.bytes_w)}
    del blk
    torch.cuda.empty_cache()
    return out


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
    quant_sample = {"qwen3-8b-decode": (synth.DENSE_LINEARS_QWEN3_8B, 64),
                    "llama31-8b-weight-sync": (synth.LLAMA31_8B_LAYER_LINEARS, 0)}
    if args.workload in quant_sample and not args.no_cpu_baseline:
        if profiled:  # a profiler's preloaded library may already hold the GPU: no processes
            quant_cpu = {"skipped": "running under a profiler"}
        else:
            try:
                lin, m = quant_sample[args.workload]
                quant_cpu = cpu_quantizers_all_cores(lin, m, seed=6000, scales=args.scales)
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
    gpu = {"gpu": dev_name, "cus": props.multi_processor_count}
    runners = {"qwen3-8b-prefill": run_prefill, "qwen3-8b-decode": run_decode,
               "llama31-8b-mlp": run_mlp, "llama31-8b-weight-sync": run_weight_sync,
               "qwen3-30b-a3b-moe": run_moe, "qwen3-8b-kv-cache": run_kv_cache,
               "qwen3-8b-backward": run_backward, "qwen3-8b-decode-fused-act": run_fused_act,
               "qwen3-30b-a3b-moe-fused-act": run_moe_fused_act}
    return runners[args.workload](args, torch, fq, synth, gpu, quant_cpu)


def run_prefill(args, torch, fq, synth, gpu, quant_cpu):
    """Default line: the Qwen3-8B decoder block at prefill (M = 8192; config "same linears at
    prefill shape"), one step = the 4 activation quantizations and 4 GEMMs of the serving layout
    replayed from a HIP graph. value = the step's GEMM TFLOP/s (2MNK over the 7 linears / step
    time). Parts: every GEMM's launch time, the 32-layer weight sync and the decode step."""
    M = 8192
    linears = synth.DENSE_LINEARS_QWEN3_8B
    groups = serving_layout(linears)
    cfg = {"workload": "Qwen3-8B decoder block, prefill (M = 8192 tokens)", "tokens_M": M,
           "hidden": 4096, "linears": [list(l) for l in linears], "gemms": [list(g) for g in groups],
           "layout": "q/k/v and gate/up weights concatenated along N (one activation "
                     "quantization and one GEMM per shared input)",
           "gemm_out": "bf16", "scales": args.scales}
    blk = DenseBlock(torch, fq, synth, groups, M, seed=1000 + args.seed, requant=False,
                     scales=args.scales)
    blk.capture()
    marks = timed_steps(torch, blk.step, args.steps, args.warmup)
    clocks = sample_clocks(marks[-1])
    ms, spread = finish_marks(torch, marks)
    value = blk.flops / (ms * 1e-3) / 1e12
    graph, gemms = dense_parts(blk, args, M)
    big = max(gemms, key=lambda g: g["N"] * g["K"])
    roof = roof_mfma(GEMM_KERNEL, 2 * M * big["N"] * big["K"], big["avg_launch_us"],
                     f"{big['gemm']}: M={M}, N={big['N']}, K={big['K']} (one launch)",
                     traffic=measured_traffic(PREFILL_TRAFFIC_FILE) if args.scales == "fp32"
                     else None)
    del blk
    torch.cuda.empty_cache()
    parts = {"act_quant_and_gemm_graph": graph, "gemms": gemms,
             "weight_sync_32_layers": weight_sync_part(torch, fq, synth, args),
             "decode_step": decode_part(torch, fq, synth, args)}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(linears, M, seed=5000, budget_linears=1, scales=args.scales,
                                 unit="TFLOP/s")
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "TFLOP/s", ms, cfg, roof, cpu, ms_per_step_p10_p50_p90=spread,
         step_gemm_flops=blk_flops(groups, M), parts=parts, clocks_during_timed_steps=clocks,
         **gpu)


def blk_flops(groups, M):
    return sum(2 * M * N * K for _, N, K in groups)


def run_decode(args, torch, fq, synth, gpu, quant_cpu):
    """The Qwen3-8B decode step (config "dense decode step", M = 64): per-step re-quantization of
    all 7 weights in one batched launch, then the 4 activation quantizations and 4 GEMMs from a
    HIP graph. value = the step's algorithmic bytes / step time (GB/s); roofline = the weight
    re-quantization kernel."""
    M = 64
    linears = synth.DENSE_LINEARS_QWEN3_8B
    groups = serving_layout(linears)
    cfg = {"workload": "Qwen3-8B decoder block, decode step (M = 64 tokens)", "tokens_M": M,
           "hidden": 4096, "linears": [list(l) for l in linears], "gemms": [list(g) for g in groups],
           "weight_requant_per_step": True, "gemm_out": "bf16", "scales": args.scales,
           "layout": "q/k/v and gate/up weights concatenated along N"}
    blk = DenseBlock(torch, fq, synth, groups, M, seed=1000 + args.seed, requant=True,
                     scales=args.scales)
    blk.capture()
    marks = timed_steps(torch, lambda: blk.step(timed=True), args.steps, args.warmup)
    clocks = sample_clocks(marks[-1])
    ms, spread = finish_marks(torch, marks)
    step_bytes = blk.bytes_w + blk.bytes_a + blk.bytes_g
    value = step_bytes / (ms * 1e-3) / 1e9
    graph, gemms = dense_parts(blk, args, M)
    r = blk.t_w.result()
    roof = roof_hbm(WQ_KERNEL, blk.bytes_w, r["avg_us"],
                    "3 B per weight element + 4 B per 128x128 block",
                    "all weights of the block (192,937,984 elements, 11,776 blocks) in one launch",
                    traffic=measured_traffic())
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(linears, M, seed=5000, budget_linears=7, scales=args.scales)
        cpu["gpu_over_oracle"] = value / cpu["value"]
        if quant_cpu is not None:
            cpu["quantizers"] = quant_cpu
            if "all_cores" in quant_cpu:
                quant_cpu["gpu_weight_requant_over_oracle_all_cores"] = (
                    r["gbs"] / quant_cpu["all_cores"]["value"])
    parts = {"act_quant_and_gemm_graph": graph, "gemms": gemms,
             "quant_weight_batched": dict(r, frac_hbm=r["gbs"] / HBM_PEAK_GBS)}
    emit(args, value, "GB/s", ms, cfg, roof, cpu, ms_per_step_p10_p50_p90=spread,
         step_bytes=step_bytes, step_gemm_flops=blk.flops, parts=parts,
         clocks_during_timed_steps=clocks, **gpu)


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


def run_fused_act(args, torch, fq, synth, gpu, quant_cpu):
    """The decode GEMMs of one Qwen3-8B block (serving layout: q/k/v, o, gate/up, down) at small
    token counts, two ways: activation quantization and GEMM as two calls per GEMM, or one call
    of the GEMM on bf16 activations (one kernel up to 4 rows; above, the call runs the same two
    kernels itself). Both are timed as the host launches them (where small batches are
    launch-bound) and replayed from a HIP graph (GPU time only). value = algorithmic GB/s of the
    fused block at M = 1 (graph replay); roofline = the fused gate/up kernel at M = 1."""
    groups = serving_layout(synth.DENSE_LINEARS_QWEN3_8B)
    pow2 = args.scales == "pow2"
    accum = "mx" if pow2 else "fp8"
    weights = []
    for i, (name, N, K) in enumerate(groups):
        w = synth.weight_bf16(N, K, seed=9100 + i, device="cuda")
        weights.append(fq.quant_weight(w, scale=args.scales))
        del w
    results = []
    roof = None
    value = ms1 = None
    for M in (1, 4, 16, 64):
        xs = [synth.act_bf16(M, K, seed=9200 + M + i, device="cuda")
              for i, (_, _, K) in enumerate(groups)]
        ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _, N, _ in groups]
        qs = [(torch.empty((M, K), dtype=torch.uint8, device="cuda"),
               torch.empty((M, K // 128), dtype=torch.float32, device="cuda")) for _, _, K in groups]
        ws = fq.new_workspace(max(fq.fp8rl_workspace_bytes(op, M, N, K) for _, N, K in groups
                                  for op in (fq.FP8RL_OP_GEMM, fq.FP8RL_OP_GEMM_FUSED_ACT)),
                              "cuda")

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
        if M == 1:
            nbytes = sum(N * K + 4 * (N // 128) * (K // 128) + 2 * M * K + 2 * M * N
                         for _, N, K in groups)
            ms1 = row["graph_fused_us"] / 1e3
            value = nbytes / (ms1 * 1e-3) / 1e9
            gi = max(range(len(groups)), key=lambda j: groups[j][1] * groups[j][2])
            _, gN, gK = groups[gi]
            x, (wq, sw), y = xs[gi], weights[gi], ys[gi]
            us = graph_launch_us(torch, lambda: fq.gemm_fused_act(
                x, wq, sw, y=y, workspace=ws, accum=accum, scale=args.scales),
                max(args.steps, 20))
            gb = gN * gK + 4 * (gN // 128) * (gK // 128) + 2 * M * gK + 2 * M * gN
            roof = roof_hbm("gemm_stream_kernel (fused activation quantization)", gb, us,
                            "weight codes + block scales + bf16 activations + bf16 output",
                            f"gate_up_proj: M={M}, N={gN}, K={gK} (one launch)")
    cfg = {"workload": "Qwen3-8B decode GEMMs (q/k/v, o, gate/up, down) on bf16 activations, "
                       "activation quantization fused into the GEMM", "tokens_M": [1, 4, 16, 64],
           "gemms": [list(gr) for gr in groups], "scales": args.scales,
           "launches_per_block": {"unfused": 2 * len(groups),
                                  "fused": {"M <= 4": len(groups), "M > 4": 2 * len(groups)}}}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(synth.DENSE_LINEARS_QWEN3_8B, 1, seed=5000, budget_linears=7,
                                 scales=args.scales)
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "GB/s", ms1, cfg, roof, cpu, results=results, **gpu)


def run_mlp(args, torch, fq, synth, gpu, quant_cpu):
    """Llama-3.1-8B MLP (config "Llama-3.1-8B-shaped MLP"): gate/up (fused, 28672 x 4096) and
    down (4096 x 14336) with their activation quantizations, at M = 4096 (the line's value, GEMM
    TFLOP/s over the step) and M = 256 (a part, against its HBM roofline)."""
    mlp = synth.LLAMA31_8B_LAYER_LINEARS[4:]
    out = {}
    for M in (256, 4096):
        blk = DenseBlock(torch, fq, synth, serving_layout(mlp), M, seed=2000 + M, requant=False,
                         scales=args.scales)
        blk.capture()
        marks = timed_steps(torch, blk.step, args.steps, args.warmup)
        ms, spread = finish_marks(torch, marks)
        graph, gemms = dense_parts(blk, args, M)
        out[M] = {"tokens_M": M, "ms_per_step": ms, "ms_per_step_p10_p50_p90": spread,
                  "gemm_tflops_incl_act_quant": blk.flops / (ms * 1e-3) / 1e12,
                  "act_quant_and_gemm_graph": graph, "gemms": gemms}
        del blk
        torch.cuda.empty_cache()
    big = max(out[4096]["gemms"], key=lambda g: g["N"] * g["K"])
    roof = roof_mfma(GEMM_KERNEL, 2 * 4096 * big["N"] * big["K"], big["avg_launch_us"],
                     f"{big['gemm']}: M=4096, N={big['N']}, K={big['K']} (one launch)")
    cfg = {"workload": "Llama-3.1-8B MLP (gate/up + down GEMMs with activation quantization), "
                       "M = 4096 (M = 256 in parts)", "tokens_M": [256, 4096],
           "gemms": [list(g) for g in serving_layout(mlp)], "gemm_out": "bf16",
           "scales": args.scales}
    value = out[4096]["gemm_tflops_incl_act_quant"]
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_dense(mlp, 4096, seed=5100, budget_linears=1, scales=args.scales,
                                 unit="TFLOP/s")
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "TFLOP/s", out[4096]["ms_per_step"], cfg, roof, cpu,
         parts={"m4096": out[4096], "m256": out[256]}, **gpu)


def run_weight_sync(args, torch, fq, synth, gpu, quant_cpu):
    """Config "weight-sync pass": every linear weight of 32 Llama-3.1-8B layers (6.98e9
    elements, 14 GB bf16) re-quantized per step in 7 batched launches. value = algorithmic GB/s
    of the pass; roofline = the weight quantizer kernel over all its launches."""
    sync = WeightSync(torch, fq, synth, scales=args.scales)
    for _ in range(args.warmup):
        sync.step()
    torch.cuda.synchronize()
    sync.timer.reset()
    marks = timed_steps(torch, sync.step, args.steps, 0)
    ms, spread = finish_marks(torch, marks)
    r = sync.timer.result()
    value = sync.bytes / (ms * 1e-3) / 1e9
    roof = roof_hbm(WQ_KERNEL, sync.bytes / len(sync.descs), r["avg_us"],
                    "3 B per weight element + 4 B per 128x128 block",
                    "32 weight matrices (about 3 GB of algorithmic traffic) per launch, 7 launches "
                    "per pass; achieved = all bytes over all launch time",
                    traffic=measured_traffic(WSYNC_TRAFFIC_FILE) if args.scales == "fp32" else None)
    roof["achieved"] = r["gbs"]
    roof["frac"] = r["gbs"] / HBM_PEAK_GBS
    cfg = {"workload": "Llama-3.1-8B weight sync: all linear weights of 32 layers re-quantized "
                       "to E4M3 with 128x128 block scales", "layers": WeightSync.LAYERS,
           "matrices": len(sync.shapes), "elements": sync.elements, "bytes": sync.bytes,
           "launches_per_pass": len(sync.descs), "scales": args.scales}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = dict(quant_cpu or {}, kind="oracle")
        best = cpu.get("all_cores") or cpu.get("one_thread")
        if best:
            cpu.update(value=best["value"], unit="GB/s", cores=best["cores"])
            cpu["gpu_over_oracle"] = value / best["value"]
    emit(args, value, "GB/s", ms, cfg, roof, cpu, ms_per_step_p10_p50_p90=spread, **gpu)


def run_kv_cache(args, torch, fq, synth, gpu, quant_cpu):
    """Per-tensor FP8 of Qwen3-8B's attention inputs over 36 layers: (1) recalibration -- the
    running amax of Q, K and V (column slices of each layer's fused [T][6144] QKV output) over a
    4096-token calibration batch in one batched call, then the 108 scales; (2) the KV-cache store
    of an 8192-token prefill chunk: each layer's K and V quantized with its scale into a
    65536-row FP8 cache at slot-mapped rows (one launch per layer for its K and V, replayed from a
    HIP graph). value = algorithmic GB/s of recalibration + store; roofline = the amax kernel."""
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
    ms = ms_cal + ms_store
    value = (cal_bytes + store_bytes) / (ms * 1e-3) / 1e9
    roof = roof_hbm("amax_bf16_kernel", cal_bytes, r_cal["avg_us"], "2 B per element read",
                    f"the running amax of {len(xs)} Q/K/V tensors ({T_cal} calibration tokens, "
                    f"36 layers) in one launch")
    cfg = {"workload": "Qwen3-8B per-tensor FP8 Q/K/V recalibration and KV-cache store, 36 "
                       "layers", "layers": layers, "calibration_tokens": T_cal,
           "new_tokens": T_new, "cache_rows": cache_rows, "kv_width": kv}
    parts = {"recalibration": {"tensors": len(xs), "bytes": cal_bytes,
                               "ms_per_pass_incl_scales": ms_cal, "amax_launch_us": r_cal["avg_us"],
                               "amax_gbs": r_cal["gbs"], "amax_frac_hbm": r_cal["gbs"] / HBM_PEAK_GBS},
             "kv_store": {"launches": layers, "bytes": store_bytes, "ms_per_pass": ms_store,
                          "gbs": store_bytes / (ms_store * 1e-3) / 1e9,
                          "frac_hbm": store_bytes / (ms_store * 1e-3) / 1e9 / HBM_PEAK_GBS,
                          "per_unit": "3 B per element + 8 B slot per row"}}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_kv(synth, min_seconds=10.0)
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "GB/s", ms, cfg, roof, cpu, parts=parts, **gpu)


def cpu_baseline_kv(synth, min_seconds=10.0):
    """The oracle's per-tensor path on layers of the KV-cache workload, cycling until
    `min_seconds`: running amax of a layer's Q, K and V over its calibration batch, the three
    scales, and the per-tensor codes of its new K and V rows."""
    import numpy as np
    import torch

    from oracle import kvcache as ok

    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    hidden, kv, T_cal, T_new = 4096, 1024, 4096, 8192
    elapsed, nbytes, layers = 0.0, 0, 0
    while elapsed < min_seconds:
        cal = bits(synth.act_bf16(T_cal, hidden + 2 * kv, seed=7500 + layers))
        new = bits(synth.act_bf16(T_new, 2 * kv, seed=8500 + layers))
        t0 = time.perf_counter()
        scales = []
        for lo, hi in ((0, hidden), (hidden, hidden + kv), (hidden + kv, hidden + 2 * kv)):
            scales.append(ok.scale_per_tensor(ok.amax(cal[:, lo:hi])))
        ok.quant_per_tensor(new[:, :kv], scales[1])
        ok.quant_per_tensor(new[:, kv:], scales[2])
        elapsed += time.perf_counter() - t0
        nbytes += 2 * cal.size + 2 * (T_new * kv * 3 + T_new * 8)
        layers += 1
    return dict(value=nbytes / elapsed / 1e9, unit="GB/s", cores=1, kind="oracle",
                seconds=elapsed, sample=f"{layers} layers: amax + scale of Q, K, V over "
                                        f"{T_cal} calibration tokens, per-tensor codes of "
                                        f"{T_new} new K and V rows; numpy, one thread")


def run_backward(args, torch, fq, synth, gpu, quant_cpu):
    """FP8 backward of the Qwen3-8B decoder block's linears (serving layout: q/k/v and gate/up
    fused) over T = 8192 tokens. Per linear: the output gradient dY quantized both ways from one
    read (1x128 rows for Dgrad, 128x1 token groups stored transposed for Wgrad), the input X in
    128x1 token groups, the weight's transposed block-quantized copy, then Dgrad = dYq WqT^T
    (blockwise-scaled GEMM) and Wgrad = dYqT XqT^T (row-scaled GEMM). Each part is captured in
    its own HIP graph and timed over replays; bf16 outputs with the library's default
    accumulation (FP8 slice sums for Dgrad, f16 ones for Wgrad) or, with --scales pow2,
    matrix-core scales for Dgrad. value = GEMM TFLOP/s of Dgrad + Wgrad over quantizers + both
    GEMMs; the opt-in FP8-slice Wgrad (outside the bf16 tolerance in rare cancelling elements)
    is timed as a part of its own."""
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

    def wgrad_part(wacc=None):
        for l in L:
            dyt, s_dyt, _, _ = l["q_dy"]
            xt, s_xt, _, _ = l["q_x"]
            fq.gemm_rowscaled(dyt, s_dyt, xt, s_xt, y=l["dw"], workspace=l["ws_dw"], accum=wacc)

    res = {}
    flops = sum(2 * T * l["N"] * l["K"] for l in L)
    qbytes = sum(T * l["N"] * (2 + 2) + T * l["N"] // 128 * 8 + T * l["K"] * 3 + T * l["K"] // 128 * 4
                 + l["N"] * l["K"] * 3 for l in L)
    parts_fn = (("quantizers", quant_part), ("dgrad", dgrad_part), ("wgrad", wgrad_part),
                ("wgrad_fp8_slices_opt_in", lambda: wgrad_part("fp8")))
    for name, fn in parts_fn:
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        res[name] = _timed(torch, g.replay, max(args.steps, 5), max(args.warmup, 2))
    # the dominant kernel: the largest Dgrad GEMM (gate/up: M = T, N = K = 4096, K = 24576),
    # timed per launch
    big = max(L, key=lambda l: l["N"] * l["K"])
    _, _, dyq, s_dy = big["q_dy"]
    wqt, swt, _, _ = big["q_w"]
    t = KernelTimer(torch)
    for _ in range(3):
        fq.gemm(dyq, s_dy, wqt, swt, y=big["dx"], workspace=big["ws_dx"], accum=acc)
    for _ in range(max(args.steps, 10)):
        t.launch(lambda: fq.gemm(dyq, s_dy, wqt, swt, y=big["dx"], workspace=big["ws_dx"],
                                 accum=acc), 0)
    torch.cuda.synchronize()
    roof = roof_mfma(GEMM_KERNEL, 2 * T * big["N"] * big["K"], t.result()["avg_us"],
                     f"Dgrad of {big['name']}: M={T}, N={big['K']}, K={big['N']} (one launch)")
    ms = res["quantizers"] + res["dgrad"] + res["wgrad"]
    value = 2 * flops / (ms * 1e-3) / 1e12
    gem = lambda k: {"ms": res[k], "tflops": flops / (res[k] * 1e-3) / 1e12,
                     "frac_mfma": flops / (res[k] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS}
    parts = {"quantizers": {"ms": res["quantizers"], "bytes": qbytes,
                            "gbs": qbytes / (res["quantizers"] * 1e-3) / 1e9,
                            "frac_hbm": qbytes / (res["quantizers"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "per_unit": "dY: 2 B read + 2 B of codes (both layouts) per element "
                                        "+ both scale sets; X: 3 B per element + scales; W: 3 B "
                                        "per element"},
             "dgrad": gem("dgrad"), "wgrad": dict(gem("wgrad"), accum="default (f16 slices)"),
             "wgrad_fp8_slices_opt_in": dict(gem("wgrad_fp8_slices_opt_in"),
                                             note="FP8 slice sums: outside the bf16 tolerance in "
                                                  "rare cancelling elements; not the default")}
    cfg = {"workload": "Qwen3-8B decoder block linears, FP8 backward (Dgrad + Wgrad), 8192 "
                       "tokens", "tokens": T, "gemms": [[l["name"], l["N"], l["K"]] for l in L],
           "scales": args.scales}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_backward(synth, T, min_seconds=10.0)
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "TFLOP/s", ms, cfg, roof, cpu, parts=parts, **gpu)


def cpu_baseline_backward(synth, T, min_seconds=10.0):
    """The oracle's FP8 backward (quantizers, Dgrad, Wgrad) of the o_proj-shaped linear
    (4096 x 4096) over T tokens, repeated until `min_seconds`."""
    import numpy as np
    import torch

    from oracle import backward as ob

    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    N = K = 4096
    elapsed, flops, reps = 0.0, 0, 0
    while elapsed < min_seconds or reps == 0:
        dy = bits(synth.act_bf16(T, N, seed=9600 + reps) * 0.01)
        x = bits(synth.act_bf16(T, K, seed=9700 + reps))
        w = bits(synth.weight_bf16(N, K, seed=9800 + reps, outlier_frac=0.001))
        t0 = time.perf_counter()
        ob.linear_backward_fp8(dy, x, w, out="bf16")
        elapsed += time.perf_counter() - t0
        flops += 2 * (2 * T * N * K)
        reps += 1
    return dict(value=flops / elapsed / 1e12, unit="TFLOP/s", cores=blas_threads(),
                kind="oracle", seconds=elapsed,
                sample=f"{reps} FP8 backward pass(es) of a 4096x4096 linear over {T} tokens "
                       f"(quantizers, Dgrad and Wgrad, fp64 BLAS)")


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def run_moe(args, torch, fq, synth, gpu, quant_cpu):
    """Qwen3-30B-A3B MoE layer (T = 4096 tokens, E = 128, top-8, Zipf(1.1)-routed): per step the
    activation quantization and grouped GEMM of the expert gate/up (2048 -> 1536) and of the
    expert down (768 -> 2048); the per-step re-quantization of all 256 expert weights is timed
    as a part (one batched launch). value = GEMM TFLOP/s over the step; roofline = the grouped
    GEMM kernel, every expert's weights read once (HBM-bound by max(flops / P, bytes / B))."""
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tg.reset()
    marks = timed_steps(torch, step, args.steps, 0)
    ms, spread = finish_marks(torch, marks)
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
    value = flops / (ms * 1e-3) / 1e12
    roof = roof_hbm("grouped_big_kernel", (b1 + b2) / 2, r["avg_us"],
                    "activation codes + scales + every expert's weight codes and block scales "
                    "once + bf16 output",
                    "one grouped GEMM (gate/up or down; average of the two)",
                    traffic=measured_traffic(MOE_TRAFFIC_FILE) if args.scales == "fp32" else None)
    roof["frac_roofline"] = roof_us / (1e3 * g_ms)
    roof["roofline_rule"] = ("per GEMM max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s), every expert's "
                             "weights read once")
    cfg = {"workload": "Qwen3-30B-A3B MoE layer (T=4096, E=128, top-8, Zipf 1.1 routing)",
           "tokens": T, "experts": E, "top_k": topk, "routed_rows": M,
           "max_expert_rows": int(counts.max()), "gemms": [["gate_up", 2 * I, H], ["down", H, I]],
           "scales": args.scales}
    parts = {"grouped_gemm": dict(r, tflops=flops / (g_ms * 1e-3) / 1e12, roofline_us=roof_us,
                                  frac_roofline=roof_us / (1e3 * g_ms)),
             "expert_requant": dict(rq, bytes=wq_bytes, frac_hbm=rq["gbs"] / HBM_PEAK_GBS,
                                    what="all 2 x 128 expert weights, one batched launch")}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_moe(synth, counts, min_seconds=10.0)
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "TFLOP/s", ms, cfg, roof, cpu, ms_per_step_p10_p50_p90=spread,
         parts=parts, **gpu)


def run_moe_fused_act(args, torch, fq, synth, gpu, quant_cpu):
    """The Qwen3-30B-A3B MoE layer's expert GEMMs on bf16 activations, two ways per step:
    one call per GEMM -- gate/up on the T token rows read through the router's token indices
    (each token quantized once), down on its input in expert order -- against the 1x128
    quantizer on the routed rows followed by the grouped GEMM (the routed gate/up input gathered
    beforehand, not timed). Both replayed from HIP graphs. value = GEMM TFLOP/s of the one-call
    step; roofline = the one-call gate/up (its quantizer and grouped GEMM launches together)
    against max(2MNK / FP8 peak, bytes / HBM peak), bytes = bf16 tokens once + every expert's
    weight codes and scales once + bf16 output."""
    T, H, I, E, topk = 4096, 2048, 768, 128, 8
    counts, ids = synth.moe_routing(T, E, topk, seed=synth.seed_of(5, 0))
    off = synth.offsets_from_counts(counts).cuda()
    ids = ids.cuda()
    M = int(counts.sum())
    xt = synth.act_bf16(T, H, seed=45, device="cuda")
    x1 = xt[ids.long()].contiguous()  # the routed gate/up input of the two-call flow
    x2 = synth.act_bf16(M, I, seed=42, device="cuda")
    wq1, sw1 = fq.quant_weight(synth.weight_bf16(2 * I, H, seed=43, batch=E, device="cuda")
                               .view(E * 2 * I, H), scale=args.scales)
    wq2, sw2 = fq.quant_weight(synth.weight_bf16(H, I, seed=44, batch=E, device="cuda")
                               .view(E * H, I), scale=args.scales)
    wq1, sw1 = wq1.view(E, 2 * I, H), sw1.view(E, 2 * I // 128, H // 128)
    wq2, sw2 = wq2.view(E, H, I), sw2.view(E, H // 128, I // 128)
    accum = "mx" if args.scales == "pow2" else None
    xq1 = torch.empty((M, H), dtype=torch.uint8, device="cuda")
    sa1 = torch.empty((M, H // 128), dtype=torch.float32, device="cuda")
    xq2 = torch.empty((M, I), dtype=torch.uint8, device="cuda")
    sa2 = torch.empty((M, I // 128), dtype=torch.float32, device="cuda")
    y1 = torch.empty((M, 2 * I), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ws = fq.new_workspace(max(fq.fp8rl_workspace_bytes(fq.FP8RL_OP_GROUPED_GEMM_FUSED_ACT, M, N, K, E)
                              for N, K in ((2 * I, H), (H, I))), "cuda")
    fused_up = lambda: fq.grouped_gemm_fused_act(xt, wq1, sw1, off, row_ids=ids, y=y1,
                                                 workspace=ws, accum=accum, scale=args.scales)
    fused_down = lambda: fq.grouped_gemm_fused_act(x2, wq2, sw2, off, y=y2, workspace=ws,
                                                   accum=accum, scale=args.scales)
    two_up = lambda: (fq.quant_act(x1, xq1, sa1, scale=args.scales),
                      fq.grouped_gemm(xq1, sa1, wq1, sw1, off, y=y1, accum=accum))
    two_down = lambda: (fq.quant_act(x2, xq2, sa2, scale=args.scales),
                        fq.grouped_gemm(xq2, sa2, wq2, sw2, off, y=y2, accum=accum))
    reps = max(10, args.steps)
    # alternating rounds, the faster of each: the engine clock settles over the first ones
    t = {k: float("inf") for k in ("fused_up", "fused_down", "two_up", "two_down")}
    for _ in range(3):
        for k, fn in (("fused_up", fused_up), ("two_up", two_up), ("fused_down", fused_down),
                      ("two_down", two_down)):
            t[k] = min(t[k], graph_launch_us(torch, fn, reps))
    flops_up, flops_down = 2 * M * (2 * I) * H, 2 * M * H * I
    ms = (t["fused_up"] + t["fused_down"]) / 1e3
    value = (flops_up + flops_down) / (ms * 1e-3) / 1e12
    b_up = 2 * T * H + E * (2 * I * H + 4 * (2 * I // 128) * (H // 128)) + 2 * M * 2 * I
    roof_us = 1e6 * max(flops_up / (FP8_PEAK_TFLOPS * 1e12), b_up / (HBM_PEAK_GBS * 1e9))
    roof = roof_hbm("quant_act_tok128_kernel + grouped_big_kernel (one call, token gather)",
                    b_up, t["fused_up"],
                    "bf16 token activations once + every expert's weight codes and block scales "
                    "once + bf16 output", "the gate/up call (two launches)")
    roof["frac_roofline"] = roof_us / t["fused_up"]
    roof["roofline_rule"] = "max(2MNK / 5.0 PFLOP/s, bytes / 8 TB/s)"
    cfg = {"workload": "Qwen3-30B-A3B MoE expert GEMMs on bf16 activations (T=4096, E=128, top-8, "
                       "Zipf 1.1 routing), activation quantization inside the GEMM call",
           "tokens": T, "experts": E, "top_k": topk, "routed_rows": M,
           "gemms": [["gate_up", 2 * I, H], ["down", H, I]], "scales": args.scales}
    parts = {"gate_up": {"one_call_us": t["fused_up"], "two_calls_us": t["two_up"],
                         "ratio": t["fused_up"] / t["two_up"],
                         "what": "one call on the token rows with the router's indices against "
                                 "the quantizer on the routed rows, then the grouped GEMM"},
             "down": {"one_call_us": t["fused_down"], "two_calls_us": t["two_down"],
                      "ratio": t["fused_down"] / t["two_down"]},
             "two_call_step_tflops": (flops_up + flops_down)
             / ((t["two_up"] + t["two_down"]) * 1e-6) / 1e12}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_moe(synth, counts, min_seconds=10.0)
        cpu["gpu_over_oracle"] = value / cpu["value"]
    emit(args, value, "TFLOP/s", ms, cfg, roof, cpu, parts=parts, **gpu)


def cpu_baseline_moe(synth, counts, min_seconds=10.0):
    """The oracle on a sample of the MoE layer: 16 experts at a time (their Zipf-routed row
    counts), activation quantization and grouped gate/up and down GEMMs, cycling through the
    experts until `min_seconds` (expert weights quantized beforehand, not timed)."""
    import numpy as np
    import torch

    from oracle import gemm as og
    from oracle import quant as oq

    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    H, I, G = 2048, 768, 16
    elapsed, flops, groups = 0.0, 0, 0
    while elapsed < min_seconds or groups == 0:
        e0 = (groups * G) % len(counts)
        c = [int(v) for v in counts[e0:e0 + G]]
        m = sum(c)
        off = np.zeros(len(c) + 1, np.int32)
        off[1:] = np.cumsum(c)
        w1 = bits(synth.weight_bf16(2 * I, H, seed=4300 + groups, batch=len(c)))
        w2 = bits(synth.weight_bf16(H, I, seed=4400 + groups, batch=len(c)))
        q1 = [oq.quant_weight_blk128(w1[e]) for e in range(len(c))]
        q2 = [oq.quant_weight_blk128(w2[e]) for e in range(len(c))]
        x1 = bits(synth.act_bf16(m, H, seed=4500 + groups))
        x2 = bits(synth.act_bf16(m, I, seed=4600 + groups))
        t0 = time.perf_counter()
        xq1, sa1 = oq.quant_act_tok128(x1)
        og.grouped_gemm_blockscaled(xq1, sa1, np.stack([a for a, _ in q1]),
                                    np.stack([b for _, b in q1]), off, out="bf16")
        xq2, sa2 = oq.quant_act_tok128(x2)
        og.grouped_gemm_blockscaled(xq2, sa2, np.stack([a for a, _ in q2]),
                                    np.stack([b for _, b in q2]), off, out="bf16")
        elapsed += time.perf_counter() - t0
        flops += 2 * m * (2 * I) * H + 2 * m * H * I
        groups += 1
    return dict(value=flops / elapsed / 1e12, unit="TFLOP/s", cores=blas_threads(),
                kind="oracle", seconds=elapsed,
                sample=f"{groups} groups of {G} experts with their routed rows: activation "
                       f"quantization + grouped gate/up and down GEMMs (fp64 BLAS); expert "
                       f"weight quantization not timed")


if __name__ == "__main__":
    main()
