#!/usr/bin/env python3
"""Benchmark of the whole-tensor Muon optimizer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over the batch:
- fused momentum;
- the Frobenius norm;
- 5 Newton-Schulz iterations (Gram, square, update);
- the weight apply.
The default workload is one Qwen3-32B decoder layer's seven projection
matrices in bf16. Inputs are seeded synthetic data, resident in HBM before the
timed region starts.

Timing follows the pages' protocol of averaging many steps (Canzona analysis
page, section 5, "Metrics"): W untimed warm-up steps, then exactly K steps
between two device synchronisations, timed with events on the step's stream.
Per-kernel durations come from HIP event pairs that the library records around
every launch during the same timed region, on the same stream. After it,
--runs fresh plans each run 3 warm-up and --run-steps timed steps (the pages'
average over runs of several steps); the line reports their mean, median and
min. The GPU's graphics clock and socket power are sampled through amdsmi
during both, because the chip runs at its power cap and its clock varies.

It prints one JSON line, with value = algorithmic TFLOP/s of the whole step.
Flops count only the triangles the method needs (see oracle.step_flops).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3     # MI355X fp32 matrix, published
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_32b_layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", default="all",
                    help="matrix indices the oracle times for the CPU baseline (comma-separated, or all)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the perf-only legs over the other workloads")
    ap.add_argument("--chains", type=int, default=0,
                    help="GEMM chains of the plan (sets MUON_CHAINS; 0: the library default)")
    ap.add_argument("--no-roofline-pass", action="store_true",
                    help="skip the separate single-chain pass that times the update kernel alone")
    ap.add_argument("--runs", type=int, default=10,
                    help="protocol runs after the timed region: each a fresh plan, 3 warm-up and "
                         "--run-steps timed steps (0: none)")
    ap.add_argument("--run-steps", type=int, default=10)
    ap.add_argument("--no-master-weights", action="store_true",
                    help="skip the step with fp32 master weights and momentum (MUON_BF16_F32_MASTER)")
    ap.add_argument("--no-mfma-probe", action="store_true",
                    help="skip the MFMA throughput probe")
    ap.add_argument("--no-tp-apply", action="store_true",
                    help="skip the measurement of the tensor-parallel local update (muon_apply)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain elementwise copy kernel (torch.add, fp32) over this "
                         "many MiB, the reference for scaling HBM byte counters")
    return ap.parse_args()


def nsflops(shapes, ns_steps):
    """Algorithmic flops per step and per kernel kind (same count as the oracle's).
    "dense" counts full products (4m^2 n + 2m^3 per iteration), the convention
    of literature that does not exploit the symmetry."""
    gram = square = update = dense = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        gram += m * (m + 1) * n
        square += m * m * (m + 1)
        update += 2 * m * m * n
        dense += 4 * m * m * n + 2 * m ** 3
    return {"gram": gram, "square": square, "update": update,
            "total": ns_steps * (gram + square + update), "dense": ns_steps * dense}


def cpu_baseline(wload, indices):
    """The fp64 oracle, as it stands, on a bounded sample of the workload's matrices."""
    import numpy as np
    from matrix_optimizer_step_muon_amd import workloads as wl
    from oracle import muon_ref as ref
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    mats = wl.generate(wload, indices)
    f64 = [tuple(wl.stored_to_f64(x, wload.dtype) for x in t) for t in mats]
    hp = wload.hparams()
    t0 = time.perf_counter()
    for (W, G, M) in f64:
        ref.muon_step(W, G, M, **hp)
    dt = time.perf_counter() - t0
    flops = sum(ref.step_flops(*wload.shapes[i], wload.ns_steps) for i in indices)
    shapes = [f"{wload.shapes[i][0]}x{wload.shapes[i][1]}" for i in indices]
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads or os.cpu_count(),
            "host_cpus": os.cpu_count(), "cpu_model": model,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"fp64 numpy oracle, full step on {len(indices)} of {len(wload.shapes)} "
                      f"matrices ({', '.join(shapes)}) of the same workload"}


class GpuSampler:
    """Samples the graphics clock and socket power of the GPU in use through
    amdsmi (the library under rocm-smi), on a background thread, while a `with`
    block runs. Best effort: where amdsmi or the device's metrics cannot be
    read, summary() says why instead."""

    def __init__(self, device_props, period_s=0.01):
        self.props = device_props
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._smi = None

    def _handle(self, smi):
        handles = smi.amdsmi_get_processor_handles()
        want = (getattr(self.props, "pci_domain_id", None), getattr(self.props, "pci_bus_id", None),
                getattr(self.props, "pci_device_id", None))
        for h in handles:
            try:
                dom, bus, rest = smi.amdsmi_get_gpu_device_bdf(h).split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    return h
            except Exception:
                continue
        if len(handles) == 1:
            return handles[0]
        raise RuntimeError(f"no amdsmi device matches PCI {want} among {len(handles)}")

    def __enter__(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = self._handle(amdsmi)
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        except Exception as e:  # noqa: BLE001 - any failure only disables sampling
            self.error = f"{type(e).__name__}: {e}"[:200]
        return self

    def _run(self):
        smi = self._smi
        while not self._stop.is_set():
            try:
                clk = smi.amdsmi_get_clock_info(self._h, smi.AmdSmiClkType.GFX)["clk"]
                pw = smi.amdsmi_get_power_info(self._h)
                self.samples.append((clk, pw.get("current_socket_power"), pw.get("power_limit")))
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"[:200]
                return
            self._stop.wait(self.period)

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        if self._smi is not None:
            try:
                self._smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass
        return False

    def summary(self):
        import numpy as np
        clk = [c for c, _, _ in self.samples if isinstance(c, (int, float))]
        if not clk:
            return {"source": "amdsmi", "samples": 0, "error": self.error or "no samples"}
        pw = [p for _, p, _ in self.samples if isinstance(p, (int, float))]
        lim = [q for _, _, q in self.samples if isinstance(q, (int, float))]
        limit = lim[-1] if lim else None
        if limit is not None and limit > 1e5:  # reported in microwatts
            limit = limit / 1e6
        return {"source": "amdsmi (the rocm-smi library): GFX clock and socket power, polled every "
                          "10 ms during the protocol runs",
                "samples": len(clk), "gfx_mhz_median": float(np.median(clk)),
                "gfx_mhz_min": min(clk), "gfx_mhz_max": max(clk),
                "socket_power_w_median": float(np.median(pw)) if pw else None,
                "power_limit_w": limit}


def protocol_runs(mu, dev, hparams, stream, runs, steps, warmup=3):
    """The pages' averaging protocol: `runs` fresh plans in this process, each
    with `warmup` untimed and `steps` timed consecutive steps on the same
    buffers. Returns the per-step times in ms."""
    import torch
    times = []
    for _ in range(runs):
        plan = mu.Plan(dev, **hparams)
        for _ in range(warmup):
            plan.step(stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for k in range(steps):
            plan.step(stream)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        times += [ev[k].elapsed_time(ev[k + 1]) for k in range(steps)]
        plan.close()
    return times


# Split kind of each matrix of a Qwen3 layer (q, k, v, o, gate, up, down):
# q, k, v, gate and up are column-parallel, o and down row-parallel.
QWEN3_LAYER_KINDS = ("column", "column", "column", "row", "column", "column", "row")


def tp_apply_measure(mu, shapes, dtype, stream, ranks=8, reps=20):
    """The tensor-parallel local update P_local += Delta W_local over every
    rank's shards of the given matrices (all ranks on this one GPU, so the
    shards cover the whole matrices), as one muon_apply launch. Inputs are
    resident; returns the average launch time and its HBM rate on the
    algorithmic bytes (read P and Delta W, write P)."""
    import torch
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    elem = 2 if dtype == "bf16" else 4
    pairs, keep, numel = [], [], 0
    for i, (r, c) in enumerate(shapes):
        kind = QWEN3_LAYER_KINDS[i % len(QWEN3_LAYER_KINDS)]
        D = torch.randn(r, c, device="cuda", dtype=torch.float32).mul_(4e-4).to(dt)
        keep.append(D)
        n = r if kind == "column" else c
        for k in range(ranks):
            a, b = k * n // ranks, (k + 1) * n // ranks
            view = D[a:b, :] if kind == "column" else D[:, a:b]
            P = torch.randn(view.shape, device="cuda", dtype=torch.float32).mul_(0.02).to(dt)
            pairs.append((P, view))
            numel += P.numel()
    plan = mu.ApplyPlan(pairs)
    plan.apply(stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        plan.apply(stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    plan.close()
    gbs = 3 * elem * numel / (ms / 1e3) / 1e9
    return {"shards": len(pairs), "ranks": ranks, "elements": numel, "avg_launch_ms": round(ms, 4),
            "alg_bytes_per_elem": 3 * elem, "achieved_gbs": round(gbs, 1), "peak_gbs": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "what": f"P_local += Delta W_local over all {ranks} ranks' TP shards of the workload's "
                    "matrices (column-parallel: row blocks; row-parallel: column blocks, strided views)"}


def master_weights_measure(mu, wload, stream, steps, warmup, alg_flops):
    """The same step with fp32 master weights and momentum and bf16 gradients
    (MUON_BF16_F32_MASTER), on the same shapes: seeded synthetic fp32 W and M
    and bf16 G, resident in HBM; `warmup` untimed and `steps` timed steps."""
    import torch
    dev = []
    for i, (r, c) in enumerate(wload.shapes):
        g = torch.Generator(device="cuda").manual_seed(1000 + i)
        W = torch.randn(r, c, device="cuda", generator=g).mul_(wload.w_std)
        G = torch.randn(r, c, device="cuda", generator=g).mul_(wload.g_std).to(torch.bfloat16)
        M = torch.randn(r, c, device="cuda", generator=g).mul_(wload.g_std)
        dev.append([W, G, M])
    plan = mu.Plan(dev, **wload.hparams())
    for _ in range(warmup):
        plan.step(stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        plan.step(stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    plan.close()
    del dev
    return {"dtype": "W, M fp32; G bf16; Newton-Schulz bf16", "ms_per_step": round(ms, 4),
            "value": round(alg_flops / (ms / 1e3) / 1e12, 2), "unit": "TFLOP/s",
            "fraction_of_peak": round(alg_flops / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "elementwise_min_bytes_per_elem": 18,
            "what": "the same shapes and step count; the elementwise minimum is 18 B per element "
                    "(read G 2, M 4, W 4; write M' 4, W' 4) against 10 B in bf16"}


def other_config_measure(mu, wload, stream, steps=10, runs=2, warmup=3):
    """A perf-only leg over another workload: the same shapes and dtype with
    seeded N(0, std^2) data drawn on the GPU (no parity here; the GPU tests
    compare these workloads with the oracle), `runs` fresh plans of `warmup`
    untimed and `steps` timed steps each, timed with events on the stream."""
    import numpy as np
    import torch
    dt = torch.bfloat16 if wload.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(7000 + wload.seed)
    dev = []
    for r, c in wload.shapes:
        W = torch.randn(r, c, device="cuda", generator=g).mul_(wload.w_std).to(dt)
        G = torch.randn(r, c, device="cuda", generator=g).mul_(wload.g_std).to(dt)
        M = (torch.randn(r, c, device="cuda", generator=g).mul_(wload.g_std).to(dt)
             if wload.momentum == "prev" else torch.zeros(r, c, device="cuda", dtype=dt))
        dev.append([W, G, M])
    torch.cuda.synchronize()
    times = []
    for _ in range(runs):
        plan = mu.Plan(dev, **wload.hparams())
        for _ in range(warmup):
            plan.step(stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            plan.step(stream)
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / steps)
        plan.close()
    del dev
    torch.cuda.empty_cache()
    ms = float(np.mean(times))
    fl = nsflops(wload.shapes, wload.ns_steps)["total"]
    out = {"matrices": len(wload.shapes), "dtype": wload.dtype, "ms_per_step": round(ms, 4),
           "ms_per_step_min": round(min(times), 4), "runs": runs, "steps_per_run": steps,
           "alg_tflop_per_step": round(fl / 1e12, 4)}
    if wload.dtype == "bf16":
        tf = fl / (ms / 1e3) / 1e12
        out.update({"tflops": round(tf, 2), "fraction_of_peak": round(tf / BF16_PEAK_TFLOPS, 4),
                    "ms_at_half_peak": round(fl / (0.5 * BF16_PEAK_TFLOPS * 1e12) * 1e3, 3)})
    else:
        out["note"] = "fp32 and latency-bound (0.0012 TFLOP per step): ms only"
    return out


def hbm_ceiling_measure(stream, mib=2048, reps=10):
    """What plain streaming kernels reach on this GPU: torch's elementwise
    copy (read 1, write 1, the momentum kernel's 1:1 mix) and add of two
    tensors (read 2, write 1, the shard apply's mix) over `mib` MiB per
    operand of fp32, resident in HBM, timed with events."""
    import torch
    n = mib * 2**20 // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
    b = torch.empty_like(a).uniform_()
    c = torch.empty_like(a)
    out = {}
    for name, fn, nbytes in (("copy", lambda: c.copy_(a), 2 * 4 * n),
                             ("add", lambda: torch.add(a, b, out=c), 3 * 4 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"gbs": round(nbytes / (ms / 1e3) / 1e9, 1), "avg_launch_ms": round(ms, 4),
                     "bytes_per_launch": nbytes}
    del a, b, c
    torch.cuda.empty_cache()
    out["what"] = (f"torch copy_ and add over {mib} MiB fp32 operands: the streaming rate a plain "
                   "elementwise kernel reaches, against which the HBM-bound kernels are read")
    return out


def dp_partition_measure(mu, wl, ranks=32, tp=8):
    """The DP static partition (host) of a Qwen3-32B-shaped buffer: one TP
    rank's local parameters in buckets, over `ranks` DP ranks, by the
    Start_Index rule and by the alpha-Balanced Greedy LPT algorithm (alpha = 1,
    loads = element counts). Reports R_LB = max/avg over ranks of the memory
    (elements) and of the Muon FLOPs per step, and the planner's time."""
    import math
    buckets = wl.qwen3_32b_param_buffer(tp=tp)
    sizes = [[math.prod(p) for p in b] for b in buckets]
    flops = [[nsflops([p], 5)["total"] if len(p) == 2 else math.prod(p) for p in b] for b in buckets]
    def r_lb(cuts, loads):
        tot = [0.0] * ranks
        for b, c in zip(loads, cuts):
            for r in range(ranks):
                tot[r] += sum(b[c[r]:c[r + 1]])
        return round(max(tot) / (sum(tot) / ranks), 3)
    out = {"buffer": f"Qwen3-32B-shaped, TP={tp} local shards, buckets of >= 40M elements",
           "buckets": len(buckets), "params": sum(len(b) for b in buckets), "dp_ranks": ranks}
    mu.dp_partition(sizes, ranks, alpha=1.0)   # first call: loads the library
    for name, alpha in (("static", None), ("alpha_balanced", 1.0)):
        t0 = time.perf_counter()
        cuts, _ = mu.dp_partition(sizes, ranks, alpha=alpha)
        ms = (time.perf_counter() - t0) * 1e3
        out[name] = {"R_LB_memory": r_lb(cuts, sizes), "R_LB_flops": r_lb(cuts, flops), "ms": round(ms, 3)}
    return out


def tp_micro_groups_measure(mu, ranks=8):
    """The TP micro-group schedule (host) of a Qwen3-32B-shaped model's
    TP-split tensors (64 layers of q, k, v, o, gate, up, down) over `ranks` host
    ranks, cost = element count, C_max = the largest tensor's cost.

    Groups run one after another and each waits for its slowest host rank, so
    the schedule's cost is the sum over groups of the largest rank load. The
    report gives that sum over the sum of the mean rank loads (1.0 = every
    group perfectly balanced), for the hosted elements and the hosted Muon
    FLOPs, against one group per layer with hosts dealt round-robin, plus the
    group count and the planner's time."""
    import math
    shapes = [(8192, 5120), (1024, 5120), (1024, 5120), (5120, 8192), (25600, 5120), (25600, 5120),
              (5120, 25600)] * 64
    numel = [float(math.prod(s)) for s in shapes]
    flops = [float(nsflops([s], 5)["total"]) for s in shapes]

    def makespan_ratio(groups, loads):
        worst = mean = 0.0
        for ids, hosts in groups:
            tot = [0.0] * ranks
            for i, h in zip(ids, hosts):
                tot[h] += loads[i]
            worst += max(tot)
            mean += sum(tot) / ranks
        return round(worst / mean, 3)

    mu.tp_micro_groups(numel, ranks, max(numel))   # first call: loads the library
    t0 = time.perf_counter()
    groups = mu.tp_micro_groups(numel, ranks, max(numel))
    ms = (time.perf_counter() - t0) * 1e3
    per_layer = [(list(range(7 * l, 7 * l + 7)), [i % ranks for i in range(7 * l, 7 * l + 7)]) for l in range(64)]
    return {"tensors": len(shapes), "host_ranks": ranks, "c_max": "the largest tensor's element count",
            "groups": len(groups), "ms": round(ms, 3),
            "micro_groups": {"makespan_ratio_memory": makespan_ratio(groups, numel),
                             "makespan_ratio_flops": makespan_ratio(groups, flops)},
            "per_layer_round_robin": {"groups": len(per_layer),
                                      "makespan_ratio_memory": makespan_ratio(per_layer, numel),
                                      "makespan_ratio_flops": makespan_ratio(per_layer, flops)}}


def mfma_probe_measure(mu, stream, reps=6, iters=400_000):
    """The bf16 MFMA rate the chip sustains on random register data: two
    workgroups of 4 waves per CU issuing 32x32x16 MFMAs back to back
    (muon_mfma_probe), `reps` timed launches after one untimed, with the GPU
    clock sampled meanwhile."""
    import torch
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * n_cu
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    mu.mfma_probe(out, blocks, iters // 10, stream)
    torch.cuda.synchronize()
    sampler = GpuSampler(torch.cuda.get_device_properties(0))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with sampler:
        a.record(stream)
        for _ in range(reps):
            mu.mfma_probe(out, blocks, iters, stream)
        b.record(stream)
        torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = blocks * 4 * iters * 8 * 32768
    clock = sampler.summary()
    return {"tflops": round(flops / (ms / 1e3) / 1e12, 1), "avg_launch_ms": round(ms, 3),
            "gfx_mhz_median": clock.get("gfx_mhz_median"), "socket_power_w_median": clock.get("socket_power_w_median"),
            "what": "bf16 32x32x16 MFMAs back to back on random register operands, 8 waves per CU"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "update_kernel_traffic_qwen3_32b_layer.txt")
KERNEL_SOURCE = os.path.join(ROOT, "matrix_optimizer_step_muon_amd", "csrc", "muon_kernels.hip")


def kernel_source_hash() -> str:
    import hashlib
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def committed_traffic(workload: str):
    """HBM bytes per update launch from the committed rocprofv3 counter summary.

    FETCH_SIZE and WRITE_SIZE of the update kernel, each scaled by what the same
    counter reads for a plain copy kernel of known size. The value is used only
    if the counters were taken on this exact kernel source and workload, and
    is None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash() or t.get("workload") != workload:
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the Muon step of one rank needs no communication, so N ranks run N independent "
              "copies of this benchmark)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from matrix_optimizer_step_muon_amd import muon as mu
    from matrix_optimizer_step_muon_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    wload = wl.WORKLOADS[args.workload]
    dt_torch = torch.bfloat16 if wload.dtype == "bf16" else torch.float32

    print(f"[bench] generating {args.workload}: {len(wload.shapes)} matrices, "
          f"{wload.numel / 1e6:.1f} M elements, {wload.dtype}", file=sys.stderr, flush=True)
    dev = []
    for i in range(len(wload.shapes)):
        W, G, M = wl.generate_matrix(wload, i)
        ts = []
        for a in (W, G, M):
            if wload.dtype == "bf16":
                ts.append(torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda())
            else:
                ts.append(torch.from_numpy(a).cuda())
        dev.append(ts)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    if args.chains > 0:
        os.environ["MUON_CHAINS"] = str(args.chains)
    plan = mu.Plan(dev, **wload.hparams())
    info = plan.info()
    print(f"[bench] plan: workspace {plan.workspace_bytes() / 2**30:.2f} GiB, {info}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        plan.step(stream)
    torch.cuda.synchronize()

    # The timed region: no per-kernel events, one event before the first
    # step and one after each step. The spans give per-step times, the
    # first-to-last span the total.
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(args.steps):
        plan.step(stream)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[-1])
    step_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    ms_per_step = total_ms / args.steps
    print(f"[bench] {args.steps} steps in {total_ms:.2f} ms", file=sys.stderr, flush=True)

    if args.copy_probe_mib:
        n = args.copy_probe_mib * 2**20 // 4
        src = torch.empty(n, dtype=torch.float32, device="cuda").uniform_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)   # one kernel: reads and writes copy_probe_mib MiB
        torch.cuda.synchronize()
        del src, dst

    # Per-kernel durations and the update kernel's roofline, from a separate
    # pass of the same steps on a single-chain plan, with the library's HIP
    # event pairs around every launch (on the stream each kernel runs on).
    # With two chains a chain's launches share the GPU with the other chain's
    # kernels in their tails, and their spans overlap, so they do not measure
    # the kernels.
    ktimes = None
    if not args.no_roofline_pass:
        saved = os.environ.get("MUON_CHAINS")
        os.environ["MUON_CHAINS"] = "1"
        try:
            plan1 = mu.Plan(dev, **wload.hparams())
        finally:
            if saved is None:
                del os.environ["MUON_CHAINS"]
            else:
                os.environ["MUON_CHAINS"] = saved
        for _ in range(args.warmup):
            plan1.step(stream)
        torch.cuda.synchronize()
        plan1.reset_timing()
        plan1.set_timing(True)
        for _ in range(args.steps):
            plan1.step(stream)
        torch.cuda.synchronize()
        plan1.set_timing(False)
        ktimes = plan1.kernel_times()
        plan1.close()
        print(f"[bench] per-kernel pass: {args.steps} single-chain steps", file=sys.stderr, flush=True)
    upd_times = ktimes["update"] if ktimes else (0.0, 0)
    mom_times = ktimes["momentum"] if ktimes else (0.0, 0)

    # The pages' protocol (runs x steps, each run a fresh plan), with the clock
    # sampled over its span of several seconds (the device's metrics refresh
    # too slowly to be sampled over the shorter timed region above).
    proto = None
    clock = None
    if args.runs > 0 and args.run_steps > 0:
        psampler = GpuSampler(torch.cuda.get_device_properties(0))
        with psampler:
            pt = protocol_runs(mu, dev, wload.hparams(), stream, args.runs, args.run_steps)
        proto = {"runs": args.runs, "steps_per_run": args.run_steps, "warmup_per_run": 3,
                 "mean_ms": round(float(np.mean(pt)), 4), "median_ms": round(float(np.median(pt)), 4),
                 "min_ms": round(min(pt), 4), "max_ms": round(max(pt), 4)}
        clock = psampler.summary()
        print(f"[bench] protocol: {args.runs} runs x {args.run_steps} steps, mean {proto['mean_ms']:.3f} ms",
              file=sys.stderr, flush=True)

    def aux(name, fn):
        """An auxiliary measurement: a failure is recorded in the line instead
        of ending the run, so the headline measurement above is never lost."""
        try:
            res = fn()
            print(f"[bench] {name}: {json.dumps(res)[:200]}", file=sys.stderr, flush=True)
            return res
        except Exception as e:  # noqa: BLE001 - any failure is reported, not raised
            print(f"[bench] {name} failed: {e}", file=sys.stderr, flush=True)
            return {"error": f"{type(e).__name__}: {e}"[:300]}

    master = None
    if wload.dtype == "bf16" and not args.no_master_weights:
        master = aux("fp32 master weights", lambda: master_weights_measure(
            mu, wload, stream, args.steps, args.warmup, nsflops(wload.shapes, wload.ns_steps)["total"]))
    probe = None if args.no_mfma_probe else aux("mfma probe", lambda: mfma_probe_measure(mu, stream))
    dp_part = aux("dp partition", lambda: dp_partition_measure(mu, wl))
    tp_groups = aux("tp micro groups", lambda: tp_micro_groups_measure(mu))
    tp_apply = None
    if not args.no_tp_apply:
        tp_apply = aux("tp apply", lambda: tp_apply_measure(mu, wload.shapes, wload.dtype, stream))
    ceiling = aux("hbm ceiling", lambda: hbm_ceiling_measure(stream))
    others = None
    if not args.no_other_configs:
        others = {}
        for name, w in wl.WORKLOADS.items():
            if name != args.workload:
                others[name] = aux(f"config {name}", lambda w=w: other_config_measure(mu, w, stream))

    fl = nsflops(wload.shapes, wload.ns_steps)
    tflops = fl["total"] / (ms_per_step / 1e3) / 1e12
    peak = BF16_PEAK_TFLOPS if wload.dtype == "bf16" else F32_PEAK_TFLOPS
    # Update launches: ns_steps per chain and step, each over its chain's
    # matrices. Flops per launch = the step's update flops / its launches.
    upd_ms, upd_n = upd_times
    upd_avg = upd_ms / max(upd_n, 1)
    upd_per_step = upd_n / args.steps if upd_n else 0
    upd_flops = fl["update"] * wload.ns_steps / upd_per_step if upd_n else 0.0
    upd_tflops = upd_flops / (upd_avg / 1e3) / 1e12 if upd_n else None
    per_kernel = None
    if ktimes:
        per_kernel = {k: {"avg_ms": round(v[0] / v[1], 4), "launches": v[1],
                          "ms_per_step": round(v[0] / args.steps, 4)} for k, v in ktimes.items() if v[1]}
        per_kernel["timed_in"] = ("a separate pass of the same steps on a single-chain plan, one HIP event "
                                  "pair per launch; the headline steps run two chains whose launches overlap")
    elem = 2 if wload.dtype == "bf16" else 4
    # Momentum kernel algorithmic bytes: read G, M; write M' and U. A step
    # runs one momentum launch per chain (or one over all matrices); its time
    # per step, from the same pass as the update roofline, covers every element.
    mom_ms = mom_times[0] / args.steps
    mom_gbs = 4 * elem * wload.numel / (mom_ms / 1e3) / 1e9 if mom_times[1] else None

    out = {
        "metric": "Muon optimizer-step ms + achieved bf16 MFMA TFLOP/s (fraction of peak) per rank share",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wload.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "matrices": len(wload.shapes),
                   "shapes": sorted({f"{r}x{c}" for r, c in wload.shapes}),
                   "elements": wload.numel, "ns_steps": wload.ns_steps, "lr": wload.lr,
                   "beta": wload.beta, "nesterov": wload.nesterov,
                   "alg_tflop_per_step": round(fl["total"] / 1e12, 3)},
        "fraction_of_peak": round(tflops / peak, 4),
        "step_ms": {"mean": round(ms_per_step, 4), "median": round(float(np.median(step_ms)), 4),
                    "min": round(min(step_ms), 4), "max": round(max(step_ms), 4)},
        "dense_equiv_tflops": round(fl["dense"] / (ms_per_step / 1e3) / 1e12, 2),
        "protocol": proto,
        "gpu_clock": clock,
        # The same rate against the dense peak scaled to the observed clock
        # (the published peak assumes 2.4 GHz; the chip runs at its power cap).
        "fraction_of_peak_at_observed_clock": (
            round(tflops / (peak * clock["gfx_mhz_median"] / 2400.0), 4)
            if clock and clock.get("gfx_mhz_median") else None),
        "roofline": {
            "kernel": "update (X' = aX + BX; weight apply on the last iteration)",
            "bound": "mfma",
            "achieved": round(upd_tflops, 2) if upd_tflops else None,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(upd_tflops / peak, 4) if upd_tflops else None,
            "traffic": committed_traffic(args.workload),
            "traffic_unit": ("bytes per launch at the L2's memory-side interface (rocprofv3 FETCH_SIZE + "
                             "WRITE_SIZE, copy-scaled): L2 misses, all addressed to DRAM; the Infinity Cache's "
                             "share of them has no counter on this GPU"),
            "alg_tflop_per_launch": round(upd_flops / 1e12, 4),
            "launches_per_step": upd_per_step,
            "timed_in": "a separate single-chain pass of the same steps",
            "avg_launch_ms": round(upd_avg, 4),
        },
        "kernels": per_kernel,
        "master_weights": master,
        "mfma_probe": probe,
        # The step's rate against the bf16 MFMA rate the chip sustains on
        # random data under its power limit (the probe above).
        "fraction_of_mfma_probe": round(tflops / probe["tflops"], 4) if probe and probe.get("tflops") else None,
        "dp_partition": dp_part,
        "tp_micro_groups": tp_groups,
        "tp_apply": tp_apply,
        "momentum_hbm": {"achieved_gbs": round(mom_gbs, 1) if mom_gbs else None,
                         "peak_gbs": HBM_PEAK_GBS, "alg_bytes_per_elem": 4 * elem},
        "hbm_ceiling": ceiling,
        "other_configs": others,
        "device": torch.cuda.get_device_name(0),
        "host": platform.node(),
    }
    plan.close()
    del dev
    torch.cuda.empty_cache()

    # The HBM-bound kernels against the streaming ceiling of the same mix.
    if ceiling and "copy" in ceiling:
        if mom_gbs:
            out["momentum_hbm"]["fraction_of_copy_ceiling"] = round(mom_gbs / ceiling["copy"]["gbs"], 4)
        if tp_apply and tp_apply.get("achieved_gbs"):
            tp_apply["fraction_of_add_ceiling"] = round(tp_apply["achieved_gbs"] / ceiling["add"]["gbs"], 4)

    if not args.no_cpu_baseline:
        idx = (list(range(len(wload.shapes))) if args.cpu_sample == "all"
               else [int(x) for x in args.cpu_sample.split(",") if x != ""])
        print(f"[bench] cpu baseline: oracle on matrices {idx}", file=sys.stderr, flush=True)
        try:
            out["cpu_baseline"] = cpu_baseline(wload, idx)
        except Exception as e:  # noqa: BLE001 - the line is still printed
            print(f"[bench] cpu baseline failed: {e}", file=sys.stderr, flush=True)
            out["cpu_baseline"] = {"value": None, "error": f"{type(e).__name__}: {e}"[:300]}
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
