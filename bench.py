"""Benchmark: forward + backward of the blocked vocabulary-projection
cross-entropy on one MI355X.

A step is one vpce_forward + one vpce_backward over the whole batch of the
one-GPU slice of a 1M-token context (N=65536 tokens, d=7168, V=129280, R=8
shards, bf16 inputs, fp32 accumulation and gradients), with the inputs already
resident in HBM. Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--cpu-seconds S] [--input-cache DIR]
                    [--no-clock] [--chunk-cols C]
    python bench.py --copy-calibration   # plain 1 GiB device copies, for
                                         # scaling HBM traffic counters

Roofline: the timed steps call the library's traced variants of the forward
and the backward, which record a HIP event pair on the library's stream (the
current torch stream, passed to the C ABI) around every kernel launch. The
line's roofline block is for the kernel with the most GPU time per step: its
algorithmic flops per launch (2*N*d*V for the forward tile kernel, 2*N*d*C
for the logit recompute of a backward chunk of C vocabulary columns and
4*N*d*C for the launch that forms both its products) over its mean launch
duration.
Every kernel kind's own figures are listed under roofline.kernels. HBM
traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE counter runs
of this same script, scaled by the counters' reading for plain device copies
of known size; it is stored in profiles/ with a hash of the built device code
and reported only while that code is unchanged.
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

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz (dense)
PEAK_F32_TFLOPS = 157.3
HEADLINE = "ctx1m_slice_n64k_d7168_v129k_r8"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_code_hash() -> str:
    """Hash of the device code built into libvpce.so (its .hip_fatbin ELF
    section), so that stored counter readings go stale exactly when the
    compiled kernels change, and not when only comments or dead code do."""
    import struct
    path = os.path.join(ROOT, "vocabulary_projection_cross_amd", "libvpce.so")
    with open(path, "rb") as f:
        elf = f.read()
    if elf[:4] != b"\x7fELF" or elf[4] != 2:
        raise RuntimeError(f"{path} is not a 64-bit ELF file")
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)

    def section(i):
        name, _, _, _, off, size = struct.unpack_from("<IIQQQQ", elf,
                                                     shoff + i * shentsize)
        return name, off, size

    _, stroff, _ = section(shstrndx)
    for i in range(shnum):
        name, off, size = section(i)
        end = elf.index(b"\0", stroff + name)
        if elf[stroff + name:end] == b".hip_fatbin":
            return hashlib.sha256(elf[off:off + size]).hexdigest()[:16]
    raise RuntimeError(f"{path} holds no .hip_fatbin section")


KERNEL_NAMES = {"forward_tile": "fwd_lse_kernel",
                "recompute": "recompute_g_kernel",
                "products": "prod_pair_kernel (dW = G^T H and dH += G W)",
                "merge": "merge_kernel", "other": "fill/loss/scale kernels"}
# algorithmic flops of one launch per backward-chunk column: the recompute
# forms one N x C logit chunk (2 N d C), the product launch both dW and dH of
# the chunk (2 x 2 N d C)
CHUNK_PRODUCTS = {"recompute": 1, "products": 2}


def chunk_widths(w, C):
    """Vocabulary columns of each backward chunk, in launch order: shards in
    ring order (the first V mod R one row wider), each cut into chunks of at
    most C columns."""
    base, extra = divmod(w.V, w.R)
    out = []
    for r in range(w.R):
        vw = base + (1 if r < extra else 0)
        out += [min(C, vw - c0) for c0 in range(0, vw, C)]
    return out


def kernel_table(w, kinds_f, fev, kinds_b, bev, C):
    """Per kernel kind: launches per step, mean duration per launch and per
    step (HIP events around each launch, averaged over the timed steps), and
    the algorithmic flops of its launches (2 N d V for the forward tile
    kernel; per backward chunk of C columns 2 N d C for the recompute and
    4 N d C for the launch holding both products)."""
    widths = chunk_widths(w, C)
    steps = len(fev)
    table = {}
    for kinds, evs in ((kinds_f, fev), (kinds_b, bev)):
        chunk = {k: 0 for k in CHUNK_PRODUCTS}
        for i, kind in enumerate(kinds):
            ms = sum(evs[s][2 * i].elapsed_time(evs[s][2 * i + 1])
                     for s in range(steps)) / steps
            if kind == "forward_tile":
                fl = 2.0 * w.N * w.d * w.V
            elif kind in chunk:
                fl = (2.0 * CHUNK_PRODUCTS[kind] * w.N * w.d *
                      widths[chunk[kind]])
                chunk[kind] += 1
            else:
                fl = 0.0
            t = table.setdefault(kind, {"kernel": KERNEL_NAMES[kind],
                                        "launches_per_step": 0,
                                        "ms_per_step": 0.0, "flops": 0.0})
            t["launches_per_step"] += 1
            t["ms_per_step"] += ms
            t["flops"] += fl
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    for t in table.values():
        n = t["launches_per_step"]
        t["launch_ms"] = t["ms_per_step"] / n
        t["flops_per_launch"] = t.pop("flops") / n
        if t["flops_per_launch"] > 0:
            tf = t["flops_per_launch"] / (t["launch_ms"] * 1e-3) / 1e12
            t["tflops"] = tf
            t["frac"] = tf / peak
    return table


def traffic_record(workload: str, kernel: str, chunk_cols=None):
    """Measured HBM bytes per launch of `kernel`, if the stored counter
    summary was taken from the device code built now (and, for the backward
    kernels, at the same chunk width)."""
    stem = kernel.split(" ")[0]
    path = os.path.join(ROOT, "profiles",
                        f"{stem}_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_code_hash") != kernel_code_hash():
        return None
    if chunk_cols is not None and rec.get("chunk_cols", chunk_cols) != \
            chunk_cols:
        return None
    return rec


class ClockSampler:
    """Samples the shader clock of every XCD with `amd-smi metric --clock`
    (a child process) while the timed steps run; reports the median of the
    per-sample XCD means, or None where the tool is missing or fails."""

    def __init__(self, enabled=True):
        import threading
        self.enabled = enabled
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import subprocess
        while not self._stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "--clock", "--json"],
                                   capture_output=True, text=True, timeout=10)
                data = json.loads(r.stdout)
                gpu = data["gpu_data"][0] if isinstance(data, dict) else data[0]
                clk = [v["clk"]["value"] for k, v in gpu["clock"].items()
                       if k.startswith("gfx_")]
                if clk:
                    self.samples.append(sum(clk) / len(clk))
            except Exception:
                return
            self._stop.wait(0.2)

    def __enter__(self):
        if self.enabled:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.enabled:
            self._thread.join(timeout=15)

    def median(self):
        if not self.samples:
            return None
        xs = sorted(self.samples)
        return float(xs[len(xs) // 2])


def cpu_baseline(inp, target_s=15.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workload: the first n tokens against the full vocabulary (forward and
    backward, 6 n d V flops). Returns tokens/s and the sample description."""
    from threadpoolctl import threadpool_info

    import oracle
    w = inp.workload
    Wf = inp.W_f64()

    def run(n):
        Hs = inp.H_f64(slice(0, n))
        ys = inp.labels[:n]
        t0 = time.perf_counter()
        oracle.forward(Hs, Wf, ys)
        oracle.backward(Hs, Wf, ys)
        return time.perf_counter() - t0

    # Grow the sample until it takes at least 70% of the target: small
    # samples carry fixed costs (the W conversion, thread start-up) that
    # make a one-shot extrapolation from a tiny probe undershoot.
    n = 32
    t = run(n)
    while t < 0.7 * target_s and n < w.N:
        grow = min(8.0, 1.25 * target_s / max(t, 1e-3))
        n = min(w.N, max(n + 32, int(n * grow) // 32 * 32))
        t = run(n)
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    blas = ",".join(sorted({d.get("internal_api", "?")
                            for d in threadpool_info()}))
    del Wf
    return {"value": n / t, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {n} of {w.N} tokens, full V={w.V}, d={w.d}; "
                      f"fp64 numpy ({blas}) forward+backward in {t:.1f} s "
                      f"({6.0 * n * w.d * w.V / t / 1e9:.1f} GFLOP/s)"}


def copy_calibration():
    """Plain device copies of known size, for scaling HBM traffic counters:
    3 copies of 1 GiB (each reads 1 GiB and writes 1 GiB)."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def load_inputs(w, cache_dir):
    """Seeded synthetic inputs; optionally kept as .npy files under cache_dir
    so repeated runs in one session skip the generation."""
    import numpy as np

    import workloads as WL
    if cache_dir:
        os.makedirs(cache_dir, exist_ok=True)
        stem = os.path.join(cache_dir, f"{w.name}_seed0")
        names = ("H", "W", "labels", "outliers")
        if all(os.path.exists(f"{stem}_{k}.npy") for k in names):
            arr = {k: np.load(f"{stem}_{k}.npy", mmap_mode="r") for k in names}
            return WL.Inputs(w, arr["H"], arr["W"], np.array(arr["labels"]),
                             np.array(arr["outliers"]))
        inp = WL.make_inputs(w, 0)
        for k, v in (("H", inp.H), ("W", inp.W), ("labels", inp.labels),
                     ("outliers", inp.outlier_rows)):
            np.save(f"{stem}_{k}.npy", v)
        return inp
    return WL.make_inputs(w, 0)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--input-cache", default=None)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--chunk-cols", type=int, default=None)
    # no shader-clock sampling (it starts amd-smi child processes, which a
    # profiler that has already initialised the GPU may not allow)
    ap.add_argument("--no-clock", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path across several GPUs "
              "(the ring of shards over RCCL) is not built, only described. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import vocabulary_projection_cross_amd as vp
    import workloads as WL

    w = WL.BY_NAME[args.workload]
    log(f"bench: generating {w.name} inputs")
    inp = load_inputs(w, args.input_cache)
    dev = torch.device("cuda:0")
    if w.dtype == "bf16":
        H = torch.from_numpy(np.ascontiguousarray(inp.H).view(np.int16)).to(
            dev).view(torch.bfloat16)
        W = torch.from_numpy(np.ascontiguousarray(inp.W).view(np.int16)).to(
            dev).view(torch.bfloat16)
    else:
        H = torch.from_numpy(np.ascontiguousarray(inp.H)).to(dev)
        W = torch.from_numpy(np.ascontiguousarray(inp.W)).to(dev)
    lab = torch.from_numpy(np.ascontiguousarray(inp.labels)).to(dev)
    dloss = torch.ones(1, dtype=torch.float32, device=dev)
    # the workspace at the widest backward chunk, or at --chunk-cols (the
    # planner's narrower chunks: less memory, more dH read-modify-writes)
    ws = torch.empty(vp.workspace_bytes(w.N, w.d, w.V, w.R, H.dtype,
                                        chunk_cols=args.chunk_cols),
                     dtype=torch.uint8, device=dev)
    chunk = args.chunk_cols or vp.plan(w.N, w.d, w.V, w.R, 1 << 62,
                                       H.dtype)["chunk_cols"]
    torch.cuda.synchronize()
    in_bytes = sum(t.numel() * t.element_size() for t in (H, W, lab))

    def step():
        loss, lse = vp.forward(H, W, lab, w.R, workspace=ws)
        dH, dW = vp.backward(H, W, lab, lse, dloss, w.R, workspace=ws)
        return loss, lse, dH, dW

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        out = step()
    torch.cuda.synchronize()
    out = None

    # The binding launches on torch's current stream; every event is
    # recorded there. Each timed step runs the traced calls, which bracket
    # every kernel launch with an event pair, so per-kernel durations come
    # from the timed steps themselves.
    stream = torch.cuda.current_stream(dev)

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
        for e in evs:          # torch creates the event on its first record
            e.record(stream)
        return evs

    _, lse0, _, n_fwd = vp.forward_traced(H, W, lab, w.R, [], workspace=ws)
    _, _, _, n_bwd = vp.backward_traced(H, W, lab, lse0, dloss, w.R, [],
                                        workspace=ws)
    del lse0
    fev = [new_events(n_fwd) for _ in range(args.steps)]
    bev = [new_events(n_bwd) for _ in range(args.steps)]
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    kinds_f = kinds_b = None
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    with ClockSampler(enabled=not args.no_clock) as clock:
        wall0 = time.perf_counter()
        t_all0.record(stream)
        for k in range(args.steps):
            ev[k][0].record(stream)
            loss, lse, kinds_f, _ = vp.forward_traced(H, W, lab, w.R, fev[k],
                                                      workspace=ws)
            ev[k][1].record(stream)
            dH, dW, kinds_b, _ = vp.backward_traced(H, W, lab, lse, dloss,
                                                    w.R, bev[k], workspace=ws)
            ev[k][2].record(stream)
        t_all1.record(stream)
        torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3 / args.steps
    total_ms = t_all0.elapsed_time(t_all1)
    fwd_ms = [a.elapsed_time(b) for a, b, _ in ev]
    bwd_ms = [b.elapsed_time(c) for _, b, c in ev]
    kernels = kernel_table(w, kinds_f, fev, kinds_b, bev, chunk)
    out_bytes = sum(t.numel() * t.element_size() for t in (loss, lse, dH, dW))
    # peak device bytes of one step, the previous outputs released
    del loss, lse, dH, dW
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    # device-level cross-check: the memory the device reports in use grows by
    # no more than torch's allocator reserved (the HIP runtime may hand back
    # memory it kept from earlier frees, so it can grow by less), so the
    # library allocated nothing of its own during the step
    free0 = torch.cuda.mem_get_info(dev)[0]
    reserved0 = torch.cuda.memory_reserved(dev)
    loss, lse, dH, dW = step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    requested_peak = torch.cuda.memory_stats()["requested_bytes.all.peak"]
    device_used_delta = free0 - torch.cuda.mem_get_info(dev)[0]
    reserved_delta = torch.cuda.memory_reserved(dev) - reserved0
    fixed = in_bytes + out_bytes
    planned = vp.plan(w.N, w.d, w.V, w.R, fixed + ws.numel(), H.dtype)
    ms = total_ms / args.steps
    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak_tf = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    # the dominant kernel: the most GPU time per step
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    dom_tf = dk["flops_per_launch"] / (dk["launch_ms"] * 1e-3) / 1e12
    trec = traffic_record(w.name, dk["kernel"], chunk)
    traffic = None
    if trec is not None:
        traffic = int(trec["hbm_bytes_per_launch"])
    result = {
        "metric": "fwd+bwd tokens/s of blocked vocab-proj CE; % bf16 MFMA "
                  "peak; peak bytes",
        "value": w.N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded; H~N(0,1), W scaled for logit std 3, "
                 "Zipf(1.1) labels over a permuted vocabulary, 2% ignored)"
                 if w.name == HEADLINE else "synthetic (seeded)"),
        "config": {"workload": w.name, "N": w.N, "d": w.d, "V": w.V,
                   "R": w.R, "chunk_cols": chunk, "global_batch": w.N,
                   "parallelism": "none"},
        "tflops": tflops,
        "pct_mfma_peak": 100.0 * tflops / peak_tf,
        "fwd_ms": float(np.mean(fwd_ms)),
        "bwd_ms": float(np.mean(bwd_ms)),
        "host_wall_ms_per_step": wall_ms,
        "peak_bytes": int(peak),
        "peak_bytes_split": {"inputs": int(in_bytes),
                             "outputs": int(out_bytes),
                             "workspace": int(ws.numel()),
                             "other": int(peak - in_bytes - out_bytes -
                                          ws.numel())},
        # exact bytes requested from the allocator at the peak (before its
        # block rounding) and the planner's prediction made before launch;
        # they differ by the 4-byte upstream-gradient scalar
        "requested_peak_bytes": int(requested_peak),
        # hipMemGetInfo's used-bytes growth over the step and the growth of
        # torch's reserved pool; the first exceeds the second only if
        # something outside torch allocated device memory
        "device_used_delta_bytes": int(device_used_delta),
        "torch_reserved_delta_bytes": int(reserved_delta),
        "planned_peak_bytes": planned["peak_bytes"],
        "roofline": {"bound": "mfma", "kernel": dk["kernel"],
                     "achieved": dom_tf, "peak": peak_tf, "unit": "TFLOP/s",
                     "frac": dom_tf / peak_tf, "traffic": traffic,
                     "flops_per_launch": dk["flops_per_launch"],
                     "launch_ms": dk["launch_ms"],
                     "launches_per_step": dk["launches_per_step"],
                     "share_of_step": dk["ms_per_step"] / ms,
                     # the whole step against the same peak, and every
                     # kernel's own figures (HIP events around each launch)
                     "step_frac": tflops / peak_tf,
                     "kernels": kernels,
                     # the published peak assumes a 2400 MHz shader clock;
                     # this is the clock the chip held during the timed steps
                     # (null when the timed steps last under 2 s: the
                     # sampler, a child process polling every 0.2 s, then
                     # mostly sees the idle clock before and after them)
                     "sclk_mhz_timed": (clock.median() if total_ms >= 2000.0
                                        else None),
                     "sclk_samples": len(clock.samples)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on a sample (CPU baseline)")
        del H, W, lab, dH, dW, ws
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
