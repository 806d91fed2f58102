#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

A step is one `attn_fwd` call over the whole workload (default: bf16, causal,
B = 2, H = 32, S = 4096, D = 128) with Q, K, V already resident in HBM.  The timed
calls go to the C entry point through the binding's raw function, with the buffers'
pointers resolved (and checked, by one call of the tensor function) beforehand.  First an
untimed clock-settle phase runs steps for a fixed wall time (`--settle-s`, 1 s by
default: from idle the GPU boosts, then drops under the power limit and takes about
50 ms to reach its steady clock); then W untimed warm-up steps; then exactly K steps
are timed between two device synchronisations.  One JSON line goes to stdout;
progress goes to stderr.

The line carries:
  value / ms_per_step   whole-job TFLOP/s (4*D FLOPs per visible query-key pair)
  roofline              the attention kernel against the dense bf16 MFMA peak, its
                        average duration measured with HIP events on the launch stream
                        over the K timed steps; the K steps are also cut into five
                        consecutive windows, each timed by its own events, and their
                        median per-launch time is reported beside the mean;
                        `traffic` is the HBM bytes per launch from the committed
                        counter summary when it matches the current kernel source
  clock                 the shader clock the driver reports while the timed steps run
                        (pp_dpm_sclk's current level, a smoothed value), the settle
                        phase's length, and the dense bf16 peak at that clock
  cpu_baseline          the fp64 CPU oracle timed on a bounded sample of the same
                        workload on this host (a reported baseline, not a target)

`--workload NAME` selects any workload of attention_attn_fwd_02_amd/workloads.py: the
forward configurations and variants, split-KV decoding (GB/s against the HBM peak),
the backward (dQ, dK, dV from the forward's O and LSE; 10*D FLOPs per visible pair)
and attention with the rotary embedding.  The library measures one GPU: `--gpus N`
with N > 1 exits with a message.

`--copy-mib N` instead runs N-MiB device copies (the calibration kernel for the
FETCH_SIZE / WRITE_SIZE counters).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CSRC = os.path.join(ROOT, "attention_attn_fwd_02_amd", "csrc")
# the sources whose hash a forward traffic summary carries: the kernels and their tile map
KERNEL_SRC = (os.path.join(CSRC, "attn_fwd_kernels.hip"), os.path.join(CSRC, "attn_fwd_tile_map.h"))
PROFILES = os.path.join(ROOT, "profiles")
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}   # dense MFMA peaks, MI355X
HBM_PEAK_GBS = 8000.0                                             # HBM3E, MI355X


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(src=KERNEL_SRC) -> str:
    """First 16 hex digits of the SHA-256 of one source file, or of several read one
    after the other."""
    h = hashlib.sha256()
    for path in ((src,) if isinstance(src, str) else src):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, prefix: str = "attn_fwd", src: str = KERNEL_SRC):
    """HBM bytes per launch of the dominant kernel from
    profiles/<prefix>_traffic_<workload>.txt, or None when the summary is absent or
    was taken on a different source of that kernel."""
    path = os.path.join(PROFILES, "%s_traffic_%s.txt" % (prefix, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class SclkSampler:
    """Samples the current shader clock the amdgpu driver reports (the line marked
    '*' in pp_dpm_sclk, in MHz) every 10 ms on a background thread."""

    def __init__(self):
        import glob
        files = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = files[0] if files else None
        self.values = []
        self._stop = False
        self._th = None

    def _read(self):
        for line in open(self.path):
            if line.rstrip().endswith("*"):
                tok = line.split(":", 1)[1].strip().split()[0].lower()
                return float(tok.replace("mhz", ""))
        return None

    def start(self):
        import threading
        if self.path is None:
            return self

        def run():
            while not self._stop:
                try:
                    v = self._read()
                    if v is not None:
                        self.values.append((time.perf_counter(), v))
                except (OSError, ValueError, IndexError):
                    pass
                time.sleep(0.01)
        self._th = threading.Thread(target=run, daemon=True)
        self._th.start()
        return self

    def stop(self):
        self._stop = True
        if self._th is not None:
            self._th.join()
        if not self.values:
            try:
                v = self._read() if self.path else None
                if v is not None:
                    self.values.append((time.perf_counter(), v))
            except (OSError, ValueError, IndexError):
                pass
        return self

    def summary(self, t0=None, t1=None):
        """Median, min and max of the samples taken between t0 and t1 (perf_counter
        seconds; all samples when no interval is given or none falls inside it)."""
        inside = [v for t, v in self.values if (t0 is None or t >= t0) and (t1 is None or t <= t1)]
        v = sorted(inside or [v for _, v in self.values])
        if not v:
            return None
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1],
                "samples": len(v), "source": "pp_dpm_sclk (driver-smoothed current level)"}


def timed_run(step, steps, stream, torch):
    """Exactly `steps` calls of `step` between two device synchronisations, cut
    into (up to) five consecutive windows, each bracketed by HIP events on the
    launch stream.  Returns (wall ms per step, event ms per launch over all steps,
    the windows' per-launch event ms, the perf_counter interval)."""
    nwin = min(5, steps)
    sizes = [steps // nwin + (1 if i < steps % nwin else 0) for i in range(nwin)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nwin + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i, n in enumerate(sizes):
        for _ in range(n):
            step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wins = [evs[i].elapsed_time(evs[i + 1]) / n for i, n in enumerate(sizes)]
    total = evs[0].elapsed_time(evs[-1]) / steps
    return (t1 - t0) * 1e3 / steps, total, wins, (t0, t1)


def copy_calibration(mib: int, steps: int):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copied %d MiB x %d" % (mib, steps))


def cpu_baseline(w, q, k, v, target_s: float):
    """Time the oracle (as it stands) on random query rows of the workload."""
    import numpy as np
    import oracle
    from attention_attn_fwd_02_amd import workloads as W
    total = w.B * w.Hq * w.Sq
    rng = np.random.default_rng(12345)
    off = w.Sk - w.Sq

    def pairs(rows):
        i = rows % w.Sq
        if not w.causal:
            return int(len(rows) * w.Sk)
        return int(np.clip(i + off + 1, 0, w.Sk).sum())

    # calibrate on a warm oracle (the first call also loads the library and
    # starts its threads), then size the timed sample for about target_s seconds
    probe = rng.integers(0, total, size=256)
    oracle.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, rows=probe[:16])
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, rows=probe)
    t_probe = time.perf_counter() - t0
    rate = pairs(probe) / max(t_probe, 1e-6)                 # pairs per second
    mean_pairs = W.visible_pairs(w.B, w.Hq, w.Sq, w.Sk, w.causal) / total
    n = int(max(16, min(total, target_s * rate / max(mean_pairs, 1.0))))
    rows = rng.integers(0, total, size=n)
    log("cpu baseline: oracle on %d rows (~%.0f s)" % (n, n * mean_pairs / rate))
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, causal=w.causal, scale=w.scale, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * pairs(rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d uniformly drawn query rows (seed 12345) of the %d rows, each over all "
                      "its visible keys; fp64; %.1f s; FLOPs = 4*D per visible pair"
                      % (n, total, dt)}


def decode_line(args, w, name, wall_ms, kern_ms, med_ms, clock):
    """JSON line of a decode workload: bound by HBM bytes (K and V read once, Q read
    and O, LSE written once), so the figure is GB/s against the 8 TB/s peak.  The
    timed step is both kernels (split-KV pass and merge); the partial results they
    exchange are not counted as algorithmic bytes."""
    nbytes = w.min_hbm_bytes()
    return {
        "metric": "attention decode GB/s (split-KV, bf16, Sk=4096 D=128) + % of HBM peak",
        "value": round(nbytes / (wall_ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Sk": w.Sk, "D": w.D, "causal": w.causal, "seed": w.seed,
                   "bytes_per_step": nbytes, "flops_per_step": w.flops()},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (kern_ms * 1e-3) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": committed_traffic(name, "attn_decode",
                                                  os.path.join(CSRC, "attn_decode_kernels.hip")),
                     "kernel_ms_per_launch": round(kern_ms, 5),
                     "kernel_ms_median_of_5": round(med_ms, 5)},
        "clock": clock,
        "cpu_baseline": None,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1,
                    help="GPUs to run on; only 1 is supported (the path has no multi-GPU part)")
    ap.add_argument("--steps", type=int, default=200, help="timed steps")
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps after the settle phase")
    ap.add_argument("--settle-s", type=float, default=1.0,
                    help="untimed clock-settle phase before the warm-up, in seconds of wall time")
    ap.add_argument("--workload", default=None,
                    help="a workload of attention_attn_fwd_02_amd/workloads.py (default: the headline, "
                         "causal bf16 B=2 H=32 S=4096 D=128)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="about how long the oracle's CPU baseline sample runs")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle's CPU baseline")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="instead of attention, time a plain device copy of this many MiB (the "
                         "reference for scaling the HBM traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: the attention library measures one GPU; --gpus %d is not supported "
              "(the attention forward shards over (batch, head) with no exchange, "
              "so N GPUs would each run this one-GPU workload on their share)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_mib:
        copy_calibration(args.copy_mib, max(1, args.steps))
        return

    from attention_attn_fwd_02_amd import (ATTN_BF16, ATTN_FP16, ATTN_FP32, AttnError, attn_bwd,
                                           attn_fwd, attn_fwd_decode, attn_fwd_rope, bwd, fwd,
                                           fwd_decode, fwd_rope, load_library)
    from attention_attn_fwd_02_amd import workloads as W
    load_library()
    name = args.workload or W.HEADLINE
    w = W.lookup(name)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log("device: %s, %d CUs; workload %s" % (props.name, props.multi_processor_count, name))

    q, k, v = W.make_inputs(w)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    decode = name in W.DECODE
    backward = name in W.BACKWARD
    rope = name in W.ROPE
    dt = {"bf16": ATTN_BF16, "fp16": ATTN_FP16, "fp32": ATTN_FP32}[w.dtype]
    shape = (w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D)
    sh = stream.cuda_stream

    # Each workload runs once through the binding's tensor function (which checks every
    # buffer); the timed steps then call the same C entry point through the binding's
    # raw function with the pointers resolved once, so that no per-call Python checks
    # sit between launches.
    def checked(st):
        if st != 0:
            raise AttnError(st)
    if rope:
        # rotary embedding on Q and K: the key pass and the attention kernel both
        # run in every step; tables and the rotated-key buffer are allocated once
        ct, st_ = (t.to(dev) for t in W.rope_tables(w.Sk, w.D))
        k_rot = torch.empty_like(kd)
        layout = W.ROPE_LAYOUT[name]
        fwd_rope(qd, kd, vd, ct, st_, layout=layout, causal=w.causal, scale=w.scale, out=o,
                 lse=lse, k_rot=k_rot, stream=stream)
        raw = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
               k_rot.data_ptr(), ct.data_ptr(), st_.data_ptr(), layout) + shape + \
              (w.scale, int(w.causal), dt, sh)

        def step():
            checked(attn_fwd_rope(*raw))
    elif backward:
        # gradients of the forward; its O and LSE are computed once, outside the timing
        from attention_attn_fwd_02_amd import attn_bwd_workspace
        dod = W.make_dout(w, q).to(dev)
        fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        st_, nbytes = attn_bwd_workspace(*shape)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        bwd(qd, kd, vd, o, lse, dod, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv,
            workspace=ws, stream=stream)
        raw = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
               dod.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()) + shape + \
              (w.scale, int(w.causal), dt, ws.data_ptr(), ws.numel(), sh)

        def step():
            checked(attn_bwd(*raw))
    elif decode:
        # split-KV pass + merge; the workspace is allocated once, outside the timing
        from attention_attn_fwd_02_amd import attn_fwd_decode_workspace
        st_, nbytes = attn_fwd_decode_workspace(*shape, 0)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
        fwd_decode(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse,
                   workspace=ws, stream=stream)
        raw = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr()) + \
              shape + (w.scale, int(w.causal), dt, 0, ws.data_ptr(), ws.numel(), sh)

        def step():
            checked(attn_fwd_decode(*raw))
    else:
        fwd(qd, kd, vd, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        raw = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr()) + \
              shape + (w.scale, int(w.causal), dt, sh)

        def step():
            checked(attn_fwd(*raw))

    # the clock sampler starts here and keeps only the samples taken during the timed
    # steps; from here on the GPU is kept busy up to the timed region (an idle GPU boosts
    # and then dips below its steady clock for its first twenty or so launches)
    sampler = SclkSampler().start()

    # clock settle: whole steps for a fixed wall time, in batches of 16; the host waits
    # for the batch before the last one, so the queue never runs dry
    settle_steps = 0
    pending = []
    t_end = time.perf_counter() + max(0.0, args.settle_s)
    while time.perf_counter() < t_end:
        for _ in range(16):
            step()
        settle_steps += 16
        ev = torch.cuda.Event()
        ev.record(stream)
        pending.append(ev)
        if len(pending) > 2:
            pending.pop(0).synchronize()

    # the warm-up runs straight into the timed region, whose opening synchronisation ends it
    for _ in range(args.warmup):
        step()
    wall_ms, kern_ms, wins, (t0, t1) = timed_run(step, args.steps, stream, torch)
    sampler.stop()
    log("clock settle: %d steps in %.2f s; warm-up: %d steps" % (settle_steps, args.settle_s, args.warmup))
    med_ms = sorted(wins)[len(wins) // 2]
    flops = W.bwd_flops(w) if backward else w.flops()
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    sclk = sampler.summary(t0, t1)
    clock = {"settle_s": args.settle_s, "settle_steps": settle_steps, "sclk": sclk}
    if sclk and w.dtype in ("bf16", "fp16"):
        # dense 16-bit MFMA: 4096 FLOP per CU per clock
        clock["bf16_peak_at_sclk_tflops"] = round(
            props.multi_processor_count * 4096 * sclk["median_mhz"] * 1e6 / 1e12, 1)
    log("timed %d steps: %.3f ms/step wall, %.4f ms/launch (events; windows %s), %.1f TFLOP/s, sclk %s"
        % (args.steps, wall_ms, kern_ms, " ".join("%.4f" % x for x in wins), achieved,
           sclk["median_mhz"] if sclk else "n/a"))

    if decode:
        print(json.dumps(decode_line(args, w, name, wall_ms, kern_ms, med_ms, clock)), flush=True)
        return

    cpu = None
    if not args.no_cpu_baseline and not backward and not rope:
        cpu = cpu_baseline(w, q, k, v, args.cpu_seconds)
        log("cpu baseline: %.4g TFLOP/s on %d threads" % (cpu["value"], cpu["cores"]))

    metric = "attention fwd TFLOP/s (bf16, causal S=4096 D=128) + % of MFMA peak"
    if backward:
        metric = "attention bwd TFLOP/s (bf16, causal S=4096 D=128, 10*D FLOP per pair) + % of MFMA peak"
    elif rope:
        metric = "attention fwd with RoPE on Q and K, TFLOP/s (bf16, causal S=4096 D=128) + % of MFMA peak"
    line = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Sk": w.Sk, "D": w.D, "causal": w.causal, "seed": w.seed,
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": (committed_traffic(name, "attn_bwd", os.path.join(CSRC, "attn_bwd_kernels.hip"))
                                 if backward else committed_traffic(name)),
                     "kernel_ms_per_launch": round(kern_ms, 5),
                     "kernel_ms_median_of_5": round(med_ms, 5)},
        "clock": clock,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
