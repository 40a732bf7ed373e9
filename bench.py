#!/usr/bin/env python3
"""Throughput of the split prefix/suffix, tail-pad-skipping, non-causal
attention forward (libjpa, gfx950) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 5]
    python bench.py --op norm_rope [--workload 4]
    python bench.py --op rank_share [--workload 4] [--sp 8] [--rank 0]
    python bench.py --op cat_pad

One step = one jpa_forward_ws call over the whole workload (all query rows of
all heads, inputs already resident in HBM).  The default workload is the
largest single-GPU one: long video with GQA 40/8, prefix 256, suffix 75600
real + 176 tail-pad slots.  The run always warms up for at least 0.25 s of
back-to-back GPU work (past the clock's power-management transient); --warmup
W only raises the minimum step count.  Without --steps it times at least
0.1 s.  Prints ONE JSON line:

* value / ms_per_step: valid-token TFLOP/s of the timed steps
  (FLOPs = sum_b Hq * 4 * D * Nq_b * Nk_b, from jpa_plan);
* roofline: the kernel's GPU time per launch from HIP events recorded on the
  launch stream at the two ends of the timed region (nothing is inserted
  between launches), against the bf16 dense MFMA peak; a separate pass with
  an event pair around each launch gives the per-launch spread;
* cpu_baseline: the fp64 oracle timed on this host's cores, on the whole
  workload when it is small, else on the seeded subset of 4096 real query rows
  per head (every head) that the parity check uses; the full-workload time is
  extrapolated linearly in valid FLOPs;
* parity: the GPU result of the timed call against that oracle run.

Options for profiling runs: --no-cpu-baseline, --copy-probe BYTES (time a plain
device copy of that many bytes; used to calibrate rocprofv3 HBM counters),
--split-wgs N (force the balanced last round over N key ranges; a step is then
the main kernel plus the merge kernel; -1 never splits), with no traffic
figure reported for either.

--op norm_rope measures the step before attention instead: per-head Q/K
RMSNorm + rotary embedding (jpa_qk_norm_rope) on the q/k shapes of a norm-rope
workload; value is GB/s of algorithmic HBM bytes, roofline against 8 TB/s.
--op rank_share measures one rank's share of a head-parallel split of the
attention workload over --sp ranks (Hq/sp and Hkv/sp heads over the whole
sequence), the replicated prefix read through head-sliced views.
--op cat_pad measures the fused cat + pad of causal Conv3D caches over the
eight synthetic decoder shapes (one step = the eight calls); GB/s of
algorithmic bytes (inputs read once, output written once) against 8 TB/s.
"""

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

METRIC = "split-KV attention fwd TFLOP/s (valid tokens) + % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0        # MI355X published dense bf16 MFMA peak
KERNEL_NAME = "jpa_fwd_kernel"
KERNEL_SOURCES = ("diffusion_transformer_joint_non_amd/csrc/jpa_kernel.hip",
                  "diffusion_transformer_joint_non_amd/csrc/jpa_params.h")
DEFAULT_WORKLOAD = 5

NR_METRIC = "Q/K RMSNorm+RoPE GB/s (algorithmic HBM bytes) + % of MI355X HBM peak"
PEAK_HBM_GBS = 8000.0            # MI355X published HBM3E bandwidth
NR_KERNEL_NAME = "jpa_norm_rope_kernel"
NR_KERNEL_SOURCES = ("diffusion_transformer_joint_non_amd/csrc/jpa_norm_rope.hip",
                     "diffusion_transformer_joint_non_amd/csrc/jpa_norm_rope_params.h")
NR_DEFAULT_WORKLOAD = 4


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name: str, kernel=KERNEL_NAME, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed_steps(step, steps: int, stream):
    """Time `steps` calls of step(): the wall clock between two synchronise
    barriers, and HIP events recorded on the launch stream at the two ends of
    the same region (the region's GPU time per step; no event sits between
    the steps, so nothing is inserted between back-to-back launches).  Then a
    separate pass with an event pair around every step gives per-launch
    spread.  Returns (wall ms/step, event ms/step, per-launch ms array)."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    region_ms = e0.elapsed_time(e1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 10))]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = np.asarray([a.elapsed_time(b) for a, b in ev])
    return wall_ms, region_ms, per


# Default warmup and timed lengths, in seconds of back-to-back GPU work.  On
# MI355X the first ~0.1 s of continuous load runs up to 25% slower while
# power management settles (a trace of 2000 back-to-back attention launches
# repeats to within ~1% from launch ~400 on); timing inside that transient
# would report the settling, not the sustained rate.
WARMUP_SECONDS = 0.25
TIMED_SECONDS = 0.1


def resolve_counts(args, step, stream):
    """Warmup and timed step counts from the duration of one step.  Warmup
    always covers at least --warmup-seconds of GPU work; a given --warmup is a
    minimum step count (default 20).  --steps is used as given, else at least
    TIMED_SECONDS of GPU work and 30 steps.  Sets args.warmup_run (the warmup
    steps actually run) and args.steps."""
    import torch
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    step()
    e1.record(stream)
    torch.cuda.synchronize()
    t = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
    floor = int(np.ceil(args.warmup_seconds / t))
    args.warmup_run = max(floor, 20 if args.warmup is None else args.warmup)
    if args.warmup is None:
        args.warmup = args.warmup_run
    if args.steps is None:
        args.steps = max(30, int(np.ceil(TIMED_SECONDS / t)))


def blas_info():
    """(threads, library description) of the BLAS NumPy calls into."""
    try:
        np.dot(np.ones((2, 2)), np.ones((2, 2)))     # make sure the BLAS is loaded
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            i = max(libs, key=lambda r: r.get("num_threads", 0))
            desc = f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')})"
            return int(i["num_threads"]), desc
    except Exception:
        pass
    return 1, "unknown"


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_facts():
    """Where the oracle ran: usable cores, BLAS threads and library, CPU model."""
    threads, lib = blas_info()
    return {"cores": len(os.sched_getaffinity(0)), "blas_threads": threads, "blas": lib,
            "cpu_model": cpu_model()}


def figure(x: float, decimals: int = 2) -> float:
    """A reported figure: `decimals` places, or four significant digits when
    that would round a small positive value (the launch-bound workload's
    TFLOP/s) to nothing."""
    r = round(x, decimals)
    return r if abs(r) >= 10 ** (2 - decimals) or x == 0 else float(f"{x:.4g}")


def _read(path):
    try:
        with open(path) as f:
            return f.read().strip()
    except OSError:
        return None


def _git_head():
    root = os.path.dirname(os.path.abspath(__file__))
    head = _read(os.path.join(root, ".git", "HEAD"))
    if head and head.startswith("ref: "):
        return _read(os.path.join(root, ".git", head[5:]))
    return head


def _sclk_levels_mhz():
    """DPM levels of the GPU clock (MHz) from sysfs, or None where hidden."""
    import glob
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        txt = _read(f)
        if txt:
            return [int(t.split()[1].lower().rstrip("mhz")) for t in txt.splitlines() if len(t.split()) > 1
                    and t.split()[1].lower().endswith("mhz")]
    return None


def descriptor(seed_base):
    """Frozen description of where and on what the line was measured: code
    revision, input seeds, software stack and the device."""
    import torch
    prop = torch.cuda.get_device_properties(0)
    return {"git": _git_head(), "kernel_source_sha256_16": kernel_source_hash(), "input_seed_base": seed_base,
            "rocm": _read("/opt/rocm/.info/version"), "hip_runtime": torch.version.hip,
            "torch": torch.__version__, "amdgpu_driver": _read("/sys/module/amdgpu/version"),
            "gpu": prop.name, "arch": prop.gcnArchName, "compute_units": prop.multi_processor_count,
            "sclk_levels_mhz": _sclk_levels_mhz()}


# Above this much valid work the oracle runs on a seeded random subset of
# 4096 real query rows per head (every head, every real key) instead of the
# whole workload: the two largest workloads.
FULL_ORACLE_MAX_FLOPS = 2.0e12
SUBSET_ROWS_PER_HEAD = 4096


def cpu_baseline(w, x, flops_total):
    """Time the oracle, as it stands, on the whole workload when that is at
    most FULL_ORACLE_MAX_FLOPS of valid work, else on the seeded subset of
    SUBSET_ROWS_PER_HEAD real rows per head (synth.sample_query_rows, every
    head).
    value = valid-token TFLOP/s of what was run; the time for the whole
    workload is extrapolated linearly in valid FLOPs."""
    import oracle
    import synth
    rows_total = int((~w.pad_query_mask()).sum())
    names = ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix", "cu_q", "cu_prefix",
             "cu_suffix_real")
    t0 = time.perf_counter()
    if flops_total <= FULL_ORACLE_MAX_FLOPS or rows_total <= SUBSET_ROWS_PER_HEAD:
        ref_o, ref_l = oracle.attention(*[x[n] for n in names], x["scale"])
        sample = f"full workload: {rows_total} real query rows x {w.hq} heads"
        flops = flops_total
        rows = None
    else:
        rows = synth.sample_query_rows(w, SUBSET_ROWS_PER_HEAD)
        ref_o, ref_l = oracle.attention_rows(*[x[n] for n in names], x["scale"], rows)
        segs = oracle.decode_segments(x["cu_q"], x["cu_prefix"], x["cu_suffix_real"])
        starts = np.asarray([s.q_start for s in segs])
        keys = np.asarray([s.keys for s in segs])
        owner = np.searchsorted(starts, rows, side="right") - 1
        flops = int(4 * w.d * keys[owner].sum())
        sample = (f"seeded subset: {rows.shape[1]} real query rows per head (of {rows_total}) "
                  f"x all {w.hq} heads, every real key")
    dt = time.perf_counter() - t0
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", **host_facts(),
            "kind": "oracle", "sample": sample, "seconds": round(dt, 3),
            "sample_gflops": round(flops / 1e9, 1),
            "sample_gflop_per_s": round(flops / dt / 1e9, 2),
            "seconds_full_workload_extrapolated": round(dt * flops_total / flops, 1)}
    return base, ref_o, ref_l, rows


def copy_probe(nbytes: int, steps: int):
    import torch
    n = nbytes // 2
    a = torch.empty(n, dtype=torch.int16, device="cuda").random_()
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes": n * 2, "read_bytes": n * 2, "write_bytes": n * 2,
                      "ms": dt * 1e3, "GB/s": 2 * n * 2 / dt / 1e9}), flush=True)


def bench_norm_rope(args):
    """One step = one jpa_qk_norm_rope call over all q and k rows."""
    import torch
    import synth
    from diffusion_transformer_joint_non_amd import jpa

    wid = NR_DEFAULT_WORKLOAD if args.workload is None else args.workload
    w = synth.NORM_ROPE_WORKLOADS[wid]
    log(f"norm-rope workload {w.wid} {w.name}: generating inputs")
    x = synth.make_norm_rope_inputs(w)
    to_dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    q, k = to_dev(x["q"]), to_dev(x["k"])
    wq, wk = torch.from_numpy(x["q_weight"]).cuda(), torch.from_numpy(x["k_weight"]).cuda()
    table = torch.from_numpy(x["table"]).cuda()
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    stream = torch.cuda.current_stream()
    # algorithmic bytes: q and k read and written once, the table and weights read once
    nbytes = (2 * 2 * w.tokens * (w.hq + w.hkv) * w.d + 4 * w.tokens * w.rotary_dim + 2 * 4 * w.d)

    def step():
        jpa.jpa_qk_norm_rope(q, k, wq, wk, table, w.rotary_dim, w.interleaved, w.eps,
                             q_out=qo, k_out=ko, stream=stream)

    resolve_counts(args, step, stream)
    for _ in range(args.warmup_run):
        step()
    torch.cuda.synchronize()
    ms_per_step, kern_ms, per_launch_ms = timed_steps(step, args.steps, stream)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": NR_METRIC,
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": args.warmup_run,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"norm_rope_{w.name}", "tokens": w.tokens, "heads_q": w.hq,
                   "heads_kv": w.hkv, "head_dim": w.d, "rotary_dim": w.rotary_dim,
                   "pairs": "interleaved" if w.interleaved else "half-split",
                   "algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic(w.name, NR_KERNEL_NAME, NR_KERNEL_SOURCES),
                     "kernel": NR_KERNEL_NAME,
                     "kernel_ms": {"mean": round(kern_ms, 4),
                                   "per_launch_pass": {"median": round(float(np.median(per_launch_ms)), 4),
                                                       "min": round(float(per_launch_ms.min()), 4),
                                                       "max": round(float(per_launch_ms.max()), 4)}},
                     "kernel_source_sha256_16": kernel_source_hash(NR_KERNEL_SOURCES)},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: timing the fp64 oracle on the whole workload")
        f64 = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)
        qs, ks, ts = f64(x["q"]), f64(x["k"]), x["table"].astype(np.float64)
        t0 = time.perf_counter()
        rq, rk = oracle.qk_norm_rope(qs, ks, x["q_weight"], x["k_weight"], ts, w.rotary_dim,
                                     w.interleaved, w.eps)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s",
                                  **host_facts(), "kind": "oracle",
                                  "sample": f"full workload: {w.tokens} tokens x {w.hq}+{w.hkv} heads",
                                  "seconds": round(dt, 3)}
        err = max(float(np.abs(qo.float().cpu().numpy() - rq).max()),
                  float(np.abs(ko.float().cpu().numpy() - rk).max()))
        within = min(float(np.mean(np.abs(qo.float().cpu().numpy() - rq) <= 2.0 ** -7 * np.abs(rq) + 1e-6)),
                     float(np.mean(np.abs(ko.float().cpu().numpy() - rk) <= 2.0 ** -7 * np.abs(rk) + 1e-6)))
        result["parity"] = {"max_abs": float(f"{err:.3e}"), "frac_within_1ulp": within}
    print(json.dumps(result), flush=True)


CP_METRIC = "causal Conv3D cat+pad GB/s (algorithmic HBM bytes) + % of MI355X HBM peak"
CP_KERNEL_NAME = "jpa_cat_pad_kernel"
CP_KERNEL_SOURCES = ("diffusion_transformer_joint_non_amd/csrc/jpa_cat_pad.hip",
                     "diffusion_transformer_joint_non_amd/csrc/jpa_cat_pad_params.h")


def bench_cat_pad(args):
    """One step = jpa_causal_cat_pad over each of the eight decoder shapes."""
    import torch
    import synth
    from diffusion_transformer_joint_non_amd import jpa

    cases = synth.CAT_PAD_CASES
    dv = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    data, nbytes = [], 0
    for c in cases:
        inp = synth.make_cat_pad_inputs(c)
        x = dv(inp["x"])
        cache = dv(inp["cache"]) if c.cache_frames else None
        out = jpa.jpa_causal_cat_pad(x, cache, c.padding)
        nbytes += 2 * (x.numel() + (cache.numel() if cache is not None else 0) + out.numel())
        data.append((c, inp, x, cache, out))
    stream = torch.cuda.current_stream()

    def step():
        for c, _, x, cache, out in data:
            jpa.jpa_causal_cat_pad(x, cache, c.padding, out=out, stream=stream)

    resolve_counts(args, step, stream)
    for _ in range(args.warmup_run):
        step()
    torch.cuda.synchronize()
    ms_per_step, kern_ms, per_step_ms = timed_steps(step, args.steps, stream)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    result = {
        "metric": CP_METRIC, "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": args.warmup_run, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "causal_conv3d_cat_pad_decoder", "shapes": [c.name for c in cases],
                   "algorithmic_bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic("decoder", CP_KERNEL_NAME, CP_KERNEL_SOURCES),
                     "kernel": CP_KERNEL_NAME,
                     "kernel_ms_per_step": {"mean": round(kern_ms, 4),
                                            "per_step_pass": {"min": round(float(per_step_ms.min()), 4),
                                                              "max": round(float(per_step_ms.max()), 4)}},
                     "kernel_source_sha256_16": kernel_source_hash(CP_KERNEL_SOURCES)},
    }
    if not args.no_cpu_baseline:
        import oracle
        sub = data
        sub_bytes = sum(2 * (x.numel() + (cache.numel() if cache is not None else 0) + out.numel())
                        for _, _, x, cache, out in sub)
        t0 = time.perf_counter()
        same = True
        for c, inp, _, _, out in sub:
            ref = oracle.cat_pad(inp["x"], inp["cache"] if c.cache_frames else None, c.padding)
            same &= bool(np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref))
            del ref
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(sub_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                                  "cpu_model": cpu_model(),
                                  "kind": "oracle", "seconds": round(dt, 3),
                                  "sample": "all eight shapes (time includes the bitwise comparison)"}
        result["parity"] = {"bit_exact": bool(same)}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: at least 0.1 s of GPU work, at least 30)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="minimum untimed steps first (default 20); warmup always covers at "
                         "least 0.25 s of GPU work")
    ap.add_argument("--warmup-seconds", type=float, default=WARMUP_SECONDS,
                    help="least GPU time of warmup (default 0.25 s; counter runs that "
                         "serialise every dispatch may set 0)")
    ap.add_argument("--workload", type=int, default=None)
    ap.add_argument("--op", choices=("attention", "norm_rope", "rank_share", "cat_pad"), default="attention")
    ap.add_argument("--sp", type=int, default=8, help="rank_share: ranks of the head split")
    ap.add_argument("--rank", type=int, default=0, help="rank_share: which rank's share")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0)
    ap.add_argument("--split-wgs", type=int, default=0,
                    help="attention: force the balanced last round over this many key ranges "
                         "(0: the library decides; -1: no workspace, jpa_forward's path)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps or 3, 1))
        return

    if args.op == "norm_rope":
        bench_norm_rope(args)
        return
    if args.op == "cat_pad":
        bench_cat_pad(args)
        return

    import synth
    from diffusion_transformer_joint_non_amd import jpa

    w = synth.WORKLOADS[DEFAULT_WORKLOAD if args.workload is None else args.workload]
    share = None
    if args.op == "rank_share":
        # One rank's share of a head-parallel (Ulysses) split over args.sp ranks:
        # Hq/sp query and Hkv/sp kv heads over the full sequence, with the
        # prefix replicated on every rank in full and read through a
        # head-sliced view (a pointer offset and the full token stride).
        if w.hq % args.sp or w.hkv % args.sp:
            print(f"--sp {args.sp} does not divide the heads {w.hq}/{w.hkv}", file=sys.stderr)
            sys.exit(2)
        full_hkv = w.hkv
        w = synth.custom_workload(w.hq // args.sp, w.hkv // args.sp, w.d, w.prefix, w.suffix_real,
                                  w.suffix_pad, w.queries, wid=w.wid, name=f"{w.name}_sp{args.sp}_rank")
        share = {"sp": args.sp, "rank": args.rank, "heads_q_total": w.hq * args.sp,
                 "heads_kv_total": full_hkv, "prefix_view": "head slice of the replicated prefix"}
    log(f"workload {w.wid} {w.name}: generating inputs")
    x = synth.make_inputs(w)
    dev = {n: torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).view(torch.bfloat16).cuda()
           for n in ("q", "k_prefix", "v_prefix", "k_suffix", "v_suffix")}
    if share is not None:
        h0 = args.rank * w.hkv
        for n in ("k_prefix", "v_prefix"):
            full = torch.zeros((dev[n].shape[0], share["heads_kv_total"], w.d), dtype=torch.bfloat16,
                               device="cuda")
            full[:, h0:h0 + w.hkv] = dev[n]
            dev[n] = full[:, h0:h0 + w.hkv]          # a view: token stride of all heads
    rows, flops = jpa.jpa_plan(x["cu_q"], x["cu_prefix"], x["cu_suffix_real"], w.hq, w.d)
    out = torch.empty_like(dev["q"])
    lse = torch.empty((w.hq, dev["q"].shape[0]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    # jpa_forward_ws with its cached workspace (allocated during warmup): the
    # library's best path (it balances a mostly idle last round of items).
    def step():
        jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                           dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                           x["scale"], out=out, lse=lse, stream=stream,
                           workspace=None if args.split_wgs < 0 else "auto",
                           split_wgs=max(args.split_wgs, 0))

    resolve_counts(args, step, stream)
    log(f"warmup {args.warmup_run} steps")
    for _ in range(args.warmup_run):
        step()
    torch.cuda.synchronize()

    # HIP events on the launch stream at the two ends of the timed region give
    # the GPU time per launch; the synchronised wall clock gives ms_per_step.
    log(f"timing {args.steps} steps")
    ms_per_step, kern_ms, per_launch_ms = timed_steps(step, args.steps, stream)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    # the committed counters cover the library's own choice of path
    traffic = load_traffic(w.name) if args.split_wgs == 0 else None
    # Launch-bound sizes: the per-call time when the host is out of the way,
    # from a HIP graph of 20 calls replayed (the library allocates nothing and
    # never synchronises, so its calls capture as they are).
    graph_us = prepared_us = None
    if kern_ms < 1.0:
        g = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        with torch.cuda.stream(cs):
            with torch.cuda.graph(g, stream=cs):
                for _ in range(20):
                    jpa.jpa_forward_ws(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                                       dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                                       x["scale"], out=out, lse=lse, stream=cs,
                                       workspace=None if args.split_wgs < 0 else jpa.workspace_for(
                                           out.device, stream.cuda_stream, w.d, args.split_wgs),
                                       split_wgs=max(args.split_wgs, 0))
        torch.cuda.synchronize()
        # the same time-based warmup and timed length as the eager steps: the
        # pause for capture lets the clocks settle back to their idle state
        per_replay_s = 20 * kern_ms * 1e-3
        n_warm = max(5, int(np.ceil(WARMUP_SECONDS / per_replay_s)))
        n_timed = max(5, int(np.ceil(TIMED_SECONDS / per_replay_s)))
        for _ in range(n_warm):
            g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(n_timed):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) * 1e3 / (n_timed * 20)
        # the same call eagerly, its arguments marshalled once (PreparedForward)
        call = jpa.prepare_forward(dev["q"], dev["k_prefix"], dev["v_prefix"], dev["k_suffix"],
                                   dev["v_suffix"], x["cu_q"], x["cu_prefix"], x["cu_suffix_real"],
                                   x["scale"], out=out, lse=lse, stream=stream,
                                   workspace=None if args.split_wgs < 0 else "auto",
                                   split_wgs=max(args.split_wgs, 0))
        n_calls = max(100, int(np.ceil(TIMED_SECONDS / (kern_ms * 1e-3))))
        for _ in range(n_calls):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_calls):
            call()
        torch.cuda.synchronize()
        prepared_us = (time.perf_counter() - t0) * 1e6 / n_calls
    # minimum bytes a call moves: real q read, every out slot written, each
    # row's real prefix/suffix K and V read once, lse written
    real_q = int(sum(r[2] for r in rows))
    real_kv = int(sum(r[8] for r in rows))
    algo_bytes = (2 * w.d * w.hq * (real_q + int(x["cu_q"][-1])) + 2 * 2 * w.d * w.hkv * real_kv
                  + 4 * w.hq * int(x["cu_q"][-1]))

    result = {
        "metric": METRIC,
        "value": figure(flops / (ms_per_step * 1e-3) / 1e12),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": args.warmup_run,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads_q": w.hq, "heads_kv": w.hkv,
                   "head_dim": w.d, "prefix": list(map(int, w.prefix)),
                   "suffix_real": list(map(int, w.suffix_real)),
                   "suffix_pad": list(map(int, w.suffix_pad)), "queries": w.queries,
                   "valid_flops": flops, **({"rank_share": share} if share else {}),
                   **({"split_wgs": args.split_wgs} if args.split_wgs else {})},
        "pct_of_bf16_peak": round(100.0 * flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": figure(achieved), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": figure(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": KERNEL_NAME,
                     "kernel_ms": {"mean": round(kern_ms, 4),
                                   "per_launch_pass": {"median": round(float(np.median(per_launch_ms)), 4),
                                                       "min": round(float(per_launch_ms.min()), 4),
                                                       "max": round(float(per_launch_ms.max()), 4)}},
                     "kernel_source_sha256_16": kernel_source_hash(),
                     "algorithmic_bytes": algo_bytes,
                     "hbm_gbs_algorithmic": round(algo_bytes / (kern_ms * 1e-3) / 1e9, 1),
                     "us_per_call": round(kern_ms * 1e3, 2),
                     "us_per_call_graph": None if graph_us is None else round(graph_us, 2),
                     "us_per_call_prepared": None if prepared_us is None else round(prepared_us, 2)},
    }

    result["descriptor"] = descriptor(1000 * w.wid)
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the fp64 oracle on the host")
        base, ref_o, ref_l, sub = cpu_baseline(w, x, flops)
        result["cpu_baseline"] = base
        import oracle
        go = out.float().cpu().numpy()
        gl = lse.cpu().numpy()
        if sub is None:
            real = ~w.pad_query_mask()
            err = oracle.compare(go[real], gl[:, real].T, ref_o[real], ref_l[:, real].T)
        else:
            err = oracle.compare(np.stack([go[sub[h], h] for h in range(w.hq)]),
                                 np.stack([gl[h, sub[h]] for h in range(w.hq)]), ref_o, ref_l)
        result["parity"] = {k: float(f"{v:.3e}") for k, v in err.items()}
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
