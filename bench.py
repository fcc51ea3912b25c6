"""Benchmark of the TP-MLP shard library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The default workload carries both halves of the
metric for the 70B-shaped TP=8 rank:

* decode (``value``, algorithmic GB/s): one step runs, for each of M = 1, 8
  and 64 tokens, the rank's forward (gate/up with fused SwiGLU, down to an
  fp32 partial) and the 8-way fp32 partial reduce of that partial with seven
  other ranks' partials.  Each phase of a step reads its own weight set out
  of eight or more (like successive layers), and the reduces rotate through
  four sets of other partials, so the bytes come from HBM and not from the
  256 MB last-level cache;
* ``prefill`` (TFLOP/s): M = 4096, the forward and the 8-way reduce of its
  4096 x 8192 partial (``reduce``: that reduce's own GB/s).

Inputs are seeded synthetic tensors (``workloads``), resident in HBM before
timing.  The MFMA-bound workloads warm up for at least 50 ms by default
(``WARMUP_MS``): the GPU's clocks settle only after about 40 ms of GEMMs.

Other workloads (--workload): decode70b and prefill70b (the two halves
alone), fp8_70b
(TP=4 fp8 weights: decode M=32 and prefill M=2048), int8_70b (TP=2 int8
weights: decode M=1 and 8, prefill M=2048), w8a8_prefill70b (fp8 activations
and weights on the fp8 matrix cores, TP=4 at 2048 tokens), prefill405b (8192 tokens),
reduce70b / reduce405b (the 8-way reduces alone), sp_prefill70b (the
sequence-parallel form: forward over eight row blocks of X, reduce-scatter),
attn70b / attn_prefill70b (the same rank's attention-block projections: QKV,
output projection to an fp32 partial, 8-way reduce; decode M=1, 8, 64 and
prefill M=4096),
copy (the reduce with one
buffer over 1 GiB: a plain copy of known size, the calibration run for the
HBM byte counters).

The ``roofline`` object is for the step's dominant kernel: algorithmic bytes
(or FLOP) of its launches divided by their summed durations, taken from HIP
events that the library attaches to each of that kernel's dispatches during
the timed steps (only that kernel's: an event-timed launch costs the host
about 20 us against 3 us for a plain one, and timing every launch would make
the decode loop host-bound).  The other kernels' durations come from a
further pass with every launch timed.  Its ``traffic`` is the HBM bytes per launch that
rocprofv3's FETCH_SIZE and WRITE_SIZE counters recorded for that kernel
(scaled by what they read for the copy), kept as text under profiles/ with
the hash of the kernel's sources at the time; it is null when no record
exists or the sources have changed since.  ``cpu_baseline`` times the float64 CPU oracle on a bounded
sample of the same workload (rank 0, one GPU only).
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "decode-shard HBM GB/s (% peak) & prefill-shard TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
N_WEIGHT_SETS = 8


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="default",
                    choices=["default", "decode70b", "prefill70b", "fp8_70b", "prefill405b", "reduce70b", "reduce405b",
                             "sp_prefill70b", "attn70b", "attn_prefill70b", "int8_70b", "w8a8_prefill70b",
                             "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weight-sets", type=int, default=N_WEIGHT_SETS)
    ap.add_argument("--row-major", action="store_true",
                    help="read the weights in the (out, in) layout instead of packed for the decode kernels "
                         "(decode and prefill phases of the MLP workloads)")
    return ap.parse_args()


KERNEL_SOURCES = {
    "gateup_decode": ("decode.hip", "common.h", "internal.h"),
    "gateup_prefill": ("prefill.hip", "common.h", "internal.h"),
    "partial_reduce": ("reduce.hip", "common.h", "internal.h"),
    "qkv_decode": ("decode.hip", "gemv.hip", "common.h", "internal.h"),
    "qkv_prefill": ("prefill.hip", "common.h", "internal.h"),
    "gateup_w8a8": ("prefill.hip", "common.h", "internal.h"),
}


def sources_sha256(kernel):
    hsh = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "tensor_transformer_mlp_tp_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` in `workload` from profiles/traffic_<kernel>_<workload>.txt,
    or None when there is no record or the kernel's sources differ from the recorded hash."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                rec[key.strip()] = val.strip()
    if rec.get("kernel_sources_sha256") != sources_sha256(kernel):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- inputs

def to_dev(arr, dt):
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    if dt == "e4m3fn":
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.float8_e4m3fn).cuda()
    if dt == "int8":
        return torch.from_numpy(np.ascontiguousarray(arr)).view(torch.int8).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def device_weights(cfg_id, h, I_s, w, std_gu, std_down, n_sets):
    import torch
    sets = []
    for s in range(n_sets):
        ws = workloads.make_shard_weights(cfg_id, h, I_s, 0, w, std_gu, std_down, weight_set=s)
        d = dict(w_gate=to_dev(ws["w_gate"], w), w_up=to_dev(ws["w_up"], w), w_down=to_dev(ws["w_down"], w))
        for k in ("s_gate", "s_up", "s_down"):
            d[k] = None if ws[k] is None else torch.from_numpy(ws[k]).cuda()
        sets.append(d)
        if s == 0:
            host0 = ws
    return sets, host0


class Phase:
    """One forward (+ optional reduce) of a rank at M tokens, buffers preallocated."""

    def __init__(self, tp, cfg_id, M, h, I_s, t, act, w, with_reduce, other_sets=1):
        import torch
        self.tp, self.M, self.h, self.I_s, self.t, self.w = tp, M, h, I_s, t, w
        self.x_host = workloads.make_x(cfg_id, M, h, act)
        self.x = to_dev(self.x_host, act)
        self.partial = torch.empty((M, h), dtype=torch.float32, device="cuda")
        wdt = {"e4m3fn": torch.float8_e4m3fn, "int8": torch.int8}.get(w, torch.bfloat16)
        # the larger of the two forwards' workspaces (packed weights: 256-token tiles above the decode sizes)
        nbytes = max(tp.workspace_bytes(M, h, I_s * t, t, torch.bfloat16, wdt),
                     tp.packed_workspace_bytes(M, h, I_s * t, t, wdt) if act == "bf16" else 0)
        self.ws = tp.alloc_workspace(nbytes, "cuda")
        self.with_reduce = with_reduce
        # the t - 1 other ranks' partials: `other_sets` distinct sets, used in turn
        self.others = []
        if with_reduce:
            for r in range(other_sets):
                others = workloads.make_partials(cfg_id, t - 1, M * h, weight_set=M + 1000 * r)
                self.others.append([torch.from_numpy(o).cuda() for o in others])

        self.calls = {}

    def run(self, wset, time_fwd=None, other=0):
        """time_fwd: (library, kind mask) to event-time this call's launches
        (forward and reduce) of those kinds only; other: which set of other
        partials the reduce reads."""
        # arguments are marshalled once per (weight set, other-partials set);
        # the loop only re-issues the C calls
        other = other % max(1, len(self.others))
        key = (id(wset), other)
        if key not in self.calls:
            if wset.get("packed") is not None:
                fwd = self.tp.prepare_shard_forward_packed(self.x, wset["packed"], k=0, s_gate=wset["s_gate"],
                                                           s_up=wset["s_up"], s_down=wset["s_down"],
                                                           partial=self.partial, workspace=self.ws)
            else:
                fwd = self.tp.prepare_shard_forward(self.x, wset["w_gate"], wset["w_up"], wset["w_down"],
                                                    t=self.t, k=0, s_gate=wset["s_gate"], s_up=wset["s_up"],
                                                    s_down=wset["s_down"], partial=self.partial, workspace=self.ws)
            # in place into the rank's own partial, as the all-reduce does
            red = self.tp.prepare_partial_reduce([self.partial.view(-1)] + self.others[other],
                                                 out=self.partial.view(-1)) if self.with_reduce else None
            self.calls[key] = (fwd, red)
        fwd, red = self.calls[key]
        if time_fwd is not None:
            time_fwd[0].tp_profile_enable(time_fwd[1])
        fwd()
        if red is not None:
            red()
        if time_fwd is not None:
            time_fwd[0].tp_profile_enable(0)

    def bytes(self, act="bf16"):
        b = workloads.forward_bytes(self.M, self.h, self.I_s, act, self.w)
        if self.with_reduce:
            b += workloads.reduce_bytes(self.M * self.h, self.t)
        return b

    def flops(self):
        return workloads.forward_flops(self.M, self.h, self.I_s)


# ----------------------------------------------------------------------------- timing

def timed(tp, step_fn, steps, warmup, kinds, dur_kind=None, dur=None):
    """Wall time of `steps` steps after `warmup`, with HIP-event timing of the
    library's launches of the kernel kinds `kinds` only (an event-timed launch
    costs the host several times a plain one, which would otherwise make the
    loop host-bound).  dur_kind, dur: append the timed steps' durations (ms)
    of that kind's timed launches, in launch order, to the list dur."""
    import torch
    # warm-up with the same timing on: counts the timed launches of a step, so
    # that every event the timed steps use exists before the clock starts
    tp.profile_collect()
    tp.profile_enable(True, kinds)
    for i in range(warmup):
        step_fn(i)
    torch.cuda.synchronize()
    tp.profile_enable(False)
    launches = sum(c for _, c in tp.profile_collect().values())
    tp.profile_reserve(launches * steps // max(warmup, 1) + 64)
    tp.profile_enable(True, kinds)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_fn(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tp.profile_enable(False)
    if dur_kind is not None:
        dur.extend(tp.profile_durations(dur_kind))
    prof = tp.profile_collect()
    return elapsed, prof


def spread(ms):
    """Median, 10th and 90th percentile (microseconds) of launch durations in ms."""
    if not ms:
        return None
    v = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(v)), 3), "p10_us": round(float(np.percentile(v, 10)), 3),
            "p90_us": round(float(np.percentile(v, 90)), 3), "launches": int(v.size)}


def breakdown(tp, step_fn, steps, first):
    """Per-kind kernel durations from a further `steps` steps with every
    launch event-timed (a pass of its own: not used for throughput)."""
    import torch
    torch.cuda.synchronize()
    tp.profile_collect()
    tp.profile_enable(True)
    for i in range(steps):
        step_fn(first + i)
    torch.cuda.synchronize()
    tp.profile_enable(False)
    return tp.profile_collect()


def timed_phase(i, nph):
    """The phase of step i whose launches are event-timed, or None: phase
    i mod P on steps with i mod P < nph, P = max(nph, 3).  At most one phase
    per step, and with fewer than three phases not every step: an event-timed
    launch costs the host several plain ones, and a loop of short kernels
    that turns host-bound starts its kernels on an idle GPU, where the
    events read high."""
    period = max(nph, 3)
    return i % period if i % period < nph else None


def breakdown_rotating(tp, run_step, nph, kinds, steps, first):
    """Per-kind kernel durations of a loop of short kernels, in the timed
    region's own regime: for each kind, a further `steps` steps in which only
    that kind's launches in the phase timed_phase(i, nph) are event-timed, as
    in the timed region.  (Timing every launch makes such a loop host-bound,
    and its kernels then start on an idle GPU.)
    run_step(i, sel): runs step i, sel(phase index) giving that phase's
    (library, kind mask) or None.  Returns {kind: (ms, launches)} of the timed
    launches and {kind: ms per step} (max(nph, 3) x ms / steps)."""
    import torch
    lib = tp.load()
    names = tp.kernel_kinds()
    rec, per_step = {}, {}
    for k in kinds:
        mask = 1 << names.index(k)
        torch.cuda.synchronize()
        tp.profile_collect()
        tp.profile_reserve(2 * steps + 64)
        for j in range(steps):
            i = first + j
            run_step(i, lambda idx, i=i: (lib, mask) if timed_phase(i, nph) == idx else None)
        torch.cuda.synchronize()
        got = tp.profile_collect()
        if k in got:
            rec[k] = got[k]
            per_step[k] = max(nph, 3) * got[k][0] / steps
    return rec, per_step


def cpu_info():
    info = {"os_cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    blas_threads = None
    try:
        import threadpoolctl
        for p in threadpoolctl.threadpool_info():
            if p.get("user_api") == "blas":
                blas_threads = max(blas_threads or 0, int(p.get("num_threads", 0)))
                info["blas"] = "%s %s" % (p.get("internal_api"), p.get("version"))
    except Exception:
        pass
    info["blas_threads"] = blas_threads
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return info


def cpu_baseline(fn_once, unit_amount, unit, sample, min_seconds=10.0, max_reps=1000):
    """Time the oracle: repeat fn_once until min_seconds have passed."""
    info = cpu_info()
    reps, t0 = 0, time.perf_counter()
    while True:
        fn_once()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    cores = info.get("blas_threads") or info["affinity"]
    return {"value": unit_amount * reps / el, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": "%s; %d repetitions in %.1f s" % (sample, reps, el), "host": info}


# ----------------------------------------------------------------------------- workloads

N_OTHER_SETS = 4   # sets of the other ranks' partials the decode reduces rotate through


def bench_decode70b(tp, args):
    """70B TP=8 decode step: for M = 1, 8 and 64 tokens, the forward and the
    8-way reduce of its partial.  Each phase of a step reads its own weight
    set (phase idx of step i: set (3 i + idx) mod n, n >= 8, so a set is read
    again only after seven others, 1.2 GB, have streamed through the 256 MB
    last-level cache), and the reduces rotate through N_OTHER_SETS sets of
    the other ranks' partials."""
    import oracle
    c = workloads.CONFIGS[2]
    h, t, I_s = c["h"], c["t"], c["I"] // c["t"]
    n_sets = max(args.weight_sets, 8)
    log("generating %d weight sets of the 70B TP=8 shard" % n_sets)
    sets, host0 = device_weights(2, h, I_s, "bf16", c["std_gu"], c["std_down"], n_sets)
    if not args.row_major:
        # the decode kernels' packed weight layout, written once per weight set
        for d in sets:
            d["packed"] = tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)
    phases = [Phase(tp, 2, M, h, I_s, t, "bf16", "bf16", True, other_sets=N_OTHER_SETS) for M in c["M"]]
    nph = len(phases)
    # An event-timed launch costs the host ~25 us against ~3 us for a plain
    # one; timing the gate/up launch of all three phases made the step
    # host-bound (144 us against 130 us untimed).  Step i times the gate/up
    # launch of phase i % 3 only, so each M is sampled on a third of the steps.
    lib = tp.load()
    gmask = 1 << tp.kernel_kinds().index("gateup_decode")

    def wset(i, idx):
        return sets[(nph * i + idx) % len(sets)]

    def run_step(i, sel):
        for idx, ph in enumerate(phases):
            ph.run(wset(i, idx), sel(idx), other=i)

    def step(i):
        run_step(i, lambda idx: (lib, gmask) if i % nph == idx else None)

    steps, warmup = args.steps or 402, args.warmup if args.warmup is not None else 42
    gu_dur = []
    elapsed, prof = timed(tp, step, steps, warmup, [], "gateup_decode", gu_dur)
    # sk_clear: the one-workgroup clear of the split-K counters (M=64 forward)
    prof_all, per_step = breakdown_rotating(tp, run_step, nph, ["gateup_decode", "down_decode", "sk_clear",
                                                                "partial_reduce"], steps, warmup + steps)
    step_bytes = sum(ph.bytes() for ph in phases)
    value = step_bytes * steps / elapsed / 1e9
    kern = {}
    for name, b in (("gateup_decode", sum(workloads.gateup_bytes(ph.M, h, I_s) for ph in phases)),
                    ("down_decode", sum(workloads.down_bytes(ph.M, h, I_s) for ph in phases)),
                    ("partial_reduce", sum(workloads.reduce_bytes(ph.M * h, t) for ph in phases)),
                    ("sk_clear", None)):
        if name not in prof_all:
            continue
        ms, cnt = prof_all[name]
        kern[name] = {"launches": cnt, "avg_us": round(1e3 * ms / max(cnt, 1), 3)}
        if b is not None:
            kern[name]["GBps"] = round(b / (per_step[name] * 1e-3) / 1e9, 1)
    ms, cnt = prof["gateup_decode"]
    assert cnt == steps
    timed_bytes = sum(workloads.gateup_bytes(ph.M, h, I_s) * sum(1 for i in range(warmup, warmup + steps)
                                                                   if i % nph == idx)
                      for idx, ph in enumerate(phases))
    achieved = timed_bytes / (ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic("gateup_decode", "decode70b" + ("_rowmajor" if args.row_major else "")),
            "kernel": "gateup_decode",
            "per_launch_bytes": {str(ph.M): workloads.gateup_bytes(ph.M, h, I_s) for ph in phases},
            "avg_us": round(1e3 * ms / cnt, 3),
            "per_M_launch_us": {str(ph.M): spread([d for j, d in enumerate(gu_dur) if (warmup + j) % nph == idx])
                                for idx, ph in enumerate(phases)},
            "source": "HIP events on the gate/up launch of one phase per timed step (phase i mod 3), "
                      "on the launch stream; achieved = their algorithmic bytes / their summed durations"}
    fwd_time_ms = sum(per_step[k] for k in ("gateup_decode", "down_decode", "sk_clear") if k in per_step)
    fwd_bytes = sum(workloads.forward_bytes(ph.M, h, I_s) for ph in phases)
    # parity sample at full size, outside the timed region: the M=1 forward alone on weight set 0
    # (the step's reduce overwrites the partial in place)
    parity = None
    if not args.no_cpu_baseline:
        import torch
        ph = phases[0]
        ph.run(sets[0])
        ph.calls[(id(sets[0]), 0)][0]()
        torch.cuda.synchronize()
        ref = oracle.rank_partial_from_storage(ph.x_host, "bf16", host0["w_gate"], host0["w_up"],
                                               host0["w_down"], "bf16")
        parity = oracle.rms_normalised_max_error(ph.partial.cpu().numpy(), ref)

    out = dict(metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * elapsed / steps, 5), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16", data="synthetic",
               config={"workload": "70B-shaped TP=8 rank decode (h=8192, I_s=3584, bf16 weights%s) at "
                                   "M=1, 8 and 64 tokens, each forward followed by the 8-way fp32 "
                                   "partial reduce" % (", (out, in) layout" if args.row_major else
                                                       ", packed for the decode kernels"),
                       "M": list(c["M"]), "h": h, "I_s": I_s, "t": t, "weight_sets": len(sets),
                       "weight_set_of_phase": "(3 * step + phase) mod weight_sets",
                       "other_partial_sets": N_OTHER_SETS},
               roofline=roof,
               frac_of_hbm_peak=round(value / HBM_PEAK_GBS, 4),
               forward_only={"GBps": round(fwd_bytes / (fwd_time_ms * 1e-3) / 1e9, 1),
                             "us_per_step": round(fwd_time_ms * 1e3, 2)},
               kernels=kern, kernels_note="kernels and forward_only: for each kernel kind a further pass of "
                                          "the same number of steps that event-times that kind's launches "
                                          "in one phase per step, like the timed region",
               parity_err_M1=parity)
    if not args.no_cpu_baseline:
        host_parts = [np.zeros(ph.M * h, np.float32) for ph in phases]

        def once():
            for ph, hp in zip(phases, host_parts):
                p = oracle.rank_partial_from_storage(ph.x_host, "bf16", host0["w_gate"], host0["w_up"],
                                                     host0["w_down"], "bf16")
                oracle.fold_fp32([p.astype(np.float32).reshape(-1)] + [hp] * (t - 1))
        log("timing the CPU oracle (decode)")
        out["cpu_baseline"] = cpu_baseline(once, step_bytes / 1e9, "GB/s",
                                           "one full step (M=1, 8, 64 rank partials from the bf16 "
                                           "weight bytes + 8-way fp32 folds), repeated >= 10 s")
    return out


# Untimed warm-up of the MFMA-bound workloads: at the start of a run of long
# GEMMs the GPU's clocks take about 40 ms to settle (70B prefill gate/up in a
# kernel trace: 437, 441, 534, 624, ... us, then down to a steady 405-415 us
# after about 40 steps), so their default warm-up covers at least 50 ms.
WARMUP_MS = 50.0


def warmup_steps(step_ms):
    return max(5, int(WARMUP_MS / step_ms + 0.999))


def bench_prefill(tp, args, cfg_id, M, label, step_ms):
    import oracle
    c = workloads.CONFIGS[cfg_id]
    h, t, I_s, w = c["h"], c["t"], c["I"] // c["t"], c["w"]
    n_sets = 1   # compute-bound: weight reuse across tokens dwarfs any cache effect
    log("generating the %s inputs" % c["name"])
    sets, host0 = device_weights(cfg_id, h, I_s, w, c["std_gu"], c["std_down"], n_sets)
    if not args.row_major:
        # the packed-weight GEMMs read the decode kernels' layout (packed once, outside the timing): the
        # same single copy of the weights as the decode phases
        sets = [dict(d, packed=tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)) for d in sets]
        label += ", weights packed for the decode kernels"
    ph = Phase(tp, cfg_id, M, h, I_s, t, "bf16", w, c["reduce_n"] is not None)

    def step(i):
        ph.run(sets[0])

    steps, warmup = args.steps or 30, args.warmup if args.warmup is not None else warmup_steps(step_ms)
    gu_dur = []
    elapsed, prof_gu = timed(tp, step, steps, warmup, ["gateup_prefill"], "gateup_prefill", gu_dur)
    prof = breakdown(tp, step, steps, warmup + steps)
    prof["gateup_prefill"] = prof_gu["gateup_prefill"]   # the timed region's own record
    flops = ph.flops()
    value = flops * steps / elapsed / 1e12
    gu_ms, gu_n = prof["gateup_prefill"]
    dn_ms, dn_n = prof["down_prefill"]
    gu_tf = (4 * M * h * I_s) * gu_n / (gu_ms * 1e-3) / 1e12
    dn_tf = (2 * M * h * I_s) * dn_n / (dn_ms * 1e-3) / 1e12
    fwd_tf = flops * steps / ((gu_ms + dn_ms) * 1e-3) / 1e12
    kern = {"gateup_prefill": {"launches": gu_n, "avg_us": round(1e3 * gu_ms / gu_n, 2), "TFLOPs": round(gu_tf, 1)},
            "down_prefill": {"launches": dn_n, "avg_us": round(1e3 * dn_ms / dn_n, 2), "TFLOPs": round(dn_tf, 1)}}
    red = None
    if "partial_reduce" in prof:
        ms, n = prof["partial_reduce"]
        rb = workloads.reduce_bytes(M * h, t)
        gbs = rb * n / (ms * 1e-3) / 1e9
        kern["partial_reduce"] = {"launches": n, "avg_us": round(1e3 * ms / n, 2), "GBps": round(gbs, 1)}
        red = {"value": round(gbs, 1), "unit": "GB/s", "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
               "config": {"workload": "%d-way fp32 partial reduce of %dx%d, in place into the rank's partial "
                                      "(the reduce of the prefill step)" % (t, M, h), "t": t, "n": M * h},
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4),
                            "traffic": recorded_traffic("partial_reduce", "reduce70b" if cfg_id == 3 else
                                                        "reduce405b"),
                            "kernel": "partial_reduce", "per_launch_bytes": rb,
                            "avg_us": round(1e3 * ms / n, 2),
                            "source": "HIP events on every reduce launch of a further pass of the same steps"}}
    roof = {"bound": "mfma", "achieved": round(gu_tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(gu_tf / BF16_PEAK_TFLOPS, 4),
            "traffic": recorded_traffic("gateup_prefill", (args.workload if args.workload != "default" else
                                                           "prefill70b") + ("_rowmajor" if args.row_major else "")),
            "kernel": "gateup_prefill", "per_launch_flop": 4 * M * h * I_s, "avg_us": round(1e3 * gu_ms / gu_n, 2),
            "launch_us": spread(gu_dur),
            "source": "HIP events on every gate/up launch of the timed steps, on the launch stream"}
    out = dict(metric=METRIC, value=round(value, 1), unit="TFLOP/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * elapsed / steps, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16", data="synthetic",
               config={"workload": label, "M": M, "h": h, "I_s": I_s, "t": t, "weights": w,
                       "step_includes_reduce": ph.with_reduce},
               roofline=roof, forward_only_TFLOPs=round(fwd_tf, 1),
               forward_frac_of_bf16_peak=round(fwd_tf / BF16_PEAK_TFLOPS, 4), kernels=kern)
    if not args.no_cpu_baseline:
        rows = np.arange(0, M, max(1, M // 16))[:16]

        def once():
            oracle.rank_partial_from_storage(ph.x_host[rows], "bf16", host0["w_gate"], host0["w_up"],
                                             host0["w_down"], w, host0["s_gate"], host0["s_up"], host0["s_down"])
        log("timing the CPU oracle (prefill)")
        out["cpu_baseline"] = cpu_baseline(once, workloads.forward_flops(len(rows), h, I_s) / 1e12, "TFLOP/s",
                                           "rank partial for %d of the %d token rows (decoding the weight "
                                           "bytes each time), repeated >= 10 s" % (len(rows), M))
        if red is not None:
            sub = max(1, (M * h) // 16)
            hp = [ph.others[0][j][:sub].cpu().numpy() for j in range(t - 1)]
            hp = [np.random.Generator(np.random.PCG64(7)).standard_normal(sub, dtype=np.float32)] + hp
            log("timing the CPU oracle (reduce)")
            red["cpu_baseline"] = cpu_baseline(lambda: oracle.fold_fp32(hp), workloads.reduce_bytes(sub, t) / 1e9,
                                               "GB/s", "fold of the first %d elements of each of the %d buffers, "
                                               "repeated >= 10 s" % (sub, t), max_reps=1 << 30)
    if red is not None:
        out["reduce"] = red
    return out


def bench_default(tp, args):
    """The metric's two halves in one line: the 70B TP=8 decode step (value,
    GB/s) and, beside it, the 70B TP=8 prefill step (TFLOP/s: forward + the
    8-way reduce of its 4096 x 8192 partial) with the reduce's own GB/s."""
    out = bench_decode70b(tp, args)
    pre = bench_prefill(tp, args, 3, 4096, PREFILL70B_LABEL, 0.85)
    red = pre.pop("reduce", None)
    out["prefill"] = {k: pre[k] for k in ("value", "unit", "steps", "warmup", "ms_per_step", "config", "roofline",
                                          "forward_only_TFLOPs", "forward_frac_of_bf16_peak", "kernels",
                                          "cpu_baseline") if k in pre}
    out["prefill"]["frac_of_bf16_peak"] = round(pre["value"] / BF16_PEAK_TFLOPS, 4)
    if red is not None:
        out["reduce"] = red
    return out


PREFILL70B_LABEL = ("70B-shaped TP=8 rank prefill, M=4096, h=8192, I_s=3584, bf16, forward + 8-way fp32 partial "
                    "reduce of 4096x8192")


W_LABEL = {"e4m3fn": "fp8 e4m3fn", "int8": "int8"}


def bench_quant(tp, args, cfg_id):
    """One-byte weights with fp32 row scales (W8A16): the decode phases of the
    configuration (value: algorithmic GB/s) and its prefill size (reported
    beside it)."""
    c = workloads.CONFIGS[cfg_id]
    h, t, I_s, w = c["h"], c["t"], c["I"] // c["t"], c["w"]
    dec_Ms, pre_M = list(c["M"][:-1]), c["M"][-1]
    # enough weight sets that a set is read again only after >= 768 MB of others
    n_sets = max(2, (768 << 20) // (3 * h * I_s * (1 if w != "bf16" else 2)) + 2)
    sets, host0 = device_weights(cfg_id, h, I_s, w, c["std_gu"], c["std_down"], n_sets)
    decs = [Phase(tp, cfg_id, M, h, I_s, t, "bf16", w, False) for M in dec_Ms]
    pre = Phase(tp, cfg_id, pre_M, h, I_s, t, "bf16", w, False)
    # the decode phases read the weights packed for the decode kernels
    dsets = sets if args.row_major else \
        [dict(d, packed=tp.pack_weights(d["w_gate"], d["w_up"], d["w_down"], t=t)) for d in sets]

    nph = len(decs)
    lib = tp.load()
    gmask = 1 << tp.kernel_kinds().index("gateup_decode")

    def run_step(i, sel):
        # each phase of a step reads its own weight set
        for idx, ph in enumerate(decs):
            ph.run(dsets[(nph * i + idx) % len(dsets)], sel(idx))

    def step(i):
        # the gate/up launch of at most one phase per step is event-timed
        run_step(i, lambda idx: (lib, gmask) if timed_phase(i, nph) == idx else None)

    steps, warmup = args.steps or 100, args.warmup if args.warmup is not None else 10
    gu_dur = []
    el_d, prof_d = timed(tp, step, steps, warmup, [], "gateup_decode", gu_dur)
    rot, _ = breakdown_rotating(tp, run_step, nph, ["down_decode", "sk_clear"], steps, warmup + steps)
    prof_d.update(rot)
    p_steps = max(10, steps // 10)
    # the prefill phase reads the same packed array (the packed-weight GEMMs: one copy of the weights for
    # both phases; 12 % faster than the (out, in) layout's four-wave kernel for fp8 at 2048 tokens), or
    # with --row-major the (out, in) layout
    pset = sets[0] if args.row_major else dsets[0]
    el_p, prof_p = timed(tp, lambda i: pre.run(pset), p_steps, warmup_steps(1.5 if w == "int8" else 0.7),
                         ["gateup_prefill", "down_prefill"])
    dec_bytes = sum(ph.bytes() for ph in decs)
    dec_gbs = dec_bytes * steps / el_d / 1e9
    pre_tf = pre.flops() * p_steps / el_p / 1e12
    gu_ms, gu_n = prof_d["gateup_decode"]
    timed_gu_bytes = sum(workloads.gateup_bytes(decs[timed_phase(warmup + j, nph)].M, h, I_s, "bf16", w)
                         for j in range(steps) if timed_phase(warmup + j, nph) is not None)
    gu_gbs = timed_gu_bytes / (gu_ms * 1e-3) / 1e9
    pgu_ms, pgu_n = prof_p["gateup_prefill"]
    pgu_tf = 4 * pre_M * h * I_s * pgu_n / (pgu_ms * 1e-3) / 1e12
    out = dict(metric=METRIC, value=round(dec_gbs, 1), unit="GB/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * el_d / steps, 5), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16 (%s weights)" % W_LABEL[w], data="synthetic",
               config={"workload": "70B-shaped TP=%d rank, %s weights + fp32 row scales: decode M=%s (value%s) "
                                   "and prefill M=%d" % (t, W_LABEL[w], ", ".join(map(str, dec_Ms)),
                                                         "" if args.row_major else ", weights packed for the decode "
                                                         "kernels, the prefill on the same packed array", pre_M),
                       "h": h, "I_s": I_s, "t": t, "weight_sets": len(sets)},
               roofline={"bound": "hbm", "achieved": round(gu_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gu_gbs / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("gateup_decode",
                                                     args.workload + ("_rowmajor" if args.row_major else "")),
                         "kernel": "gateup_decode",
                         "avg_us": round(1e3 * gu_ms / gu_n, 3), "launch_us": spread(gu_dur),
                         "source": "HIP events on the gate/up launch of phase i mod %d on the timed steps i "
                                   "with i mod %d < %d" % (max(nph, 3), max(nph, 3), nph)},
               prefill={"M": pre_M, "weights": "packed" if pset is not sets[0] else "(out, in)",
                        "TFLOPs": round(pre_tf, 1), "frac_bf16_peak": round(pre_tf / BF16_PEAK_TFLOPS, 4),
                        "gateup_TFLOPs": round(pgu_tf, 1), "kernels": {k: {"avg_us": 1e3 * v[0] / v[1]}
                                                                      for k, v in prof_p.items()}},
               kernels={k: {"avg_us": 1e3 * v[0] / v[1]} for k, v in prof_d.items()})
    if not args.no_cpu_baseline:
        import oracle

        def once():
            for ph in decs:
                oracle.rank_partial_from_storage(ph.x_host, "bf16", host0["w_gate"], host0["w_up"],
                                                 host0["w_down"], w, host0["s_gate"], host0["s_up"],
                                                 host0["s_down"])
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(once, dec_bytes / 1e9, "GB/s",
                                           "one decode step's rank partials (M=%s) from the %s weight bytes "
                                           "and scales, repeated >= 10 s" % (", ".join(map(str, dec_Ms)),
                                                                             W_LABEL[w]))
    return out


FP8_PEAK_TFLOPS = 5000.0


def bench_w8a8(tp, args):
    """fp8 x fp8 forward of the 70B-shaped TP=4 rank at 2048 tokens (the fp8
    weight configuration's prefill size): per-token quantisation of X, gate/up
    on the fp8 matrix cores, quantisation of A, down."""
    import torch
    import oracle
    cfg_id, M = 4, 2048
    c = workloads.CONFIGS[cfg_id]
    h, t, I_s = c["h"], c["t"], c["I"] // c["t"]
    sets, host0 = device_weights(cfg_id, h, I_s, "e4m3fn", c["std_gu"], c["std_down"], 1)
    x_host = workloads.make_x(cfg_id, M, h, "bf16")
    x = to_dev(x_host, "bf16")
    w = sets[0]
    call = tp.prepare_shard_forward_w8a8(x, w["w_gate"], w["w_up"], w["w_down"], t=t, k=0, s_gate=w["s_gate"],
                                         s_up=w["s_up"], s_down=w["s_down"])
    steps, warmup = args.steps or 30, args.warmup if args.warmup is not None else warmup_steps(0.45)
    gu_dur = []
    elapsed, prof_gu = timed(tp, lambda i: call(), steps, warmup, ["gateup_w8a8"], "gateup_w8a8", gu_dur)
    prof = breakdown(tp, lambda i: call(), steps, warmup + steps)
    prof["gateup_w8a8"] = prof_gu["gateup_w8a8"]
    flops = workloads.forward_flops(M, h, I_s)
    value = flops * steps / elapsed / 1e12
    gu_ms, gu_n = prof["gateup_w8a8"]
    gu_tf = 4 * M * h * I_s * gu_n / (gu_ms * 1e-3) / 1e12
    dn_ms, dn_n = prof["down_w8a8"]
    dn_tf = 2 * M * h * I_s * dn_n / (dn_ms * 1e-3) / 1e12
    out = dict(metric=METRIC, value=round(value, 1), unit="TFLOP/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * elapsed / steps, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="fp8 e4m3fn x e4m3fn (per-token activation scales, row weight scales)",
               data="synthetic",
               config={"workload": "70B-shaped TP=4 rank W8A8 forward at M=2048 (h=8192, I_s=7168): quantise X, "
                                   "gate/up + SwiGLU, quantise A, down to the fp32 partial", "M": M, "h": h,
                       "I_s": I_s, "t": t},
               roofline={"bound": "mfma", "achieved": round(gu_tf, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gu_tf / FP8_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("gateup_w8a8", "w8a8_prefill70b"), "kernel": "gateup_w8a8",
                         "per_launch_flop": 4 * M * h * I_s, "avg_us": round(1e3 * gu_ms / gu_n, 2),
                         "launch_us": spread(gu_dur), "source": "HIP events on every gate/up launch of the timed steps"},
               kernels={k: {"launches": v[1], "avg_us": 1e3 * v[0] / v[1]} for k, v in prof.items()},
               gemm_TFLOPs={"gateup_w8a8": round(gu_tf, 1), "down_w8a8": round(dn_tf, 1)})
    if not args.no_cpu_baseline:
        rows = np.arange(0, M, M // 16)

        def once():
            oracle.rank_partial_w8a8_from_storage(x_host[rows], host0["w_gate"], host0["w_up"], host0["w_down"],
                                                  host0["s_gate"], host0["s_up"], host0["s_down"])
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(once, workloads.forward_flops(len(rows), h, I_s) / 1e12, "TFLOP/s",
                                           "W8A8 rank partial for %d of the %d token rows (quantisation and "
                                           "decoding included), repeated >= 10 s" % (len(rows), M))
    return out


def bench_reduce(tp, args, cfg_id):
    import torch
    import oracle
    c = workloads.CONFIGS[cfg_id]
    n, t = c["reduce_n"], c["t"]
    parts_host = workloads.make_partials(cfg_id, t, n)
    parts = [torch.from_numpy(p).cuda() for p in parts_host]
    # in place into partial 0, as the all-reduce leaves the sum in each rank's own buffer
    # (the values grow step by step; the work and the bytes do not change)
    out = parts[0]
    steps, warmup = args.steps or 50, args.warmup if args.warmup is not None else 5
    red_dur = []
    elapsed, prof = timed(tp, lambda i: tp.partial_reduce(parts, out=out), steps, warmup, ["partial_reduce"],
                          "partial_reduce", red_dur)
    b = workloads.reduce_bytes(n, t)
    ms, cnt = prof["partial_reduce"]
    achieved = b * cnt / (ms * 1e-3) / 1e9
    value = b * steps / elapsed / 1e9
    res = dict(metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * elapsed / steps, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="f32", data="synthetic",
               config={"workload": "%d-way fp32 partial reduce of %d elements, in place into partial 0"
                                   % (t, n), "t": t, "n": n, "in_place": True},
               roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("partial_reduce", args.workload), "kernel": "partial_reduce",
                         "avg_us": round(1e3 * ms / cnt, 2), "launch_us": spread(red_dur),
                         "source": "HIP events on every reduce launch of the timed steps"})
    if not args.no_cpu_baseline:
        sub = max(1, n // 16)
        hp = [p[:sub] for p in parts_host]
        res["cpu_baseline"] = cpu_baseline(lambda: oracle.fold_fp32(hp), workloads.reduce_bytes(sub, t) / 1e9,
                                           "GB/s", "fold of the first %d elements of each buffer, repeated "
                                           ">= 10 s" % sub, max_reps=1 << 30)
    return res


def bench_sp_prefill(tp, args):
    """Sequence-parallel form of the 70B TP=8 prefill step: the forward reads X
    from the eight ranks' 512-token row blocks, and the 8-way sum is the
    reduce-scatter that leaves rank 0 its 512 rows."""
    import torch
    import oracle
    cfg_id, M = 3, 4096
    c = workloads.CONFIGS[cfg_id]
    h, t, I_s, w = c["h"], c["t"], c["I"] // c["t"], c["w"]
    sets, host0 = device_weights(cfg_id, h, I_s, w, c["std_gu"], c["std_down"], 1)
    x_host = workloads.make_x(cfg_id, M, h, "bf16")
    r = M // t
    blocks = [to_dev(np.ascontiguousarray(x_host[j * r:(j + 1) * r]), "bf16") for j in range(t)]
    partial = torch.empty((M, h), dtype=torch.float32, device="cuda")
    nbytes = tp.workspace_bytes(M, h, I_s * t, t, torch.bfloat16, torch.bfloat16)
    ws = tp.alloc_workspace(nbytes, "cuda")
    others = [torch.from_numpy(o).cuda().view(M, h) for o in workloads.make_partials(cfg_id, t - 1, M * h)]
    out = torch.empty((r, h), dtype=torch.float32, device="cuda")
    fwd = tp.prepare_shard_forward_sp(blocks, sets[0]["w_gate"], sets[0]["w_up"], sets[0]["w_down"], t=t, k=0,
                                      partial=partial, workspace=ws)
    rs = tp.prepare_partial_reduce_scatter([partial] + others, 0, out=out)

    def step(i):
        fwd()
        rs()

    steps, warmup = args.steps or 30, args.warmup if args.warmup is not None else warmup_steps(0.85)
    elapsed, prof_gu = timed(tp, step, steps, warmup, ["gateup_prefill"])
    prof = breakdown(tp, step, steps, warmup + steps)
    flops = workloads.forward_flops(M, h, I_s)
    value = flops * steps / elapsed / 1e12
    gu_ms, gu_n = prof_gu["gateup_prefill"]
    gu_tf = 4 * M * h * I_s * gu_n / (gu_ms * 1e-3) / 1e12
    rs_ms, rs_n = prof["partial_reduce"]
    rs_bytes = workloads.reduce_bytes(r * h, t)
    out_d = dict(metric=METRIC, value=round(value, 1), unit="TFLOP/s", n_gpus=1, steps=steps, warmup=warmup,
                 ms_per_step=round(1e3 * elapsed / steps, 4), higher_is_better=True, scaling="weak",
                 vs_baseline=None, dtype="bf16", data="synthetic",
                 config={"workload": "sequence-parallel 70B-shaped TP=8 rank prefill: forward over 8 row blocks "
                                     "of 512 tokens (h=8192, I_s=3584, bf16) + reduce-scatter of rank 0's 512 "
                                     "rows of the 8-way fp32 sum", "M": M, "h": h, "I_s": I_s, "t": t},
                 roofline={"bound": "mfma", "achieved": round(gu_tf, 1), "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(gu_tf / BF16_PEAK_TFLOPS, 4),
                           "traffic": recorded_traffic("gateup_prefill", "sp_prefill70b"), "kernel": "gateup_prefill"},
                 kernels={k: {"launches": v[1], "avg_us": 1e3 * v[0] / v[1]} for k, v in prof.items()},
                 reduce_scatter={"GBps": round(rs_bytes * rs_n / (rs_ms * 1e-3) / 1e9, 1),
                                 "frac_hbm": round(rs_bytes * rs_n / (rs_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
    if not args.no_cpu_baseline:
        rows = np.arange(0, M, r)[:8]

        def once():
            xg = oracle.gather_rows([x_host[j * r:(j + 1) * r] for j in range(t)])
            oracle.rank_partial_from_storage(xg[rows], "bf16", host0["w_gate"], host0["w_up"], host0["w_down"],
                                             "bf16")
        log("timing the CPU oracle")
        out_d["cpu_baseline"] = cpu_baseline(once, workloads.forward_flops(len(rows), h, I_s) / 1e12, "TFLOP/s",
                                             "gather of the row blocks + rank partial for %d token rows, "
                                             "repeated >= 10 s" % len(rows))
    return out_d


class AttnPhase:
    """The attention block's two projections of a rank at M tokens (+ the
    8-way reduce of the output projection's partial), buffers preallocated."""

    def __init__(self, tp, cfg_id, M, c, with_reduce):
        import torch
        self.tp, self.M, self.c = tp, M, c
        self.h, self.t = c["h"], c["t"]
        self.n_loc, self.k_o = workloads.attn_widths(c["n_heads"], c["n_kv_heads"], c["head_dim"], c["t"])
        self.x_host = workloads.make_x(cfg_id, M, self.h, "bf16")
        self.o_host = workloads.make_attn_out_input(cfg_id, M, self.k_o, "bf16")
        self.x, self.o = to_dev(self.x_host, "bf16"), to_dev(self.o_host, "bf16")
        self.qkv = torch.empty((M, self.n_loc), dtype=torch.bfloat16, device="cuda")
        self.partial = torch.empty((M, self.h), dtype=torch.float32, device="cuda")
        self.with_reduce = with_reduce
        if with_reduce:
            self.others = [torch.from_numpy(o).cuda()
                           for o in workloads.make_partials(cfg_id, self.t - 1, M * self.h, weight_set=M)]
        self.calls = {}

    def run(self, wset, time_qkv=None):
        """time_qkv: (library, kind mask) to event-time this call's launches of
        those kinds only."""
        key = id(wset)
        if key not in self.calls:
            c = self.c
            q = self.tp.prepare_attn_qkv_forward(self.x, wset["w_qkv"], n_heads=c["n_heads"],
                                                 n_kv_heads=c["n_kv_heads"], head_dim=c["head_dim"], t=self.t,
                                                 k=0, s_qkv=wset["s_qkv"], out=self.qkv)
            o = self.tp.prepare_attn_out_forward(self.o, wset["w_o"], n_heads=c["n_heads"], head_dim=c["head_dim"],
                                                 t=self.t, k=0, s_o=wset["s_o"], partial=self.partial)
            red = self.tp.prepare_partial_reduce([self.partial.view(-1)] + self.others,
                                                 out=self.partial.view(-1)) if self.with_reduce else None
            self.calls[key] = (q, o, red)
        q, o, red = self.calls[key]
        if time_qkv is not None:
            time_qkv[0].tp_profile_enable(time_qkv[1])
        q()
        o()
        if red is not None:
            red()
        if time_qkv is not None:
            time_qkv[0].tp_profile_enable(0)

    def qkv_bytes(self, w="bf16"):
        return workloads.linear_bytes(self.M, self.n_loc, self.h, "bf16", w, "bf16")

    def oproj_bytes(self, w="bf16"):
        return workloads.linear_bytes(self.M, self.h, self.k_o, "bf16", w, "f32")

    def bytes(self, w="bf16"):
        b = self.qkv_bytes(w) + self.oproj_bytes(w)
        if self.with_reduce:
            b += workloads.reduce_bytes(self.M * self.h, self.t)
        return b

    def flops(self):
        return workloads.linear_flops(self.M, self.n_loc, self.h) + workloads.linear_flops(self.M, self.h, self.k_o)


def attn_weight_sets(cfg_id, c, n_sets):
    import torch
    n_loc, k_o = workloads.attn_widths(c["n_heads"], c["n_kv_heads"], c["head_dim"], c["t"])
    sets = []
    for s in range(n_sets):
        ws = workloads.make_attn_weights(cfg_id, c["h"], n_loc, k_o, 0, c["w"], c["std_w"], weight_set=s)
        sets.append(dict(w_qkv=to_dev(ws["w_qkv"], c["w"]), w_o=to_dev(ws["w_o"], c["w"]),
                         s_qkv=None if ws["s_qkv"] is None else torch.from_numpy(ws["s_qkv"]).cuda(),
                         s_o=None if ws["s_o"] is None else torch.from_numpy(ws["s_o"]).cuda()))
        if s == 0:
            host0 = ws
    return sets, host0


def bench_attn_decode(tp, args):
    """70B-shaped TP=8 rank, attention projections at decode: for M = 1, 8 and
    64 tokens, the column-parallel QKV projection (8 query heads + 1 KV head:
    1280 columns), the row-parallel output projection (1024 -> 8192, fp32
    partial) and the 8-way reduce of that partial."""
    import oracle
    cfg_id = 6
    c = workloads.ATTN_CONFIGS[cfg_id]
    h, t = c["h"], c["t"]
    # 36 MiB of weights per set: enough sets that a step's weights come from HBM
    n_sets = max(args.weight_sets, 16)
    log("generating %d weight sets of the 70B TP=8 attention projections" % n_sets)
    sets, host0 = attn_weight_sets(cfg_id, c, n_sets)
    phases = [AttnPhase(tp, cfg_id, M, c, True) for M in (1, 8, 64)]
    # An event-timed launch costs the host ~25 us against ~3 us for a plain
    # one, and this step's kernels are short: timing all three QKV launches
    # would make the loop host-bound.  Step i times the QKV launch of phase
    # i % 3 only, so each M is sampled on a third of the timed steps.
    lib = tp.load()
    qmask = 1 << tp.kernel_kinds().index("qkv_decode")

    # each phase of a step reads its own weight set: phase idx of step i takes set (3 i + idx) mod n
    def run_step(i, sel):
        for idx, ph in enumerate(phases):
            ph.run(sets[(3 * i + idx) % len(sets)], sel(idx))

    def step(i):
        run_step(i, lambda idx: (lib, qmask) if i % 3 == idx else None)

    steps, warmup = args.steps or 402, args.warmup if args.warmup is not None else 42
    q_dur = []
    elapsed, prof = timed(tp, step, steps, warmup, [], "qkv_decode", q_dur)
    prof_all, per_step = breakdown_rotating(tp, run_step, 3, ["qkv_decode", "oproj_decode", "sk_clear",
                                                              "partial_reduce"], steps, warmup + steps)
    step_bytes = sum(ph.bytes() for ph in phases)
    value = step_bytes * steps / elapsed / 1e9
    per = {"qkv_decode": sum(ph.qkv_bytes() for ph in phases), "oproj_decode": sum(ph.oproj_bytes() for ph in phases),
           "partial_reduce": sum(workloads.reduce_bytes(ph.M * h, t) for ph in phases), "sk_clear": None}
    kern = {}
    for name, b in per.items():
        if name not in prof_all:
            continue
        ms, cnt = prof_all[name]
        kern[name] = {"launches": cnt, "avg_us": round(1e3 * ms / max(cnt, 1), 3)}
        if b is not None:
            kern[name]["GBps"] = round(b / (per_step[name] * 1e-3) / 1e9, 1)
    ms, cnt = prof["qkv_decode"]
    # the timed launches: phase idx on the steps i with i % 3 == idx
    timed_bytes = sum(ph.qkv_bytes() * sum(1 for i in range(warmup, warmup + steps) if i % 3 == idx)
                      for idx, ph in enumerate(phases))
    assert cnt == steps
    achieved = timed_bytes / (ms * 1e-3) / 1e9
    parity = None
    if not args.no_cpu_baseline:
        import torch
        ph = phases[0]
        ph.run(sets[0])
        ph.calls[id(sets[0])][1]()   # the output projection alone (the step's reduce ran in place)
        torch.cuda.synchronize()
        ref_q = oracle.linear_from_storage(ph.x_host, "bf16", host0["w_qkv"], "bf16")
        ref_p = oracle.linear_from_storage(ph.o_host, "bf16", host0["w_o"], "bf16")
        q_bits = ph.qkv.view(torch.int16).cpu().numpy().view(np.uint16)
        parity = {"qkv": oracle.rms_normalised_max_error(oracle.bf16_bits_to_f64(q_bits), ref_q),
                  "oproj": oracle.rms_normalised_max_error(ph.partial.cpu().numpy(), ref_p)}
    out = dict(metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * elapsed / steps, 5), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16", data="synthetic",
               config={"workload": "70B-shaped TP=8 rank attention projections at decode (h=8192, 64/8 heads "
                                   "of 128: QKV 8192->1280 bf16 out, o_proj 1024->8192 fp32 partial, bf16 "
                                   "weights) at M=1, 8 and 64, each o_proj partial followed by the 8-way "
                                   "fp32 reduce", "M": [1, 8, 64], "h": h, "t": t, "weight_sets": n_sets},
               roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": recorded_traffic("qkv_decode", "attn70b"), "kernel": "qkv_decode",
                         "per_launch_bytes": {str(ph.M): ph.qkv_bytes() for ph in phases},
                         "avg_us": round(1e3 * ms / cnt, 3),
                         "per_M_launch_us": {str(ph.M): spread([d for j, d in enumerate(q_dur)
                                                                if (warmup + j) % 3 == idx])
                                             for idx, ph in enumerate(phases)},
                         "source": "HIP events on the QKV launch of one phase per timed step (phase i mod 3)"},
               frac_of_hbm_peak=round(value / HBM_PEAK_GBS, 4), kernels=kern,
               kernels_note="kernels: for each kernel kind a further pass of the same number of steps that "
                            "event-times that kind's launches in one phase per step, like the timed region",
               parity_err_M1=parity)
    if not args.no_cpu_baseline:
        hp = [[np.zeros(ph.M * h, np.float32)] * (t - 1) for ph in phases]

        def once():
            for ph, others in zip(phases, hp):
                oracle.linear_from_storage(ph.x_host, "bf16", host0["w_qkv"], "bf16")
                p = oracle.linear_from_storage(ph.o_host, "bf16", host0["w_o"], "bf16")
                oracle.fold_fp32([p.astype(np.float32).reshape(-1)] + others)
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(once, step_bytes / 1e9, "GB/s",
                                           "one full step (M=1, 8, 64 QKV and o_proj from the bf16 weight "
                                           "bytes + 8-way fp32 folds), repeated >= 10 s")
    return out


def bench_attn_prefill(tp, args):
    """70B-shaped TP=8 rank, attention projections at prefill (M = 4096):
    QKV, output projection and the 8-way reduce of its partial."""
    import oracle
    cfg_id, M = 6, 4096
    c = workloads.ATTN_CONFIGS[cfg_id]
    h, t = c["h"], c["t"]
    sets, host0 = attn_weight_sets(cfg_id, c, 1)
    ph = AttnPhase(tp, cfg_id, M, c, True)

    def step(i):
        ph.run(sets[0])

    steps, warmup = args.steps or 30, args.warmup if args.warmup is not None else warmup_steps(0.4)
    q_dur = []
    elapsed, prof_q = timed(tp, step, steps, warmup, ["qkv_prefill"], "qkv_prefill", q_dur)
    prof = breakdown(tp, step, steps, warmup + steps)
    prof["qkv_prefill"] = prof_q["qkv_prefill"]
    value = ph.flops() * steps / elapsed / 1e12
    f = {"qkv_prefill": workloads.linear_flops(M, ph.n_loc, h), "oproj_prefill": workloads.linear_flops(M, h, ph.k_o)}
    kern = {}
    for name, fl in f.items():
        ms, n = prof[name]
        kern[name] = {"launches": n, "avg_us": 1e3 * ms / n, "TFLOPs": round(fl * n / (ms * 1e-3) / 1e12, 1)}
    ms, n = prof["partial_reduce"]
    kern["partial_reduce"] = {"launches": n, "avg_us": 1e3 * ms / n,
                              "GBps": round(workloads.reduce_bytes(M * h, t) * n / (ms * 1e-3) / 1e9, 1)}
    q_tf = kern["qkv_prefill"]["TFLOPs"]
    out = dict(metric=METRIC, value=round(value, 1), unit="TFLOP/s", n_gpus=1, steps=steps, warmup=warmup,
               ms_per_step=round(1e3 * elapsed / steps, 4), higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype="bf16", data="synthetic",
               config={"workload": "70B-shaped TP=8 rank attention projections at prefill, M=4096 (QKV "
                                   "8192->1280, o_proj 1024->8192 fp32 partial, bf16) + 8-way fp32 reduce of "
                                   "4096x8192", "M": M, "h": h, "t": t},
               roofline={"bound": "mfma", "achieved": q_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(q_tf / BF16_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic("qkv_prefill", "attn_prefill70b"), "kernel": "qkv_prefill",
                         "per_launch_flop": f["qkv_prefill"], "avg_us": round(kern["qkv_prefill"]["avg_us"], 2),
                         "launch_us": spread(q_dur),
                         "source": "HIP events on every QKV launch of the timed steps"},
               kernels=kern)
    if not args.no_cpu_baseline:
        rows = np.arange(0, M, M // 16)

        def once():
            oracle.linear_from_storage(ph.x_host[rows], "bf16", host0["w_qkv"], "bf16")
            oracle.linear_from_storage(ph.o_host[rows], "bf16", host0["w_o"], "bf16")
        log("timing the CPU oracle")
        fl = workloads.linear_flops(len(rows), ph.n_loc, h) + workloads.linear_flops(len(rows), h, ph.k_o)
        out["cpu_baseline"] = cpu_baseline(once, fl / 1e12, "TFLOP/s",
                                           "QKV and o_proj for %d of the %d token rows (decoding the weight "
                                           "bytes each time), repeated >= 10 s" % (len(rows), M))
    return out


def bench_copy(tp, args):
    """One-buffer reduce over 1 GiB: reads n*4 bytes and writes n*4 bytes, nothing else."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    out = torch.empty_like(src)
    steps, warmup = args.steps or 20, args.warmup if args.warmup is not None else 3
    elapsed, prof = timed(tp, lambda i: tp.partial_reduce([src], out=out), steps, warmup, ["partial_reduce"])
    b = workloads.reduce_bytes(n, 1)
    ms, cnt = prof["partial_reduce"]
    achieved = b * cnt / (ms * 1e-3) / 1e9
    return dict(metric="copy GB/s (HBM counter calibration)", value=round(b * steps / elapsed / 1e9, 1),
                unit="GB/s", n_gpus=1, steps=steps, warmup=warmup, ms_per_step=round(1e3 * elapsed / steps, 4),
                higher_is_better=True, scaling="weak", vs_baseline=None, dtype="f32", data="synthetic",
                config={"workload": "copy of %d fp32 (one-buffer partial reduce)" % n, "n": n,
                        "bytes_read": 4 * n, "bytes_written": 4 * n},
                roofline={"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                          "kernel": "partial_reduce"})


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the TP exchange "
              "across GPUs is design-only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import tensor_transformer_mlp_tp_amd as tp
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    tp.load()
    if args.workload == "default":
        out = bench_default(tp, args)
    elif args.workload == "decode70b":
        out = bench_decode70b(tp, args)
    elif args.workload == "prefill70b":
        out = bench_prefill(tp, args, 3, 4096, PREFILL70B_LABEL, 0.85)
    elif args.workload == "prefill405b":
        out = bench_prefill(tp, args, 5, 8192, "405B-shaped TP=8 rank prefill, M=8192, h=16384, I_s=6656, "
                                               "bf16, forward + 8-way fp32 partial reduce of 8192x16384", 5.5)
    elif args.workload == "fp8_70b":
        out = bench_quant(tp, args, 4)
    elif args.workload == "int8_70b":
        out = bench_quant(tp, args, 9)
    elif args.workload == "w8a8_prefill70b":
        out = bench_w8a8(tp, args)
    elif args.workload == "reduce70b":
        out = bench_reduce(tp, args, 3)
    elif args.workload == "copy":
        out = bench_copy(tp, args)
    elif args.workload == "sp_prefill70b":
        out = bench_sp_prefill(tp, args)
    elif args.workload == "attn70b":
        out = bench_attn_decode(tp, args)
    elif args.workload == "attn_prefill70b":
        out = bench_attn_prefill(tp, args)
    else:
        out = bench_reduce(tp, args, 5)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
