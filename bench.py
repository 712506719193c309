"""Benchmark of the GSA hot path on one MI355X.

A step is one chunkwise GSA forward (gate prep, both passes, slot softmax,
state carry; all phases of the launch sequence) over one batch of the
training-shape workload: B=8, H=4, T=2048, dk=dv=128, m=64 slots, C=64,
bf16 inputs, fp32 state (seeded synthetic data).  `value` is B*T tokens/s
with inputs resident in HBM, rotating over enough input copies that the
256 MB last-level cache cannot hold them.  The timed region runs the steps
with no timing hooks; the dominant kernel's duration comes from an identical
pass whose kernels' own dispatches stamp HIP events (start and end) on the
library's stream.

Also reported: the standalone GLA forward (T=4096), the long-context GSA
forward (T=16384, initial state), and the batched decode step (HBM GB/s),
and the float64 CPU oracle timed on this host on the training-shape batch.
"""
import argparse
import ctypes
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP32_VALU_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ HIP events
class Events:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            out.append(e.value)
        return out

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def ms(self, a, b):
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return float(f.value)


def kernel_source_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "slot_memory_sequence_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get("%s@%s" % (kernel, workload))
    except Exception:
        return None
    if not rec or rec.get("source_sha") != kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------ workloads
def gsa_alg(B, H, T, dk, dv, m, C, dtype_bytes, init_state=False, final_state=False):
    th = B * H * T
    flops = th * ((C + 1) * (dk + 2 * m + dv) + 4 * m * (dk + dv))
    nbytes = th * (2 * dk + dv + m + dv) * dtype_bytes
    if init_state:
        nbytes += B * H * m * (dk + dv) * 4
    if final_state:
        nbytes += B * H * m * (dk + dv) * 4
    return flops, nbytes


def gla_alg(B, H, T, dk, dv, C, dtype_bytes):
    th = B * H * T
    return th * ((C + 1) * (dk + dv) + 4 * dk * dv), th * (3 * dk + 2 * dv) * dtype_bytes


def gsa_bwd_alg(B, H, T, dk, dv, m, dtype_bytes):
    """Per launch: fp32 vector flops of the forward token walk (state
    updates, the two reads, dq and the reverse maps: 2 m (4 dk + 3 dv) per
    token and head) and of the reverse walk (adjoint updates, the two gate
    dots, dk, dv, the decay: 7 m (dk + dv)); and the backward's algorithmic
    HBM bytes: q, k, v, g, dO read and dq, dk, dv, dg written once."""
    th = B * H * T
    return (th * 2 * m * (4 * dk + 3 * dv), th * 7 * m * (dk + dv),
            th * (4 * dk + 3 * dv + 2 * m) * dtype_bytes)


def rel_err(x, y):
    """max |x - y| / max |y| over one tensor (y the oracle)."""
    import numpy as np
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        return float("inf")
    den = float(np.max(np.abs(y))) if y.size else 0.0
    num = float(np.max(np.abs(x - y))) if y.size else 0.0
    return num / den if den > 0 else num


def gsa_bwd_chunk_alg(B, H, T, dk, dv, m, C, dtype_bytes):
    """The chunk-form backward on the matrix cores, per launch.  Algorithmic
    flops (causal halves only, 2 per multiply-add) of the forward sweep (z,
    ds, dq with their intra-chunk scores, the state carry, the reverse map)
    and of the reverse sweep (the two score sets, A_dq / A_2, dk and dv inter
    and intra, di inter and intra, the adjoint update); and algorithmic bytes:
    forward sweep q, k, v, g, dO read and dq written, reverse sweep the same
    reads and dk, dv, dg written, the whole backward each input read and each
    gradient written once."""
    th = B * H * T
    h = (C + 1) / 2.0
    fwd = (m * dk + h * dk + h * m) + (m * dv + h * dv + h * m) + (m * dk + h * m + h * dk) + 2 * m * (dk + dv)
    rev = (h * (dk + dv) + 2 * h * m + m * (dk + dv) + h * (dk + dv) + m * (dk + dv) + 2 * h * m +
           m * (dk + dv))
    reads = (2 * dk + 2 * dv + m) * dtype_bytes
    return {"flops_fwd": 2 * fwd * th, "flops_rev": 2 * rev * th,
            "bytes_fwd": th * (reads + dk * dtype_bytes), "bytes_rev": th * (reads + (dk + dv + m) * dtype_bytes),
            "bytes": th * (4 * dk + 3 * dv + 2 * m) * dtype_bytes}


def dev_sets(torch, inp, names, nsets):
    from synth import to_dev
    base = {n: to_dev(inp[n], torch) for n in names if inp.get(n) is not None}
    sets = [base]
    for _ in range(nsets - 1):
        sets.append({n: t.clone() for n, t in base.items()})
    return sets


def time_op(torch, ev, call, sets, steps, warmup):
    """Warmup, then the timed region: exactly `steps` steps rotating over the
    input sets, bracketed by device synchronisations, with no timing hooks
    (wall-clock seconds).  Then the same steps again with the kernels'
    dispatch-stamped events, which give each kernel's execution time; the
    stamps cost the stream a few microseconds per stamped launch, which is
    why they stay out of the throughput loop.  Returns (wall seconds,
    per-step phase times in ms)."""
    evs = ev.create(4 * steps)
    for i in range(warmup):
        call(sets[i % len(sets)], None)
    torch.cuda.synchronize()
    quiesce()
    t0 = time.perf_counter()
    for i in range(steps):
        call(sets[i % len(sets)], None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        call(sets[i % len(sets)], evs[4 * i: 4 * i + 4])
    torch.cuda.synchronize()
    phases = []
    for i in range(steps):
        e = evs[4 * i: 4 * i + 4]
        phases.append((ev.ms(e[0], e[1]), ev.ms(e[1], e[2]), ev.ms(e[2], e[3]), ev.ms(e[0], e[3])))
    return wall, phases


def quiesce():
    """Start of a timed GPU region: run the cyclic garbage collector now.
    Automatic collection is off in the benchmark process (main), because a
    full pass over its heap took tens of milliseconds between two steps of a
    timed loop."""
    gc.collect()


def mean(xs):
    return sum(xs) / len(xs)


def stats(xs):
    """Mean, median, p10 and p90 (nearest rank) of per-step times in ms."""
    ys = sorted(xs)
    n = len(ys)

    def q(f):
        return ys[min(n - 1, max(0, int(round(f * (n - 1)))))]
    return {"mean": round(mean(ys), 4), "median": round(q(0.5), 4), "p10": round(q(0.1), 4),
            "p90": round(q(0.9), 4), "n": n}


def cpu_threads():
    """Host threads the oracle runs on: the CPUs this process may use (its
    share of the host), and os.cpu_count() beside it."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, avail), os.cpu_count()


def timed_runs(fn, budget_s):
    """Run fn until budget_s seconds have passed (at least once): (runs, s)."""
    t0 = time.perf_counter()
    runs = 0
    while True:
        fn()
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            return runs, dt


def op_roofline(bytes_alg, t_ms):
    """The whole op against HBM: algorithmic bytes over the wall-clock step
    (every launch of the sequence and the gaps between them)."""
    a = bytes_alg / (t_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBPS, 4), "basis": "wall-clock ms_per_step"}


def roofline(bytes_alg, t_ms, kernel, workload):
    achieved = bytes_alg / (t_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": load_traffic(kernel, workload),
            "kernel": kernel, "basis": "the workload's algorithmic bytes over this kernel's "
                                       "mean dispatch time"}


def bench_gsa(torch, gsa, ev, w, name, steps, warmup, nsets, warm_too=True, nonlinearity="softmax"):
    import synth
    inp = synth.gsa_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                           seed=0, qkv_scale=w["qkv_scale"], g_shift=w["g_shift"],
                           init_std=w["init_std"], fast_slots=w.get("fast_slots", 0),
                           fast_shift=w.get("fast_shift", 0.0))
    sets = dev_sets(torch, inp, ["q", "k", "v", "g", "k0", "v0"], nsets)
    init = inp["k0"] is not None
    B, H, T, dk, dv, m = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"]
    bf16 = w["dtype"] == "bf16"
    tdt = torch.bfloat16 if bf16 else torch.float32
    outs = [torch.empty((B, H, T, dv), dtype=tdt, device="cuda") for _ in sets]
    kfs = [torch.empty((B, H, m, dk), dtype=torch.float32, device="cuda") for _ in sets] if init else None
    vfs = [torch.empty((B, H, m, dv), dtype=torch.float32, device="cuda") for _ in sets] if init else None
    nb = gsa.gsa_fwd_workspace_bytes(B, H, T, dk, dv, m, w["C"], 1 if bf16 else 0, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def call(s, events):
        i = next(j for j, x in enumerate(sets) if x is s)
        gsa.gsa_fwd(s["q"], s["k"], s["v"], s["g"], s.get("k0"), s.get("v0"), tau=w["tau"],
                    final_state=init, out=outs[i], k_final=kfs[i] if init else None,
                    v_final=vfs[i] if init else None, workspace=ws, events=events,
                    nonlinearity=nonlinearity)

    wall, ph = time_op(torch, ev, call, sets, steps, warmup)
    flops, nbytes = gsa_alg(B, H, T, dk, dv, m, w["C"], 2 if bf16 else 4, init_state=init,
                            final_state=init)
    t_op = mean([p[3] for p in ph])
    t_out = mean([p[2] for p in ph])
    t_wall = wall / steps * 1e3
    res = {
        "tokens_per_s": B * T * steps / wall, "ms_per_step": t_wall,
        "ms_phases": {"state_maps": round(mean([p[0] for p in ph]), 4),
                      "scan": round(mean([p[1] for p in ph]), 4),
                      "outputs": round(t_out, 4), "op": round(t_op, 4)},
        "ms_op_stamped": stats([p[3] for p in ph]),
        "ms_out_kernel": stats([p[2] for p in ph]),
        "alg_flops": flops, "alg_bytes": nbytes,
        "alg_tflops": flops / (t_wall * 1e-3) / 1e12,
        "roofline": roofline(nbytes, t_out, "gsa_bf16_out" if bf16 else "gsa_seg_out", name),
        "op_roofline": op_roofline(nbytes, t_wall),
        "input_sets": nsets, "out": outs[0], "inp": inp,
    }
    res["mfma_frac_alg"] = res["alg_tflops"] / PEAK_BF16_TFLOPS
    if warm_too:
        wall_w, ph_w = time_op(torch, ev, call, sets[:1], steps, 2)
        res["warm_tokens_per_s"] = B * T * steps / wall_w
        res["warm_ms_op"] = round(mean([p[3] for p in ph_w]), 4)
    return res


def bench_gla(torch, gsa, ev, w, steps, warmup, name="gla_bf16_T4096"):
    import synth
    gate = "log_decay" if w.get("log_decay_scale") else "logit"
    inp = synth.gla_inputs(w["B"], w["H"], w["T"], w["dk"], w["dv"], dtype=w["dtype"], seed=0,
                           qkv_scale=w["qkv_scale"], log_decay_scale=w.get("log_decay_scale"))
    sets = dev_sets(torch, inp, ["q", "k", "v", "g"], 2)
    B, H, T, dk, dv = w["B"], w["H"], w["T"], w["dk"], w["dv"]
    outs = [torch.empty((B, H, T, dv), dtype=torch.bfloat16, device="cuda") for _ in sets]
    nb = gsa.gla_fwd_workspace_bytes(B, H, T, dk, dv, w["C"], 1, 0)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def call(s, events):
        i = next(j for j, x in enumerate(sets) if x is s)
        gsa.gla_fwd(s["q"], s["k"], s["v"], s["g"], tau=w["tau"], out=outs[i], workspace=ws,
                    events=events, gate=gate)

    wall, ph = time_op(torch, ev, call, sets, steps, warmup)
    flops, nbytes = gla_alg(B, H, T, dk, dv, w["C"], 2)
    t_op, t_out = mean([p[3] for p in ph]), mean([p[2] for p in ph])
    t_wall = wall / steps * 1e3
    return {"value": round(B * T * steps / wall, 1), "unit": "tokens/s",
            "ms_per_step": round(t_wall, 4),
            "ms_phases": {"state_maps": round(mean([p[0] for p in ph]), 4),
                          "scan": round(mean([p[1] for p in ph]), 4), "outputs": round(t_out, 4),
                          "op": round(t_op, 4)},
            "ms_op_stamped": stats([p[3] for p in ph]),
            "ms_out_kernel": stats([p[2] for p in ph]),
            "alg_tflops": round(flops / (t_wall * 1e-3) / 1e12, 2),
            "mfma_frac_alg": round(flops / (t_wall * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "roofline": roofline(nbytes, t_out, "gla_bf16_out", name),
            "op_roofline": op_roofline(nbytes, t_wall),
            "_inp": inp, "_out": outs[0]}


def bench_decode(torch, gsa, ev, w, steps, warmup, name="gsa_decode_N256"):
    import synth
    from synth import to_dev
    inp = synth.decode_inputs(w["N"], w["H"], w["dk"], w["dv"], w["m"], dtype=w["dtype"], seed=0,
                              qkv_scale=w["qkv_scale"], state_std=w["state_std"])
    tok = {n: to_dev(inp[n], torch) for n in "qkvg"}
    states = [(to_dev(inp["kstate"], torch), to_dev(inp["vstate"], torch)) for _ in range(2)]
    out = torch.empty((w["N"], w["H"], w["dv"]), dtype=torch.bfloat16, device="cuda")
    evs = ev.create(2 * steps)
    for i in range(warmup):
        ks, vs = states[i % 2]
        gsa.gsa_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], ks, vs, tau=w["tau"], out=out)
    torch.cuda.synchronize()
    quiesce()
    t0 = time.perf_counter()
    for i in range(steps):
        ks, vs = states[i % 2]
        gsa.gsa_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], ks, vs, tau=w["tau"], out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):  # the same steps with the kernel's dispatch stamps
        ks, vs = states[i % 2]
        gsa.gsa_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], ks, vs, tau=w["tau"], out=out,
                            events=evs[2 * i: 2 * i + 2])
    torch.cuda.synchronize()
    tk = [ev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)]
    t = mean(tk)
    units = w["N"] * w["H"]
    # both fp32 states read and written once, plus the bf16 token I/O (q, k, v, g in, o out)
    nbytes = units * (2 * 4 * w["m"] * (w["dk"] + w["dv"]) + 2 * (2 * w["dk"] + 2 * w["dv"] + w["m"]))
    r = roofline(nbytes, t, "gsa_decode_kernel", name)
    return {"value": r["achieved"], "unit": "GB/s", "ms_kernel": round(t, 4),
            "ms_kernel_stats": stats(tk), "steps_per_s": round(steps / wall, 1),
            "tokens_per_s": round(w["N"] * steps / wall, 1), "roofline": r, "_inp": inp}


def bench_gla_decode(torch, gsa, ev, steps, warmup):
    """The recurrent GLA step at the decode batch's shape (256 sequences x 16
    heads, d = 128, tau = 16): one fp32 state of 64 KB per unit read and
    written once, in place."""
    import synth
    from synth import to_dev
    N, H, d = 256, 16, 128
    inp = synth.gla_inputs(N, H, 1, d, d, dtype="bf16", seed=0, init_std=0.1)
    tok = {n: to_dev(inp[n], torch)[:, :, 0].contiguous() for n in "qkvg"}
    states = [to_dev(inp["s0"], torch) for _ in range(2)]
    out = torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda")
    evs = ev.create(2 * steps)
    for i in range(warmup):
        gsa.gla_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], states[i % 2], out=out)
    torch.cuda.synchronize()
    quiesce()
    t0 = time.perf_counter()
    for i in range(steps):
        gsa.gla_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], states[i % 2], out=out)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        gsa.gla_decode_step(tok["q"], tok["k"], tok["v"], tok["g"], states[i % 2], out=out,
                            events=evs[2 * i: 2 * i + 2])
    torch.cuda.synchronize()
    t = mean([ev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)])
    units = N * H
    nbytes = units * (2 * 4 * d * d + 2 * (4 * d))
    r = roofline(nbytes, t, "gla_decode_kernel", "gla_decode_N256")
    return {"value": r["achieved"], "unit": "GB/s", "ms_kernel": round(t, 4),
            "steps_per_s": round(steps / wall, 1), "roofline": r}


def bwd_cpu_oracle(w, inp, budget_s=3.0):
    """The oracle's backward (fp64, reverse-mode through the recurrence) on
    one thread over one (batch, head) unit of the batch, scaled to the batch's
    tokens/s (every unit costs the same)."""
    import oracle
    one = {n: inp[n].f64[:1, :1].copy() for n in ("q", "k", "v", "g", "do")}
    t0 = time.perf_counter()
    runs = 0
    while True:
        oracle.gsa_bwd(one["q"], one["k"], one["v"], one["g"], one["do"], tau=w["tau"], nthreads=1)
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(w["T"] * runs / dt / (w["B"] * w["H"]) * w["B"], 1), "unit": "tokens/s",
            "cores": 1, "kind": "oracle",
            "sample": "one (b,h) unit of the batch (T=%d), %d run(s) in %.1f s, scaled to B*T tokens "
                      "over B*H units" % (w["T"], runs, dt)}


def bwd_parity(torch, w, inp, grads):
    """Max over dq, dk, dv, dg of max |x - y| / max |y| on (batch, head)
    unit 0 of the benched call against the oracle's backward."""
    import oracle
    from synth import to_np
    torch.cuda.synchronize()
    one = {n: inp[n].f64[:1, :1] for n in ("q", "k", "v", "g", "do")}
    ref = oracle.gsa_bwd(one["q"], one["k"], one["v"], one["g"], one["do"], tau=w["tau"])
    return float("%.3e" % max(rel_err(to_np(x[:1, :1]), ref[n])
                               for x, n in zip(grads, ("dq", "dk", "dv", "dg"))))


def bench_bwd(torch, gsa, ev, w, steps, warmup, name="gsa_bf16_train_T2048_bwd", cpu=True, pair=True):
    """The GSA backward at a workload's shape (the training shape B8 H4 T2048
    bf16 with zero states, or the long-context one with initial states and
    final-state gradients), dO ~ N(0, 1); two input sets rotated."""
    import synth
    B, H, T, dk, dv, m = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"]
    inp = synth.gsa_inputs(B, H, T, dk, dv, m, dtype=w["dtype"], seed=0, qkv_scale=w["qkv_scale"],
                           g_shift=w["g_shift"], init_std=w["init_std"], fast_slots=w.get("fast_slots", 0),
                           fast_shift=w.get("fast_shift", 0.0))
    states = inp["k0"] is not None
    gi = synth.gsa_grad_inputs(B, H, T, dk, dv, m, dtype=w["dtype"], seed=1,
                               final_std=1.0 if states else None)
    inp["do"], inp["dkf"], inp["dvf"] = gi["do"], gi["dkf"], gi["dvf"]
    sets = dev_sets(torch, inp, ["q", "k", "v", "g", "do", "k0", "v0", "dkf", "dvf"], 2)
    outs = [tuple(torch.empty_like(s[n]) for n in "qkvg") for s in sets]
    ws = torch.empty(gsa.gsa_bwd_workspace_bytes(B, H, T, dk, dv, m, 1), dtype=torch.uint8, device="cuda")

    def call(s, events):
        i = next(j for j, x in enumerate(sets) if x is s)
        gsa.gsa_bwd(s["q"], s["k"], s["v"], s["g"], s["do"], s.get("k0"), s.get("v0"), s.get("dkf"),
                    s.get("dvf"), tau=w["tau"], out=outs[i], workspace=ws, events=events)

    wall, ph = time_op(torch, ev, call, sets, steps, warmup)
    t_f, t_r = mean([p[0] for p in ph]), mean([p[2] for p in ph])
    al = gsa_bwd_chunk_alg(B, H, T, dk, dv, m, w["C"], 2)
    nbytes = al["bytes"]
    kern, kb, t = ("bwd_bf16_fwd", al["bytes_fwd"], t_f) if t_f >= t_r else ("bwd_bf16_rev", al["bytes_rev"], t_r)
    t_op = wall / steps * 1e3
    fl = al["flops_fwd"] + al["flops_rev"]
    res = {"value": round(B * T * steps / wall, 1), "unit": "tokens/s",
           "ms_per_step": round(t_op, 4),
           "ms_kernels": {"bwd_bf16_fwd": round(t_f, 4), "bwd_bf16_rev": round(t_r, 4)},
           "ms_kernel_stats": {"bwd_bf16_fwd": stats([p[0] for p in ph]),
                               "bwd_bf16_rev": stats([p[2] for p in ph])},
           "kernel_alg_tflops": {"bwd_bf16_fwd": round(al["flops_fwd"] / (t_f * 1e-3) / 1e12, 2),
                                 "bwd_bf16_rev": round(al["flops_rev"] / (t_r * 1e-3) / 1e12, 2)},
           "roofline": dict(roofline(kb, t, kern, name),
                            basis="this kernel's algorithmic bytes (q, k, v, g, dO read and its gradients "
                                  "written once) over its mean dispatch time"),
           "op_roofline": op_roofline(nbytes, t_op),
           "mfma": {"alg_tflops": round(fl / (t_op * 1e-3) / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(fl / (t_op * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "basis": "the chunk form's algorithmic flops (causal halves) over the wall-clock step"}}
    if not pair:
        return res
    # one training step of the op as gsa_autograd runs it: the training forward
    # (keeping the segment start states), then the backward reading them
    o_buf = [torch.empty_like(s_["v"]) for s_ in sets]
    nbf = int(gsa.lib.gsa_fwd_train_workspace_bytes(B, H, T, dk, dv, m, 1))
    wsf = torch.empty(max(nbf, 1), dtype=torch.uint8, device="cuda")
    nst = gsa.gsa_train_states_bytes(B, H, T, dk, dv, m)
    st_buf = [torch.empty(max(nst, 1), dtype=torch.uint8, device="cuda") for _ in sets]

    def fwd_train(i):
        s_ = sets[i % len(sets)]
        gsa.gsa_fwd_train(s_["q"], s_["k"], s_["v"], s_["g"], s_.get("k0"), s_.get("v0"), tau=w["tau"],
                          out=o_buf[i % len(sets)], workspace=wsf, states=st_buf[i % len(sets)])

    def bwd_saved(i, events=None):
        s_ = sets[i % len(sets)]
        gsa.gsa_bwd_train(s_["q"], s_["k"], s_["v"], s_["g"], s_["do"], st_buf[i % len(sets)], s_.get("k0"),
                          s_.get("v0"), s_.get("dkf"), s_.get("dvf"), tau=w["tau"], out=outs[i % len(sets)],
                          workspace=ws, events=events)

    def train_step(i):
        fwd_train(i)
        bwd_saved(i)

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        quiesce()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    wall_train = timed(train_step)
    for i in range(len(sets)):  # states for every set, then the backward alone
        fwd_train(i)
    wall_saved = timed(bwd_saved)
    evs = ev.create(4 * steps)
    for i in range(steps):
        bwd_saved(i, evs[4 * i: 4 * i + 4])
    torch.cuda.synchronize()
    saved_f = mean([ev.ms(evs[4 * i], evs[4 * i + 1]) for i in range(steps)])
    saved_r = mean([ev.ms(evs[4 * i + 2], evs[4 * i + 3]) for i in range(steps)])
    res.update({
            "saved_states": {"value": round(B * T * steps / wall_saved, 1), "unit": "tokens/s",
                             "ms_per_step": round(wall_saved / steps * 1e3, 4),
                             "ms_kernels": {"bwd_bf16_fwd": round(saved_f, 4), "bwd_bf16_rev": round(saved_r, 4)},
                             "op_roofline": op_roofline(nbytes, wall_saved / steps * 1e3),
                             "states_bytes": nst,
                             "what": "gsa_bwd_train: the backward reading the segment start states "
                                     "gsa_fwd_train kept (no state maps or scan of its own)"},
            "train_step": {"value": round(B * T * steps / wall_train, 1), "unit": "tokens/s",
                           "ms_per_step": round(wall_train / steps * 1e3, 4),
                           "what": "gsa_fwd_train then gsa_bwd_train on the same batch, per step "
                                   "(what gsa_autograd runs)"},
            "cpu_oracle": bwd_cpu_oracle(w, inp) if cpu else None,
            "parity_rel_err": bwd_parity(torch, w, inp, outs[0]) if cpu else None})
    return res


def bench_bwd_saved_only(torch, gsa, w, steps, warmup):
    """The backward from a training forward's kept states alone (for profiler
    runs: one gsa_fwd_train per input set, then only gsa_bwd_train)."""
    import synth
    B, H, T, dk, dv, m = w["B"], w["H"], w["T"], w["dk"], w["dv"], w["m"]
    inp = synth.gsa_inputs(B, H, T, dk, dv, m, dtype=w["dtype"], seed=0, qkv_scale=w["qkv_scale"],
                           g_shift=w["g_shift"], init_std=w["init_std"])
    gi = synth.gsa_grad_inputs(B, H, T, dk, dv, m, dtype=w["dtype"], seed=1,
                               final_std=1.0 if inp["k0"] is not None else None)
    inp["do"], inp["dkf"], inp["dvf"] = gi["do"], gi["dkf"], gi["dvf"]
    sets = dev_sets(torch, inp, ["q", "k", "v", "g", "do", "k0", "v0", "dkf", "dvf"], 2)
    states = [gsa.gsa_fwd_train(s_["q"], s_["k"], s_["v"], s_["g"], s_.get("k0"), s_.get("v0"),
                                tau=w["tau"])[3] for s_ in sets]
    ws = torch.empty(gsa.gsa_bwd_workspace_bytes(B, H, T, dk, dv, m, 1), dtype=torch.uint8, device="cuda")
    outs = [tuple(torch.empty_like(s_[n]) for n in "qkvg") for s_ in sets]

    def step(i):
        s_ = sets[i % 2]
        gsa.gsa_bwd_train(s_["q"], s_["k"], s_["v"], s_["g"], s_["do"], states[i % 2], s_.get("k0"),
                          s_.get("v0"), s_.get("dkf"), s_.get("dvf"), tau=w["tau"], out=outs[i % 2], workspace=ws)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    quiesce()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return {"value": round(B * T * steps / wall, 1), "unit": "tokens/s", "ms_per_step": round(wall / steps * 1e3, 4)}


def bench_bwd_varlen(torch, gsa, ev, w, steps, warmup, name="gsa_bf16_serve_N256_bwd"):
    """The backward over the serving workload's packed batch (256 sequences x
    H16, log-uniform lengths), dO ~ N(0, 1): training on packed sequences of
    mixed lengths.  Tokens/s counts sequence tokens (sum of lengths)."""
    import synth
    lengths = synth.varlen_lengths(w["N"], w["len_lo"], w["len_hi"], seed=0)
    inp = synth.varlen_inputs(lengths, w["H"], w["dk"], w["dv"], w["m"], dtype=w["dtype"], seed=0,
                              qkv_scale=w["qkv_scale"], g_shift=w["g_shift"])
    inp["do"] = synth.varlen_grad_inputs(lengths, w["H"], w["dk"], w["dv"], w["m"], dtype=w["dtype"],
                                         seed=1)["do"]
    cu = inp["cu_seqlens"]
    H, dk, dv, m = w["H"], w["dk"], w["dv"], w["m"]
    total = int(cu[-1])
    sets = dev_sets(torch, inp, ["q", "k", "v", "g", "do"], 2)
    ws = torch.empty(gsa.gsa_bwd_varlen_workspace_bytes(cu, H, dk, dv, m), dtype=torch.uint8, device="cuda")

    def call(s_, events):
        gsa.gsa_bwd_varlen(s_["q"], s_["k"], s_["v"], s_["g"], s_["do"], cu, tau=w["tau"], workspace=ws,
                           events=events)

    wall, ph = time_op(torch, ev, call, sets, steps, warmup)
    t_f, t_r = mean([p[0] for p in ph]), mean([p[2] for p in ph])
    # per token-head the same work as the dense backward (one sequence's tokens)
    f_f, f_r, nbytes = gsa_bwd_alg(1, H, total, dk, dv, m, 2)
    kern, fl, t = ("bwd_walk_fwd", f_f, t_f) if t_f >= t_r else ("bwd_walk_rev", f_r, t_r)
    ach = fl / (t * 1e-3) / 1e12
    return {"value": round(total * steps / wall, 1), "unit": "tokens/s", "sequences": w["N"], "H": H,
            "tokens": total, "ms_per_step": round(wall / steps * 1e3, 4),
            "ms_kernels": {"bwd_walk_fwd": round(t_f, 4), "bwd_walk_rev": round(t_r, 4)},
            "roofline": {"bound": "alu", "achieved": round(ach, 2), "peak": PEAK_FP32_VALU_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(ach / PEAK_FP32_VALU_TFLOPS, 4),
                         "traffic": load_traffic(kern, name), "kernel": kern}}


def cpu_baseline(w, inp, budget_s):
    import oracle
    threads, host_cpus = cpu_threads()
    args = [inp[n].f64 for n in "qkvg"]
    ref = None
    t0 = time.perf_counter()
    runs = 0
    while True:
        ref = oracle.gsa_fwd(*args, tau=w["tau"], want_states=False, nthreads=threads)
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    tokens = w["B"] * w["T"] * runs
    # one thread on one (batch, head) unit of the same batch, scaled to the
    # batch's tokens/s (every unit costs the same)
    one = [a[:1, :1].copy() for a in args]
    t1 = time.perf_counter()
    runs1 = 0
    while True:
        oracle.gsa_fwd(*one, tau=w["tau"], want_states=False, nthreads=1)
        runs1 += 1
        if time.perf_counter() - t1 >= min(2.0, budget_s):
            break
    dt1 = time.perf_counter() - t1
    single = {"value": round(w["T"] * runs1 / dt1 / (w["B"] * w["H"]) * w["B"], 1), "cores": 1,
              "sample": "one (b,h) unit of the batch (T=%d), %d run(s) in %.1f s, scaled to B*T tokens "
                        "over B*H units" % (w["T"], runs1, dt1)}
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads,
            "host_cpu_count": host_cpus, "kind": "oracle",
            "sample": "full %s batch (B=%d H=%d T=%d), %d run(s) in %.1f s, fp64 recurrence, "
                      "OpenMP over (b,h) units on the %d CPUs this process may use" % (
                          "training-shape", w["B"], w["H"], w["T"], runs, dt, threads),
            "single_thread": single}, ref


def oracle_gsa_sample(w, inp, out, budget_s):
    """The oracle's forward on one thread over (batch, head) unit 0 of a GSA
    workload (its initial state included), scaled to the batch's tokens/s
    (every unit costs the same); and the device output of that unit against
    it."""
    import oracle
    from synth import to_np
    one = {n: (None if inp[n] is None else inp[n].f64[:1, :1].copy()) for n in ("q", "k", "v", "g", "k0", "v0")}
    ref = {}

    def run():
        ref["o"] = oracle.gsa_fwd(one["q"], one["k"], one["v"], one["g"], one["k0"], one["v0"],
                                  tau=w["tau"], want_states=False, nthreads=1)["o"]
    runs, dt = timed_runs(run, budget_s)
    return {"value": round(w["T"] * runs / dt / (w["B"] * w["H"]) * w["B"], 1), "unit": "tokens/s",
            "cores": 1, "kind": "oracle",
            "sample": "one (b,h) unit (T=%d) on one thread, %d run(s) in %.1f s, scaled to B*T tokens "
                      "over B*H units" % (w["T"], runs, dt),
            "parity_rel_err_unit0": float("%.3e" % rel_err(to_np(out[:1, :1]), ref["o"]))}


def oracle_gla_sample(w, inp, out, budget_s):
    """As oracle_gsa_sample for the GLA workload."""
    import oracle
    from synth import to_np
    one = {n: inp[n].f64[:1, :1].copy() for n in "qkvg"}
    gate = "log_decay" if w.get("log_decay_scale") else "logit"
    ref = {}

    def run():
        ref["o"] = oracle.gla_fwd(one["q"], one["k"], one["v"], one["g"], tau=w["tau"],
                                  want_state=False, nthreads=1, gate=gate)["o"]
    runs, dt = timed_runs(run, budget_s)
    return {"value": round(w["T"] * runs / dt / (w["B"] * w["H"]) * w["B"], 1), "unit": "tokens/s",
            "cores": 1, "kind": "oracle",
            "sample": "one (b,h) unit (T=%d) on one thread, %d run(s) in %.1f s, scaled to B*T tokens "
                      "over B*H units" % (w["T"], runs, dt),
            "parity_rel_err_unit0": float("%.3e" % rel_err(to_np(out[:1, :1]), ref["o"]))}


def oracle_decode_sample(w, inp, budget_s, nseq=4):
    """The oracle's decode step on one thread over the first nseq sequences
    (x all heads) of the decode batch, scaled to whole-batch steps/s."""
    import oracle
    sl = {n: inp[n].f64[:nseq].copy() for n in ("q", "k", "v", "g", "kstate", "vstate")}

    def run():
        oracle.gsa_decode_step(sl["q"], sl["k"], sl["v"], sl["g"], sl["kstate"], sl["vstate"],
                               tau=w["tau"], nthreads=1)
    runs, dt = timed_runs(run, budget_s)
    return {"value": round(runs / dt * nseq / w["N"], 2), "unit": "steps/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d of %d sequences x H%d on one thread, %d run(s) in %.1f s, scaled to the "
                      "whole batch" % (nseq, w["N"], w["H"], runs, dt)}


def bench_small_f32(torch, gsa, ev, steps, warmup, budget_s):
    """The small float32 workload (B1 H2 T256 d64 m32): launch-latency bound,
    timed for completeness with the full-batch oracle beside it."""
    import oracle
    import synth
    from synth import to_np
    w = synth.WORKLOADS["gsa_f32_small"]
    r = bench_gsa(torch, gsa, ev, w, "gsa_f32_small", steps, warmup, 2, warm_too=False)
    args = [r["inp"][n].f64 for n in "qkvg"]
    ref = {}

    def run():
        ref["o"] = oracle.gsa_fwd(*args, tau=w["tau"], want_states=False, nthreads=1)["o"]
    runs, dt = timed_runs(run, budget_s)
    return {"value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(r["ms_per_step"], 4), "ms_op_stamped": r["ms_op_stamped"],
            "note": "launch-latency bound: no roofline claim",
            "parity_rel_err": float("%.3e" % rel_err(to_np(r["out"]), ref["o"])),
            "cpu_oracle": {"value": round(w["B"] * w["T"] * runs / dt, 1), "unit": "tokens/s",
                           "cores": 1, "kind": "oracle",
                           "sample": "the full batch, %d run(s) in %.1f s" % (runs, dt)}}


def environment(torch):
    """Where the numbers were taken: GPU arch, ROCm/HIP, torch, and the
    sources (git commit when a checkout is present, else a content hash)."""
    import subprocess
    props = torch.cuda.get_device_properties(0)
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(path):
            rocm = open(path).read().strip()
            break
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10).stdout.strip() or None
    except Exception:
        sha = None
    return {"gpu": props.name, "gfx_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm, "hip": torch.version.hip,
            "torch": torch.__version__, "git_sha": sha, "source_sha": source_sha()}


def source_sha():
    """Hash of the committed sources this run executes (kernels, ABI header,
    binding, bench)."""
    h = hashlib.sha256()
    paths = [os.path.join(ROOT, "include", "gsa.h"), os.path.join(ROOT, "bench.py"),
             os.path.join(ROOT, "slot_memory_sequence_amd", "__init__.py")]
    csrc = os.path.join(ROOT, "slot_memory_sequence_amd", "csrc")
    paths += [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    for pth in paths:
        h.update(open(pth, "rb").read())
    return h.hexdigest()[:16]


def copy_calibration(torch, ev, steps):
    """A plain device copy of known size (512 MiB read + 512 MiB written), the
    reference for scaling the profiler's FETCH_SIZE / WRITE_SIZE counters."""
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream
    evs = ev.create(2 * steps)
    for i in range(steps):
        ev.record(evs[2 * i], stream)
        dst.copy_(src)
        ev.record(evs[2 * i + 1], stream)
    torch.cuda.synchronize()
    t = mean([ev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)])
    return {"workload": "copy_512MiB", "bytes_read": n, "bytes_written": n, "ms": round(t, 4),
            "GBps": round(2 * n / (t * 1e-3) / 1e9, 1)}


def bench_serve(torch, gsa, ev, w, steps, warmup):
    """The serving path: the prefill of 256 prompts of mixed lengths as one
    packed variable-length call (final states written), then decode steps of
    all 256 x H units from those states.  Prefill tokens/s counts prompt
    tokens (sum of lengths) per second."""
    import synth
    from synth import to_dev
    lengths = synth.varlen_lengths(w["N"], w["len_lo"], w["len_hi"], seed=0)
    inp = synth.varlen_inputs(lengths, w["H"], w["dk"], w["dv"], w["m"], dtype=w["dtype"], seed=0,
                              qkv_scale=w["qkv_scale"], g_shift=w["g_shift"])
    cu = inp["cu_seqlens"]
    n, H, dk, dv, m = w["N"], w["H"], w["dk"], w["dv"], w["m"]
    total = int(cu[-1])
    sets = dev_sets(torch, inp, ["q", "k", "v", "g"], 2)
    outs = [torch.empty((H, total, dv), dtype=torch.bfloat16, device="cuda") for _ in sets]
    kfs = [torch.empty((n, H, m, dk), dtype=torch.float32, device="cuda") for _ in sets]
    vfs = [torch.empty((n, H, m, dv), dtype=torch.float32, device="cuda") for _ in sets]
    nb = gsa.gsa_fwd_varlen_workspace_bytes(cu, H, dk, dv, m)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

    def call(s, events):
        i = next(j for j, x in enumerate(sets) if x is s)
        gsa.gsa_fwd_varlen(s["q"], s["k"], s["v"], s["g"], cu, tau=w["tau"], final_state=True,
                           out=outs[i], k_final=kfs[i], v_final=vfs[i], workspace=ws, events=events)

    wall, ph = time_op(torch, ev, call, sets, steps, warmup)
    # each prompt token-head: q, k, v, g read and o written once; final states written once
    nbytes = H * total * (2 * dk + 2 * dv + m) * 2 + n * H * m * (dk + dv) * 4
    t_op, t_out = mean([p[3] for p in ph]), mean([p[2] for p in ph])
    # decode steps from the prefill's final states (one new token per sequence)
    tok = synth.decode_inputs(n, H, dk, dv, m, dtype=w["dtype"], seed=1, qkv_scale=w["qkv_scale"])
    td = {x: to_dev(tok[x], torch) for x in "qkvg"}
    ks, vs = kfs[0], vfs[0]
    dout = torch.empty((n, H, dv), dtype=torch.bfloat16, device="cuda")
    devs = ev.create(2 * steps)
    for i in range(steps):
        gsa.gsa_decode_step(td["q"], td["k"], td["v"], td["g"], ks, vs, tau=w["tau"], out=dout,
                            events=devs[2 * i: 2 * i + 2])
    torch.cuda.synchronize()
    t_dec = mean([ev.ms(devs[2 * i], devs[2 * i + 1]) for i in range(steps)])
    dec_bytes = n * H * (2 * 4 * m * (dk + dv) + 2 * (2 * dk + 2 * dv + m))
    return {"value": round(total * steps / wall, 1), "unit": "prompt tokens/s",
            "prompts": n, "H": H, "prompt_tokens": total, "len_min": min(lengths),
            "len_max": max(lengths), "ms_per_prefill": round(wall / steps * 1e3, 4),
            "ms_phases": {"state_maps": round(mean([p[0] for p in ph]), 4),
                          "scan": round(mean([p[1] for p in ph]), 4), "outputs": round(t_out, 4),
                          "op": round(t_op, 4)},
            "roofline": roofline(nbytes, t_out, "gsa_bf16_out", "gsa_bf16_serve_N256"),
            "decode_ms_kernel": round(t_dec, 4),
            "decode_roofline": roofline(dec_bytes, t_dec, "gsa_decode_kernel", "gsa_decode_N256")}


def bench_ablations(torch, gsa, ev, steps, warmup, nsets):
    """The training-shape GSA forward with each element-wise slot read of the
    ablation study in place of the softmax (same launch sequence; only the
    read inside the output kernel differs)."""
    import synth
    w = synth.WORKLOADS["gsa_bf16_train_T2048"]
    out = {}
    for nl in ("identity", "swish", "relu", "relu2"):
        r = bench_gsa(torch, gsa, ev, w, "gsa_bf16_train_T2048", steps, warmup, nsets,
                      warm_too=False, nonlinearity=nl)
        rf = dict(r["roofline"])
        rf["traffic"] = None  # counters are taken on the softmax kernel only
        out[nl] = {"value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
                   "ms_per_step": round(r["ms_per_step"], 4), "ms_phases": r["ms_phases"],
                   "roofline": rf}
        del r
    return out


def measure_peaks(torch, gsa, ev, reps=20):
    """What this GPU sustains, with the library's own calibration kernels: a
    streaming copy of 1 GiB and an in-place update of 1 GiB (bytes read +
    written per second; the forward kernels read their inputs and write
    elsewhere, the decode step updates its states in place), and a
    register-only bf16 MFMA loop (dense flops per second).  Median and best of
    `reps` event-timed runs after warm-up."""
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for name, args in (("copy", (dst, src)), ("update", (dst,))):
        evs = ev.create(2 * reps)
        for _ in range(5):
            gsa.measure_hbm(*args)
        for i in range(reps):
            gsa.measure_hbm(*args, events=evs[2 * i: 2 * i + 2])
        torch.cuda.synchronize()
        t = sorted(ev.ms(evs[2 * i], evs[2 * i + 1]) for i in range(reps))
        out["hbm_%s_GBps" % name] = round(2 * n / (t[len(t) // 2] * 1e-3) / 1e9, 1)
        out["hbm_%s_GBps_best" % name] = round(2 * n / (t[0] * 1e-3) / 1e9, 1)
    del src, dst
    out["hbm_GBps"] = max(out["hbm_copy_GBps"], out["hbm_update_GBps"])
    iters = 10000
    sink, flops = gsa.measure_mfma_bf16(iters)
    for _ in range(3):
        gsa.measure_mfma_bf16(iters, sink=sink)
    evm = ev.create(2 * reps)
    for i in range(reps):
        gsa.measure_mfma_bf16(iters, sink=sink, events=evm[2 * i: 2 * i + 2])
    torch.cuda.synchronize()
    tm = sorted(ev.ms(evm[2 * i], evm[2 * i + 1]) for i in range(reps))
    out["mfma_bf16_TFLOPs"] = round(flops / (tm[len(tm) // 2] * 1e-3) / 1e12, 1)
    out["mfma_bf16_TFLOPs_best"] = round(flops / (tm[0] * 1e-3) / 1e12, 1)
    out["mfma_check"] = bool(torch.all(sink == 1024.0 * iters + 496.0).item())
    out["kernels"] = ("gsa_measure_hbm (1 GiB copy / in-place update, non-temporal float4, 32 KB "
                      "per workgroup), gsa_measure_mfma_bf16 (16x16x32, 8 chains/wave, 4 waves/SIMD)")
    torch.cuda.empty_cache()
    return out


def with_measured(rf, peaks):
    """A roofline record with the fraction of the measured peak beside the
    published one's."""
    if rf and peaks and rf.get("unit") == "GB/s":
        rf = dict(rf)
        rf["frac_of_measured"] = round(rf["achieved"] / peaks["hbm_GBps"], 4)
    return rf


# the training shape with a set of fast-forgetting slots, one decay regime each
FORGET_WORKLOADS = (
    ("gsa_bf16_train_T2048_fast_forget",
     "the training shape with 8 of 64 slots at gate logits N(-6, 1): 64-token decay "
     "products near 2^-69, inside the chunk form's range"),
    ("gsa_bf16_train_T2048_rapid_forget",
     "the training shape with 8 of 64 slots at gate logits N(-10, 1): 64-token decay "
     "products near 2^-115, below the chunk form's range (every chunk in the 16-token "
     "sub-chunk form)"),
    ("gsa_bf16_train_T2048_extreme_forget",
     "the training shape with 8 of 64 slots at gate logits N(-40, 1): 16-token decay "
     "products near 2^-115, below the sub-chunk form's range too (every chunk an exact walk)"))


def run_only(args, torch, gsa, ev):
    import synth
    if args.only == "rapid":
        w = synth.WORKLOADS["gsa_bf16_train_T2048_rapid_forget"]
        r = bench_gsa(torch, gsa, ev, w, "gsa_bf16_train_T2048_rapid_forget", args.steps, args.warmup, args.sets,
                      warm_too=False)
        return {k: r[k] for k in ("tokens_per_s", "ms_per_step", "ms_phases", "roofline")}
    if args.only == "bwd_rapid":
        return bench_bwd(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_train_T2048_rapid_forget"], args.steps,
                         args.warmup, name="gsa_bf16_train_T2048_rapid_forget_bwd", cpu=False, pair=False)
    if args.only == "bwd_forget":
        return {fname + "_bwd": bench_bwd(torch, gsa, ev, synth.WORKLOADS[fname], args.steps, args.warmup,
                                          name=fname + "_bwd", cpu=False)
                for fname, _ in FORGET_WORKLOADS[1:]}
    if args.only == "forget":
        out = {}
        for fname, _ in FORGET_WORKLOADS:
            r = bench_gsa(torch, gsa, ev, synth.WORKLOADS[fname], fname, args.steps, args.warmup, args.sets,
                          warm_too=False)
            out[fname] = {k: r[k] for k in ("tokens_per_s", "ms_per_step", "ms_phases")}
        return out
    if args.only == "copy":
        return copy_calibration(torch, ev, args.steps)
    if args.only == "peaks":
        return measure_peaks(torch, gsa, ev)
    if args.only == "gsa":
        r = bench_gsa(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_train_T2048"], "gsa_bf16_train_T2048",
                      args.steps, args.warmup, args.sets, warm_too=False)
        return {k: r[k] for k in ("tokens_per_s", "ms_per_step", "ms_phases", "roofline")}
    if args.only == "long":
        r = bench_gsa(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_long_T16384"], "gsa_bf16_long_T16384",
                      args.steps, args.warmup, 3, warm_too=False)
        return {k: r[k] for k in ("tokens_per_s", "ms_per_step", "ms_phases", "roofline")}
    if args.only == "bwd_long":
        return bench_bwd(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_long_T16384"], args.steps,
                         args.warmup, name="gsa_bf16_long_T16384_bwd", cpu=False, pair=False)
    if args.only == "bwd_serve":
        return bench_bwd_varlen(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_serve_N256"], args.steps,
                                args.warmup)
    if args.only == "bwd_saved":
        return bench_bwd_saved_only(torch, gsa, synth.WORKLOADS["gsa_bf16_train_T2048"], args.steps, args.warmup)
    if args.only == "bwd_long_saved":
        return bench_bwd_saved_only(torch, gsa, synth.WORKLOADS["gsa_bf16_long_T16384"], args.steps, args.warmup)
    if args.only == "bwd":
        return bench_bwd(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_train_T2048"], args.steps,
                         args.warmup, cpu=False, pair=False)
    if args.only == "gla_decode":
        return bench_gla_decode(torch, gsa, ev, args.steps, args.warmup)
    if args.only == "m128":
        r = bench_gsa(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_train_T2048_m128"], "gsa_bf16_train_T2048_m128",
                      args.steps, args.warmup, args.sets, warm_too=False)
        return {k: r[k] for k in ("tokens_per_s", "ms_per_step", "ms_phases", "roofline")}
    if args.only == "bwd_m128":
        return bench_bwd(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_train_T2048_m128"], args.steps,
                         args.warmup, name="gsa_bf16_train_T2048_m128_bwd", cpu=False, pair=False)
    if args.only == "decode_m128":
        r = bench_decode(torch, gsa, ev, synth.WORKLOADS["gsa_decode_N256_m128"], args.steps, args.warmup,
                         name="gsa_decode_N256_m128")
        r.pop("_inp")
        return r
    if args.only == "serve":
        return bench_serve(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_serve_N256"], args.steps,
                           args.warmup)
    if args.only == "ablations":
        return bench_ablations(torch, gsa, ev, args.steps, args.warmup, args.sets)
    if args.only == "gla":
        return bench_gla(torch, gsa, ev, synth.WORKLOADS["gla_bf16_T4096"], args.steps, args.warmup)
    if args.only == "gla_log_decay":
        return bench_gla(torch, gsa, ev, synth.WORKLOADS["gla_bf16_T4096_log_decay"], args.steps,
                         args.warmup, "gla_bf16_T4096_log_decay")
    return bench_decode(torch, gsa, ev, synth.WORKLOADS["gsa_decode_N256"], args.steps, args.warmup)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=6, help="input copies rotated through (cache-cold)")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["gsa", "long", "gla", "gla_log_decay", "decode", "copy", "ablations", "serve",
                             "peaks", "gla_decode", "bwd", "bwd_serve", "bwd_long", "m128", "bwd_m128", "decode_m128", "bwd_saved", "bwd_long_saved", "forget", "bwd_forget",
                             "rapid", "bwd_rapid"],
                    default=None,
                    help="run one workload and print its record (for profiler runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark runs on exactly one GPU (the workload is one GPU's share; "
              "nothing here uses collectives). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import slot_memory_sequence_amd as gsa
    import synth
    from synth import to_np

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gc.disable()  # collections run at the start of each timed region (quiesce)
    ev = Events()
    if args.only is not None:
        rec = run_only(args, torch, gsa, ev)
        if isinstance(rec, dict):  # the records' private entries (inputs, outputs) stay out
            rec = {k: v for k, v in rec.items() if not k.startswith("_")}
        print(json.dumps(rec), flush=True)
        return
    wname = "gsa_bf16_train_T2048"
    w = synth.WORKLOADS[wname]
    log("bench: %s steps=%d warmup=%d sets=%d" % (wname, args.steps, args.warmup, args.sets))
    main_res = bench_gsa(torch, gsa, ev, w, wname, args.steps, args.warmup, args.sets)
    log("bench: main done %.3g tokens/s" % main_res["tokens_per_s"])

    comps = {}
    ocpu = 0.0 if args.no_cpu else max(1.0, args.cpu_seconds / 5)  # per sampled oracle timing
    if not args.no_components:
        wl = synth.WORKLOADS["gsa_bf16_long_T16384"]
        r = bench_gsa(torch, gsa, ev, wl, "gsa_bf16_long_T16384", args.steps, args.warmup, 3,
                      warm_too=False)
        comps["gsa_bf16_long_T16384"] = {
            "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(r["ms_per_step"], 4), "ms_phases": r["ms_phases"],
            "ms_op_stamped": r["ms_op_stamped"],
            "alg_tflops": round(r["alg_tflops"], 2), "mfma_frac_alg": round(r["mfma_frac_alg"], 4),
            "roofline": r["roofline"], "op_roofline": r["op_roofline"],
            "cpu_oracle": oracle_gsa_sample(wl, r["inp"], r["out"], ocpu) if ocpu else None}
        del r
        log("bench: long-context done")
        for fname, what in FORGET_WORKLOADS:
            wf = synth.WORKLOADS[fname]
            r = bench_gsa(torch, gsa, ev, wf, fname, args.steps, args.warmup, args.sets,
                          warm_too=False)
            comps[fname] = {
                "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
                "vs_headline": round(r["tokens_per_s"] / main_res["tokens_per_s"], 4),
                "what": what,
                "ms_per_step": round(r["ms_per_step"], 4), "ms_phases": r["ms_phases"],
                "ms_op_stamped": r["ms_op_stamped"], "roofline": r["roofline"],
                "op_roofline": r["op_roofline"],
                "cpu_oracle": oracle_gsa_sample(wf, r["inp"], r["out"], ocpu) if ocpu else None}
            del r
        log("bench: fast-forgetting slots done")
        # 128 slots: the forward (two slot groups and their merge), decode, backward
        wm = synth.WORKLOADS["gsa_bf16_train_T2048_m128"]
        r = bench_gsa(torch, gsa, ev, wm, "gsa_bf16_train_T2048_m128", args.steps, args.warmup, args.sets,
                      warm_too=False)
        comps["gsa_bf16_train_T2048_m128"] = {
            "value": round(r["tokens_per_s"], 1), "unit": "tokens/s",
            "vs_m64": round(r["tokens_per_s"] / main_res["tokens_per_s"], 4),
            "ms_per_step": round(r["ms_per_step"], 4), "ms_phases": r["ms_phases"],
            "ms_op_stamped": r["ms_op_stamped"], "roofline": r["roofline"], "op_roofline": r["op_roofline"],
            "alg_tflops": round(r["alg_tflops"], 2),
            "cpu_oracle": oracle_gsa_sample(wm, r["inp"], r["out"], ocpu) if ocpu else None}
        del r
        comps["gsa_decode_N256_m128"] = bench_decode(torch, gsa, ev, synth.WORKLOADS["gsa_decode_N256_m128"],
                                                     args.steps, args.warmup, name="gsa_decode_N256_m128")
        comps["gsa_decode_N256_m128"].pop("_inp")
        log("bench: 128 slots forward and decode done")
        r = bench_gla(torch, gsa, ev, synth.WORKLOADS["gla_bf16_T4096"], args.steps, args.warmup)
        gi, go = r.pop("_inp"), r.pop("_out")
        r["cpu_oracle"] = oracle_gla_sample(synth.WORKLOADS["gla_bf16_T4096"], gi, go, ocpu) if ocpu else None
        comps["gla_bf16_T4096"] = r
        del gi, go
        log("bench: gla done")
        r = bench_gla(torch, gsa, ev, synth.WORKLOADS["gla_bf16_T4096_log_decay"],
                      max(1, args.steps // 2), args.warmup, "gla_bf16_T4096_log_decay")
        r.pop("_inp"), r.pop("_out")
        comps["gla_bf16_T4096_log_decay"] = r
        log("bench: gla with log-decay gates done")
        r = bench_decode(torch, gsa, ev, synth.WORKLOADS["gsa_decode_N256"], args.steps, args.warmup)
        di = r.pop("_inp")
        r["cpu_oracle"] = oracle_decode_sample(synth.WORKLOADS["gsa_decode_N256"], di, ocpu) if ocpu else None
        comps["gsa_decode_N256"] = r
        del di
        log("bench: decode done")
        comps["gsa_f32_small"] = bench_small_f32(torch, gsa, ev, args.steps, args.warmup, ocpu or 0.2)
        log("bench: small fp32 done")
        comps["gla_decode_N256"] = bench_gla_decode(torch, gsa, ev, args.steps, args.warmup)
        log("bench: GLA decode done")
        comps["gsa_bf16_train_T2048_bwd"] = bench_bwd(torch, gsa, ev, w, max(1, args.steps // 4),
                                                      args.warmup, cpu=not args.no_cpu)
        log("bench: backward done")
        comps["gsa_bf16_serve_N256_bwd"] = bench_bwd_varlen(
            torch, gsa, ev, synth.WORKLOADS["gsa_bf16_serve_N256"], max(1, args.steps // 4), args.warmup)
        log("bench: packed-batch backward done")
        comps["gsa_bf16_long_T16384_bwd"] = bench_bwd(
            torch, gsa, ev, synth.WORKLOADS["gsa_bf16_long_T16384"], max(1, args.steps // 4), args.warmup,
            name="gsa_bf16_long_T16384_bwd", cpu=False)
        log("bench: long-context backward done")
        for fname, what in FORGET_WORKLOADS[1:]:
            r = bench_bwd(torch, gsa, ev, synth.WORKLOADS[fname], max(1, args.steps // 4), args.warmup,
                          name=fname + "_bwd", cpu=False)
            r["what"] = "the backward (and a training step) on " + what
            comps[fname + "_bwd"] = r
        log("bench: fast-forgetting backward done")
        comps["gsa_bf16_train_T2048_m128_bwd"] = bench_bwd(
            torch, gsa, ev, synth.WORKLOADS["gsa_bf16_train_T2048_m128"], max(1, args.steps // 4), args.warmup,
            name="gsa_bf16_train_T2048_m128_bwd", cpu=False)
        log("bench: 128-slot backward done")
        comps["gsa_bf16_serve_N256"] = bench_serve(torch, gsa, ev, synth.WORKLOADS["gsa_bf16_serve_N256"],
                                                   max(1, args.steps // 2), args.warmup)
        log("bench: serving prefill + decode done")
        torch.cuda.empty_cache()
        comps["gsa_bf16_train_T2048_read_ablations"] = bench_ablations(
            torch, gsa, ev, max(1, args.steps // 2), args.warmup, args.sets)
        log("bench: read ablations done")
        torch.cuda.empty_cache()

    peaks = measure_peaks(torch, gsa, ev)
    log("bench: measured peaks %s" % peaks)
    main_res["roofline"] = with_measured(main_res["roofline"], peaks)
    main_res["op_roofline"] = with_measured(main_res["op_roofline"], peaks)
    for c in comps.values():
        for key in ("roofline", "op_roofline", "decode_roofline"):
            if key in c:
                c[key] = with_measured(c[key], peaks)
        if "identity" in c:  # the read ablations
            for v in c.values():
                v["roofline"] = with_measured(v["roofline"], peaks)

    cpu, err = None, None
    if not args.no_cpu:
        cpu, ref = cpu_baseline(w, main_res["inp"], args.cpu_seconds)
        err = rel_err(to_np(main_res["out"]), ref["o"])
        log("bench: cpu baseline done, parity rel err %.3e" % err)

    line = {
        "metric": "GSA fwd tokens/s (B*T/s) at T=2048; % bf16 MFMA peak; decode HBM GB/s",
        "value": round(main_res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q,k,v scaled 1/sqrt(128), gate logits N(0,1))",
        "config": {"workload": wname, "B": w["B"], "H": w["H"], "T": w["T"], "dk": w["dk"],
                   "dv": w["dv"], "m": w["m"], "C": w["C"], "tau": w["tau"],
                   "input_sets_rotated": main_res["input_sets"]},
        "roofline": main_res["roofline"],
        "op_roofline": main_res["op_roofline"],
        "ms_phases": main_res["ms_phases"],
        "ms_op_stamped": main_res["ms_op_stamped"],
        "ms_out_kernel": main_res["ms_out_kernel"],
        "alg_tflops": round(main_res["alg_tflops"], 2),
        "mfma_frac_alg": round(main_res["mfma_frac_alg"], 4),
        "mfma": {"alg_tflops": round(main_res["alg_tflops"], 2), "peak": PEAK_BF16_TFLOPS,
                 "unit": "TFLOP/s", "frac": round(main_res["mfma_frac_alg"], 4),
                 "basis": "algorithmic flops (causal halves) over the wall-clock step"},
        "warm_cache_tokens_per_s": round(main_res.get("warm_tokens_per_s", 0.0), 1),
        "decode_GBps": comps.get("gsa_decode_N256", {}).get("value"),
        "measured_peaks": peaks,
        "components": comps,
        "cpu_baseline": cpu,
        "parity_rel_err": None if err is None else float("%.3e" % err),
        "kernel_source_sha": kernel_source_sha(),
        "environment": environment(torch),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
