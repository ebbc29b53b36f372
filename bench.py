#!/usr/bin/env python3
"""Benchmark of the integer training step on one MI355X.

Main line: the large int8 Linear training step (tokens 8192, in 4096,
out 4096): forward, dgrad and wgrad contractions (each 8192x4096x4096,
int8 x int8 -> int32, with the fused max-abs) and the NITI update of the
16.8M weights.  Throughput counts 2*M*N*K ops per contraction (824.6 G int8
ops per step); requantisation and update ALU work is not counted.  Inputs are
seeded synthetic tensors with the workload's distributions, resident in HBM
before the timed region.

Timing protocol: --warmup W steps, then untimed steps until the clocks have
left their idle state (at least --settle-s seconds and two consecutive K-step
windows within 1%; the first K-step window after the W steps is reported
beside it), then K steps between one HIP event pair (the reported step time),
K steps with an event pair each (median and minimum), and K steps with every
launch bracketed by events (per-kernel averages, the roofline figure; an
event between two kernels makes the first end with a system-scope release,
so these steps run slightly slower).  Socket power, the power-limit
residency and the graphics clock are read from the driver's metrics over a
few seconds of back-to-back steps.  The NITI update is also timed on its
own, with the last-level cache flushed before every launch and warm.

Also reported: the single-layer and MLP workloads (latency-bound), the
oracle (plain C, CPU) timed on bounded samples of the large step on this
host with every thread and with one, and secondary measurements of the conv,
DFP-16, offsets, model-driver and adaptive-precision paths.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-s S]
       [--power-window-s P] [--no-secondary] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
PEAK_INT8_TOPS = 5000.0     # MI355X dense int8 matrix peak (5.0 POP/s)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_VALU_TOPS = 39.32      # 256 CUs x 4 SIMDs x 16 int32 lane-ops per cycle x 2.4 GHz
T, IN, OUT = 8192, 4096, 4096


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="after the --warmup steps, keep stepping (untimed) for at least this long and "
                         "until two consecutive K-step windows agree within 1%%: the clocks leave their "
                         "idle state over the first tens of milliseconds")
    ap.add_argument("--power-window-s", type=float, default=3.2,
                    help="seconds of back-to-back steps over which socket power, power-limit residency "
                         "and the graphics clock are read (0: skip)")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run a read-only and a write-only streaming kernel over 256 MiB "
                         "(scale for the HBM byte counters)")
    ap.add_argument("--cpu-sample-rows", type=int, default=1024,
                    help="token rows of the workload the CPU oracle runs on all host threads")
    ap.add_argument("--cpu-sample-rows-1t", type=int, default=64,
                    help="token rows of the workload the CPU oracle runs on one thread")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """HIP events on the current stream around named launches."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self, name):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append((name, e))

    def per_name(self):
        out = {}
        for (name, e0), (_, e1) in zip(self.marks, self.marks[1:]):
            if name is None:
                continue
            out.setdefault(name, []).append(e0.elapsed_time(e1))
        return out


class PowerMonitor:
    """Socket power, power-limit residency and graphics clock of the GPU from
    the driver's metrics table (amdsmi).  The table is refreshed about once a
    second; its energy accumulator, firmware timestamp (10 ns units), PPT
    (package power tracking) residency and accumulation counter (1 ms units)
    are exact between two refreshes, so averages are taken over whole
    refresh intervals.  Unavailable (None) when amdsmi cannot read the
    device."""

    def __init__(self, torch):
        self.h = None
        self.err = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            want = None
            try:
                p = torch.cuda.get_device_properties(0)
                want = "%04x:%02x:%02x" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
            except Exception:
                pass
            for h in hs:
                if want is None or amdsmi.amdsmi_get_gpu_device_bdf(h).lower().startswith(want):
                    self.h = h
                    break
            if self.h is None and len(hs) == 1:
                self.h = hs[0]
            self.amdsmi = amdsmi
            if self.h is None:
                self.err = f"no amdsmi handle matches the device ({want})"
        except Exception as e:   # no amdsmi, no permission: report the reason
            self.err = repr(e)

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, int) and c > 0]
        return dict(t=time.perf_counter(), fw=m.get("firmware_timestamp"), energy=m.get("energy_accumulator"),
                    acc=m.get("accumulation_counter"), ppt=m.get("ppt_residency_acc"),
                    clk=float(np.mean(clks)) if clks else None, clks=clks,
                    power=m.get("current_socket_power"))

    def static(self):
        out = {}
        try:
            cap = self.amdsmi.amdsmi_get_power_cap_info(self.h)
            out["power_cap_w"] = round(cap["power_cap"] / 1e6, 1)
        except Exception as e:
            out["power_cap_w"] = None
            out["power_cap_error"] = repr(e)
        try:
            ci = self.amdsmi.amdsmi_get_clock_info(self.h, self.amdsmi.AmdSmiClkType.GFX)
            out["gfxclk_max_mhz"] = ci.get("max_clk")
        except Exception:
            out["gfxclk_max_mhz"] = None
        try:
            out["energy_resolution_uj"] = float(self.amdsmi.amdsmi_get_energy_count(self.h)["counter_resolution"])
        except Exception:
            out["energy_resolution_uj"] = 15.3
        return out

    def window(self, step, torch, seconds):
        """Run step() back to back for `seconds` while sampling the metrics
        table every 2 ms; average power (energy / firmware time), PPT
        residency and the graphics clock over the refresh intervals that lie
        wholly inside the stepping."""
        import threading
        st = self.static()
        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                try:
                    samples.append(self.read())
                except Exception:
                    pass
                time.sleep(0.002)

        th = threading.Thread(target=sampler, daemon=True)
        torch.cuda.synchronize()
        th.start()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(25):
                step()
            n += 25
            torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join()
        # refreshes: samples whose firmware timestamp changed, inside [t0, t1]
        ref, last = [], None
        for s in samples:
            if s["fw"] is not None and s["fw"] != last:
                if t0 + 0.05 < s["t"] < t1:
                    ref.append(s)
                last = s["fw"]
        out = dict(st, window_s=round(t1 - t0, 3), steps=n, refreshes=len(ref),
                   source="amdsmi gpu_metrics: energy accumulator over firmware time, PPT residency "
                          "over the accumulation counter, current_gfxclks (8 XCDs) at each refresh")
        if len(ref) >= 2:
            a, b = ref[0], ref[-1]
            dt = (b["fw"] - a["fw"]) * 1e-8
            out["avg_socket_power_w"] = round((b["energy"] - a["energy"]) * st["energy_resolution_uj"] * 1e-6 / dt, 1)
            out["ppt_limited_frac"] = round((b["ppt"] - a["ppt"]) / max(1, b["acc"] - a["acc"]), 3)
            clks = [r["clk"] for r in ref[1:] if r["clk"]]
            out["gfxclk_mhz_mean"] = round(float(np.mean(clks)), 1) if clks else None
            out["gfxclk_mhz_per_xcd"] = ref[-1]["clks"]
            out["interval_s"] = round(dt, 3)
        try:
            # the driver's per-limiter residencies (percent of time), for the
            # reasons the clock sat below its maximum
            v = self.amdsmi.amdsmi_get_violation_status(self.h)
            out["violation_pct"] = {k: v[k] for k in ("per_ppt_pwr", "per_socket_thrm", "per_vr_thrm",
                                                      "per_hbm_thrm", "per_prochot_thrm",
                                                      "per_gfx_clk_below_host_limit") if k in v}
        except Exception as e:
            out["violation_pct"] = {"error": repr(e)}
        return out


def settle(torch, step, k, min_s, max_s=5.0, tol=0.01):
    """Untimed steps until at least min_s seconds have passed and two
    consecutive windows of k steps agree within tol (at most max_s).
    Returns (steps run, seconds, window times in ms/step)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wins, n = [], 0
    t0 = time.perf_counter()
    while True:
        e0.record()
        for _ in range(k):
            step()
        e1.record()
        torch.cuda.synchronize()
        n += k
        wins.append(e0.elapsed_time(e1) / k)
        el = time.perf_counter() - t0
        if el >= max_s or (el >= min_s and len(wins) >= 2 and abs(wins[-1] - wins[-2]) <= tol * wins[-2]):
            return n, el, wins


def bench_linear(torch, steps_mod, args, pm):
    from integer_only_nn_amd import ops
    import ionn_synth
    dev = torch.device("cuda:0")
    log("generating the large-linear inputs")
    d = ionn_synth.large_linear()
    X = torch.from_numpy(d["X"]).to(dev)
    W = torch.from_numpy(d["W"]).to(dev)
    dY = torch.from_numpy(d["dY"]).to(dev)
    buf = steps_mod.LinearStepBuffers.make(T, IN, OUT, dev)
    s = buf.scal
    res = {}
    if pm.h is not None:
        try:
            res["idle_gfxclk_mhz"] = pm.read()["clk"]
        except Exception:
            pass
    # the maxima alternate between two scalar sets: each step's update
    # clears the set the next step max-combines into (no fill launch per
    # step); sets[ph] is the current step's
    sets = (s[8:11], s[12:15])
    ph = [0]

    def step(tm=None):
        m = tm.mark if tm else (lambda n: None)
        cur, nxt = sets[ph[0]], sets[ph[0] ^ 1]
        ph[0] ^= 1
        m("fwd")
        ops.int_linear_fwd(X, W, buf.Y, absmax_Y=cur[0:1])
        m("dgrad")
        ops.int_linear_dgrad(dY, W, buf.dX, absmax_dX=cur[1:2])
        m("wgrad")
        ops.int_linear_wgrad(dY, X, buf.G, absmax_G=cur[2:3])
        m("update")
        ops.niti_quantize_update_clear(buf.G, cur[2:3], 8, 2, W, nxt, shifts_out=s[4:6])

    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)

    def timed(nsteps):
        torch.cuda.synchronize()
        t0.record()
        for _ in range(nsteps):
            step()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / nsteps

    for _ in range(args.warmup):
        step()
    # the first K-step window right after the warm-up steps, from idle clocks
    res["first_window_ms_per_step"] = timed(args.steps)
    n_set, s_set, wins = settle(torch, step, args.steps, args.settle_s)
    res["settle"] = {"steps": n_set, "seconds": round(s_set, 3),
                     "first_windows_ms_per_step": [round(w, 4) for w in wins[:6]],
                     "last_windows_ms_per_step": [round(w, 4) for w in wins[-2:]]}
    res["ms"] = timed(args.steps)

    # per-step times (an event pair per step) for the median and the minimum
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    res["per_step_ms"] = {"median": float(np.median(per_step)), "min": float(np.min(per_step)),
                          "max": float(np.max(per_step))}

    # the same steps with every launch bracketed by events: per-kernel averages
    tm = Timer(torch)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step(tm)
    tm.mark(None)
    t1.record()
    torch.cuda.synchronize()
    res["ms_instr"] = t0.elapsed_time(t1) / args.steps
    res["per"] = {k: float(np.mean(v)) for k, v in tm.per_name().items()}

    # each contraction timed inside the step by one event pair around it
    # alone (the other launches run unbracketed), and back to back on its own
    def only(name, e_a, e_b):
        def st_():
            cur, nxt = sets[ph[0]], sets[ph[0] ^ 1]
            ph[0] ^= 1
            if name == "fwd":
                e_a.record()
            ops.int_linear_fwd(X, W, buf.Y, absmax_Y=cur[0:1])
            if name == "fwd":
                e_b.record()
            elif name == "dgrad":
                e_a.record()
            ops.int_linear_dgrad(dY, W, buf.dX, absmax_dX=cur[1:2])
            if name == "dgrad":
                e_b.record()
            elif name == "wgrad":
                e_a.record()
            ops.int_linear_wgrad(dY, X, buf.G, absmax_G=cur[2:3])
            if name == "wgrad":
                e_b.record()
            ops.niti_quantize_update_clear(buf.G, cur[2:3], 8, 2, W, nxt, shifts_out=s[4:6])
        return st_
    # kernels launched back to back on their own (maxima into the spare
    # set s[0:3], which no step reads)
    launch = {"fwd": lambda: ops.int_linear_fwd(X, W, buf.Y, absmax_Y=s[0:1]),
              "dgrad": lambda: ops.int_linear_dgrad(dY, W, buf.dX, absmax_dX=s[1:2]),
              "wgrad": lambda: ops.int_linear_wgrad(dY, X, buf.G, absmax_G=s[2:3]),
              "update": lambda: ops.niti_quantize_update(buf.G, s[2:3], 8, 2, W, shifts_out=s[4:6])}
    in_step, b2b = {}, {}
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for name in ("fwd", "dgrad", "wgrad"):
        torch.cuda.synchronize()
        for a, b in evs:
            only(name, a, b)()
        torch.cuda.synchronize()
        in_step[name] = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    for name, fn in launch.items():
        fn()
        t0.record()
        for _ in range(args.steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        b2b[name] = t0.elapsed_time(t1) / args.steps
    res["kernel_in_step"] = in_step
    res["kernel_back_to_back"] = b2b

    # the same step with the propagated delta requantised to 7 bits (untimed above)
    def step_req():
        cur = sets[ph[0]]
        step()
        ops.niti_quantize(buf.dX, cur[1:2], 7, False, buf.delta, shift_out=s[3:4])
    for _ in range(2):
        step_req()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step_req()
    t1.record()
    torch.cuda.synchronize()
    res["ms_req"] = t0.elapsed_time(t1) / args.steps
    res["shifts"] = buf.scal.cpu().tolist()
    # max |Y|, |dX|, |G| of the last step (the tests compare them with the
    # oracle's for this workload)
    res["last_maxima"] = [int(v) & 0xFFFFFFFF for v in sets[ph[0] ^ 1].cpu().tolist()]

    # power and clock over a few seconds of back-to-back steps
    if args.power_window_s > 0 and pm.h is not None:
        try:
            res["power"] = pm.window(step, torch, args.power_window_s)
        except Exception as e:
            res["power"] = {"error": repr(e)}

    # the NITI update on its own: G cold (the 256 MB last-level cache flushed
    # by a 1 GiB pass before every launch: a write pass, as the measurement
    # protocol states, and a read-only pass, which leaves no dirty lines to
    # write back during the update) and warm (launched back to back)
    flush = torch.empty(256 << 20, dtype=torch.int32, device=dev)    # 1 GiB
    fam = torch.zeros(1, dtype=torch.int32, device=dev)
    ops.ionn_fill_u32(flush, 1)
    upd = {}
    for kind in ("write", "read"):
        torch.cuda.synchronize()
        for a, b in evs:
            if kind == "write":
                ops.ionn_fill_u32(flush, 0)
            else:
                ops.ionn_absmax_i32(flush, fam)
            a.record()
            launch["update"]()
            b.record()
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in evs]
        upd[kind] = {"median_ms": float(np.median(ts)), "min_ms": float(np.min(ts))}
    upd["warm"] = {"median_ms": b2b["update"], "min_ms": b2b["update"]}
    del flush
    res["update_alone"] = upd
    return res


def bench_small(torch, nsteps):
    """The two latency-bound workloads: the single int8 linear layer (batch
    16, 64 -> 32, one NITI step) and the 784-256-128-10 MLP trained for 10
    steps at batch 256, each eagerly (one library call per launch) and
    replayed from one captured HIP graph.  The MLP's weights are restored
    from their seeded values before every 10-step run, outside the timed
    region."""
    import ionn_synth
    from integer_only_nn_amd import steps as st
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}

    d = ionn_synth.single_linear()
    X, W0, dY = to(d["X"]), to(d["W"]), to(d["dY"])
    W = W0.clone()
    buf = st.LinearStepBuffers.make(16, 64, 32, dev)

    def one(stream=None):
        st.linear_step(X, W, dY, buf, stream=stream)

    def eager_ms(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def graph_ms(fn, reps, nreplay=20):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            fn(s.cuda_stream)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for _ in range(reps):
                    fn(s.cuda_stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(nreplay):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (nreplay * reps)

    ems = eager_ms(one, nsteps)
    gms = graph_ms(one, 10)
    ops1 = 3 * 2.0 * 16 * 64 * 32
    out["single_linear_16x64x32"] = {
        "us_per_step": round(ems * 1e3, 2), "graph_us_per_step": round(gms * 1e3, 2),
        "GOPS": round(ops1 / (ems * 1e-3) / 1e9, 3), "graph_GOPS": round(ops1 / (gms * 1e-3) / 1e9, 3),
        "launches_per_step": 6, "note": "W evolves from step to step; the kernels' work does not depend on it"}
    # the same step in one launch (one workgroup, operands in LDS)
    bufs = st.LinearStepBuffers.make(16, 64, 32, dev)

    def one_small(stream=None):
        st.linear_step_small(X, W, dY, bufs, stream=stream)

    fms = eager_ms(one_small, nsteps)
    fgms = graph_ms(one_small, 10)
    out["single_linear_16x64x32"]["one_launch"] = {
        "entry_point": "int_linear_step_small", "us_per_step": round(fms * 1e3, 2),
        "graph_us_per_step": round(fgms * 1e3, 2), "GOPS": round(ops1 / (fms * 1e-3) / 1e9, 3),
        "graph_GOPS": round(ops1 / (fgms * 1e-3) / 1e9, 3), "launches_per_step": 1}

    m = ionn_synth.mlp()
    Ws0 = [to(w) for w in m["Ws"]]
    Ws = [w.clone() for w in Ws0]
    Xm, lab = to(m["X"]), to(m["labels"].astype(np.int32))
    net = st.MLP.make(Ws, 256)

    def ten(stream=None):
        for _ in range(10):
            net.step(Xm, lab, stream=stream)

    def restore():
        for w, w0 in zip(Ws, Ws0):
            w.copy_(w0)

    ten()
    torch.cuda.synchronize()
    ts = []
    for _ in range(nsteps):
        restore()
        torch.cuda.synchronize()
        e0.record()
        ten()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    t_eager = float(np.median(ts))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        ten(s.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            ten(s.cuda_stream)
    torch.cuda.synchronize()
    tg = []
    for _ in range(nsteps):
        restore()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        tg.append(e0.elapsed_time(e1))
    t_graph = float(np.median(tg))
    sizes = (784, 256, 128, 10)
    ops_step = 2.0 * 256 * sum(a * b for a, b in zip(sizes[:-1], sizes[1:])) * 3
    out["mlp_784_256_128_10_b256_10steps"] = {
        "ms_10_steps": round(t_eager, 4), "samples_per_s": round(2560 / (t_eager * 1e-3), 1),
        "graph_ms_10_steps": round(t_graph, 4), "graph_samples_per_s": round(2560 / (t_graph * 1e-3), 1),
        "TOPS": round(10 * ops_step / (t_eager * 1e-3) / 1e12, 4),
        "graph_TOPS": round(10 * ops_step / (t_graph * 1e-3) / 1e12, 4),
        "launches_per_step": 1 + 2 * 3 + 2 + 4 * 3,
        "note": "median of runs; weights restored to their seeded values before each 10-step run, "
                "outside the timed region"}
    return out


def _timed(torch, step, nsteps):
    """Step time over nsteps (one event pair) and per-launch averages from a
    second, event-bracketed run, after the clocks have settled on this
    workload as for the headline (at least 0.3 s of untimed steps and two
    consecutive nsteps windows within 1%)."""
    settle(torch, lambda: step(None), nsteps, 0.3)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(nsteps):
        step(None)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / nsteps
    tm = Timer(torch)
    for _ in range(nsteps):
        step(tm)
    tm.mark(None)
    torch.cuda.synchronize()
    return ms, {k: float(np.mean(v)) for k, v in tm.per_name().items()}


def bench_conv(torch, steps_mod, nsteps):
    """The 128x56x56, 64 -> 64 channel conv NITI step, launch by launch as
    steps.conv_step runs it."""
    import ionn_synth
    from integer_only_nn_amd import ops
    dev = torch.device("cuda:0")
    d = ionn_synth.conv3x3()
    X, Wt, dY = (torch.from_numpy(d[k]).to(dev) for k in ("X", "W", "dY"))
    buf = steps_mod.ConvStepBuffers.make(128, 56, 56, 64, 64, dev)
    desc = ops.conv_desc(128, 56, 56, 64, 64)
    s = buf.scal
    # the maxima alternate between two scalar sets: each step's update
    # clears the set the next step max-combines into (no fill launch)
    sets = (s[8:11], s[12:15])
    ph = [0]

    def cur_next():
        c, n = sets[ph[0]], sets[ph[0] ^ 1]
        ph[0] ^= 1
        return c, n

    def step(tm):
        m = tm.mark if tm else (lambda n: None)
        c, n = cur_next()
        m("fwd")
        ops.int_conv_fwd(X, Wt, buf.Y, desc, absmax_Y=c[0:1])
        m("requant_y")
        ops.niti_quantize(buf.Y, c[0:1], 7, False, buf.y8, shift_out=s[3:4])
        m("dgrad")
        ops.int_conv_dgrad(dY, Wt, buf.dX, desc, absmax_dX=c[1:2])
        m("requant_dx")
        ops.niti_quantize(buf.dX, c[1:2], 7, False, buf.dx8, shift_out=s[4:5])
        m("wgrad")
        ops.int_conv_wgrad(dY, X, buf.G, desc, absmax_G=c[2:3], workspace=buf.ws)
        m("update")
        ops.niti_quantize_update_clear(buf.G, c[2:3], 8, 2, Wt, n, shifts_out=s[5:7])

    def step_fused(tm):
        # the requantisation fused into the contractions (steps.conv_step_fused):
        # one contraction pass stores each 32-pixel block's int8 value at the
        # block's own shift with its rounding bits, a streaming pass applies
        # the tensor's shift; the int32 sums are never stored
        m = tm.mark if tm else (lambda n: None)
        c, n = cur_next()
        m("fwd_requant")
        ops.int_conv_fwd_requant(X, Wt, buf.y8, desc, 7, False, c[0:1], shift_out=s[3:4], workspace=buf.rws)
        m("dgrad_requant")
        ops.int_conv_dgrad_requant(dY, Wt, buf.dx8, desc, 7, c[1:2], shift_out=s[4:5], workspace=buf.rws)
        m("wgrad")
        ops.int_conv_wgrad(dY, X, buf.G, desc, absmax_G=c[2:3], workspace=buf.ws)
        m("update")
        ops.niti_quantize_update_clear(buf.G, c[2:3], 8, 2, Wt, n, shifts_out=s[5:7])
    return _timed(torch, step, nsteps), _timed(torch, step_fused, nsteps)


def bench_dfp16(torch, steps_mod, nsteps):
    """The DFP-16 step (fwd, dgrad, wgrad contractions with down-conversion,
    then Gavg) on M=25088 K=256 N=1024."""
    import ionn_synth
    from integer_only_nn_amd import ops
    dev = torch.device("cuda:0")
    d = ionn_synth.dfp16_gemm()
    X, W, dY = (torch.from_numpy(d[k]).to(dev) for k in ("X", "W", "dY"))
    e = lambda v: torch.tensor([v], dtype=torch.int32, device=dev)
    eX, eW, edY = e(d["eX"]), e(d["eW"]), e(d["edY"])
    buf = steps_mod.DfpStepBuffers.make(25088, 256, 1024, dev)
    ex = buf.exps

    def step(tm):
        m = tm.mark if tm else (lambda n: None)
        m("fwd")
        ops.dfp16_gemm_fwd(X, eX, W, eW, buf.Y, ex[0:1], buf.ws, status_out=ex[3:4])
        m("dgrad")
        ops.dfp16_gemm_dgrad(dY, edY, W, eW, buf.dX, ex[1:2], buf.ws, status_out=ex[4:5])
        m("wgrad")
        ops.dfp16_gemm_wgrad(dY, edY, X, eX, buf.G, ex[2:3], buf.ws, status_out=ex[5:6])
        m("gavg")
        ops.dfp16_gavg(buf.G, ex[2:3], eW, buf.gavg)
    return _timed(torch, step, nsteps)


def bench_dfp16_paper(torch, nsteps):
    """The DFP-16 layer (M=25088, K=256, N=1024) stepped as the DFP page
    runs it: FP32 input, weights and incoming gradient converted to DFP-16
    (shared exponent from the absolute maximum), the three contractions
    with FP32 chunk partials and the one-bit input shift, the FP32 output
    re-quantised for the next layer, and the FP32 weight update with its
    DFP-16 copy.  The forward on Blocked-DFP operands (exponent per 64
    values) is timed beside it."""
    from integer_only_nn_amd import ops
    dev = torch.device("cuda:0")
    M, K, N = 25088, 256, 1024
    g = torch.Generator(device="cpu").manual_seed(5)
    X32 = (torch.randn(M, K, generator=g) * 2.0).to(dev)
    W32 = (torch.randn(N, K, generator=g) * 0.05).to(dev)
    dY32 = (torch.randn(M, N, generator=g) * 1e-3).to(dev)
    i16 = lambda *shape: torch.empty(*shape, dtype=torch.int16, device=dev)
    f32 = lambda *shape: torch.empty(*shape, dtype=torch.float32, device=dev)
    ex = torch.zeros(8, dtype=torch.int32, device=dev)       # eX, eW, edY, eY, status
    X16, W16, dY16, Y16 = i16(M, K), i16(N, K), i16(M, N), i16(M, N)
    Y, dX, G = f32(M, N), f32(M, K), f32(N, K)
    cws = torch.empty(ops.dfp_convert_workspace_bytes(), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(ops.dfp16_f32_workspace_bytes(M, K, N, w) for w in range(3)), dtype=torch.uint8, device=dev)
    Xb, Wb = i16(M, K), i16(N, K)
    eXb = torch.empty(M * (K // 64), dtype=torch.int32, device=dev)
    eWb = torch.empty(N * (K // 64), dtype=torch.int32, device=dev)

    def step(tm):
        m = tm.mark if tm else (lambda name: None)
        m("to_dfp_inputs")
        ops.dfp_from_f32(X32, X16, ex[0:1], cws)
        ops.dfp_from_f32(dY32, dY16, ex[2:3], cws)
        m("to_dfp_weights")
        ops.dfp_from_f32(W32, W16, ex[1:2], cws)
        m("fwd")
        ops.dfp16_gemm_fwd_f32(X16, ex[0:1], W16, ex[1:2], Y, ws)
        m("requant_y")
        ops.dfp_from_f32(Y, Y16, ex[3:4], cws)
        m("dgrad")
        ops.dfp16_gemm_dgrad_f32(dY16, ex[2:3], W16, ex[1:2], dX, ws)
        m("wgrad")
        ops.dfp16_gemm_wgrad_f32(dY16, ex[2:3], X16, ex[0:1], G, ws)
        m("sgd_update")
        ops.dfp16_sgd_update(W32, G, 1e-4, W16, ex[1:2], cws)
        # the Blocked-DFP variant of the forward (one exponent per 64 values)
        m("to_blocked")
        ops.dfp_from_f32_blocked(X32, Xb, eXb)
        ops.dfp_from_f32_blocked(W32, Wb, eWb)
        m("fwd_blocked")
        ops.dfp16_gemm_fwd_f32_blocked(Xb, eXb, Wb, eWb, Y, ws)
    ms, per = _timed(torch, step, nsteps)
    # the step proper: conversions, the three contractions, re-quantisation
    # and the update (the blocked variant is timed beside it, not in it)
    return ms - per["to_blocked"] - per["fwd_blocked"], per


def bench_offsets(torch, nsteps):
    """Offsets (bias) and the static OSS chain on the large-linear workload:
    the forward with the chain in the contraction's epilogue (int8 out), the
    same as an int32 contraction plus the OSS pass, and the offsets' backward
    (gradient over the 8192 error rows, its max, the int32 NITI update).
    Per-channel parameters are seeded: offset U[-2^18, 2^18), mult
    U[1, 2^11) with every seventh negated, k U[16, 22)."""
    import ionn_synth
    from integer_only_nn_amd import ops
    dev = torch.device("cuda:0")
    d = ionn_synth.large_linear()
    X, W, dY = (torch.from_numpy(d[k]).to(dev) for k in ("X", "W", "dY"))
    rng = np.random.default_rng(11)
    off = rng.integers(-2**18, 2**18, OUT, dtype=np.int64).astype(np.int32)
    mult = rng.integers(1, 2**11, OUT, dtype=np.int64).astype(np.int32)
    mult[::7] *= -1
    k = rng.integers(16, 22, OUT).astype(np.int8)
    off, mult, k = (torch.from_numpy(a).to(dev) for a in (off, mult, k))
    Y8 = torch.empty(T, OUT, dtype=torch.int8, device=dev)
    acc = torch.empty(T, OUT, dtype=torch.int32, device=dev)
    gb = torch.empty(OUT, dtype=torch.int32, device=dev)
    gws = torch.empty(ops.ionn_bias_grad_workspace_bytes(T, OUT), dtype=torch.uint8, device=dev)
    P = torch.zeros(OUT, dtype=torch.int32, device=dev)
    am = torch.zeros(1, dtype=torch.int32, device=dev)
    sh = torch.zeros(2, dtype=torch.int32, device=dev)

    def step(tm):
        m = tm.mark if tm else (lambda n: None)
        m("fwd_oss_fused")
        ops.int_linear_fwd_oss(X, W, off, mult, k, Y8)
        m("fwd_int32")
        ops.int_linear_fwd(X, W, acc)
        m("oss_pass")
        ops.ionn_oss_requant(acc, off, mult, k, Y8)
        m("bias_grad")
        ops.ionn_bias_grad(dY, gb, gws)
        m("fill")
        ops.ionn_fill_u32(am, 0)
        m("absmax")
        ops.ionn_absmax_i32(gb, am)
        m("update_i32")
        ops.niti_quantize_update_i32(gb, am, 8, 2, P, shifts_out=sh)
    return _timed(torch, step, nsteps)


def bench_model(torch, nsteps):
    """The example network of the on-device training page (arc-fault
    detection: Conv 16x2 valid + ReLU, Linear 160 + ReLU, Linear 2) trained
    by the library's model driver: whole steps (forward, MSE gradient,
    backward, updates) at the page's batch of 8, eagerly and replayed from
    one captured HIP graph, and at batch 65536."""
    import ionn_synth
    from integer_only_nn_amd import steps as st
    dev = torch.device("cuda:0")
    res = {}
    for B in (8, 65536):
        d = ionn_synth.arc_fault(B=B)
        layers = _model_layers(d)
        m = st.Model(layers, B, dev)
        X, lab, tmc, tmw = (torch.from_numpy(np.ascontiguousarray(d[k])).to(dev)
                            for k in ("X", "labels", "tmc", "tmw"))
        for _ in range(5):
            m.step(X, lab, tmc, tmw)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(nsteps):
            m.step(X, lab, tmc, tmw)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / nsteps
        r = {"ms_per_step": round(ms, 4), "samples_per_s": round(B / (ms * 1e-3), 1)}
        if B == 8:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s):
                m.step(X, lab, tmc, tmw, stream=s.cuda_stream)   # warm the capture stream
                torch.cuda.synchronize()
                with torch.cuda.graph(g, stream=s):
                    m.step(X, lab, tmc, tmw, stream=s.cuda_stream)
            torch.cuda.synchronize()
            t0.record()
            for _ in range(nsteps):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            gms = t0.elapsed_time(t1) / nsteps
            r["graph_ms_per_step"] = round(gms, 4)
            r["graph_samples_per_s"] = round(B / (gms * 1e-3), 1)
        res[f"batch_{B}"] = r
    return res


def _graph_ms(torch, fn, reps, nreplay=20):
    """Average time of one fn(stream) call, from a HIP graph holding `reps`
    back-to-back calls replayed `nreplay` times (no host gaps between the
    launches, unlike an eager loop whose per-call Python cost exceeds a
    short kernel)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn(s.cuda_stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn(s.cuda_stream)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(nreplay):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (nreplay * reps)


def bench_apt(torch, nsteps):
    """Adaptive per-layer precision: the k-bit update of one 4096 x 4096
    layer (16.8 M int16 weights; reads W and G, writes W: 6 algorithmic bytes
    per weight) plain and with Gavg sampling; the update of all 20 weight
    layers of a ResNet-20 in one launch, per training step; and the move of
    all 20 layers' precision between epochs (every layer raised or lowered
    by one bit, so each rescale pass does real work).  Kernel times come
    from graph replays of back-to-back calls; the eager per-call times
    (HIP events around each call) are reported beside them."""
    import ionn_synth
    from integer_only_nn_amd import steps as st
    dev = torch.device("cuda:0")
    n = IN * OUT
    W, _ = ionn_synth.apt_weights([n], k0=12, seed=3)
    big = st.AptLayers(W, [12], [-10], dev)
    Gb = [torch.from_numpy(ionn_synth.apt_grad(9, n, 3000.0, seed=3)).to(dev)]
    egb = torch.tensor([-22], dtype=torch.int32, device=dev)
    sizes = ionn_synth.RESNET20_SIZES
    Ws, es = ionn_synth.apt_weights(sizes, k0=6)
    rn = st.AptLayers(Ws, [6] * len(sizes), es, dev)
    rn8 = st.AptLayers(Ws, [6] * len(sizes), es, dev, int8_layers=tuple(range(len(sizes))))
    Gr = [torch.from_numpy(ionn_synth.apt_grad(l, m, 500.0)).to(dev) for l, m in enumerate(sizes)]
    egr = torch.full((len(sizes),), -14, dtype=torch.int32, device=dev)
    big.bind_grads(Gb)
    rn.bind_grads(Gr)
    rn8.bind_grads(Gr)
    flip = [0]

    def step(tm):
        m = tm.mark if tm else (lambda name: None)
        m("update_16M")
        big.step(None, egb, 6)
        m("update_16M_sampling")
        big.step(None, egb, 6, sample=True)
        m("resnet20_update")
        rn.step(None, egr, 3)
        m("resnet20_update_sampling")
        rn.step(None, egr, 3, sample=True)
        m("set_sums")
        flip[0] ^= 1
        rn.gsum.fill_(0.0 if flip[0] else 1e9)   # below T_min: raise; far above T_max: lower
        m("resnet20_adjust")
        rn.end_epoch(1.0, 100.0, 2, 16)
    _, per = _timed(torch, step, nsteps)
    g = {"update_16M": _graph_ms(torch, lambda s: big.step(None, egb, 6, stream=s), 10),
         "update_16M_sampling": _graph_ms(torch, lambda s: big.step(None, egb, 6, sample=True, stream=s), 10),
         "resnet20_update": _graph_ms(torch, lambda s: rn.step(None, egr, 3, stream=s), 10),
         "resnet20_update_sampling": _graph_ms(torch, lambda s: rn.step(None, egr, 3, sample=True, stream=s), 10),
         "resnet20_int8_update": _graph_ms(torch, lambda s: rn8.step(None, egr, 3, stream=s), 10)}
    gbs = 6.0 * n / (g["update_16M"] * 1e-3) / 1e9
    r4 = lambda v: round(v, 4)
    return {"layer_16M": {"shape": "4096 x 4096 int16 weights, k = 12",
                          "update_ms": r4(g["update_16M"]), "update_sampling_ms": r4(g["update_16M_sampling"]),
                          "eager_update_ms": r4(per["update_16M"]),
                          "roofline": {"bound": "hbm", "kernel": "apt_update", "achieved": round(gbs, 1),
                                       "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                       "bytes_per_launch": 6.0 * n}},
            "resnet20": {"layers": len(sizes), "weights": sum(sizes),
                         "update_ms": r4(g["resnet20_update"]), "update_sampling_ms": r4(g["resnet20_update_sampling"]),
                         "eager_update_ms": r4(per["resnet20_update"]),
                         "eager_adjust_ms": r4(per["resnet20_adjust"]),
                         "weight_bytes_int16": sum(w.numel() * w.element_size() for w in rn.W),
                         "int8_storage": {"update_ms": r4(g["resnet20_int8_update"]),
                                          "weight_bytes": sum(w.numel() * w.element_size() for w in rn8.W),
                                          "note": "every layer held in int8 (k <= 8, never raised past 8)"}}}


def _model_layers(d):
    """The example network's layer dicts (geometry of the page, parameters
    from ionn_synth.arc_fault)."""
    prm = [dict(weight=q["W"], offset=q["offset"], mult=q["mult"], k=q["k"]) for q in d["layers"]]
    return [dict(kind="conv", relu=True, H=64, W=2, Cin=1, Cout=3, KH=16, KW=2, pad=0, **prm[0]),
            dict(kind="linear", relu=True, IN=147, OUT=160, **prm[1]),
            dict(kind="linear", relu=False, IN=160, OUT=2, **prm[2])]


# The translation units (and the headers they include) that build the
# contraction and update kernels the traffic figures describe.
TRAFFIC_SOURCES = ("common.h", "gemm_core.h", "gemm256.h", "gemm_skinny.h", "wgrad_long.h", "gemm_i8.hip", "niti.hip")


def _kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in TRAFFIC_SOURCES:
        h.update(name.encode())
        with open(os.path.join(HERE, "integer_only_nn_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM-side bytes per launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, if it was taken on the kernel sources as they are
    now (else {}: the counters describe an older kernel)."""
    path = os.path.join(HERE, "profiles", "gemm256_linear_step_8192x4096x4096_hbm_traffic.txt")
    if not os.path.exists(path):
        return {}
    out, src = {}, None
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] == "source_sha256":
                src = parts[1]
            elif len(parts) == 3 and parts[0] == "traffic_bytes_per_launch":
                out[parts[1]] = float(parts[2])
    return out if src == _kernel_source_hash() else {}


def _cpu_model():
    """The host CPU's model name, with its family, model and stepping
    numbers (a virtual machine may report only a generic name)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = (x.strip() for x in line.split(":", 1))
                    info.setdefault(k, v)
                elif info:
                    break
    except OSError:
        return None
    name = info.get("model name")
    if name is None:
        return None
    ids = [f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info]
    return f"{name} ({', '.join(ids)})" if ids else name


def cpu_baseline(rows, threads=None):
    """The oracle (plain C, OpenMP) on a bounded sample of the large-linear
    step: `rows` token rows through fwd and dgrad, wgrad over `rows` tokens,
    then the NITI update of all 16.8M weights.  threads=None: the oracle's
    default (every host thread).  Returns (TOPS of the sample, seconds,
    threads used)."""
    import oracle
    import ionn_synth
    d = ionn_synth.large_linear(T=rows, IN=IN, OUT=OUT)
    X, W, dY = d["X"], d["W"], d["dY"]
    prev = oracle.get_threads()
    if threads is not None:
        oracle.set_threads(threads)
    try:
        used = oracle.get_threads()
        t0 = time.perf_counter()
        oracle.linear_fwd(X, W)
        oracle.linear_dgrad(dY, W)
        G = oracle.linear_wgrad(dY, X)
        oracle.niti_update(G, W, 8, 2)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_threads(prev)
    ops_done = 3 * 2.0 * rows * IN * OUT
    return ops_done / dt / 1e12, dt, used


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the step is "
              "timed on one GPU at its full per-GPU shape (a data-parallel split over tokens would "
              "reduce-scatter the int32 weight gradient and max-combine every per-tensor maximum)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from integer_only_nn_amd import lib, steps as steps_mod
    lib()  # fail loudly if the HIP library is missing
    assert torch.cuda.is_available(), "no ROCm device visible"
    pm = PowerMonitor(torch)

    L = bench_linear(torch, steps_mod, args, pm)
    ms, per = L["ms"], L["per"]
    ops_step = 3 * 2.0 * T * IN * OUT
    tops = ops_step / (ms * 1e-3) / 1e12
    # the roofline kernel: the slowest contraction, timed inside the step by
    # one event pair around it alone (per-launch brackets on every kernel
    # slow the step down; they only give the breakdown in kernel_ms)
    gemm = dict(L["kernel_in_step"])
    dom = max(gemm, key=gemm.get)
    achieved = 2.0 * T * IN * OUT / (gemm[dom] * 1e-3) / 1e12
    b2b = L["kernel_back_to_back"]
    upd_bytes = 6.0 * IN * OUT
    traffic = measured_traffic()
    upd_gbs = upd_bytes / (per["update"] * 1e-3) / 1e9
    gbs = lambda t_ms: round(upd_bytes / (t_ms * 1e-3) / 1e9, 1)
    ua = L["update_alone"]
    log(f"step {ms:.3f} ms  {tops:.1f} TOPS  per-kernel ms {per}")
    shifts = L["shifts"]
    power = L.get("power") or {"error": pm.err}
    roof = {"bound": "mfma", "kernel": f"int_linear_{dom}", "achieved": round(achieved, 1),
            "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": traffic.get(f"int_linear_{dom}"),
            "duration_ms": round(gemm[dom], 4),
            "duration_source": "HIP events around this kernel alone inside each timed step (the "
                               "interval also holds the system-scope release the end event forces)",
            "achieved_back_to_back": round(2.0 * T * IN * OUT / (b2b[dom] * 1e-3) / 1e12, 1)}
    clk = power.get("gfxclk_mhz_mean")
    if clk:
        # the same peak at the graphics clock the power limit held during the
        # steps (matrix rate scales with the clock)
        roof["peak_at_measured_clock"] = round(PEAK_INT8_TOPS * clk / 2400.0, 1)
        roof["frac_at_measured_clock"] = round(achieved / roof["peak_at_measured_clock"], 4)

    result = {
        "metric": "INT8 training-step TOPS (fwd+dgrad+wgrad+NITI update), % of INT8 MFMA peak",
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded SplitMix64: X~round(N(0,40)), W~round(N(0,20)), dY~U[-64,63])",
        "config": {"workload": "large int8 linear training step", "tokens": T, "in": IN,
                   "out": OUT, "target_bits_weight": 8, "mu_weight": 2, "parallelism": "none"},
        "pct_of_int8_peak": round(100.0 * tops / PEAK_INT8_TOPS, 2),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "per_step_ms": {k: round(v, 4) for k, v in L["per_step_ms"].items()},
        "warmup_protocol": {"warmup_steps": args.warmup, "settle": L["settle"],
                            "first_window_after_warmup_ms_per_step": round(L["first_window_ms_per_step"], 4),
                            "idle_gfxclk_mhz": L.get("idle_gfxclk_mhz")},
        "kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "ms_per_step_events_per_launch": round(L["ms_instr"], 4),
        "kernel_ms_in_step": {k: round(v, 4) for k, v in L["kernel_in_step"].items()},
        "kernel_ms_back_to_back": {k: round(v, 4) for k, v in L["kernel_back_to_back"].items()},
        "roofline": roof,
        "clock_power": power,
        "update_pass": {"bound": "hbm", "achieved": round(upd_gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(upd_gbs / PEAK_HBM_GBS, 4),
                        "bytes_per_launch": upd_bytes,
                        "in_step_event_interval_ms": round(per["update"], 4),
                        "alone": {k: {"median_ms": round(v["median_ms"], 4), "min_ms": round(v["min_ms"], 4),
                                      "GBps": gbs(v["median_ms"]),
                                      "frac": round(gbs(v["median_ms"]) / PEAK_HBM_GBS, 4)}
                                  for k, v in ua.items()},
                        "alone_note": "write / read: the last-level cache flushed before every launch by a "
                                      "1 GiB write (resp. read-only) pass; warm: launched back to back",
                        "traffic": traffic.get("niti_quantize_update"),
                        "traffic_source": "profiles/ FETCH_SIZE + WRITE_SIZE summary of the committed "
                                          "kernels (null when the sources changed since)"},
        "ms_per_step_with_delta_requant": round(L["ms_req"], 4),
        "shifts": {"s_delta": shifts[3], "s_weight": shifts[4], "ws": shifts[5]},
        "maxima_last_step": L["last_maxima"],
    }
    result["small_workloads"] = bench_small(torch, 20)
    if args.calibrate:
        from integer_only_nn_amd import ops
        cal = torch.ones(64 << 20, dtype=torch.int32, device="cuda:0")   # 256 MiB
        am = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        for _ in range(3):
            ops.ionn_absmax_i32(cal, am)     # reads exactly 256 MiB
            ops.ionn_fill_u32(cal, 0)        # writes exactly 256 MiB
        torch.cuda.synchronize()
        result["calibration"] = {"read_kernel": "absmax_kernel", "write_kernel": "fill_u32_kernel",
                                 "bytes": 256 << 20}
    if not args.no_secondary:
        log("secondary: conv and DFP-16 steps, offsets and OSS, the example network")
        (c_ms, c_per), (cf_ms, cf_per) = bench_conv(torch, steps_mod, 20)
        f_ms, f_per = bench_dfp16(torch, steps_mod, 20)
        conv_ops = 3 * 2.0 * 128 * 56 * 56 * 64 * 9 * 64
        dfp_ops = 3 * 2.0 * 25088 * 256 * 1024
        # conv contractions are HBM-bound: int8 image in, int32 result out
        img = 128 * 56 * 56 * 64
        conv_bytes = {"fwd": img + 4 * img, "dgrad": img + 4 * img, "wgrad": 2 * img + 4 * 64 * 9 * 64}
        cdom = max(conv_bytes, key=lambda k: c_per[k])
        cgbs = conv_bytes[cdom] / (c_per[cdom] * 1e-3) / 1e9
        # fused path: the contractions run twice with no int32 traffic and are
        # bound by the matrix cores; the algorithmic work per call is one
        # contraction, 2 * pixels * 64 * 576 int8 ops
        conv_op1 = 2.0 * 128 * 56 * 56 * 64 * 9 * 64
        fdom_c = max(("fwd_requant", "dgrad_requant"), key=lambda k: cf_per[k])
        cf_tops = conv_op1 / (cf_per[fdom_c] * 1e-3) / 1e12
        # VALU view of the DFP-16 contractions: 5 int32 operations per output
        # element per 64-term chunk (digit combination mad_i24 + lshl_add,
        # then the rounding shift, its rounding bit and the add)
        dfp_alu = {"fwd": 5.0 * 25088 * 1024 * (256 // 64), "dgrad": 5.0 * 25088 * 256 * (1024 // 64),
                   "wgrad": 5.0 * 1024 * 256 * (25088 // 64)}
        # the method's own work: 2*M*N*K int16 multiply-adds per contraction,
        # each 4 int8 digit products on the matrix cores (every role has the
        # same M*N*K); the VALU view of the epilogue is kept beside it
        dfp_i8 = 4 * 2.0 * 25088 * 256 * 1024
        fdom = max(dfp_alu, key=lambda k: f_per[k])
        falu = dfp_alu[fdom] / (f_per[fdom] * 1e-3) / 1e12
        p_ms, p_per = bench_dfp16_paper(torch, 20)
        # the same count for the FP32 form: per output element and 64-term
        # chunk three operations of digit combination, one int32 -> FP32
        # conversion and one FP32 addition
        pdom = max(("fwd", "dgrad", "wgrad"), key=lambda k: p_per[k])
        palu = dfp_alu[pdom] / (p_per[pdom] * 1e-3) / 1e12
        o_ms, o_per = bench_offsets(torch, 20)
        o_gemm = 2.0 * T * IN * OUT / (o_per["fwd_oss_fused"] * 1e-3) / 1e12
        o_oss = 5.0 * T * OUT / (o_per["oss_pass"] * 1e-3) / 1e9
        o_bg = 1.0 * T * OUT / (o_per["bias_grad"] * 1e-3) / 1e9
        offsets = {"shape": f"T{T} IN{IN} OUT{OUT}",
                   "kernel_ms": {k2: round(v, 4) for k2, v in o_per.items()},
                   "fwd_with_oss_ms": {"fused": round(o_per["fwd_oss_fused"], 4),
                                       "int32_then_oss_pass": round(o_per["fwd_int32"] + o_per["oss_pass"], 4)},
                   "offset_backward_ms": round(o_per["bias_grad"] + o_per["fill"] + o_per["absmax"]
                                               + o_per["update_i32"], 4),
                   "roofline": {"bound": "mfma", "kernel": "int_linear_fwd_oss", "achieved": round(o_gemm, 1),
                                "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                                "frac": round(o_gemm / PEAK_INT8_TOPS, 4)},
                   "oss_pass": {"bound": "hbm", "achieved": round(o_oss, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(o_oss / PEAK_HBM_GBS, 4), "bytes_per_launch": 5.0 * T * OUT},
                   "bias_grad": {"bound": "hbm", "achieved": round(o_bg, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(o_bg / PEAK_HBM_GBS, 4), "bytes_per_launch": 1.0 * T * OUT}}
        result["secondary"] = {
            "conv3x3_step": {"shape": "N128 56x56 64->64 NHWC", "path": "requantisation fused (one contraction pass + streaming pass)",
                             "ms_per_step": round(cf_ms, 4),
                             "TOPS": round(conv_ops / (cf_ms * 1e-3) / 1e12, 2),
                             "images_per_s": round(128 / (cf_ms * 1e-3), 1),
                             "kernel_ms": {k: round(v, 4) for k, v in cf_per.items()},
                             "roofline": {"bound": "mfma", "kernel": f"int_conv_{fdom_c}",
                                          "achieved": round(cf_tops, 1), "peak": PEAK_INT8_TOPS,
                                          "unit": "TFLOP/s", "frac": round(cf_tops / PEAK_INT8_TOPS, 4),
                                          "ops_per_launch": conv_op1},
                             "int32_path": {"ms_per_step": round(c_ms, 4),
                                            "kernel_ms": {k: round(v, 4) for k, v in c_per.items()},
                                            "roofline": {"bound": "hbm", "kernel": f"int_conv_{cdom}",
                                                         "achieved": round(cgbs, 1), "peak": PEAK_HBM_GBS,
                                                         "unit": "GB/s", "frac": round(cgbs / PEAK_HBM_GBS, 4),
                                                         "bytes_per_launch": conv_bytes[cdom]}}},
            "dfp16_step": {"shape": "M25088 K256 N1024", "ms_per_step": round(f_ms, 4),
                           "int16_TOPS": round(dfp_ops / (f_ms * 1e-3) / 1e12, 2),
                           "images_per_s": round(128 / (f_ms * 1e-3), 1),
                           "kernel_ms": {k: round(v, 4) for k, v in f_per.items()},
                           "roofline": {"bound": "mfma", "kernel": f"dfp16_gemm_{fdom}",
                                        "achieved": round(dfp_i8 / (f_per[fdom] * 1e-3) / 1e12, 1),
                                        "peak": PEAK_INT8_TOPS, "unit": "TOPS (int8 digit products)",
                                        "frac": round(dfp_i8 / (f_per[fdom] * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                                        "ops_per_launch": dfp_i8,
                                        "work": "2*M*N*K int16 multiply-adds = 4 int8 digit products each"},
                           "roofline_valu": {"bound": "alu", "kernel": f"dfp16_gemm_{fdom}",
                                             "achieved": round(falu, 2), "peak": PEAK_VALU_TOPS,
                                             "unit": "T int32 op/s", "frac": round(falu / PEAK_VALU_TOPS, 4),
                                             "ops_per_launch": dfp_alu[fdom],
                                             "work": "the kernel's per-chunk epilogue: 5 int32 ops per output per chunk"}},
            "dfp16_paper_step": {"shape": "M25088 K256 N1024, FP32 chunk partials, 1-bit input shift",
                                 "ms_per_step": round(p_ms, 4),
                                 "int16_TOPS": round(dfp_ops / (p_ms * 1e-3) / 1e12, 2),
                                 "kernel_ms": {k: round(v, 4) for k, v in p_per.items()},
                                 "roofline": {"bound": "mfma", "kernel": f"dfp16_gemm_{pdom}_f32",
                                              "achieved": round(dfp_i8 / (p_per[pdom] * 1e-3) / 1e12, 1),
                                              "peak": PEAK_INT8_TOPS, "unit": "TOPS (int8 digit products)",
                                              "frac": round(dfp_i8 / (p_per[pdom] * 1e-3) / 1e12 / PEAK_INT8_TOPS, 4),
                                              "ops_per_launch": dfp_i8},
                                 "roofline_valu": {"bound": "alu", "kernel": f"dfp16_gemm_{pdom}_f32",
                                                   "achieved": round(palu, 2), "peak": PEAK_VALU_TOPS,
                                                   "unit": "T int32 op/s", "frac": round(palu / PEAK_VALU_TOPS, 4),
                                                   "ops_per_launch": dfp_alu[pdom]}},
            "offsets_oss": offsets,
            "arc_fault_model": dict(shape="Conv 16x2 valid 1->3 + ReLU, Linear 147->160 + ReLU, Linear 160->2",
                                    **bench_model(torch, 50)),
            "adaptive_precision": bench_apt(torch, 20),
        }
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on bounded samples, all host threads then one thread")
        ctops, dt, threads = cpu_baseline(args.cpu_sample_rows)
        ctops1, dt1, _ = cpu_baseline(args.cpu_sample_rows_1t, threads=1)
        sample = lambda r, t: (f"{r} of {T} token rows through fwd, dgrad and wgrad "
                               f"(3 x 2 x {r} x {IN} x {OUT} ops) plus the full 16.8M-weight update; {t:.1f} s")
        result["cpu_baseline"] = {
            "value": round(ctops, 5), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": sample(args.cpu_sample_rows, dt), "cpu_model": _cpu_model(),
            "host_threads": os.cpu_count(),
            "one_thread": {"value": round(ctops1, 5), "unit": "TOPS", "cores": 1,
                           "sample": sample(args.cpu_sample_rows_1t, dt1)}}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
