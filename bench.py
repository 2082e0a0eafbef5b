#!/usr/bin/env python3
"""Benchmark of the W4A16 GEMM library on one MI355X.

Headline (the step that is timed): one W4A16 GEMM at the decode workload
M=1, N=17408, K=5120, group 128 (bf16 activations, packed int4 weights,
fp32 accumulation, bf16 output), reported as effective weight bandwidth:
(N*K/2 packed bytes + N*K/128*2 scale bytes) per step / time per step.

All inputs are synthetic (seeded, see synth/gen.py) and resident in HBM
before the timed region: W eager warm-up steps, then untimed graph replays
of the K steps that let the GPU clocks settle, then exactly K eager steps
between HIP events, enqueued behind enough untimed replays that the GPU runs
them back to back. Weights and scales are rotated over enough copies
(>= 512 MB) that the 256 MB Infinity Cache cannot serve them from one step
to the next. The other workloads (small-batch split-K decode, deep prefill,
grouped, batched, the four decoder GEMMs of a layer at M=1322 with group
sizes 32 and 128) are measured the same way and reported under "workloads".

Output: one JSON line on stdout. `--gpus N` with N > 1 exits with a message:
the library is single-GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s at M=1 decode; TFLOP/s at M=1322 prefill (1x MI355X)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ROTATE_BYTES = 512 << 20
# GPU work run back to back before the timed replay (clock settling)
SETTLE_S = 0.1
SETTLE_MAX_S = 1.0
# GPU work queued ahead of the timed eager steps, at least (see time_steps)
LEAD_S = 0.02
# untimed eager steps between the lead's replays and the timed steps
LEAD_EAGER = 4
# host enqueue time per step assumed when there is no warmup to measure it
HOST_STEP_GUESS_S = 100e-6
# the decode GEMV at M=1, N=17408, K=5120, split_k 1 (40 groups per slice ->
# 2-row blocks, 5 instructions per block; a two-deep ring of weight blocks per
# wave; one 8-wave workgroup per compute unit, x in registers)
DECODE_KERNEL = "w4a16::gemv_mfma_kernel<2, 5, 2, 8>"
# HBM bytes per launch of the decode GEMV from rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE, KiB per dispatch, taken on this kernel), scaled by the factors a
# plain copy kernel of known size reads from the same counters (FETCH x2.00,
# WRITE x1.00); None when the kernel has changed since the counters were taken
TRAFFIC_DECODE_GEMV = {
    "kernel": DECODE_KERNEL,
    "fetch_kib_counter": 22545.51, "fetch_factor": 2.00,
    "write_kib_counter": 40.01, "write_factor": 1.00,
    "bytes": int((22545.51 * 2.00 + 40.01 * 1.00) * 1024),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def eff_weight_bytes(N, K, G=1):
    return G * (N * K // 2 + N * (K // 128) * 2)


class Dev:
    """Device copies of a workload, with `copies` rotated weight/scale sets."""

    def __init__(self, c, copies=1):
        import torch
        import bf16_activation_quantized_amd as w4
        d = torch.device("cuda:0")
        self.x = torch.from_numpy(c.x.view(np.int16)).to(d).view(torch.bfloat16)
        s = torch.from_numpy(c.s.view(np.int16)).to(d).view(torch.bfloat16)
        q = torch.from_numpy(c.q).to(d)
        w = w4.w4a16_pack_int4(q)
        del q
        self.w = [w] + [w.clone() for _ in range(copies - 1)]
        self.s = [s] + [s.clone() for _ in range(copies - 1)]
        self.m_sizes = None if c.m_sizes is None else torch.from_numpy(c.m_sizes).to(d)
        torch.cuda.synchronize()


def time_steps(step, steps, warmup, settle_s=SETTLE_S):
    """W untimed eager warmup steps (their host enqueue time is measured);
    then the K steps are captured once in a HIP graph on a side stream (the
    library enqueues only kernels, so the capture is exact) and replayed
    untimed, in chunks of about 20 ms of GPU work, until at least `settle_s`
    seconds have run back to back and the shader clock has settled: it has
    reached 95 % of its highest DPM level, or stopped rising from one chunk to
    the next (under the decode GEMV's load it climbs from idle for a few
    hundred milliseconds; under prefill's it sinks to a power-limited level),
    at most SETTLE_MAX_S. The timed region is then exactly K eager calls of
    the step, enqueued between two HIP events on that stream behind untimed
    replays that keep the GPU busy for longer than the host takes to enqueue
    them (at least LEAD_S, and three times the warmup's host enqueue time for
    K steps), and behind LEAD_EAGER untimed eager steps: t0 .. t1 spans the K steps' GPU execution back to back, with no
    host gap and no graph-launch boundary inside (a replay of a 20-step graph
    carries several microseconds of launch cost of its own). All of it is
    bracketed by synchronisations. The shader and memory clocks are sampled
    while the settling replays run. Returns (total seconds, seconds per step,
    record of clocks and of the lead)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        h0 = time.perf_counter()
        for i in range(warmup):
            step(i)
        # host enqueue time per step (first calls included: an overestimate)
        h_step = (time.perf_counter() - h0) / warmup if warmup > 0 else HOST_STEP_GUESS_S
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        one = max(time.perf_counter() - w0, 1e-6)
        chunk = max(1, int(math.ceil(0.02 / one)))
        top = CLOCKS.top_sclk()

        def queue():
            for _ in range(chunk):
                g.replay()
            e = torch.cuda.Event()
            e.record(s)
            return e
        # one chunk always queued behind the one being waited for, so that the
        # GPU never idles between chunks
        t_settle = time.perf_counter()
        pending = [queue(), queue()]
        n, samples, prev = 2 * chunk, [], None
        while True:
            e = pending.pop(0)
            rec = CLOCKS.sample_while(e)          # while the replays run
            e.synchronize()
            elapsed = time.perf_counter() - t_settle
            last = rec.get("sclk_mhz_last") if rec else None
            if rec and "sclk_mhz_first" in rec:
                samples.append(rec)
            if elapsed >= SETTLE_MAX_S or (elapsed >= settle_s and (
                    last is None or (top and last >= 0.95 * top) or (prev is not None and last <= prev))):
                break
            prev = last
            pending.append(queue())
            n += chunk
        settled_s = time.perf_counter() - t_settle
        clocks = None
        if samples:
            clocks = dict(sclk_mhz_settle_first=samples[0]["sclk_mhz_first"],
                          sclk_mhz_median=samples[-1]["sclk_mhz_median"],
                          sclk_mhz_last=samples[-1]["sclk_mhz_last"], sclk_mhz_top=top,
                          sclk_samples=sum(r["sclk_samples"] for r in samples), mclk=samples[-1]["mclk"])
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        # the lead: untimed replays queued ahead of the first event keep the
        # GPU under the same load (clocks as settled) while the host enqueues
        # the K timed calls
        n_lead = max(1, int(math.ceil(max(LEAD_S, 3.0 * h_step * (steps + LEAD_EAGER)) / one)))
        h1 = time.perf_counter()
        for _ in range(n_lead):
            g.replay()
        # a few untimed eager steps after the replays: the switch from graph
        # replays to eager launches stays out of the timed region
        for i in range(LEAD_EAGER):
            step(i)
        t0.record(s)
        for i in range(steps):
            step(i)
        t1.record(s)
        host_s = time.perf_counter() - h1
        torch.cuda.synchronize()
    total = t0.elapsed_time(t1) / 1e3
    clocks = dict(clocks or {}, settle_replays=n, settle_ms=round(settled_s * 1e3, 2),
                  lead_ms=round(n_lead * one * 1e3, 2), host_enqueue_ms=round(host_s * 1e3, 2),
                  host_ahead=bool(host_s < n_lead * one))
    if not clocks["host_ahead"]:
        log(f"time_steps: the host took {host_s * 1e3:.2f} ms to enqueue the lead and the {steps} timed steps, "
            f"longer than the lead's {n_lead * one * 1e3:.2f} ms of GPU work: the GPU may have idled")
    return total, total / steps, clocks


class _Clocks:
    """Shader / memory clock of the visible GPU from sysfs (the current DPM
    level, marked '*'), found through the device's PCI address; None where
    the files are not readable."""

    def __init__(self):
        self.dev_dir = None

    def _find(self):
        if self.dev_dir is not None:
            return self.dev_dir
        self.dev_dir = ""
        try:
            import torch
            p = torch.cuda.get_device_properties(0)
            bus = "%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
            d = os.path.join("/sys/bus/pci/devices", bus)
            if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                self.dev_dir = d
        except Exception:
            pass
        return self.dev_dir

    @staticmethod
    def _current(path):
        try:
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return line.split(":", 1)[1].strip(" *\n")
        except OSError:
            return None
        return None

    def sample(self):
        d = self._find()
        if not d:
            return None
        return dict(sclk=self._current(os.path.join(d, "pp_dpm_sclk")),
                    mclk=self._current(os.path.join(d, "pp_dpm_mclk")))

    def top_sclk(self):
        """The highest shader clock DPM level (MHz), or None."""
        d = self._find()
        if not d:
            return None
        try:
            with open(os.path.join(d, "pp_dpm_sclk")) as f:
                lv = [int(l.split(":", 1)[1].strip(" *\n").lower().replace("mhz", "")) for l in f if ":" in l]
            return max(lv) if lv else None
        except (OSError, ValueError):
            return None

    def sample_while(self, event, every_s=0.01, most=40):
        """Samples every few milliseconds until `event` has completed (the
        GPU work queued before it is done): the first, median and last sclk
        (MHz) and the last mclk."""
        if not self._find():
            return None
        sclk, last = [], None
        while len(sclk) < most:
            last = self.sample()
            try:
                sclk.append(int(str(last["sclk"]).lower().replace("mhz", "")))
            except ValueError:
                pass
            if event.query():
                break
            time.sleep(every_s)
        if not sclk:
            return dict(mclk=last["mclk"] if last else None)
        return dict(sclk_mhz_first=sclk[0], sclk_mhz_median=int(np.median(sclk)), sclk_mhz_last=sclk[-1],
                    sclk_samples=len(sclk), mclk=last["mclk"])


CLOCKS = _Clocks()


def bench_decode(name, steps, warmup, split_k=0, path=None, variant=None):
    import torch
    import bf16_activation_quantized_amd as w4
    from synth import make_config, CONFIGS
    cfg = CONFIGS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    wb = eff_weight_bytes(N, K)
    copies = max(1, math.ceil(ROTATE_BYTES / wb))
    c = make_config(name)
    d = Dev(c, copies)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, split_k, path=path, variant=variant)
    ws = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device="cuda")
    sk = split_k if split_k else w4.w4a16_gemm_auto_split_k(M, N, K)

    def step(i):
        j = i % copies
        w4.w4a16_gemm(d.x, d.w[j], d.s[j], y=y, split_k=split_k, workspace=ws, path=path, variant=variant)

    total, t, clk = time_steps(step, steps, warmup)
    return dict(M=M, N=N, K=K, split_k=sk, weight_copies=copies, eff_weight_bytes=wb,
                us_per_step=t * 1e6, gbs=wb / t / 1e9, frac_hbm=wb / t / 1e9 / HBM_PEAK_GBS, clocks=clk), d, y


def bench_prefill(name, steps, warmup, variant=None):
    import torch
    import bf16_activation_quantized_amd as w4
    from synth import make_config, CONFIGS
    cfg = CONFIGS[name]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    c = make_config(name)
    d = Dev(c, 1)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    need = w4.w4a16_gemm_workspace_bytes(M, N, K, 0, path=None if variant is None else w4.PATH_TILE, variant=variant)
    ws = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device="cuda")
    path = None if variant is None else w4.PATH_TILE

    def step(i):
        w4.w4a16_gemm(d.x, d.w[0], d.s[0], y=y, workspace=ws, path=path, variant=variant)

    total, t, clk = time_steps(step, steps, warmup)
    flops = 2.0 * M * N * K
    return dict(M=M, N=N, K=K, us_per_step=t * 1e6,
                tflops=flops / t / 1e12, frac_bf16=flops / t / 1e12 / BF16_PEAK_TFLOPS, clocks=clk), d, y


def bench_grouped(name, steps, warmup, variant=None):
    import torch
    import bf16_activation_quantized_amd as w4
    from synth import make_config, CONFIGS
    cfg = CONFIGS[name]
    G, Mt, N, K = cfg["G"], cfg["M_total"], cfg["N"], cfg["K"]
    c = make_config(name)
    d = Dev(c, 1)
    y = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda")

    def step(i):
        w4.w4a16_gemm_grouped(d.x, d.w[0], d.s[0], d.m_sizes, y=y, variant=variant)

    total, t, clk = time_steps(step, steps, warmup)
    flops = 2.0 * Mt * N * K
    return dict(G=G, M_total=Mt, N=N, K=K, m_sizes=[int(v) for v in c.m_sizes], us_per_step=t * 1e6,
                tflops=flops / t / 1e12, frac_bf16=flops / t / 1e12 / BF16_PEAK_TFLOPS, clocks=clk), d, y


def bench_batched(name, steps, warmup, variant=None, split_k=0):
    import torch
    import bf16_activation_quantized_amd as w4
    from synth import make_config, CONFIGS
    cfg = CONFIGS[name]
    B, M, N, K = cfg["B"], cfg["M"], cfg["N"], cfg["K"]
    c = make_config(name)
    d = Dev(c, 1)
    x = d.x.view(B, M, K)
    y = torch.empty((B, M, N), dtype=torch.bfloat16, device="cuda")
    need = w4.w4a16_gemm_batched_workspace_bytes(B, M, N, K, split_k, variant)
    ws = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device="cuda")

    def step(i):
        w4.w4a16_gemm_batched(x, d.w[0], d.s[0], y=y, split_k=split_k, workspace=ws, variant=variant)

    total, t, clk = time_steps(step, steps, warmup)
    flops = 2.0 * B * M * N * K
    return dict(B=B, M=M, N=N, K=K, us_per_step=t * 1e6,
                tflops=flops / t / 1e12, frac_bf16=flops / t / 1e12 / BF16_PEAK_TFLOPS, clocks=clk), d, y


# the four decoder GEMMs of one layer at M = 1322 (N, K), after the per-GEMM
# table of the gfx1151 skinny-GEMM page (its model quantises with one scale
# per 32 k)
LAYER_GEMMS = (("gate_up", 19456, 2560), ("qkv", 6144, 2560), ("o_proj", 4096, 2560), ("down", 2560, 9728))
LAYER_M = 1322


def bench_layers(steps, warmup, group):
    """Each of the four layer GEMMs on its own (default path and tile choice)
    at the given group size, and the per-layer aggregate: total flops / total
    time of the four."""
    import torch
    import bf16_activation_quantized_amd as w4
    from synth import make_inputs
    M = LAYER_M
    out, tot_flops, tot_s = {}, 0.0, 0.0
    for name, N, K in LAYER_GEMMS:
        c = make_inputs(M, N, K, 1322 + N + K, group=group)
        d = Dev(c, 1)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        need = w4.w4a16_gemm_workspace_bytes(M, N, K, 0, group_size=group)
        ws = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device="cuda")

        def step(i, d=d, y=y, ws=ws):
            w4.w4a16_gemm(d.x, d.w[0], d.s[0], y=y, workspace=ws, group_size=group)

        _, t, _ = time_steps(step, steps, warmup)
        flops = 2.0 * M * N * K
        out[name] = dict(N=N, K=K, us_per_step=round(t * 1e6, 2), tflops=round(flops / t / 1e12, 1))
        tot_flops += flops
        tot_s += t
        del d, y, ws
    out["per_layer"] = dict(us=round(tot_s * 1e6, 2), tflops=round(tot_flops / tot_s / 1e12, 1),
                            frac_bf16=round(tot_flops / tot_s / 1e12 / BF16_PEAK_TFLOPS, 4))
    return dict(M=M, group_size=group, gemms=out)


def bench_pack(steps, warmup):
    import torch
    import bf16_activation_quantized_amd as w4
    from synth import CONFIGS
    N, K = CONFIGS["decode_gemv"]["N"], CONFIGS["decode_gemv"]["K"]
    q = torch.randint(0, 16, (N, K), dtype=torch.uint8, device="cuda")
    out = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")

    def step(i):
        w4.w4a16_pack_int4(q, out=out)

    total, t, _ = time_steps(step, steps, warmup)
    return dict(rows=N, K=K, us_per_step=t * 1e6, gbs=(N * K * 1.5) / t / 1e9)


def bench_dispatch(N, K, Ms, steps=20):
    """Path / tile height / split-K selection over M at one N x K: every
    explicit choice and the automatic one (split_k=0, no path), each
    timed over `steps` calls (time_steps) with rotated weight copies, in two passes
    (forward, then reverse order, so that the drift of the clocks under load
    favours no candidate; the faster pass counts). One JSON line per M: the
    automatic choice (path, variant, SK) and its time, the best explicit
    choice and their ratio."""
    import torch
    import bf16_activation_quantized_amd as w4
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    q = torch.randint(0, 16, (N, K), dtype=torch.uint8, device="cuda", generator=g)
    w = w4.w4a16_pack_int4(q)
    del q
    s = (torch.rand(N, K // 128, device="cuda", generator=g) * 0.015 + 0.005).to(torch.bfloat16)
    wb = eff_weight_bytes(N, K)
    copies = max(1, math.ceil(ROTATE_BYTES / wb))
    ws_ = [w] + [w.clone() for _ in range(copies - 1)]
    ss_ = [s] + [s.clone() for _ in range(copies - 1)]
    names = {w4.PATH_GEMV: "gemv", w4.PATH_SKINNY: "small-batch", w4.PATH_TILE: "tile"}
    sks = (1, 2, 4, 8, 16)
    out = []
    for M in Ms:
        x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        cands = [("auto", None, None, 0)]
        if M == 1:
            cands += [("gemv", w4.PATH_GEMV, 0, sk) for sk in sks]
        if M <= 48:
            for tiles in ((1, 2) if M <= 32 else (1,)):
                cands += [(f"small-batch{tiles}", w4.PATH_SKINNY, tiles, sk) for sk in sks]
        if M <= 16:   # the LDS-staged small-batch kernel, stage geometries 0 and 3
            for var in (3, 6):
                cands += [(f"small-batch-lds{var - 3}", w4.PATH_SKINNY, var, sk) for sk in sks]
        if M > 1:
            for rows in (48, 64, 80, 96, 112, 128, 144):
                for sk in (sks if M < 1024 else (1, 2)):
                    cands.append((f"tile{rows}", w4.PATH_TILE, rows, sk))
        apath, avar, ask = w4.w4a16_gemm_auto_config(M, N, K)
        times = {}
        for order in (cands, cands[::-1]):
            for name, path, var, sk in order:
                need = w4.w4a16_gemm_workspace_bytes(M, N, K, sk, path=path, variant=var)
                wsp = torch.empty(max(need // 4, 1) + 4, dtype=torch.float32, device="cuda")

                def step(i, path=path, var=var, sk=sk, wsp=wsp):
                    w4.w4a16_gemm(x, ws_[i % copies], ss_[i % copies], y=y, split_k=sk, workspace=wsp,
                                  path=path, variant=var)
                try:
                    _, t, _ = time_steps(step, steps, 3)
                    key = (name, var, sk)
                    times[key] = min(times.get(key, float("inf")), t * 1e6)
                except RuntimeError as e:   # a combination the library refuses
                    if order is cands:
                        log(f"dispatch M={M} {name} sk={sk}: {e}")
                del wsp
        auto_us = times[("auto", None, 0)]
        explicit = {k: v for k, v in times.items() if k[0] != "auto"}
        best = min(explicit.items(), key=lambda kv: kv[1])
        aname = f"{names[apath]}{'' if apath != w4.PATH_SKINNY else ('-lds' + str(avar - 3) if avar >= 3 else avar)}"
        if apath == w4.PATH_TILE:
            aname += str(avar)
        twin = [v for (n, var, sk), v in explicit.items()
                if sk == ask and var == avar and n.startswith(names[apath])]
        r = dict(N=N, K=K, M=M, auto=[aname, ask], auto_us=round(auto_us, 2),
                 auto_explicit_us=round(twin[0], 2) if twin else None,
                 best=[best[0][0], best[0][2], round(best[1], 2)], auto_vs_best=round(auto_us / best[1], 3),
                 auto_tflops=round(2.0 * M * N * K / auto_us / 1e6, 1), auto_gbs=round(wb / auto_us / 1e3, 1),
                 candidates=len(explicit),
                 times={f"{n}:{sk}": round(v, 2) for (n, var, sk), v in sorted(explicit.items(), key=lambda kv: kv[1])})
        print(json.dumps(r), flush=True)
        out.append(r)
        del x, y
    return out


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def oracle_time(name, budget_s=6.0, max_runs=3):
    """The CPU oracle (unpack + dequant + fp64 GEMM, numpy with a threaded
    BLAS) on the whole of workload `name`, timed on the host cores: the median
    of up to `max_runs` runs, fewer once `budget_s` has passed (at least one).
    Returns seconds per run and the number of runs."""
    import oracle
    from synth import make_config
    c = make_config(name)
    p = oracle.pack_int4(c.q)
    if name == "grouped":
        run = lambda: oracle.gemm_grouped(c.x, p, c.s, c.m_sizes)
    elif name == "batched":
        B = c.G
        xb = c.x.reshape(B, c.M // B, c.K)
        run = lambda: oracle.gemm_batched(xb, p, c.s)
    else:
        run = lambda: oracle.gemm(c.x, p, c.s)
    times = []
    t_start = time.perf_counter()
    while len(times) < max_runs:
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s:
            break
    return float(np.median(times)), len(times)


def cpu_oracle_record(name, work, unit, budget_s=6.0):
    """Per-workload oracle timing: `work` is the workload's effective weight
    bytes (unit GB/s) or flops (unit TFLOP/s)."""
    t, n = oracle_time(name, budget_s)
    val = work / t / (1e9 if unit == "GB/s" else 1e12)
    return dict(ms=round(t * 1e3, 2), value=val, unit=unit, runs=n, cores=int(_blas_threads()), kind="oracle",
                sample=f"whole workload, unpack + dequant + fp64 GEMM, median of {n}")


def cpu_baseline(budget_s=12.0):
    """The oracle (unpack + dequant + fp64 GEMV) on the decode workload, timed
    on the host cores."""
    from synth import CONFIGS
    blas_threads = _blas_threads()
    cfg = CONFIGS["decode_gemv"]
    t, n = oracle_time("decode_gemv", budget_s, max_runs=20)
    wb = eff_weight_bytes(cfg["N"], cfg["K"])
    return dict(value=wb / t / 1e9, unit="GB/s", cores=int(blas_threads), kind="oracle",
                sample=f"full decode workload M=1 N={cfg['N']} K={cfg['K']} (unpack + dequant + fp64 GEMV), "
                       f"{n} runs, median {t * 1e3:.1f} ms; numpy element-wise steps single-threaded, "
                       f"BLAS with {blas_threads} threads",
                host_cpus=os.cpu_count(), affinity_cpus=len(os.sched_getaffinity(0)),
                cpu_model=_cpu_model())


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", default=None,
                    choices=["decode_gemv", "decode_splitk", "prefill", "grouped", "batched", "pack", "tiny",
                             "dispatch", "layers"],
                    help="measure one workload only and print its record (for profiling)")
    ap.add_argument("--split-k", type=int, default=0)
    ap.add_argument("--variant", type=int, default=None)
    ap.add_argument("--path", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--shape", default="17408,5120", help="N,K of --only dispatch")
    ap.add_argument("--ms", default="1,2,16,32,64,96,128,192,256,384,512,1024,2048",
                    help="M values of --only dispatch")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this W4A16 GEMM library runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    import bf16_activation_quantized_amd as w4
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    w4._lib()   # fails loudly if the HIP library is not built

    if args.only == "dispatch":
        N, K = (int(v) for v in args.shape.split(","))
        bench_dispatch(N, K, [int(v) for v in args.ms.split(",")])
        return
    if args.only:
        if args.only in ("decode_gemv", "decode_splitk", "tiny"):
            r, _, _ = bench_decode(args.only, args.steps, args.warmup, args.split_k, args.path, args.variant)
        elif args.only == "prefill":
            r, _, _ = bench_prefill("prefill", args.steps, args.warmup, args.variant)
        elif args.only == "grouped":
            r, _, _ = bench_grouped("grouped", args.steps, args.warmup, args.variant)
        elif args.only == "batched":
            r, _, _ = bench_batched("batched", args.steps, args.warmup, args.variant, args.split_k)
        elif args.only == "layers":
            r = {f"g{g}": bench_layers(args.steps, args.warmup, g) for g in (32, 128)}
        else:
            r = bench_pack(args.steps, args.warmup)
        print(json.dumps({"workload": args.only, **r}), flush=True)
        return

    log("bench: decode_gemv (headline)")
    head, _, _ = bench_decode("decode_gemv", args.steps, args.warmup)
    log(f"bench: decode_gemv: {head['us_per_step']:.3f} us per step, clocks {head.get('clocks')}")
    wb = head["eff_weight_bytes"]
    ms_per_step = head["us_per_step"] / 1e3
    # dominant kernel of the step: the decode GEMV, one launch per step at
    # split_k 1; its average launch duration is the timed region / K (HIP
    # events on the launch stream around K back-to-back launches), so it
    # includes the dispatch gap between consecutive launches
    kern_s = head["us_per_step"] / 1e6
    achieved = wb / kern_s / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=TRAFFIC_DECODE_GEMV["bytes"] if TRAFFIC_DECODE_GEMV else None,
                    traffic_detail=TRAFFIC_DECODE_GEMV,
                    kernel=DECODE_KERNEL, bytes_per_launch=wb,
                    launch_us=round(head["us_per_step"], 3))

    workloads = {}
    if not args.no_extras:
        steps2 = max(20, args.steps // 2)
        log("bench: tiny")
        workloads["tiny"], _, _ = bench_decode("tiny", steps2, args.warmup)
        for sk in (0, 1, 2, 4, 8):
            log(f"bench: decode_splitk sk={sk}")
            workloads[f"decode_splitk_sk{sk if sk else 'auto'}"], _, _ = bench_decode(
                "decode_splitk", steps2, args.warmup, split_k=sk)
        log("bench: prefill")
        workloads["prefill"], _, _ = bench_prefill("prefill", steps2, args.warmup)
        log("bench: grouped")
        workloads["grouped"], _, _ = bench_grouped("grouped", steps2, args.warmup)
        log("bench: batched")
        workloads["batched"], _, _ = bench_batched("batched", steps2, args.warmup)
        for g in (32, 128):
            log(f"bench: layer GEMMs group {g}")
            workloads[f"layers_g{g}"] = bench_layers(steps2, args.warmup, g)
        log("bench: pack")
        workloads["pack_int4"] = bench_pack(steps2, args.warmup)
        torch.cuda.empty_cache()
        for k, r in workloads.items():
            if "us_per_step" in r:
                log(f"bench: {k}: {r['us_per_step']:.2f} us per step")

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline()
        # the oracle beside every workload, same process (the whole workload
        # each time, median of up to 3 runs)
        for key, name in (("tiny", "tiny"), ("decode_splitk_skauto", "decode_splitk"), ("prefill", "prefill"),
                          ("grouped", "grouped"), ("batched", "batched")):
            r = workloads.get(key)
            if r is None:
                continue
            log(f"bench: cpu oracle {name}")
            if "gbs" in r:
                rec = cpu_oracle_record(name, r["eff_weight_bytes"], "GB/s")
                rec["gpu_over_cpu"] = round(r["gbs"] / rec["value"], 1)
            else:
                rows = r["M_total"] if "M_total" in r else r["M"] * r.get("B", 1)
                flops = 2.0 * rows * r["N"] * r["K"]
                rec = cpu_oracle_record(name, flops, "TFLOP/s")
                rec["gpu_over_cpu"] = round(r["tflops"] / rec["value"], 1)
            r["cpu_oracle"] = rec
        head["cpu_oracle"] = dict(ms=round(head["eff_weight_bytes"] / cpu["value"] / 1e6, 2), value=cpu["value"],
                                  unit="GB/s", cores=cpu["cores"], kind="oracle",
                                  gpu_over_cpu=round(head["gbs"] / cpu["value"], 1))

    out = {
        "metric": METRIC,
        "value": round(head["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV M=1 N=17408 K=5120 group=128 (bf16 x packed int4, fp32 acc, bf16 out)",
                   "M": 1, "N": 17408, "K": 5120, "split_k": head["split_k"],
                   "weight_copies_rotated": head["weight_copies"], "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "clocks": head.get("clocks"),
        "workloads": dict(decode_gemv=head, **workloads),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
