#!/usr/bin/env python3
"""Router benchmark on one MI355X: quantize + gate GEMM + top-k per step.

A step is one router call, router_forward: runtime NVFP4 quantization of the
step's bf16 activations, the block-scaled gate projection and the six-step
routing epilogue. At T <= 4 tokens the library runs the whole call as one
kernel launch. The default workload is the decode router: T=1, D=7168,
E=256, k=8, with 61 independent layer sets (token, NVFP4 gate weights, bias)
cycled call by call, inputs resident in HBM before timing. Gate weights are
quantized once at load time by the library itself (untimed).

The K timed steps are replayed from one HIP graph (decode loops are
graph-captured), bracketed by HIP events recorded on the stream the graph is
launched on; the eager rate and the two-call path (router_quantize, then
router_gate_topk) are reported alongside. The roofline's `traffic` comes from
the FETCH_SIZE / WRITE_SIZE counter summary committed under profiles/ and is
null when the kernel sources have changed since it was taken. The CPU
baseline is the oracle, timed on a bounded sample, with the host's core
count, CPU model and BLAS build.

The decode line also carries a `prefill` block: the same metric at T=8192
(D=7168, E=256, k=8), timed the same way, with the MFMA roofline of its gate
kernel (FLOP over the event-timed launch duration) against the fp16 peak and
against the library's MFMA probe. `--no-prefill` leaves it out.

`--copy-calibration MiB` instead times a plain device-to-device copy of that
size (the reference kernel for scaling the byte counters).

Prints one JSON line on stdout; progress goes to stderr.
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

METRIC = "router tokens/s (quant+gate GEMM+top-k) D=7168,E=256,k=8; µs/call at T=1"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_forward_T1_D7168_E256_k8_traffic.txt")


# Every source the decode kernel's translation unit is built from.
DECODE_SOURCES = ("gate_decode.hip", "gate_common.hpp", "nvfp4_device.hpp", "router_internal.hpp")


def kernel_source_hash():
    """sha256 over the decode kernel's sources, so a stale counter summary is not reported for a changed kernel."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "nvfp4_block_scaled_06_amd", "csrc")
    for name in DECODE_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(d, name), "rb").read())
    return h.hexdigest()


def committed_traffic(path=TRAFFIC_FILE):
    """HBM bytes per launch (fetch + write, copy-calibrated) from the committed counter summary, or None."""
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quant_bytes(c):
    """Algorithmic bytes of one quantize call: x read once (single pass) or twice, codes+scales written."""
    reads = 2 if c.T * c.D // 16 > 2048 else 1
    return reads * 2 * c.T * c.D + c.T * c.D * 9 // 16 + 4


def forward_bytes(c):
    """Algorithmic bytes of one single-launch router call: W, x (bf16) and bias read; codes, scales, gsa and
    routing written."""
    return c.E * c.D * 9 // 16 + 2 * c.T * c.D + 4 * c.E + c.T * c.D * 9 // 16 + 4 + 8 * c.T * c.k


def gate_flops(c):
    return 2 * c.T * c.E * c.D


def cpu_baseline(cfg, seconds):
    """The oracle as it stands, one router call after another on the host, for about `seconds`."""
    from nvfp4_block_scaled_06_amd import workloads as wl
    from oracle import quant_ref, router_ref

    c = wl.CONFIGS[cfg]
    nlayers = min(c.layers, 4)
    wq = [quant_ref.quantize_ref(wl.make_w(cfg, l)) for l in range(nlayers)]  # load time, untimed
    bias = [wl.make_bias(cfg, l) for l in range(nlayers)]
    if c.T * c.D > 64 * 7168:
        rows = 64
        xs = [wl.make_x(cfg)[:rows]]
    else:
        rows = c.T
        xs = [wl.make_x(cfg, l) for l in range(nlayers)]
    calls, t0 = 0, time.perf_counter()
    while True:
        l = calls % nlayers
        xq = quant_ref.quantize_ref(xs[l % len(xs)])
        L, _ = router_ref.logits_ref(*xq, *wq[l])
        router_ref.route_ref(L, bias[l], c.k, c.routed_scale)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # The oracle's only multi-threaded work is the BLAS matrix product, so the threads it actually uses are
    # BLAS's (the rest of it is single-threaded numpy).
    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])
    except Exception:
        cores = 1
    return {"value": calls * rows / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} oracle router calls of {rows} token(s) cycling {nlayers} of the layer sets "
                      f"({el:.1f} s; numpy float64, weights quantized beforehand)"}


def copy_calibration(torch, mib, reps):
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE readings calibrate the
    counters (reads and writes `mib` MiB per launch)."""
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)  # the runtime's device-to-device copy kernel
    # The same bytes through an elementwise kernel (read n, write n), in case the runtime copy is not counted.
    for _ in range(reps):
        torch.bitwise_not(src.view(torch.int32), out=dst.view(torch.int32))
    torch.cuda.synchronize()
    assert torch.equal(torch.bitwise_not(src), dst)
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": reps}), flush=True)


def probe_rates(torch, rt, c, nbytes, time_graph, steps, t_launch, eager):
    """What a kernel that only reads can reach: the library's streaming-read probe over a footprint of the
    gate's algorithmic bytes, cycled over as many buffers as there are layer sets and replayed like the
    router (the achievable rate for this footprint), and over 1 GiB (the achievable HBM bandwidth)."""
    dev = torch.device("cuda:0")
    fb = (nbytes + 15) // 16 * 16
    gen = torch.Generator(device=dev).manual_seed(0)
    bufs = [torch.randint(0, 256, (fb,), dtype=torch.uint8, device=dev, generator=gen) for _ in range(c.layers)]
    sink = torch.empty(8192, dtype=torch.int32, device=dev)

    def step_probe(i):
        rt.probe_read(bufs[i % len(bufs)], sink)

    for i in range(20):
        step_probe(i)
    torch.cuda.synchronize()
    if eager:
        cur = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for i in range(200):
            step_probe(i)
        e1.record(cur)
        torch.cuda.synchronize()
        t_small = e0.elapsed_time(e1) * 1e-3 / 200
    else:
        _, ev = time_graph(step_probe)
        t_small = ev / steps
    big = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    rt.probe_read(big, sink)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ev:
        a.record(cur)
        rt.probe_read(big, sink)
        b.record(cur)
    torch.cuda.synchronize()
    t_big = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    # One buffer read over and over (hot in L2), replayed like the router: the latency floor of such a read.
    t_one = None
    if not eager:
        _, ev_one = time_graph(lambda i: rt.probe_read(bufs[0], sink))
        t_one = ev_one / steps
    del big, bufs
    log(f"probe: {fb} B in {t_small * 1e6:.2f} us per launch; 1 GiB at {(1 << 30) / t_big / 1e9:.0f} GB/s")
    return {"kernel": "probe_read_kernel", "footprint_bytes": fb, "buffers": c.layers,
            "launch_us": t_small * 1e6, "achievable_gbs": fb / t_small / 1e9,
            "frac_of_achievable": t_small / t_launch, "hbm_1gib_gbs": (1 << 30) / t_big / 1e9,
            "one_hot_buffer_launch_us": None if t_one is None else t_one * 1e6}


def mfma_probe_tflops(torch, rt, iters=4000):
    """fp16 MFMA rate the chip sustains at its running clock: the library's MFMA probe (four independent
    32x32x16 chains per wavefront, four wavefronts per SIMD, no memory traffic), median of 5 launches."""
    sink = torch.empty(rt.MFMA_PROBE_SINK, dtype=torch.float32, device="cuda:0")
    rt.probe_mfma(iters, sink)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
    for a, b in ev:
        a.record(cur)
        rt.probe_mfma(iters, sink)
        b.record(cur)
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3
    tflops = 1024 * 4 * iters * 4 * 32768 / t / 1e12
    log(f"MFMA probe: {tflops:.0f} TFLOP/s fp16")
    return tflops


def lmhead_bench(torch, K, W, T=1, D=7168, N=129280):
    """Greedy NVFP4 lm_head (lmhead_argmax) over an N x D vocabulary matrix: K calls graph-replayed after W
    warm-ups, each streaming the packed weights (N D 9/16 bytes; 521 MB at the default size, twice the
    Infinity Cache, so every call reads HBM). Prints one JSON line with the HBM roofline."""
    from nvfp4_block_scaled_06_amd import router as rt

    rt.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ws = rt.Workspace(max(rt.lmhead_workspace_bytes(T, D, N), rt.workspace_bytes(N, D, 1, 1)), dev)
    g = torch.Generator(device=dev).manual_seed(1234)
    w = (torch.randn((N, D), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
    wq = rt.quantize(w, ws)
    del w
    xs = [rt.quantize((torch.randn((T, D), generator=g, device=dev)).to(torch.bfloat16), ws) for _ in range(8)]
    torch.cuda.synchronize()
    for i in range(W):
        rt.lmhead_argmax(xs[i % 8], wq, ws)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(gr, stream=st):
            for i in range(K):
                rt.lmhead_argmax(xs[i % 8], wq, ws)
    torch.cuda.current_stream().wait_stream(st)
    gr.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(cur)
    gr.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / K
    nbytes = N * D * 9 // 16 + T * D * 9 // 16 + 8 + 8 * T
    big = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    rt.probe_read(big, sink)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for a, b in ev:
        a.record(cur)
        rt.probe_read(big, sink)
        b.record(cur)
    torch.cuda.synchronize()
    probe = (1 << 30) / (float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3) / 1e9
    achieved = nbytes / t / 1e9
    log(f"lm_head N={N} D={D} T={T}: {t * 1e6:.1f} us per call, {achieved:.0f} GB/s; read probe {probe:.0f} GB/s")
    print(json.dumps({
        "metric": f"greedy NVFP4 lm_head GEMV+argmax calls/s, N={N} D={D} T={T}", "value": 1.0 / t, "unit": "calls/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "nvfp4 operands, f16 products, f32 accumulate", "data": "synthetic",
        "config": {"workload": f"lm_head decode T={T} D={D} N={N}", "entry": "lmhead_argmax", "launch": "hipgraph",
                   "us_per_call": t * 1e6},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "lmhead_argmax_kernel",
                     "algorithmic": f"{nbytes} B per launch", "read_probe_1gib_gbs": probe,
                     "frac_of_read_probe": achieved / probe},
        "cpu_baseline": None}), flush=True)


def grouped_bench(torch, gcfg, K, W):
    """The grouped NVFP4 layer (grouped_offsets + router_quantize over the flattened groups + grouped_gemm)
    on a GroupedConfig: K calls graph-replayed after W warm-ups, weights resident and quantized beforehand.
    Prints one JSON line; the roofline is the GEMM kernel's: HBM bytes at decode size (the weight stream),
    fp16 MFMA FLOP at prefill size."""
    from nvfp4_block_scaled_06_amd import router as rt
    from nvfp4_block_scaled_06_amd import workloads as wl

    rt.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    c = wl.GROUPED_CONFIGS[gcfg]
    R = c.G * c.P
    log(f"grouped layer {c.name}: G={c.G} P={c.P} D={c.D} N={c.N}")
    ws = rt.Workspace(max(rt.workspace_bytes(R, c.D, 16, 1), rt.workspace_bytes(c.N, c.D, 16, 1)), dev)
    w = torch.from_numpy(np.stack([wl.make_grouped_w(gcfg, g) for g in range(c.G)]).view(np.int16)).to(dev)
    wg = rt.quantize_grouped_weights(w, ws)  # load time
    del w
    x = torch.from_numpy(wl.make_grouped_x(gcfg).view(np.int16)).to(dev)
    rng_buf = torch.arange(c.G + 1, dtype=torch.int32, device=dev)  # allocated once, reused
    off = torch.empty(c.G + 1, dtype=torch.int32, device=dev)
    xq = rt.empty_nvfp4(R, c.D, dev)
    out = torch.empty((R, c.N), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        rt.grouped_offsets(rng_buf, c.P, out=off)
        rt.quantize(x, ws, out=xq)
        rt.grouped_gemm(xq, wg, off, c.P, out=out)

    for _ in range(W):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(K):
                step()
    torch.cuda.current_stream().wait_stream(st)
    g.replay()
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(cur)
    g.replay()
    e1.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t = e0.elapsed_time(e1) * 1e-3 / K
    # The GEMM kernel alone, event-timed per launch.
    n = min(K, 200)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(cur)
        rt.grouped_gemm(xq, wg, off, c.P, out=out)
        b.record(cur)
    torch.cuda.synchronize()
    tk = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3
    flops = 2 * R * c.N * c.D
    nbytes = c.G * c.N * c.D * 9 // 16 + 4 * c.G + R * c.D * 9 // 16 + 4 + 4 * (c.G + 1) + 4 * R * c.N
    gemv = c.P <= 4 and c.P * c.D <= 32768 and c.D <= 16384  # grouped_gemm's decode-size (GEMV) path
    if c.P <= 4:
        achieved = nbytes / tk / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "kernel": "grouped_gemv_kernel" if gemv else "grouped_mfma_kernel",
                "kernel_launch_us": tk * 1e6, "algorithmic": f"{nbytes} B per launch"}
    else:
        achieved = flops / tk / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None, "kernel": "grouped_mfma_kernel",
                "kernel_launch_us": tk * 1e6, "algorithmic": f"{flops} FLOP per launch"}
    log(f"{c.name}: {t * 1e6:.2f} us per call (offsets + quantize + GEMM); GEMM {tk * 1e6:.2f} us, "
        f"{roof['achieved']:.0f} {roof['unit']}")
    print(json.dumps({
        "metric": f"grouped NVFP4 layer rows/s, G={c.G} P={c.P} D={c.D} N={c.N}", "value": R / t, "unit": "rows/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": wall / K * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": ("nvfp4 operands, exact f16 products on the VALU (v_dot2), f32 accumulate" if gemv else
                  "nvfp4 operands, exact f16 products on 32x32x16 f16 MFMA, f32 accumulate"), "data": "synthetic",
        "config": {"workload": f"{c.name} G={c.G} P={c.P} D={c.D} N={c.N}",
                   "entry": "grouped_offsets + router_quantize + grouped_gemm", "launch": "hipgraph",
                   "us_per_call": t * 1e6, "gemm_launch_us": tk * 1e6},
        "roofline": roof, "cpu_baseline": None}), flush=True)


def path_dtype(c):
    """The arithmetic each gate path computes in (the operands stay NVFP4 throughout)."""
    if c.T <= 4:
        return "nvfp4 operands, exact f16 products on the VALU (v_dot2), f32 accumulate"
    if c.T <= 256:
        return "nvfp4 operands, exact f16 products on 16x16x32 f16 MFMA, f32 accumulate"
    return "nvfp4 operands, exact f16 products on 32x32x16 f16 MFMA, f32 accumulate"


class RouterBench:
    """One router shape made resident on the GPU, with the timing helpers its measurements share."""

    def __init__(self, torch, rt, wl, cfg, K, W):
        self.torch, self.rt, self.c, self.K, self.W = torch, rt, wl.CONFIGS[cfg], K, W
        c, dev = self.c, torch.device("cuda:0")
        log(f"workload cfg {c.cfg} {c.name}: T={c.T} D={c.D} E={c.E} k={c.k} layers={c.layers}")
        self.ws = rt.Workspace.for_shapes([(c.T, c.D, c.E, c.k), (c.E, c.D, c.E, c.k)], dev)
        self.wq, self.bias, self.xs = [], [], []
        for l in range(c.layers):
            w = torch.from_numpy(wl.make_w(c.cfg, l).view(np.int16)).to(dev)
            self.wq.append(rt.quantize(w, self.ws))  # load time
            del w
            self.bias.append(torch.from_numpy(wl.make_bias(c.cfg, l)).to(dev))
            self.xs.append(torch.from_numpy(wl.make_x(c.cfg, l).view(np.int16)).to(dev))
        self.xq = rt.empty_nvfp4(c.T, c.D, dev)
        self.out = (torch.empty((c.T, c.k), dtype=torch.int32, device=dev),
                    torch.empty((c.T, c.k), dtype=torch.float32, device=dev), None)
        torch.cuda.synchronize()
        log("inputs resident")

    def step_forward(self, i):
        c, l = self.c, i % self.c.layers
        self.rt.forward(self.xs[l], self.wq[l], self.bias[l], c.k, c.routed_scale, self.ws, xq=self.xq, out=self.out)

    def step_two_calls(self, i):
        c, l = self.c, i % self.c.layers
        self.rt.quantize(self.xs[l], self.ws, out=self.xq)
        self.rt.gate_topk(self.xq, self.wq[l], self.bias[l], c.k, c.routed_scale, self.ws, out=self.out)

    def time_eager(self, step):
        torch = self.torch
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(self.K):
            step(self.W + i)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    def time_graph(self, step):
        """(wall seconds, HIP-event seconds) of one replay of K captured steps."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(self.K):
                    step(self.W + i)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()  # untimed warm replay
        torch.cuda.synchronize()
        cur = torch.cuda.current_stream()  # replay() launches the graph on this stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(cur)
        g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        del g
        return dt, e0.elapsed_time(e1) * 1e-3

    def event_time(self, fn, n):
        """Mean duration of n eager launches of fn, each bracketed by HIP events on the launch stream."""
        torch = self.torch
        cur = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            ev[i][0].record(cur)
            fn(self.W + i)
            ev[i][1].record(cur)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e-3

    def run(self, eager_only):
        """Warm-up, then the timed router calls. Returns the measured figures."""
        c, K, rt = self.c, self.K, self.rt
        for step in (self.step_forward, self.step_two_calls):
            for i in range(self.W):
                step(i)
        self.torch.cuda.synchronize()
        r = {"eager_fwd": self.time_eager(self.step_forward), "eager_two": self.time_eager(self.step_two_calls),
             "graph_fwd": None, "graph_two": None, "ev_fwd": None}
        log(f"eager: forward {r['eager_fwd'] / K * 1e6:.2f} us/call, quantize+gate "
            f"{r['eager_two'] / K * 1e6:.2f} us/call")
        if not eager_only:
            r["graph_two"], _ = self.time_graph(self.step_two_calls)
            r["graph_fwd"], r["ev_fwd"] = self.time_graph(self.step_forward)
            log(f"graph: forward {r['graph_fwd'] / K * 1e6:.2f} us/call (events {r['ev_fwd'] / K * 1e6:.2f}), "
                f"quantize+gate {r['graph_two'] / K * 1e6:.2f} us/call")
        r["timed_s"] = r["eager_fwd"] if r["graph_fwd"] is None else r["graph_fwd"]
        nk = min(K, 500)
        r["tf"] = self.event_time(self.step_forward, nk)
        r["tq"] = self.event_time(lambda i: rt.quantize(self.xs[i % c.layers], self.ws, out=self.xq), nk)
        r["tg"] = self.event_time(lambda i: rt.gate_topk(self.xq, self.wq[i % c.layers], self.bias[i % c.layers],
                                                         c.k, c.routed_scale, self.ws, out=self.out), nk)
        log(f"launch times: forward {r['tf'] * 1e6:.2f} us, quantize {r['tq'] * 1e6:.2f} us, "
            f"gate {r['tg'] * 1e6:.2f} us")
        return r

    def config_fields(self, r):
        c, K = self.c, self.K
        return {
            "workload": f"{c.name} router T={c.T} D={c.D} E={c.E} k={c.k}, {c.layers} layer set(s) cycled",
            "T": c.T, "D": c.D, "E": c.E, "k": c.k,
            "entry": "router_forward",
            "launch": "eager" if r["graph_fwd"] is None else "hipgraph",
            "us_per_call": r["timed_s"] / K * 1e6,
            "eager_us_per_call": r["eager_fwd"] / K * 1e6,
            "two_call_us_per_call": (r["eager_two"] if r["graph_two"] is None else r["graph_two"]) / K * 1e6,
            "forward_launch_us": r["tf"] * 1e6,
            "quantize_launch_us": r["tq"] * 1e6,
            "gate_launch_us": r["tg"] * 1e6,
        }

    def prefill_roofline(self, r):
        """MFMA roofline of the prefill gate: its FLOP over its event-timed launch duration."""
        c = self.c
        achieved = gate_flops(c) / r["tg"] / 1e12
        probe = mfma_probe_tflops(self.torch, self.rt)
        return {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None, "kernel": "gate_mfma_kernel",
                "kernel_launch_us": r["tg"] * 1e6, "algorithmic": f"{gate_flops(c)} FLOP per launch",
                "mfma_probe_tflops": probe, "frac_of_mfma_probe": achieved / probe}


def cpu_host_facts():
    """Host facts for the CPU baseline: cores available to this process, CPU model, BLAS build and threads."""
    facts = {"host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None}
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                facts["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info

        facts["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
                         for i in threadpool_info()]
    except Exception:
        pass
    return facts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=2, help="router shape 1..5 (2 = decode T=1)")
    ap.add_argument("--eager", action="store_true", help="time eager launches only (no graph replay)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill block (T=8192) that the decode line carries by default")
    ap.add_argument("--cold", action="store_true",
                    help="also time router calls that each follow a 1 GiB read (weights no longer in the Infinity Cache)")
    ap.add_argument("--lmhead", action="store_true",
                    help="time the greedy NVFP4 lm_head (129280 x 7168, T=1) instead of the router")
    ap.add_argument("--grouped", type=int, default=0, metavar="CFG",
                    help="time the grouped NVFP4 layer instead of the router (12 = decode size, 13 = prefill size)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="time a plain device copy of this many MiB instead of the router")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the router path is single-GPU.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration, max(args.steps, 1))
        return
    if args.lmhead:
        lmhead_bench(torch, min(args.steps, 200), min(args.warmup, 20))
        return
    if args.grouped:
        grouped_bench(torch, args.grouped, min(args.steps, 200), min(args.warmup, 20))
        return

    from nvfp4_block_scaled_06_amd import router as rt
    from nvfp4_block_scaled_06_amd import workloads as wl

    rt.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup
    rb = RouterBench(torch, rt, wl, args.config, K, W)
    c = rb.c
    r = rb.run(args.eager)

    if c.T > 256:
        roof = rb.prefill_roofline(r)
    elif c.T > 4:
        # Batched decode: a few hundred MFLOP against a megabyte of weights; bytes bound it (in practice the
        # loads' and the handoff's latency). router_forward is two launches here (the amax pass, then the
        # fused quantize + gate + route kernel); the events around the timed replay give the call's duration,
        # both launches and the gap between them included.
        nbytes = forward_bytes(c)
        t_call = r["tf"] if r["ev_fwd"] is None else r["ev_fwd"] / K
        achieved = nbytes / t_call / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                "kernel": "batch_amax_zero_kernel + gate_batch_kernel (router_forward: two launches)",
                "launch_us": t_call * 1e6,
                "algorithmic": f"{nbytes} B per call",
                "probe": probe_rates(torch, rt, c, nbytes, rb.time_graph, K, t_call, args.eager)}
    else:
        # One launch per step: the events around the timed replay give the average launch duration.
        nbytes = forward_bytes(c)
        t_launch = r["tf"] if r["ev_fwd"] is None else r["ev_fwd"] / K
        achieved = nbytes / t_launch / 1e9
        traffic = committed_traffic() if (c.cfg == 2 and not args.eager) else None
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": "gate_decode_kernel (quantizing; the whole call is one launch)",
                "launch_us": t_launch * 1e6,
                "algorithmic": f"{nbytes} B per launch",
                "probe": probe_rates(torch, rt, c, nbytes, rb.time_graph, K, t_launch, args.eager)}

    cold = None
    if args.cold:
        # A 1 GiB streaming read before every call evicts the 256 MB Infinity Cache, so the call's weights
        # come from HBM. Graphs of 100 (read, call) pairs and of 100 reads alone are replayed; the
        # difference per pair is the cold call.
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.empty(8192, dtype=torch.int32, device=dev)

        def replay(with_call):
            g = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(g, stream=s):
                    for i in range(100):
                        rt.probe_read(flush, sink)
                        if with_call:
                            rb.step_forward(W + i)
            torch.cuda.current_stream().wait_stream(s)
            g.replay()
            torch.cuda.synchronize()
            cs = torch.cuda.current_stream()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(cs)
            g.replay()
            e1.record(cs)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3

        cold = (replay(True) - replay(False)) / 100
        del flush
        log(f"cold (after a 1 GiB read): forward {cold * 1e6:.2f} us per call")

    timed_s = r["timed_s"]
    ms = timed_s / K * 1e3
    config = rb.config_fields(r)
    if cold is not None:
        config["cold_forward_launch_us"] = cold * 1e6
    config["parallelism"] = "single GPU"
    line = {
        "metric": METRIC,
        "value": c.T * K / timed_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype(c),
        "data": "synthetic",
        "config": config,
        "roofline": roof,
    }

    if c.T <= 4 and not args.no_prefill:
        # The same metric at the prefill shape (T=8192, D=7168, E=256, k=8): tokens/s of router_forward and
        # the MFMA roofline of its gate kernel, timed the same way with the same step counts.
        del rb
        torch.cuda.empty_cache()
        pb = RouterBench(torch, rt, wl, 4, K, min(W, 5))
        pr = pb.run(args.eager)
        line["prefill"] = {"value": pb.c.T * K / pr["timed_s"], "unit": "tokens/s", "dtype": path_dtype(pb.c),
                           "config": pb.config_fields(pr), "roofline": pb.prefill_roofline(pr)}
        del pb

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        cpu = cpu_baseline(c.cfg, args.cpu_seconds)
        cpu.update(cpu_host_facts())
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
