"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Codes, scale bytes and gsa must match bit for bit; logits within 1e-5 of the
|x||w| scale; top-k and weights under the near-tie rules of oracle.check. Small
shapes are compared in full; the 8192- and 32768-token shapes run in full on
the GPU and are compared on sampled rows that the oracle computes one by one.
"""

import numpy as np
import pytest
import torch

from conftest import bf16_exact, hex_bytes, load_golden
from nvfp4_block_scaled_06_amd import router as rt
from nvfp4_block_scaled_06_amd import workloads as wl
from oracle import check, quant_ref, router_ref

pytestmark = pytest.mark.gpu

WS_BYTES = 32 << 20


def log(msg):
    print(f"[gpu-parity] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rt.load_library()
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


@pytest.fixture(scope="module")
def ws(dev):
    # Large enough for every workload's call (the library sizes its own needs).
    need = max(rt.workspace_bytes(c.T, c.D, c.E, c.k) for c in wl.CONFIGS.values())
    return rt.Workspace(max(WS_BYTES, need), dev)


def to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def gpu_quant(bits, dev, ws, override=None):
    x = to_dev(bits, dev)
    ov = None if override is None else torch.tensor([override], dtype=torch.float32, device=dev)
    q = rt.quantize(x, ws, gsa_override=ov)
    torch.cuda.synchronize()
    return q


def host(q):
    return q.codes.cpu().numpy(), q.scales.cpu().numpy(), q.gscale.cpu().numpy()


def assert_quant(q, ref, what):
    fails = check.check_quant(*host(q), ref)
    assert not fails, f"{what}:\n" + "\n".join(fails)


def full_gsa(bits, chunk=4096):
    """The oracle's global scale of a large tensor, its amax taken chunk by chunk."""
    amax = max(quant_ref.amax_ref(bits[i:i + chunk]) for i in range(0, bits.shape[0], chunk))
    return quant_ref.gsa_ref(amax)


# ----------------------------------------------------------------------------- quantizer


@pytest.mark.parametrize("case", load_golden("quant_worked_examples.json")["cases"], ids=lambda c: c["name"])
def test_quant_worked_examples(dev, ws, case):
    log(f"quant worked example {case['name']}")
    bits = bf16_exact(case["x"])[None, :]
    c, s, g = host(gpu_quant(bits, dev, ws, case["gsa_override"]))
    assert f"{int(g.view(np.uint32)[0]):08X}" == case["expect_gsa_hex"]
    assert s[0].tolist() == hex_bytes(case["expect_scales_hex"]).tolist()
    assert c[0].tolist() == hex_bytes(case["expect_codes_hex"]).tolist()


def all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[((b >> 7) & 0xFF) != 0xFF]  # 65280 patterns, a multiple of 16


@pytest.mark.parametrize("override", [None, 1.0, 1e-3, 0.37, 7e-39, 1e-44, 1e30])
def test_quant_every_bf16_pattern(dev, ws, override):
    """Each finite bf16 value once, shuffled into blocks, under several global scales."""
    log(f"quant every bf16 pattern, override={override}")
    b = all_finite_bf16()
    b = b[np.random.default_rng(17).permutation(b.size)].reshape(-1, 256)
    assert_quant(gpu_quant(b, dev, ws, override), quant_ref.quantize_ref(b, override), f"override {override}")
    # The single-workgroup kernel on a slice of the same data.
    sub = b[:128]
    assert_quant(gpu_quant(sub, dev, ws, override), quant_ref.quantize_ref(sub, override), "single-wg slice")


def test_quant_near_threshold_values(dev, ws):
    """bf16 values sitting on or next to every E2M1 threshold of their block (forces the exact path)."""
    log("quant near-threshold values")
    rng = np.random.default_rng(23)
    rows = []
    for _ in range(64):
        s = float(2.0 ** rng.integers(-8, 8)) * (1 + rng.integers(0, 8) / 8)
        t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]) * s
        v = np.concatenate([t, t * (1 + 2 ** -8), t * (1 - 2 ** -8), -t])
        rows.append(v[:32].astype(np.float32))
    bits = wl.bf16_bits(np.stack(rows))
    for ov in (None, 1.0, 3e-3):
        assert_quant(gpu_quant(bits, dev, ws, ov), quant_ref.quantize_ref(bits, ov), f"override {ov}")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_quant_small_configs(dev, ws, cfg):
    c = wl.CONFIGS[cfg]
    for layer in range(min(c.layers, 3)):
        log(f"quant cfg {cfg} layer {layer}: x [{c.T},{c.D}], W [{c.E},{c.D}]")
        x = wl.make_x(cfg, layer)
        assert_quant(gpu_quant(x, dev, ws), quant_ref.quantize_ref(x), f"x cfg {cfg} layer {layer}")
        w = wl.make_w(cfg, layer)
        assert_quant(gpu_quant(w, dev, ws), quant_ref.quantize_ref(w), f"W cfg {cfg} layer {layer}")


@pytest.fixture(scope="module")
def big_inputs():
    return {}


def get_big(big_inputs, cfg):
    if cfg not in big_inputs:
        log(f"generating full-size inputs for cfg {cfg}")
        big_inputs[cfg] = (wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg))
    return big_inputs[cfg]


@pytest.mark.parametrize("cfg", [4, 5])
def test_quant_full_size_sampled(dev, ws, big_inputs, cfg):
    c = wl.CONFIGS[cfg]
    x, w, _ = get_big(big_inputs, cfg)
    log(f"quant full size cfg {cfg}: [{c.T},{c.D}]")
    q = gpu_quant(x, dev, ws)
    gsa = full_gsa(x)
    rows = wl.sample_rows(c.T, 64, seed=cfg)
    ref = quant_ref.quantize_ref(x[rows], gsa_override=gsa)
    got = (q.codes[torch.from_numpy(rows).to(dev)].cpu().numpy(), q.scales[torch.from_numpy(rows).to(dev)].cpu().numpy(),
           q.gscale.cpu().numpy())
    fails = check.check_quant(*got, ref)
    assert not fails, "\n".join(fails)
    # Every scale byte is a finite E4M3 value (never the NaN pattern, never above 448).
    assert int(q.scales.max().item()) <= 0x7E


def test_quant_edges(dev, ws):
    cases = {
        "zeros": np.zeros((3, 64), dtype=np.uint16),
        "negative zeros": np.full((2, 32), 0x8000, dtype=np.uint16),
        "one block": wl.bf16_bits(np.random.default_rng(1).standard_normal((1, 16)).astype(np.float32)),
        "tiny values (subnormal gsa)": wl.bf16_bits(
            (np.random.default_rng(2).standard_normal((4, 64)) * 2.0 ** -128).astype(np.float32)),
    }
    for nblocks in (2047, 2048, 2049, 4097):
        cases[f"{nblocks} blocks"] = wl.bf16_bits(
            np.random.default_rng(nblocks).standard_normal((nblocks, 16)).astype(np.float32))
    cases["ragged rows"] = wl.bf16_bits(np.random.default_rng(3).standard_normal((37, 48)).astype(np.float32))
    for name, bits in cases.items():
        log(f"quant edge {name} {bits.shape}")
        assert_quant(gpu_quant(bits, dev, ws), quant_ref.quantize_ref(bits), name)
    # A too-small static scale: block scales saturate at 448 (the failure the runtime scale fixed).
    bits = wl.make_x(3)
    ov = float(quant_ref.gsa_ref(quant_ref.amax_ref(bits))) / 10
    log("quant static-scale saturation")
    q = gpu_quant(bits, dev, ws, ov)
    ref = quant_ref.quantize_ref(bits, ov)
    assert_quant(q, ref, "saturating override")
    assert (ref[1] == 0x7E).any()
    # Empty input: gsa 0, nothing else written.
    log("quant empty")
    q = gpu_quant(np.zeros((0, 64), dtype=np.uint16), dev, ws)
    assert float(q.gscale.cpu()[0]) == 0.0


# ----------------------------------------------------------------------------- gate + routing


def run_router(dev, ws, x_bits, w_bits, bias, k, r, want_logits=True):
    xq = gpu_quant(x_bits, dev, ws)
    wq = gpu_quant(w_bits, dev, ws)
    b = torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(dev)
    idx, w, logits = rt.gate_topk(xq, wq, b, k, r, ws, want_logits=want_logits)
    torch.cuda.synchronize()
    return xq, wq, idx.cpu().numpy(), w.cpu().numpy(), None if logits is None else logits.cpu().numpy()


def assert_route(ref, idx, w, logits, k, r, what, rows=None):
    fails = []
    if logits is not None:
        fails += check.check_logits(logits, ref["L"], ref["A"])
    fails += check.check_topk(idx, w, ref["s"], ref["b"], k, r, rows=rows)
    assert not fails, f"{what}:\n" + "\n".join(fails)
    if logits is not None:
        ra, rel = check.logit_error_stats(logits, ref["L"], ref["A"])
        log(f"{what}: max |dL|/A = {ra:.3g}, max rel err (|L| >= median) = {rel:.3g}")


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_gate_small_configs(dev, ws, cfg):
    c = wl.CONFIGS[cfg]
    for layer in range(min(c.layers, 3)):
        log(f"gate cfg {cfg} layer {layer}")
        x, w, bias = wl.make_x(cfg, layer), wl.make_w(cfg, layer), wl.make_bias(cfg, layer)
        xq, wq, idx, wts, logits = run_router(dev, ws, x, w, bias, c.k, c.routed_scale)
        ref = router_ref.router_ref(x, w, bias, c.k, c.routed_scale)
        assert_quant(xq, ref["xq"], "x")
        assert_quant(wq, ref["wq"], "W")
        assert_route(ref, idx, wts, logits, c.k, c.routed_scale, f"cfg {cfg} layer {layer}")


@pytest.mark.parametrize("cfg", [4, 5])
def test_gate_full_size_sampled(dev, ws, big_inputs, cfg):
    c = wl.CONFIGS[cfg]
    x, w, bias = get_big(big_inputs, cfg)
    log(f"gate full size cfg {cfg}: T={c.T} E={c.E}")
    xq, wq, idx, wts, logits = run_router(dev, ws, x, w, bias, c.k, c.routed_scale)
    rows = wl.sample_rows(c.T, 64, seed=cfg)
    gsa = full_gsa(x)
    xr = quant_ref.quantize_ref(x[rows], gsa_override=gsa)
    wr = quant_ref.quantize_ref(w)
    L, A = router_ref.logits_ref(*xr, *wr)
    ridx, rw, s, b = router_ref.route_ref(L, bias, c.k, c.routed_scale)
    ref = {"L": L, "A": A, "s": s, "b": b}
    assert_route(ref, idx[rows], wts[rows], logits[rows], c.k, c.routed_scale, f"cfg {cfg} sampled", rows=rows)
    # Properties that hold on every row: distinct valid experts, weights summing to r.
    assert np.all((idx >= 0) & (idx < c.E))
    srt = np.sort(idx, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1])
    np.testing.assert_allclose(wts.sum(axis=1), c.routed_scale, rtol=1e-5)


def synth(shape, seed, scale=1.0):
    return wl.bf16_bits((np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("T,D,E,k", [
    (1, 32, 16, 1),        # smallest D, top-1
    (5, 256, 16, 16),      # k = E
    (7, 512, 20, 3),       # E not a multiple of 16
    (3, 1024, 512, 32),    # largest E and k
    (17, 768, 256, 8),     # ragged 16-row tiles
    (256, 1024, 256, 8),   # largest split-gate T
    (257, 1024, 256, 8),   # smallest MFMA-gate T, ragged row tile
    (300, 2048, 384, 8),   # MFMA gate, 3 expert tiles per wave
    (65, 4096, 100, 6),    # E not a multiple of 32 (tile gate at this T)
    (96, 8192, 64, 4),
    (33, 1056, 64, 4),     # tile gate: D not a multiple of 128, ragged row tile
    (200, 160, 48, 5),     # tile gate: fewer K steps than wavefronts
    (600, 1056, 100, 6),   # MFMA gate: D not a multiple of 128, E not a multiple of 32
    (640, 384, 200, 8),    # MFMA gate, experts split over workgroups, second block partly empty
    (512, 512, 512, 32),   # MFMA gate, largest E and k
    (8200, 256, 256, 8),   # split experts, ragged last token block
])
def test_gate_shapes(dev, ws, T, D, E, k):
    log(f"gate shape T={T} D={D} E={E} k={k}")
    x, w = synth((T, D), T * 1000 + D), synth((E, D), E * 1000 + D, 0.02)
    bias = np.random.default_rng(E).uniform(-0.01, 0.01, E).astype(np.float32)
    xq, wq, idx, wts, logits = run_router(dev, ws, x, w, bias, k, 2.5)
    ref = router_ref.router_ref(x, w, bias, k, 2.5)
    assert_quant(xq, ref["xq"], "x")
    assert_route(ref, idx, wts, logits, k, 2.5, f"T={T} D={D} E={E} k={k}")


@pytest.mark.parametrize("T", [4, 300])
def test_gate_zero_input_ties_go_to_lower_expert(dev, ws, T):
    """x == 0: every score is 0.5, selection is the top-k of bias with exact ties broken by index."""
    E, D, k = 64, 256, 8
    bias = np.round(np.random.default_rng(5).uniform(-1, 1, E), 1).astype(np.float32)  # many exact ties
    x = np.zeros((T, D), dtype=np.uint16)
    w = synth((E, D), 9, 0.02)
    log(f"gate zero input T={T}")
    xq, wq, idx, wts, logits = run_router(dev, ws, x, w, bias, k, 2.5)
    want = np.lexsort((np.arange(E), -bias.astype(np.float64)))[:k]
    assert np.all(idx == want[None, :]), (idx[0], want)
    assert np.all(wts == np.float32(2.5 / k))
    assert np.all(logits == 0.0)


def test_gate_empty_batch(dev, ws):
    log("gate T=0")
    w = synth((16, 64), 1, 0.02)
    wq = gpu_quant(w, dev, ws)
    xq = rt.empty_nvfp4(0, 64, dev)
    b = torch.zeros(16, dtype=torch.float32, device=dev)
    idx, wts, _ = rt.gate_topk(xq, wq, b, 2, 1.0, ws)
    torch.cuda.synchronize()
    assert idx.shape == (0, 2)


def test_gate_is_deterministic(dev, ws):
    c = wl.CONFIGS[3]
    x, w, bias = wl.make_x(3), wl.make_w(3), wl.make_bias(3)
    log("gate determinism cfg 3")
    a = run_router(dev, ws, x, w, bias, c.k, c.routed_scale)
    b = run_router(dev, ws, x, w, bias, c.k, c.routed_scale)
    assert np.array_equal(a[2], b[2]) and np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))
    assert np.array_equal(a[4].view(np.uint32), b[4].view(np.uint32))


@pytest.mark.parametrize("cfg", [2, 3])
def test_graph_capture_replays_match_eager(dev, ws, cfg):
    """Both calls captured in a HIP graph (no syncs, allocations or memset nodes inside) and replayed."""
    c = wl.CONFIGS[cfg]
    x, w, bias = wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg)
    log(f"graph capture cfg {cfg}")
    xd = to_dev(x, dev)
    wq = gpu_quant(w, dev, ws)
    bd = torch.from_numpy(bias).to(dev)
    xq = rt.empty_nvfp4(c.T, c.D, dev)
    out = (torch.empty((c.T, c.k), dtype=torch.int32, device=dev), torch.empty((c.T, c.k), dtype=torch.float32, device=dev),
           torch.empty((c.T, c.E), dtype=torch.float32, device=dev))
    rt.quantize(xd, ws, out=xq)
    rt.gate_topk(xq, wq, bd, c.k, c.routed_scale, ws, out=out)
    torch.cuda.synchronize()
    eager = [t.clone() for t in out]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rt.quantize(xd, ws, out=xq)
            rt.gate_topk(xq, wq, bd, c.k, c.routed_scale, ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in out:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, eager):
            assert torch.equal(a, b), f"replay {rep} differs"


# ----------------------------------------------------------------------------- router_forward


@pytest.mark.parametrize("cfg,T,D,E,k", [(2, 1, 7168, 256, 8), (None, 3, 7168, 256, 8), (None, 4, 2048, 384, 8),
                                         (None, 2, 16384, 64, 4), (None, 9, 7168, 256, 8), (1, 4, 256, 16, 2),
                                         (None, 4, 16384, 512, 32),  # single launch at its largest D, E and k
                                         (None, 1, 16416, 100, 5)])  # D past the single launch: two-call path
def test_forward_matches_oracle(dev, ws, cfg, T, D, E, k):
    """router_forward (single launch at decode sizes) gives the quantizer's bytes and the oracle's routing."""
    if cfg is not None:
        x, w, bias = wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg)
        r = wl.CONFIGS[cfg].routed_scale
    else:
        x, w = synth((T, D), 7 * T + D), synth((E, D), 11 * E + D, 0.02)
        bias = np.random.default_rng(E + T).uniform(-0.01, 0.01, E).astype(np.float32)
        r = 2.5
    log(f"forward T={T} D={D} E={E} k={k}")
    wq = gpu_quant(w, dev, ws)
    b = torch.from_numpy(bias).to(dev)
    xq, (idx, wts, logits) = rt.forward(to_dev(x, dev), wq, b, k, r, ws, want_logits=True)
    torch.cuda.synchronize()
    ref = router_ref.router_ref(x, w, bias, k, r)
    assert_quant(xq, ref["xq"], "x via router_forward")
    assert_route(ref, idx.cpu().numpy(), wts.cpu().numpy(), logits.cpu().numpy(), k, r, f"forward T={T}")


def test_forward_static_scale_override(dev, ws):
    c = wl.CONFIGS[2]
    x, w, bias = wl.make_x(2, 3), wl.make_w(2, 3), wl.make_bias(2, 3)
    ov = float(quant_ref.gsa_ref(quant_ref.amax_ref(x))) / 4
    log("forward with gsa override")
    wq = gpu_quant(w, dev, ws)
    xq, (idx, wts, logits) = rt.forward(to_dev(x, dev), wq, torch.from_numpy(bias).to(dev), c.k, c.routed_scale, ws,
                                        gsa_override=torch.tensor([ov], dtype=torch.float32, device=dev),
                                        want_logits=True)
    torch.cuda.synchronize()
    ref = router_ref.router_ref(x, w, bias, c.k, c.routed_scale, gsa_override=ov)
    assert_quant(xq, ref["xq"], "x (override)")
    assert_route(ref, idx.cpu().numpy(), wts.cpu().numpy(), logits.cpu().numpy(), c.k, c.routed_scale, "override")


def test_forward_graph_replay_cycles_layers(dev, ws):
    """Decode loop as the benchmark runs it: several layer sets captured in one graph, replayed twice."""
    c = wl.CONFIGS[2]
    L = 5
    xs = [to_dev(wl.make_x(2, l), dev) for l in range(L)]
    wqs = [gpu_quant(wl.make_w(2, l), dev, ws) for l in range(L)]
    bs = [torch.from_numpy(wl.make_bias(2, l)).to(dev) for l in range(L)]
    xq = [rt.empty_nvfp4(1, c.D, dev) for _ in range(L)]
    outs = [(torch.empty((1, c.k), dtype=torch.int32, device=dev), torch.empty((1, c.k), dtype=torch.float32, device=dev),
             None) for _ in range(L)]
    log("forward graph replay")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for l in range(L):
                rt.forward(xs[l], wqs[l], bs[l], c.k, c.routed_scale, ws, xq=xq[l], out=outs[l])
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(2):
        for o in outs:
            o[0].zero_()
            o[1].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            ref = router_ref.router_ref(wl.make_x(2, l), wl.make_w(2, l), wl.make_bias(2, l), c.k, c.routed_scale)
            fails = check.check_topk(outs[l][0].cpu().numpy(), outs[l][1].cpu().numpy(), ref["s"], ref["b"], c.k,
                                     c.routed_scale)
            assert not fails, f"replay {rep} layer {l}: " + "; ".join(fails)
