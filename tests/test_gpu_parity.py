"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Codes, scale bytes and gsa must match bit for bit; logits within 1e-5 of the
|x||w| scale; top-k and weights under the near-tie rules of oracle.check. Every
gate call runs twice, with and without the logits output (the benchmark times
the call without it, which takes other code in the kernels' epilogues), and
both runs are compared with the oracle. Every shape is compared in full,
including the 8192- and 32768-token ones (the oracle works through them in
4096-row chunks under the whole tensor's global scale).
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


@pytest.mark.parametrize("bad", ["inf", "-inf", "nan"])
@pytest.mark.parametrize("T,D", [(1, 7168), (4, 256), (64, 7168), (300, 1024)])
def test_nonfinite_input_makes_gsa_nonfinite(dev, ws, bad, T, D):
    """Inf or NaN in x is a precondition violation whose device-visible flag is a non-finite global scale, on
    every quantizer path (one workgroup, two passes, and the single-launch router); nothing else is checked."""
    log(f"non-finite x ({bad}) T={T} D={D}")
    a = np.random.default_rng(T + D).standard_normal((T, D)).astype(np.float32)
    a[T // 2, D // 3] = {"inf": np.inf, "-inf": -np.inf, "nan": np.nan}[bad]
    x = wl.bf16_bits(a)
    q = gpu_quant(x, dev, ws)
    g = float(q.gscale.cpu()[0])
    assert (np.isnan(g) if bad == "nan" else g == np.inf), g
    E, k = 64, 4
    wq = gpu_quant(synth((E, D), 5, 0.02), dev, ws)
    xq, _ = rt.forward(to_dev(x, dev), wq, torch.zeros(E, dtype=torch.float32, device=dev), k, 2.5, ws)
    torch.cuda.synchronize()
    g = float(xq.gscale.cpu()[0])
    assert (np.isnan(g) if bad == "nan" else g == np.inf), g


# ----------------------------------------------------------------------------- gate + routing


def run_router(dev, ws, x_bits, w_bits, bias, k, r, want_logits=True):
    xq = gpu_quant(x_bits, dev, ws)
    wq = gpu_quant(w_bits, dev, ws)
    b = torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(dev)
    idx, w, logits = rt.gate_topk(xq, wq, b, k, r, ws, want_logits=want_logits)
    torch.cuda.synchronize()
    return xq, wq, idx.cpu().numpy(), w.cpu().numpy(), None if logits is None else logits.cpu().numpy()


def run_router_both(dev, ws, x_bits, w_bits, bias, k, r):
    """The gate with the logits output, then again without it (the timed configuration).

    Returns (xq, wq, idx, w, logits, idx_nolog, w_nolog)."""
    xq, wq, idx, w, logits = run_router(dev, ws, x_bits, w_bits, bias, k, r, want_logits=True)
    b = torch.from_numpy(np.ascontiguousarray(bias, dtype=np.float32)).to(dev)
    i2, w2, _ = rt.gate_topk(xq, wq, b, k, r, ws, want_logits=False)
    torch.cuda.synchronize()
    return xq, wq, idx, w, logits, i2.cpu().numpy(), w2.cpu().numpy()


# Plain relative logit error over the logits with |L| at or above their row's
# median |L| (the reading of "relative 1e-5" that the tolerance scale A relaxes
# only near cancellation): measured and bounded here.
PLAIN_REL_BOUND = 1e-5


def assert_route(ref, idx, w, logits, k, r, what, rows=None):
    fails = []
    if logits is not None:
        fails += check.check_logits(logits, ref["L"], ref["A"])
    fails += check.check_topk(idx, w, ref["s"], ref["b"], k, r, rows=rows)
    assert not fails, f"{what}:\n" + "\n".join(fails)
    if logits is not None:
        ra, rel = check.logit_error_stats(logits, ref["L"], ref["A"])
        log(f"{what}: max |dL|/A = {ra:.3g}, max rel err (|L| >= median) = {rel:.3g}")
        assert rel <= PLAIN_REL_BOUND, f"{what}: plain relative logit error {rel:.3g} above {PLAIN_REL_BOUND}"


def assert_route_both(ref, res, k, r, what):
    """Both runs of run_router_both against the oracle; the no-logits run must also equal the other bit for bit."""
    _, _, idx, w, logits, i2, w2 = res
    assert_route(ref, idx, w, logits, k, r, what)
    assert_route(ref, i2, w2, None, k, r, what + " (no logits)")
    assert np.array_equal(idx, i2) and np.array_equal(w.view(np.uint32), w2.view(np.uint32)), \
        f"{what}: routing differs between the runs with and without logits"


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_gate_small_configs(dev, ws, cfg):
    c = wl.CONFIGS[cfg]
    for layer in range(min(c.layers, 3)):
        log(f"gate cfg {cfg} layer {layer}")
        x, w, bias = wl.make_x(cfg, layer), wl.make_w(cfg, layer), wl.make_bias(cfg, layer)
        res = run_router_both(dev, ws, x, w, bias, c.k, c.routed_scale)
        ref = router_ref.router_ref(x, w, bias, c.k, c.routed_scale)
        assert_quant(res[0], ref["xq"], "x")
        assert_quant(res[1], ref["wq"], "W")
        assert_route_both(ref, res, c.k, c.routed_scale, f"cfg {cfg} layer {layer}")


CHUNK = 4096
FULL_CASES = [(4, i) for i in range(wl.CONFIGS[4].T // CHUNK)] + [(5, i) for i in range(wl.CONFIGS[5].T // CHUNK)]


@pytest.fixture(scope="module")
def full_size_runs():
    return {}


def get_full_run(full_size_runs, big_inputs, dev, ws, cfg):
    """Every entry point at the prefill sizes, once per config: router_quantize, router_gate_topk with and
    without logits, and router_forward without logits (the call the benchmark times). Host copies."""
    if cfg not in full_size_runs:
        c = wl.CONFIGS[cfg]
        x, w, bias = get_big(big_inputs, cfg)
        log(f"full size cfg {cfg}: GPU runs at T={c.T} D={c.D} E={c.E} k={c.k}")
        xd = to_dev(x, dev)
        wq = gpu_quant(w, dev, ws)
        bd = torch.from_numpy(bias).to(dev)
        xq = rt.quantize(xd, ws)
        idx, wts, logits = rt.gate_topk(xq, wq, bd, c.k, c.routed_scale, ws, want_logits=True)
        i2, w2, _ = rt.gate_topk(xq, wq, bd, c.k, c.routed_scale, ws, want_logits=False)
        xq3, (i3, w3, _) = rt.forward(xd, wq, bd, c.k, c.routed_scale, ws, want_logits=False)
        torch.cuda.synchronize()
        run = {"xq": host(xq), "wq": host(wq), "idx": idx.cpu().numpy(), "w": wts.cpu().numpy(),
               "logits": logits.cpu().numpy(), "idx_nolog": i2.cpu().numpy(), "w_nolog": w2.cpu().numpy(),
               "fwd_xq": host(xq3), "fwd_idx": i3.cpu().numpy(), "fwd_w": w3.cpu().numpy(), "gsa": full_gsa(x),
               "wq_ref": quant_ref.quantize_ref(w)}
        del xd, xq, xq3, idx, wts, logits, i2, w2, i3, w3
        torch.cuda.empty_cache()
        # The runs with and without logits, and router_forward, route identically and quantize identically.
        assert np.array_equal(run["idx"], run["idx_nolog"]) and np.array_equal(run["idx"], run["fwd_idx"])
        assert np.array_equal(run["w"].view(np.uint32), run["w_nolog"].view(np.uint32))
        assert np.array_equal(run["w"].view(np.uint32), run["fwd_w"].view(np.uint32))
        for a, b in zip(run["xq"], run["fwd_xq"]):
            assert np.array_equal(a, b)
        full_size_runs.clear()  # one config's host copies at a time
        full_size_runs[cfg] = run
    return full_size_runs[cfg]


@pytest.mark.parametrize("cfg,chunk", FULL_CASES, ids=[f"cfg{c}-rows{i * CHUNK}" for c, i in FULL_CASES])
def test_full_size_chunk(dev, ws, big_inputs, full_size_runs, cfg, chunk):
    """Prefill sizes in full: each 4096-row chunk's codes, scales, logits, top-k and weights against the oracle
    (quantized under the whole tensor's global scale), for the runs with and without logits."""
    c = wl.CONFIGS[cfg]
    x, w, bias = get_big(big_inputs, cfg)
    run = get_full_run(full_size_runs, big_inputs, dev, ws, cfg)
    r0, r1 = chunk * CHUNK, (chunk + 1) * CHUNK
    log(f"full size cfg {cfg}: rows {r0}..{r1 - 1}")
    xr = quant_ref.quantize_ref(x[r0:r1], gsa_override=run["gsa"])
    codes, scales, gsa = run["xq"]
    fails = check.check_quant(codes[r0:r1], scales[r0:r1], gsa, xr)
    if chunk == 0:
        fails += check.check_quant(*run["wq"], run["wq_ref"])
    assert not fails, "\n".join(fails)
    assert int(scales[r0:r1].max()) <= 0x7E
    L, A = router_ref.logits_ref(*xr, *run["wq_ref"])
    _, _, s, b = router_ref.route_ref(L, bias, c.k, c.routed_scale)
    ref = {"L": L, "A": A, "s": s, "b": b}
    rows = np.arange(r0, r1)
    assert_route(ref, run["idx"][r0:r1], run["w"][r0:r1], run["logits"][r0:r1], c.k, c.routed_scale,
                 f"cfg {cfg} rows {r0}..", rows=rows)
    assert_route(ref, run["idx_nolog"][r0:r1], run["w_nolog"][r0:r1], None, c.k, c.routed_scale,
                 f"cfg {cfg} rows {r0}.. (no logits)", rows=rows)
    np.testing.assert_allclose(run["w"][r0:r1].sum(axis=1), c.routed_scale, rtol=1e-5)


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
    (300, 2304, 256, 8),   # MFMA gate, 18 K steps: scale windows of 8 steps, the last one partial
    (700, 3328, 384, 8),   # one K group, 26 K steps (four windows), E not a multiple of 256
    (300, 256, 64, 4),     # MFMA gate with fewer experts than one expert block (64 of 128 columns)
    (600, 512, 16, 2),     # likewise, 16 experts
    (2, 7168, 100, 8),     # decode gate: E not a multiple of 16
    (3, 4128, 256, 8),     # decode gate: 5 K slices, the last one two blocks
    (4, 4128, 100, 5),     # decode gate: both ragged
])
def test_gate_shapes(dev, ws, T, D, E, k):
    log(f"gate shape T={T} D={D} E={E} k={k}")
    x, w = synth((T, D), T * 1000 + D), synth((E, D), E * 1000 + D, 0.02)
    bias = np.random.default_rng(E).uniform(-0.01, 0.01, E).astype(np.float32)
    res = run_router_both(dev, ws, x, w, bias, k, 2.5)
    ref = router_ref.router_ref(x, w, bias, k, 2.5)
    assert_quant(res[0], ref["xq"], "x")
    assert_route_both(ref, res, k, 2.5, f"T={T} D={D} E={E} k={k}")


ALL_TIED = [(T, E, k) for T in (4, 64, 300, 8200) for E in (256, 384) for k in (8, 16)]


@pytest.mark.parametrize("T,E,k", ALL_TIED)
def test_gate_all_scores_tied(dev, ws, T, E, k):
    """x == 0 and bias == 0: every expert has the same selection score, so the k lowest experts are chosen in
    index order and each weight is r/k exactly. Every kernel's many-survivor selection takes this (the checker
    accepts any set at a full tie, so the test asserts the rule itself)."""
    D = 256
    log(f"gate all tied T={T} E={E} k={k}")
    x = np.zeros((T, D), dtype=np.uint16)
    w = synth((E, D), 3 * E, 0.02)
    bias = np.zeros(E, dtype=np.float32)
    for want_logits in (True, False):
        xq, wq, idx, wts, logits = run_router(dev, ws, x, w, bias, k, 2.5, want_logits=want_logits)
        assert np.all(idx == np.arange(k)[None, :]), (want_logits, idx[:2])
        assert np.all(wts == np.float32(2.5 / k)), (want_logits, wts[:2])
        # The single-launch path as well (T <= 4).
        xq2, (i2, w2, _) = rt.forward(to_dev(x, dev), wq, torch.from_numpy(bias).to(dev), k, 2.5, ws,
                                      want_logits=want_logits)
        torch.cuda.synchronize()
        assert np.array_equal(i2.cpu().numpy(), idx) and np.array_equal(w2.cpu().numpy(), wts)


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
                                         (None, 1, 16416, 100, 5),   # D past the single launch: two-call path
                                         (None, 2, 7168, 100, 8),    # single launch, E not a multiple of 16
                                         (None, 3, 4128, 256, 8),    # single launch, ragged last K slice
                                         (None, 4, 4128, 100, 5),    # both
                                         (3, 64, 7168, 256, 8),      # batched decode (timed by the benchmark)
                                         (None, 5, 7168, 256, 8),    # smallest batched-decode T
                                         (None, 17, 4128, 100, 6),   # batched: ragged rows, last slice, experts
                                         (None, 8, 32, 16, 1),       # batched: one K step, one expert tile, top-1
                                         (None, 40, 1056, 64, 4),    # batched: second slice two blocks
                                         (None, 64, 7168, 300, 8),   # batched: ragged last expert quarter
                                         (None, 255, 2048, 512, 32),  # batched: largest E and k, ragged rows
                                         (None, 256, 16384, 256, 8),  # batched: largest T and D
                                         (None, 100, 16416, 64, 4),  # D past the batched path: two-call path
                                         (None, 257, 1024, 256, 8)])  # T past the batched path
@pytest.mark.parametrize("want_logits", [True, False], ids=["logits", "nologits"])
def test_forward_matches_oracle(dev, ws, cfg, T, D, E, k, want_logits):
    """router_forward (one launch at T <= 4, two fused launches up to T = 256) gives the quantizer's bytes and the
    oracle's routing."""
    if cfg is not None:
        x, w, bias = wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg)
        r = wl.CONFIGS[cfg].routed_scale
    else:
        x, w = synth((T, D), 7 * T + D), synth((E, D), 11 * E + D, 0.02)
        bias = np.random.default_rng(E + T).uniform(-0.01, 0.01, E).astype(np.float32)
        r = 2.5
    log(f"forward T={T} D={D} E={E} k={k} logits={want_logits}")
    wq = gpu_quant(w, dev, ws)
    b = torch.from_numpy(bias).to(dev)
    xq, (idx, wts, logits) = rt.forward(to_dev(x, dev), wq, b, k, r, ws, want_logits=want_logits)
    torch.cuda.synchronize()
    ref = router_ref.router_ref(x, w, bias, k, r)
    assert_quant(xq, ref["xq"], "x via router_forward")
    assert_route(ref, idx.cpu().numpy(), wts.cpu().numpy(), None if logits is None else logits.cpu().numpy(), k, r,
                 f"forward T={T}")


@pytest.mark.parametrize("cfg", [2, 3])
def test_forward_is_deterministic(dev, ws, cfg):
    """router_forward twice on the same inputs (one launch at T = 1, two at T = 64): identical bits."""
    c = wl.CONFIGS[cfg]
    x, w, bias = wl.make_x(cfg), wl.make_w(cfg), wl.make_bias(cfg)
    log(f"forward determinism cfg {cfg}")
    wq = gpu_quant(w, dev, ws)
    xd, b = to_dev(x, dev), torch.from_numpy(bias).to(dev)
    runs = []
    for _ in range(2):
        xq, (idx, wts, logits) = rt.forward(xd, wq, b, c.k, c.routed_scale, ws, want_logits=True)
        torch.cuda.synchronize()
        runs.append((xq.codes.cpu().numpy(), idx.cpu().numpy(), wts.cpu().numpy().view(np.uint32),
                     logits.cpu().numpy().view(np.uint32)))
    for a, b2 in zip(*runs):
        assert np.array_equal(a, b2)


@pytest.mark.parametrize("cfg", [2, 3])
def test_forward_static_scale_override(dev, ws, cfg):
    c = wl.CONFIGS[cfg]
    x, w, bias = wl.make_x(cfg, 3), wl.make_w(cfg, 3), wl.make_bias(cfg, 3)
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


@pytest.mark.parametrize("cfg", [2, 3])
def test_forward_graph_replay_cycles_layers(dev, ws, cfg):
    """Decode loop as the benchmark runs it: several layer sets captured in one graph, replayed twice."""
    c = wl.CONFIGS[cfg]
    L = 5
    xs = [to_dev(wl.make_x(cfg, l), dev) for l in range(L)]
    wqs = [gpu_quant(wl.make_w(cfg, l), dev, ws) for l in range(L)]
    bs = [torch.from_numpy(wl.make_bias(cfg, l)).to(dev) for l in range(L)]
    xq = [rt.empty_nvfp4(c.T, c.D, dev) for _ in range(L)]
    outs = [(torch.empty((c.T, c.k), dtype=torch.int32, device=dev),
             torch.empty((c.T, c.k), dtype=torch.float32, device=dev), None) for _ in range(L)]
    log(f"forward graph replay cfg {cfg}")
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
            ref = router_ref.router_ref(wl.make_x(cfg, l), wl.make_w(cfg, l), wl.make_bias(cfg, l), c.k,
                                        c.routed_scale)
            fails = check.check_topk(outs[l][0].cpu().numpy(), outs[l][1].cpu().numpy(), ref["s"], ref["b"], c.k,
                                     c.routed_scale)
            assert not fails, f"replay {rep} layer {l}: " + "; ".join(fails)
