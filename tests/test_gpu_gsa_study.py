"""Static versus runtime global scale: the failure that motivates the runtime
gsa (commit 04cf8ca8, dsv4/layers/router.py, runtime-gsa paragraph).

A static gsa calibrated on ordinary tokens lets x / gsa exceed 6 * 448 on a
batch whose max is larger: block scales saturate at 448 and those blocks lose
magnitude. The runtime gsa = max|x| / 2688 keeps every quotient in range. Both
runs go through router_forward on the GPU (the static one with gsa_override);
each is compared with routing on unquantized activations (bf16 x times the
NVFP4 gate weights, float64, the oracle's epilogue), which isolates the error
the activation quantization adds.

Scenarios, 7168 hidden, 256 experts, top 8, routed scale 2.5:
  A  in distribution: 31 N(0,1) decode tokens; static gsa from 30 other such
     tokens;
  B  outlier channels: the 64-token batched-decode batches (1 % of channels
     x50), four layer sets; the same static gsa.
"""

import numpy as np
import pytest
import torch

from nvfp4_block_scaled_06_amd import router as rt
from nvfp4_block_scaled_06_amd import workloads as wl
from oracle import check, quant_ref, router_ref

pytestmark = pytest.mark.gpu

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def log(msg):
    print(f"[gsa-study] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rt.load_library()
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    return d


def to_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)


def saturated_fraction(x_bits, gsa):
    """Share of 16-element blocks whose ideal scale bmax / (6 gsa) exceeds 448 (they lose magnitude). The
    block holding the tensor's max can exceed it by gsa's one rounding (a relative 2^-23), which is no loss."""
    v = np.abs(quant_ref.bf16_bits_to_f64(x_bits))
    bmax = v.reshape(v.shape[0], -1, 16).max(axis=2)
    return float(np.mean(bmax / (E2M1_MAX * float(gsa)) > E4M3_MAX * (1 + 2.0 ** -20)))


def metrics(idx, wts, logits, ref_idx, ref_w, L_ref, E, k, r):
    """Logit error relative to each token's largest reference logit, top-k overlap, weight distance."""
    T = idx.shape[0]
    rel = np.abs(logits - L_ref).max(axis=1) / np.abs(L_ref).max(axis=1)
    overlap = np.mean([len(set(idx[t]) & set(ref_idx[t])) / k for t in range(T)])
    flips = np.mean([set(idx[t]) != set(ref_idx[t]) for t in range(T)])
    dense = np.zeros((T, E))
    dense_ref = np.zeros((T, E))
    np.put_along_axis(dense, idx.astype(np.int64), wts, axis=1)
    np.put_along_axis(dense_ref, ref_idx, ref_w, axis=1)
    wdist = np.abs(dense - dense_ref).sum(axis=1).mean() / r
    return {"logit_rel_err_median": float(np.median(rel)), "topk_overlap": float(overlap),
            "tokens_with_flips": float(flips), "weight_l1_over_r": float(wdist)}


def run_scenario(dev, ws, name, x_bits, w_bits, bias, gsa_static, k, r):
    E = w_bits.shape[0]
    wq = rt.quantize(to_dev(w_bits, dev), ws)
    torch.cuda.synchronize()
    w_hat = quant_ref.dequant_ref(wq.codes.cpu().numpy(), wq.scales.cpu().numpy(), wq.gscale.cpu().numpy()[0])
    L_ref = quant_ref.bf16_bits_to_f64(x_bits) @ w_hat.T
    ref_idx, ref_w, _, _ = router_ref.route_ref(L_ref, bias, k, r)
    b = torch.from_numpy(bias).to(dev)
    out = {}
    for mode, ov in (("runtime", None), ("static", gsa_static)):
        ovt = None if ov is None else torch.tensor([ov], dtype=torch.float32, device=dev)
        xq, (idx, wts, logits) = rt.forward(to_dev(x_bits, dev), wq, b, k, r, ws, gsa_override=ovt,
                                            want_logits=True)
        torch.cuda.synchronize()
        gsa = float(xq.gscale.cpu().numpy()[0])
        # The quantized activations are the oracle's, bit for bit, for either scale.
        fails = check.check_quant(xq.codes.cpu().numpy(), xq.scales.cpu().numpy(), xq.gscale.cpu().numpy(),
                                  quant_ref.quantize_ref(x_bits, gsa_override=ov))
        assert not fails, "\n".join(fails[:10])
        m = metrics(idx.cpu().numpy(), wts.cpu().numpy(), logits.cpu().numpy().astype(np.float64), ref_idx, ref_w,
                    L_ref, E, k, r)
        m["gsa"] = gsa
        m["max_x_over_gsa"] = quant_ref.amax_ref(x_bits) / gsa
        m["saturated_blocks"] = saturated_fraction(x_bits, gsa)
        out[mode] = m
        log(f"{name:22s} {mode:8s} gsa={gsa:.4e} max|x|/gsa={m['max_x_over_gsa']:9.1f} "
            f"saturated={m['saturated_blocks']:.4f} logit_err={m['logit_rel_err_median']:.2e} "
            f"topk_overlap={m['topk_overlap']:.4f} flips={m['tokens_with_flips']:.3f} "
            f"w_l1/r={m['weight_l1_over_r']:.4f}")
    return out


def test_static_versus_runtime_global_scale(dev):
    c2, c3 = wl.CONFIGS[2], wl.CONFIGS[3]
    ws = rt.Workspace(max(rt.workspace_bytes(c3.T, c3.D, c3.E, c3.k), rt.workspace_bytes(c3.E, c3.D, c3.E, c3.k)),
                      dev)
    calib = np.concatenate([wl.make_x(2, l) for l in range(30)])
    gsa_static = float(quant_ref.gsa_ref(quant_ref.amax_ref(calib)))
    log(f"static gsa from 30 calibration tokens: {gsa_static:.4e}")

    xa = np.concatenate([wl.make_x(2, l) for l in range(30, 61)])
    a = run_scenario(dev, ws, "A in distribution", xa, wl.make_w(2, 0), wl.make_bias(2, 0), gsa_static, c2.k,
                     c2.routed_scale)
    bs = [run_scenario(dev, ws, f"B outliers, layer {l}", wl.make_x(3, l), wl.make_w(3, l), wl.make_bias(3, l),
                       gsa_static, c3.k, c3.routed_scale) for l in range(4)]

    bound = 6 * 448 * (1 + 2.0 ** -23)
    for res in [a] + bs:
        # Runtime gsa: x / gsa stays within 6 * 448 (up to gsa's one rounding), no block saturates.
        assert res["runtime"]["max_x_over_gsa"] <= bound
        assert res["runtime"]["saturated_blocks"] == 0.0
    for res in bs:
        st, rt_ = res["static"], res["runtime"]
        # The static scale saturates the outlier blocks, and routing drifts further from the unquantized one.
        assert st["max_x_over_gsa"] > 10 * 6 * 448
        assert st["saturated_blocks"] > 0.005
        assert st["logit_rel_err_median"] > 2 * rt_["logit_rel_err_median"]
        assert st["topk_overlap"] < rt_["topk_overlap"]
