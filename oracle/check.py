"""Comparison rules between a device result and the oracle.

TEST INFRASTRUCTURE (CPU oracle); see the package docstring.

* Codes, scale bytes and the global scale: bitwise equal (integer work).
* Logits: |L_dev - L_ref| <= tol * A_ref elementwise, A_ref = sum |xhat*what|.
  A plain relative test fails for a correct fp32 sum whenever the logit
  nearly cancels, so the error is measured against the dot product's
  condition scale (tol = 1e-5).
* Top-k set: with b_k and b_k1 the oracle's k-th and (k+1)-th selection
  scores, a gap >= tol demands the oracle's set exactly. Inside a near-tie,
  experts with b >= b_k1 + tol must be chosen, experts with b <= b_k - tol
  must not, and the rest are free.
* Order: descending, enforced between chosen entries whose oracle b differ
  by at least tol.
* Weights: |w_dev - w_ref(G)| <= tol, where w_ref(G) re-applies steps 4-6
  on the device's own chosen set G in its order.

Every check returns a list of human-readable failures (empty == pass).
"""

import numpy as np


def check_bytes(name, dev, ref, limit=10):
    dev = np.asarray(dev)
    ref = np.asarray(ref)
    if dev.shape != ref.shape:
        return [f"{name}: shape {dev.shape} != {ref.shape}"]
    bad = np.argwhere(dev != ref)
    out = []
    for pos in bad[:limit]:
        p = tuple(int(i) for i in pos)
        out.append(f"{name}{list(p)}: dev 0x{int(dev[p]):02X} ref 0x{int(ref[p]):02X}")
    if len(bad) > limit:
        out.append(f"{name}: {len(bad)} mismatches in total")
    return out


def check_quant(dev_codes, dev_scales, dev_gsa, ref):
    """Bitwise comparison of (codes, scales, gsa) against ``quantize_ref``'s tuple."""
    ref_codes, ref_scales, ref_gsa = ref
    out = check_bytes("codes", dev_codes, ref_codes)
    out += check_bytes("scales", dev_scales, ref_scales)
    dg = np.asarray(dev_gsa, dtype=np.float32).reshape(()).view(np.uint32)
    rg = np.asarray(ref_gsa, dtype=np.float32).reshape(()).view(np.uint32)
    if int(dg) != int(rg):
        out.append(f"gsa: dev 0x{int(dg):08X} ref 0x{int(rg):08X}")
    return out


def check_logits(L_dev, L_ref, A_ref, tol=1e-5, limit=10):
    L_dev = np.asarray(L_dev, dtype=np.float64)
    err = np.abs(L_dev - L_ref)
    bound = tol * A_ref
    bad = np.argwhere(~(err <= bound))
    out = []
    for pos in bad[:limit]:
        p = tuple(int(i) for i in pos)
        out.append(f"logit{list(p)}: dev {L_dev[p]!r} ref {L_ref[p]!r} A {A_ref[p]!r}")
    if len(bad) > limit:
        out.append(f"logits: {len(bad)} outside tolerance")
    return out


def logit_error_stats(L_dev, L_ref, A_ref):
    """max |err|/A and the plain relative error over logits with |L| >= row median."""
    L_dev = np.asarray(L_dev, dtype=np.float64)
    err = np.abs(L_dev - L_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel_a = np.where(A_ref > 0, err / A_ref, 0.0)
        big = np.abs(L_ref) >= np.median(np.abs(L_ref), axis=1, keepdims=True)
        rel = np.where(big & (L_ref != 0), err / np.abs(L_ref), 0.0)
    return float(np.max(rel_a, initial=0.0)), float(np.max(rel, initial=0.0))


def check_topk(idx_dev, w_dev, s_ref, b_ref, k, routed_scale, tol=1e-5, rows=None, limit=10):
    """Apply the set / order / weight rules row by row.

    ``s_ref``/``b_ref`` are the oracle's float64 scores [T, E]; ``rows`` maps
    device rows to oracle rows when only a sample was computed.
    """
    idx_dev = np.asarray(idx_dev)
    w_dev = np.asarray(w_dev, dtype=np.float64)
    T, E = b_ref.shape
    out = []
    for t in range(T):
        if len(out) >= limit:
            out.append("... (more rows not checked)")
            break
        tag = f"row {t if rows is None else rows[t]}"
        ids = [int(i) for i in idx_dev[t]]
        if len(ids) != k or len(set(ids)) != k or min(ids) < 0 or max(ids) >= E:
            out.append(f"{tag}: invalid index list {ids}")
            continue
        b = b_ref[t]
        order = np.lexsort((np.arange(E), -b))
        bk = b[order[k - 1]]
        bk1 = b[order[k]] if k < E else -np.inf
        chosen = set(ids)
        if bk - bk1 >= tol:
            want = {int(i) for i in order[:k]}
            if chosen != want:
                out.append(f"{tag}: set {sorted(chosen)} != oracle {sorted(want)} (gap {bk - bk1:.3g})")
                continue
        else:
            must = {int(e) for e in np.nonzero(b >= bk1 + tol)[0]}
            never = {int(e) for e in np.nonzero(b <= bk - tol)[0]}
            if not must <= chosen or chosen & never:
                out.append(f"{tag}: near-tie set {sorted(chosen)} violates must={sorted(must)} never")
                continue
        bs = b[ids]
        inverted = [(i, j) for i in range(k) for j in range(i + 1, k) if bs[j] - bs[i] >= tol]
        if inverted:
            out.append(f"{tag}: order {ids} not descending at positions {inverted[0]}")
        s_sel = s_ref[t][ids]
        w_want = float(routed_scale) * s_sel / s_sel.sum()
        werr = np.abs(w_dev[t] - w_want)
        if not np.all(werr <= tol):
            out.append(f"{tag}: weights {w_dev[t].tolist()} vs {w_want.tolist()} (max err {werr.max():.3g})")
    return out
