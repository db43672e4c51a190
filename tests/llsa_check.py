"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, and compare under the tolerances of
the method's contract:
  - index lists and transposes bit-exact on the fp32 path;
  - on the bf16 path a selection may differ from the oracle's only in rows whose
    oracle score gap (K-th kept minus best rejected) is below 1e-3, checked
    level by level with the oracle re-run on the GPU's parent lists;
  - bf16 outputs: max-abs <= 2e-2 and mean-abs <= 2e-3; gradients max-abs
    <= 5e-2, with the oracle recomputing on the GPU's index lists;
  - fp32 outputs: max-abs <= 1e-5 (out, lse) and 1e-4 (gradients).
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

BS = 16
GAP = 1e-3
TOL = {"bf16": dict(out_max=2e-2, out_mean=2e-3, grad_max=5e-2),
       "f32": dict(out_max=1e-5, out_mean=1e-5, grad_max=1e-4)}


def level_k(w, l):
    """top-k of level l (1-based): w.topk is an int or one value per level"""
    return w.topk if isinstance(w.topk, int) else w.topk[l - 1]


def to_device(arr, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def ws_array(ws, off, count, np_dtype):
    import torch
    nbytes = count * np.dtype(np_dtype).itemsize
    return ws[off:off + nbytes].cpu().numpy().view(np_dtype).copy()


def gpu_run(w, inp, flags=0, backward=True, q64=None):
    """HIP path on raster-order inputs: grid-order gather, forward, backward.
    Returns numpy float64 results in Z-order plus workspace contents."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    B, H, N, d = w.B, w.H, w.N, w.d
    dt = lib.BF16 if w.dtype == "bf16" else lib.F32
    q_r, k_r, v_r = (to_device(inp[n], w.dtype) for n in ("q", "k", "v"))
    q, k, v = (lib.grid_order(x, w.frames, w.rows, w.side) for x in (q_r, k_r, v_r))
    out, lse, ws = lib.forward(q, k, v, w.topk, w.levels, flags)
    res = {"q": q, "k": k, "v": v, "out_t": out, "lse_t": lse, "ws": ws}
    if backward:
        do = to_device(inp["do"], w.dtype)
        dq, dk, dv = lib.backward(q, k, v, out, lse, do, w.topk, w.levels, ws, flags)
        res.update(dq_t=dq, dk_t=dk, dv_t=dv)
    torch.cuda.synchronize()
    lay = (lib.llsa_workspace_layout(B, H, N, d, BS, w.topk, w.levels, dt)
           if isinstance(w.topk, int) else
           lib.llsa_workspace_layout_lk(B, H, N, d, BS, w.topk, w.levels, dt))
    G = B * H
    res["lay"] = lay
    res["idx"], res["qbar"], res["kbar"], res["vbar"] = [], [], [], []
    res["rowptr"], res["col"] = [], []
    for l in range(1, w.levels + 1):
        n = N // BS ** l
        K = level_k(w, l)
        res["idx"].append(ws_array(ws, lay["idx"][l - 1], G * n * K, np.int32)
                          .reshape(G, n, K))
        for name in ("qbar", "kbar", "vbar"):
            res[name].append(ws_array(ws, lay[name][l - 1], G * n * d, np.float32)
                             .reshape(G, n, d).astype(np.float64))
        if backward:
            res["rowptr"].append(ws_array(ws, lay["rowptr"][l - 1], G * (n + 1), np.int32)
                                 .reshape(G, n + 1))
            res["col"].append(ws_array(ws, lay["col"][l - 1], G * n * K, np.int32)
                              .reshape(G, n * K))
    res["out"] = to_f64(out).reshape(G, N, d)
    res["lse"] = lse.cpu().numpy().astype(np.float64).reshape(G, N)
    if backward:
        for n_ in ("dq", "dk", "dv"):
            res[n_] = to_f64(res[n_ + "_t"]).reshape(G, N, d)
    return res


def oracle_inputs(w, inp):
    """Exact float64 values of the stored inputs, grid-ordered by the oracle."""
    G, N, d = w.G, w.N, w.d
    z = {}
    for n in ("q", "k", "v"):
        z[n] = oracle.grid_order(inp[n + "64"].reshape(G, N, d), w.frames, w.rows, w.side)
    z["do"] = inp["do64"].reshape(G, N, d) if "do64" in inp else None
    return z


def check_selection(w, gpu, orc_pyr, exact: bool):
    """Level-by-level comparison; returns the number of rows that differ."""
    qp, kp = orc_pyr
    scale = 1.0 / np.sqrt(w.d)
    diffs = 0
    for l in range(w.levels, 0, -1):
        parent = None if l == w.levels else gpu["idx"][l]
        want, gap = oracle.select_level(qp[l - 1], kp[l - 1], parent, level_k(w, l), BS, scale)
        got = gpu["idx"][l - 1]
        bad = np.any(got != want, axis=2)
        if exact:
            assert not bad.any(), "level %d: %d rows differ" % (l, bad.sum())
        else:
            assert np.all(gap[bad] < GAP), \
                "level %d: mismatch in rows with gap >= %g: %s" % (l, GAP, gap[bad][gap[bad] >= GAP][:5])
        # every GPU row is a valid selection: ascending, distinct, children of parent
        assert np.all(np.diff(got, axis=2) > 0)
        if parent is not None:
            par = np.repeat(parent, BS, axis=1)
            assert np.all(np.any((got[..., :, None] // BS) == par[..., None, :], axis=3))
        diffs += int(bad.sum())
    return diffs


def check_transpose(gpu, w):
    for l in range(w.levels):
        rp, col = oracle.transpose(gpu["idx"][l])
        np.testing.assert_array_equal(gpu["rowptr"][l], rp)
        np.testing.assert_array_equal(gpu["col"][l], col)


def assert_close(got, want, max_abs, mean_abs=None, what=""):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    assert err.max() <= max_abs, "%s: max-abs %.3g > %.3g" % (what, err.max(), max_abs)
    if mean_abs is not None:
        assert err.mean() <= mean_abs, "%s: mean-abs %.3g > %.3g" % (what, err.mean(), mean_abs)
    return float(err.max()), float(err.mean())
