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

import os
from concurrent.futures import ThreadPoolExecutor

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
    """HIP path on raster-order inputs: grid-order gather and forward
    (llsa_forward_grid; llsa_grid_order and llsa_forward_lk for a top-k per
    level), backward.
    Returns numpy float64 results in Z-order plus workspace contents."""
    import torch
    import sparse_attention_diffusion_order_amd as lib
    B, H, N, d = w.B, w.H, w.N, w.d
    dt = lib.BF16 if w.dtype == "bf16" else lib.F32
    q_r, k_r, v_r = (to_device(inp[n], w.dtype) for n in ("q", "k", "v"))
    if isinstance(w.topk, int):
        # the forward with the grid order folded into its pooling pass
        q, k, v, out, lse, ws = lib.forward_grid(q_r, k_r, v_r, w.frames, w.rows, w.side,
                                                 w.topk, w.levels, flags)
    else:
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
        n = -(-N // BS ** l)  # the last block of a level may be partial
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


def host_workers(limit: int = 16) -> int:
    """CPU threads for oracle work: the cores this process may use, at most
    `limit` (a GPU machine gives one GPU's process a share of 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def per_head(fn, G: int, workers: int = 0):
    """[fn(h) for h in range(G)], run in a thread pool.  The oracle's C
    routines release the GIL (ctypes), so heads run in parallel on the host
    cores; each head's arithmetic is the oracle's own, unchanged."""
    workers = workers or host_workers()
    if workers == 1 or G == 1:
        return [fn(h) for h in range(G)]
    with ThreadPoolExecutor(max_workers=min(workers, G)) as ex:
        return list(ex.map(fn, range(G)))


def oracle_values(w, z, kp, vp, idx, flags=0, backward=True):
    """The oracle's out, lse (and dq, dk, dv) for every head and token, on the
    given index lists, one head per host thread."""
    scale = 1.0 / np.sqrt(w.d)

    def head(h):
        sl = slice(h, h + 1)
        q, k, v = (z[n][sl] for n in ("q", "k", "v"))
        kph, vph, ih = [x[sl] for x in kp], [x[sl] for x in vp], [x[sl] for x in idx]
        o, lse = oracle.forward(q, k, v, kph, vph, ih, BS, scale, flags)
        if not backward:
            return o, lse
        return (o, lse) + oracle.backward(q, k, v, kph, vph, ih, o, lse, z["do"][sl], BS,
                                          scale, flags)

    parts = per_head(head, w.G)
    return [np.concatenate([p_[i] for p_ in parts]) for i in range(len(parts[0]))]


def grad_tol(ref, base: float) -> float:
    """Max-abs bound of a bf16-path gradient: the stated 5e-2 (for unit-scale
    inputs), or 2^-6 of the tensor's largest magnitude when that is larger --
    eight bf16 roundings (2^-9 each) of the largest value -- since every
    rounding on the bf16 path (the P and dS operands, lse, the stored result)
    is relative to the values it rounds."""
    return max(base, float(np.abs(ref).max()) * 2.0 ** -6)


def check_selection(w, gpu, orc_pyr, exact: bool, causal: bool = False):
    """Level-by-level comparison; returns the number of rows that differ.
    causal: the causal selection (the row's own block plus its best K-1
    earlier candidates, -1 in the slots left)."""
    qp, kp = orc_pyr
    scale = 1.0 / np.sqrt(w.d)
    diffs = 0
    for l in range(w.levels, 0, -1):
        parent = None if l == w.levels else gpu["idx"][l]

        def head(h, l=l, parent=parent):
            sl = slice(h, h + 1)
            return oracle.select_level(qp[l - 1][sl], kp[l - 1][sl],
                                       None if parent is None else parent[sl], level_k(w, l), BS,
                                       scale, causal=causal)

        parts = per_head(head, w.G)
        want = np.concatenate([p_[0] for p_ in parts])
        gap = np.concatenate([p_[1] for p_ in parts])
        got = gpu["idx"][l - 1]
        bad = np.any(got != want, axis=2)
        if exact:
            assert not bad.any(), "level %d: %d rows differ" % (l, bad.sum())
        else:
            assert np.all(gap[bad] < GAP), \
                "level %d: mismatch in rows with gap >= %g: %s" % (l, GAP, gap[bad][gap[bad] >= GAP][:5])
        # every GPU row is a valid selection: ascending, distinct, children of
        # the parent's picks (causal: the valid picks first, the row itself
        # among them and none after it, then -1)
        valid = got >= 0
        if causal:
            assert np.all(valid[..., :1]) and np.all(valid[..., :-1] | ~valid[..., 1:])
            rows = np.arange(got.shape[1])[None, :, None]
            assert np.all(np.any(got == rows, axis=2)) and np.all(~valid | (got <= rows))
            pairs = valid[..., 1:]
            assert np.all(np.diff(got, axis=2)[pairs] > 0)
        else:
            assert np.all(valid) and np.all(np.diff(got, axis=2) > 0)
        if parent is not None:
            par = np.repeat(parent, BS, axis=1)[:, :got.shape[1]]
            par = np.where(par >= 0, par, -2)  # an unused parent slot has no children
            hit = np.any((got[..., :, None] // BS) == par[..., None, :], axis=3)
            assert np.all(hit | ~valid)
        diffs += int(bad.sum())
    return diffs


def check_transpose(gpu, w):
    """The key->query lists, exactly: rowptr, and col up to rowptr[n] (causal
    rows hold fewer than K picks, so the n K slots of a head end in unused
    ones, which the library leaves untouched)."""
    for l in range(w.levels):
        rp, col = oracle.transpose(gpu["idx"][l])
        np.testing.assert_array_equal(gpu["rowptr"][l], rp)
        for h in range(rp.shape[0]):
            np.testing.assert_array_equal(gpu["col"][l][h, :rp[h, -1]], col[h, :rp[h, -1]])


def assert_close(got, want, max_abs, mean_abs=None, what=""):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    assert err.max() <= max_abs, "%s: max-abs %.3g > %.3g" % (what, err.max(), max_abs)
    if mean_abs is not None:
        assert err.mean() <= mean_abs, "%s: mean-abs %.3g > %.3g" % (what, err.mean(), mean_abs)
    return float(err.max()), float(err.mean())


def full_check(w, flags=0, inp=None):
    """Every stage of the HIP path against the oracle, for every head, block
    and token: pyramid, selection (gap rule on bf16, exact on fp32),
    transposes (exact), out and lse, and the gradients."""
    inp = synth.make_inputs(w) if inp is None else inp
    gpu = gpu_run(w, inp, flags=flags)
    z = oracle_inputs(w, inp)
    tol = TOL[w.dtype]
    qp, kp, vp = (oracle.pool(z[n], BS, w.levels) for n in ("q", "k", "v"))
    for l in range(w.levels):  # pyramid: fp32 sums of exact inputs
        for name, ref in (("qbar", qp), ("kbar", kp), ("vbar", vp)):
            assert_close(gpu[name][l], ref[l], 2e-6, what="%s level %d" % (name, l + 1))
    check_selection(w, gpu, (qp, kp), exact=(w.dtype == "f32"),
                    causal=bool(flags & oracle.CAUSAL))
    check_transpose(gpu, w)
    o, lse, dq, dk, dv = oracle_values(w, z, kp, vp, gpu["idx"], flags)
    assert_close(gpu["out"], o, tol["out_max"], tol["out_mean"], "out")
    assert_close(gpu["lse"], lse, tol["out_max"], tol["out_mean"], "lse")
    for n_, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(gpu[n_], ref, tol["grad_max"], what=n_)
    return gpu
