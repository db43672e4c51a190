#!/usr/bin/env python3
"""LLSA hot-path benchmark on one MI355X.

One step = the whole hot path over one batch of seeded synthetic input already
resident in HBM: grid-order gather of Q, K, V (raster -> quadtree order), the
forward (pool pyramid, hierarchical Top-K, sparse attention with enrichment)
and the backward (index transpose, dQ, pooled-token gradients, dK/dV), all
through the C ABI of libllsa.so on one stream: llsa_forward_grid (the gather
folded into the pooling pass, which writes the grid-ordered Q, K, V) and
llsa_backward.  Prints ONE JSON line.

The headline times K whole steps between two HIP events on the caller's
stream.  A second pass of K steps runs the same work stage by stage, with
the gather as its own launches (llsa_grid_order, llsa_forward_part,
llsa_backward_part, one stream), and records an event after every stage for
the per-stage times; the roofline object is computed from it for the stage
kernel that takes the longest.  Then per-rep distributions (median, p10, p90) of the
forward, forward+backward and grid-order gather: warm, and cold with a
512 MiB write before each rep so that nothing stays in the 256 MB MALL.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_PEAK_TFLOPS = 157.3
DEFAULT_WORKLOAD = "grid256_bf16_l2_k16"


def grid_name(w):
    return ("%dx%dx%d" % (w.frames, w.rows, w.side) if w.frames > 1
            else "%dx%d" % (w.rows, w.side))


def metric(w):
    """The headline metric, named for the workload's size (for the default
    workload: 'LLSA fwd & fwd+bwd ms and TFLOP/s at N=65536 (256x256), d=64, bf16')."""
    return "LLSA fwd & fwd+bwd ms and TFLOP/s at N=%d (%s), d=%d, %s" % (
        w.N, grid_name(w), w.d, w.dtype)


def flops(w):
    """Algorithmic FLOPs: attention fwd = 4*G*N*n_kv*d with n_kv = 16K + L*K
    entries per query; bwd = 2.5 x fwd (five products, recomputation not
    counted); selection = 2*d*G*(n_L^2 + sum_{l<L} n_l*16K)."""
    n = [w.N // 16 ** l for l in range(w.levels + 1)]
    n_kv = 16 * w.topk + w.levels * w.topk
    attn_fwd = 4.0 * w.G * w.N * n_kv * w.d
    sel = 2.0 * w.d * w.G * (n[w.levels] ** 2 + sum(n[l] * 16 * w.topk for l in range(1, w.levels)))
    return {"attn_fwd": attn_fwd, "attn_bwd": 2.5 * attn_fwd, "select": sel,
            "fwd": attn_fwd + sel, "fwdbwd": 3.5 * attn_fwd + sel, "n_kv": n_kv}


def algo_bytes(w):
    """Algorithmic (unique) HBM bytes per launch of each stage kernel: every
    tensor the stage must read or write, counted once.  Per query block of 16
    tokens the attention forward moves q, k, v, out (bf16: 4 x 16 x 128 B)
    plus lse (64 B)."""
    e = 2 if w.dtype == "bf16" else 4
    tok = w.G * w.N * w.d * e
    n = [w.N // 16 ** l for l in range(w.levels + 1)]
    pyr = sum(w.G * n[l] * w.d * 4 for l in range(1, w.levels + 1))
    idx = sum(w.G * n[l] * w.topk * 4 for l in range(1, w.levels + 1))
    lse = w.G * w.N * 4
    return {
        "zorder": 2 * 3 * tok,
        "pool": 3 * tok + 3 * pyr,
        "select": 2 * pyr + idx,
        "attn_fwd": 4 * tok + lse + idx,
        "transpose": 3 * idx + sum(w.G * (n[l] + 1) * 4 for l in range(1, w.levels + 1)),
        "dq": 5 * tok + 2 * lse + idx,           # q k v o dout in, dq out; lse in, delta out
        "dkdv": 6 * tok + 2 * lse + 2 * idx,     # q k v dout in, dk dv out; lse, delta
    }


def sha_of_sources():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_diffusion_order_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


PMC_SUMMARY = "pmc_fetch_write_llsa_kernels_%s.json"
TRACE_SUMMARY = "kernel_trace_llsa_kernels_%s.md"
KERNEL_OF_STAGE = {"zorder": ("zorder_kernel",), "pool": ("pool_l12",),
                   "select": ("select_top2", "select_mfma", "select_kernel"),
                   "attn_fwd": ("attn_fwd_u4", "attn_fwd_bf16"),
                   "transpose": ("transpose_fill",), "dq": ("dq_bf16",),
                   "enrich": ("enrich_bwd_bf16",), "dkdv": ("dkdv_bf16",)}


def load_traffic(stage, w):
    """Measured HBM bytes per launch of a stage's kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this workload, if it was taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", PMC_SUMMARY % w.name)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha") != sha_of_sources():
        return None
    for want in KERNEL_OF_STAGE.get(stage, (stage,)):
        for name, k in rec.get("kernels", {}).items():
            if name.split("<")[0] == want:
                return k.get("hbm_bytes_per_launch")
    return None


def _short_kernel(name):
    n = name.replace("llsa::(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].replace("HIP_vector_type<unsigned int, 4u> ", "uint4")


def summarize_trace(db, out, cmd, bench_json=None):
    """Markdown summary of a rocprofv3 --kernel-trace --stats results database."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, total_calls, total_duration, average, percentage "
                          "from top_kernels"))
    with open(out, "w") as f:
        f.write("# rocprofv3 kernel trace: LLSA kernels, workload %s\n\n" % os.path.basename(out)
                .replace("kernel_trace_llsa_kernels_", "").replace(".md", ""))
        f.write("Command (on the MI355X, from the repository root):\n\n    %s\n\n" % cmd)
        f.write("Sources: csrc sha256 prefix %s\n\n" % sha_of_sources())
        f.write("`top_kernels` view of the results database; durations in microseconds.\n\n")
        f.write("| kernel | calls | total us | avg us | % |\n|---|---|---|---|---|\n")
        for r in rows:
            f.write("| %s | %d | %.0f | %.2f | %.2f |\n" % (_short_kernel(r[0]), r[1], r[2],
                                                         r[3], r[4]))
        if bench_json:
            b = json.loads(open(bench_json).read().strip().splitlines()[-1])
            f.write("\nHIP-event stage times of the same (profiled) bench run, ms per launch:\n\n")
            f.write("    %s\n\nms_per_step %.4f, value %.2f TFLOP/s\n"
                    % (json.dumps(b["stage_ms"]), b["ms_per_step"], b["value"]))


def summarize_pmc(fetch_db, write_db, out, cmd, workload):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every kernel, scaled by what
    the same counter reads for the plain device copy of known size that the
    profiled bench run ends with (--calib-copy-mib)."""
    import sqlite3

    def per_kernel(db, counter):
        c = sqlite3.connect(db)
        acc = {}
        for name, val in c.execute("select kernel_name, value from counters_collection "
                                   "where counter_name = ?", (counter,)):
            acc.setdefault(_short_kernel(name), []).append(val)
        return {k: sum(v) / len(v) for k, v in acc.items()}

    fet, wri = per_kernel(fetch_db, "FETCH_SIZE"), per_kernel(write_db, "WRITE_SIZE")
    copy = [k for k in fet if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise SystemExit("no copy kernel in the FETCH_SIZE run (use --calib-copy-mib)")
    ck = copy[0]
    copy_kib = CALIB_COPY_MIB * 1024.0
    f_fac = copy_kib / fet[ck]
    w_fac = copy_kib / wri[ck]
    kernels = {}
    for k in sorted(set(fet) | set(wri)):
        if k == ck:
            continue
        fb = fet.get(k, 0.0) * f_fac * 1024
        wb = wri.get(k, 0.0) * w_fac * 1024
        kernels[k] = {"fetch_kib_raw": round(fet.get(k, 0.0), 1),
                      "write_kib_raw": round(wri.get(k, 0.0), 1),
                      "hbm_bytes_per_launch": int(fb + wb),
                      "fetch_bytes": int(fb), "write_bytes": int(wb)}
    rec = {"workload": workload, "sources_sha": sha_of_sources(), "commands": cmd,
           "calibration": {"kernel": ck, "copy_bytes": CALIB_COPY_MIB << 20,
                           "fetch_kib_raw": round(fet[ck], 1), "write_kib_raw": round(wri[ck], 1),
                           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
           "kernels": kernels}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


CALIB_COPY_MIB = 256
N_CU = 256


def summarize_counters(db, out, cmd, workload):
    """Per-kernel averages of the counters of one rocprofv3 --pmc pass; with
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE also the MFMA-busy fraction
    busy / (active cycles x 256 CUs)."""
    import sqlite3
    c = sqlite3.connect(db)
    acc = {}
    for name, ctr, val in c.execute("select kernel_name, counter_name, value "
                                    "from counters_collection"):
        acc.setdefault(_short_kernel(name), {}).setdefault(ctr, []).append(val)
    kernels = {}
    for k, ctrs in sorted(acc.items()):
        row = {ctr: round(sum(v) / len(v), 1) for ctr, v in sorted(ctrs.items())}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in row and row.get("GRBM_GUI_ACTIVE"):
            row["mfma_busy_frac"] = round(row["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                          (row["GRBM_GUI_ACTIVE"] * N_CU), 4)
        kernels[k] = row
    rec = {"workload": workload, "sources_sha": sha_of_sources(), "commands": cmd,
           "kernels": kernels}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")


def _host_threads(limit=16):
    """host threads for the oracle: the cores this process may use, at most
    `limit` (the share of one GPU's process on the GPU machine)"""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(limit, n))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            return next((ln.split(":", 1)[1].strip() for ln in fh
                         if ln.startswith("model name")), "")
    except OSError:
        return ""


def oracle_workload(w, inp, threads, heads=None):
    """The oracle (plain fp64 C, unchanged) over whole heads of the workload:
    grid order, pool and selection per head, then the forward in query-block
    chunks, then the backward per head, each phase on a pool of `threads`
    host threads (the C routines release the GIL).  Returns seconds per
    phase and the number of heads."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    G, N, d = w.G, w.N, w.d
    heads = list(range(G)) if heads is None else list(heads)
    scale = 1.0 / np.sqrt(d)
    st = {}

    def prep(h):
        x = {n: oracle.grid_order(inp[n + "64"].reshape(G, N, d)[h:h + 1], w.frames, w.rows,
                                  w.side) for n in ("q", "k", "v")}
        x["do"] = inp["do64"].reshape(G, N, d)[h:h + 1]
        return x

    ins = {h: prep(h) for h in heads}  # input staging: not timed
    n1 = N // 16
    chunks = max(1, -(-threads // len(heads)))
    bounds = [(c * n1 // chunks, (c + 1) * n1 // chunks) for c in range(chunks)]
    t = {}
    with ThreadPoolExecutor(max_workers=threads) as ex:
        def sel(h):
            x = ins[h]
            qp, kp, vp = (oracle.pool(x[n], 16, w.levels) for n in ("q", "k", "v"))
            idx, _ = oracle.select(qp, kp, w.topk, 16, scale)
            st[h] = dict(kp=kp, vp=vp, idx=idx, out=np.zeros((1, N, d)), lse=np.zeros((1, N)))

        def fwd(task):
            h, (a, b) = task
            x, s_ = ins[h], st[h]
            oracle.forward(x["q"], x["k"], x["v"], s_["kp"], s_["vp"], s_["idx"], 16, scale,
                           qblocks=np.arange(a, b), out=s_["out"], lse=s_["lse"])

        def bwd(h):
            x, s_ = ins[h], st[h]
            oracle.backward(x["q"], x["k"], x["v"], s_["kp"], s_["vp"], s_["idx"], s_["out"],
                            s_["lse"], x["do"], 16, scale)

        t0 = time.perf_counter()
        list(ex.map(sel, heads))
        t1 = time.perf_counter()
        list(ex.map(fwd, [(h, ab) for h in heads for ab in bounds]))
        t2 = time.perf_counter()
        list(ex.map(bwd, heads))
        t3 = time.perf_counter()
    t = {"select_s": t1 - t0, "fwd_s": t2 - t1, "bwd_s": t3 - t2, "total_s": t3 - t0}
    return t, len(heads), chunks


def cpu_baseline(w, inp):
    """The oracle timed on the host's cores (a baseline, not the target):
    the whole workload (every head: pool, selection, forward, backward) on
    all threads this process may use (at most 16), and one head on a single
    thread.  TFLOP/s by the same FLOP convention as the GPU figures."""
    threads = _host_threads()
    f = flops(w)
    tm, nh, chunks = oracle_workload(w, inp, threads)
    t1, _, _ = oracle_workload(w, inp, 1, heads=[0])
    return {"value": round(f["fwdbwd"] / tm["total_s"] / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads, "kind": "oracle",
            "seconds": round(tm["total_s"], 3),
            "phases_s": {k_: round(v_, 3) for k_, v_ in tm.items() if k_ != "total_s"},
            "fwd_ms": round((tm["select_s"] + tm["fwd_s"]) * 1e3, 1),
            "fwdbwd_ms": round(tm["total_s"] * 1e3, 1),
            "one_thread": {"value": round(f["fwdbwd"] / w.G / t1["total_s"] / 1e12, 6),
                           "seconds": round(t1["total_s"], 3), "sample": "head 0"},
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(),
            "sample": "the whole workload (%d heads): per head pool + selection, then the "
                      "forward in %d query-block chunks per head, then the backward one head "
                      "per thread (%d busy), on a pool of %d threads; fp64 C oracle"
                      % (nh, chunks, min(nh, threads), threads)}


def dense_reference(w, q, k, v, do, reps=3):
    """torch scaled_dot_product_attention, non-causal, same shapes and dtype."""
    import torch
    import torch.nn.functional as F
    res = {}
    import contextlib
    from torch.nn.attention import SDPBackend, sdpa_kernel
    # the fused backend that takes these shapes: flash attention, else the
    # memory-efficient kernel (recorded, as the comparison depends on it)
    ctx, res["backend"] = contextlib.nullcontext(), "default"
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION),
                     ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                F.scaled_dot_product_attention(q[:, :1, :256], k[:, :1, :256], v[:, :1, :256])
            torch.cuda.synchronize()
            ctx, res["backend"] = sdpa_kernel([be]), name
            break
        except Exception:
            continue
    with ctx:
        qq, kk, vv = (x.detach().clone().requires_grad_(True) for x in (q, k, v))
        for mode in ("fwd", "fwdbwd"):
            times = []
            for r in range(reps + 1):
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                s.record()
                o = F.scaled_dot_product_attention(qq, kk, vv, dropout_p=0.0, is_causal=False)
                if mode == "fwdbwd":
                    o.backward(do)
                e.record()
                torch.cuda.synchronize()
                if r:
                    times.append(s.elapsed_time(e))
            res[mode + "_ms"] = float(np.median(times))
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(synth.WORKLOADS))
    ap.add_argument("--flags", type=int, default=0,
                    help="llsa flags of the timed calls (e.g. 16: causal); the headline uses 0. "
                         "With other flags FLOPs are still counted as for flags 0, and the "
                         "measured-traffic and CPU-baseline fields are left out")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-dist", action="store_true",
                    help="skip the per-rep warm/cold distributions (for profiled runs)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this size (for PMC scaling)")
    ap.add_argument("--summarize-trace", metavar="DB",
                    help="write the markdown summary of a rocprofv3 --kernel-trace --stats "
                         "database to --out and exit (no GPU)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the JSON summary of rocprofv3 --pmc FETCH_SIZE and "
                         "WRITE_SIZE databases to --out and exit (no GPU)")
    ap.add_argument("--summarize-counters", metavar="DB",
                    help="per-kernel averages of one rocprofv3 --pmc pass")
    ap.add_argument("--oracle-only", action="store_true",
                    help="time only the CPU oracle on the workload (all threads and one "
                         "thread on one head) and print its JSON line; no GPU")
    ap.add_argument("--out")
    ap.add_argument("--cmd", default="", help="the profiling command, recorded in the summary")
    ap.add_argument("--bench-json", help="bench output of the profiled run (trace summary)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.cmd, args.bench_json)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.cmd, args.workload)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.out, args.cmd,
                      args.workload)
        return
    if args.oracle_only:
        w = synth.WORKLOADS[args.workload]
        print("[bench] workload %s: generating inputs" % w.name, file=sys.stderr, flush=True)
        inp = synth.make_inputs(w)
        print("[bench] CPU oracle", file=sys.stderr, flush=True)
        rec = {"workload": w.name, "gflop": {k_: round(v_ / 1e9, 3)
                                             for k_, v_ in flops(w).items() if k_ != "n_kv"}}
        rec.update(cpu_baseline(w, inp))
        print(json.dumps(rec), flush=True)
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the hot path shards over heads "
              "with no communication); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_diffusion_order_amd as lib

    w = synth.WORKLOADS[args.workload]
    print("[bench] workload %s: generating inputs" % w.name, file=sys.stderr, flush=True)
    inp = synth.make_inputs(w)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dcode = lib.BF16 if w.dtype == "bf16" else lib.F32

    def up(a):
        a = np.ascontiguousarray(a)
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    B, H, N, d, K, L = w.B, w.H, w.N, w.d, w.topk, w.levels
    q_r, k_r, v_r, do = (up(inp[n]) for n in ("q", "k", "v", "do"))
    q, k, v = (torch.empty_like(q_r) for _ in range(3))
    out, dq, dk, dv = (torch.empty_like(q_r) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws_bytes = lib.llsa_workspace_bytes(B, H, N, d, 16, K, L, dcode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    row_bytes = d * q_r.element_size()
    shape = (B, H, N, d, 16, K, L, dcode, args.flags, ws, ws_bytes, sh)

    stages = ["zorder", "pool", "select", "attn_fwd", "transpose", "dq", "enrich", "dkdv"]

    def run_stage(name):
        if name == "zorder":
            for src, dst in ((q_r, q), (k_r, k), (v_r, v)):
                lib.llsa_grid_order(src, dst, B * H, w.frames, w.rows, w.side, row_bytes, 0, sh)
        elif name in ("pool", "select", "attn_fwd"):
            part = {"pool": lib.PART_POOL, "select": lib.PART_SELECT, "attn_fwd": lib.PART_ATTN}[name]
            lib.llsa_forward_part(part, q, k, v, out, lse, *shape)
        else:
            part = {"transpose": lib.PART_TRANSPOSE, "dq": lib.PART_DQ,
                    "enrich": lib.PART_ENRICH, "dkdv": lib.PART_DKDV}[name]
            lib.llsa_backward_part(part, q, k, v, out, lse, do, dq, dk, dv, *shape)

    def fwd():
        lib.llsa_forward(q, k, v, out, lse, *shape)

    def fwdbwd():
        lib.llsa_forward(q, k, v, out, lse, *shape)
        lib.llsa_backward(q, k, v, out, lse, do, dq, dk, dv, *shape)

    gshape = (B, H, w.frames, w.rows, w.side, d, 16, K, L, dcode, args.flags, ws, ws_bytes, sh)

    def fwd_grid():
        """the forward on raster-order inputs, the grid order folded into its
        pooling pass (llsa_forward_grid writes q, k, v in grid order)"""
        lib.llsa_forward_grid(q_r, k_r, v_r, q, k, v, out, lse, *gshape)

    def step():
        """one pass of the whole path through the public entry points: grid
        order, pool, select and attention (llsa_forward_grid), then the
        backward"""
        fwd_grid()
        lib.llsa_backward(q, k, v, out, lse, do, dq, dk, dv, *shape)

    def step_parts(evs):
        """the same work stage by stage, one stream, an event after each"""
        for si, name in enumerate(stages):
            run_stage(name)
            evs[si + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def timed(body):
        """ms per call of body over K calls, one start and one end event"""
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record(stream)
        for _ in range(args.steps):
            body()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    # headline: K whole steps
    ms_per_step = timed(step)
    # the forward (llsa_forward) and forward + backward on grid-ordered
    # inputs, and the forward with the grid order folded in, same protocol
    fwd_ms = timed(fwd)
    fwdbwd_ms = timed(fwdbwd)
    fwd_grid_ms = timed(fwd_grid)

    # breakdown: K more steps with an event after every stage (each record
    # adds a few microseconds between stages, so these are not summed into
    # the headline); each stage's time is that of its kernel launches
    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    # a head start for the host: whole steps enqueued first (the GPU stays
    # busy at full clock meanwhile), so that every stage below is enqueued
    # before the GPU reaches it and no host-side gap lands between two events
    for _ in range(max(args.steps, 20)):
        step()
    for s in range(args.steps):
        all_evs[s][0].record(stream)
        step_parts(all_evs[s])
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([ev[i].elapsed_time(ev[i + 1]) for ev in all_evs]))
                for i, name in enumerate(stages)}

    # per-rep distributions: warm (inputs and workspace may sit in the 256 MB
    # MALL from the previous rep) and cold (a 512 MiB write before each rep
    # evicts them); one event pair around each rep on the library's stream
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def reps(body, cold, n):
        out_ms = []
        for _ in range(n):
            if cold:
                flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            body()
            e1.record(stream)
            torch.cuda.synchronize()
            out_ms.append(e0.elapsed_time(e1))
        p10, p50, p90 = np.percentile(out_ms, [10, 50, 90])
        return {"p50": round(float(p50), 5), "p10": round(float(p10), 5),
                "p90": round(float(p90), 5)}

    nrep = max(args.steps, 20)
    timing = {"reps": nrep}
    for cold in (() if args.no_dist else (False, True)):
        tag = "cold" if cold else "warm"
        timing["fwd_ms_" + tag] = reps(fwd, cold, nrep)
        timing["fwdbwd_ms_" + tag] = reps(fwdbwd, cold, nrep)
        timing["grid_order_ms_" + tag] = reps(lambda: run_stage("zorder"), cold, nrep)
    del flush

    f = flops(w)
    value = f["fwdbwd"] / (ms_per_step * 1e-3) / 1e12

    # roofline of the longest single-kernel stage (attention fwd, dq or dkdv)
    peak_mfma = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    abytes = algo_bytes(w)
    # FLOPs per kernel: the backward's five products (S recomputed, dP, dQ,
    # dK, dV; 0.5 x the forward's FLOPs each) counted once, S and dP split
    # between the two kernels that both compute them: dq 1.0 x, dkdv 1.5 x
    # (sum 2.5 x).  kflops_exec: what each kernel executes, recomputation
    # included (dq: S, dP, dQ = 1.5 x; dkdv: S, dP, dK, dV = 2.0 x).
    kflops = {"attn_fwd": f["attn_fwd"], "dq": 1.0 * f["attn_fwd"], "dkdv": 1.5 * f["attn_fwd"]}
    kflops_exec = {"attn_fwd": f["attn_fwd"], "dq": 1.5 * f["attn_fwd"],
                   "dkdv": 2.0 * f["attn_fwd"]}
    kname = max(("attn_fwd", "dq", "dkdv"), key=lambda s: stage_ms[s])
    kms = stage_ms[kname]
    achieved = abytes[kname] / (kms * 1e-3) / 1e9
    # (the committed counter summaries were taken with flags 0)
    traffic = load_traffic(kname, w) if not args.flags else None
    roofline = {"kernel": kname, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic,
                "algo_bytes_per_launch": abytes[kname], "avg_launch_ms": round(kms, 5),
                "mfma_tflops": round(kflops[kname] / (kms * 1e-3) / 1e12, 2),
                "mfma_frac": round(kflops[kname] / (kms * 1e-3) / 1e12 / peak_mfma, 4),
                "mfma_tflops_incl_recompute": round(kflops_exec[kname] / (kms * 1e-3) / 1e12, 2)}

    res = {
        "metric": metric(w), "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "block_size": 16,
                   "topk": K, "levels": L, "grid": grid_name(w),
                   "sigma_px": w.sigma, "seed": w.seed,
                   **({"flags": args.flags,
                       "flops_counted_as": "flags 0 (the work of the default, non-causal path)"}
                      if args.flags else {})},
        "fwd_ms": round(fwd_ms, 5), "fwd_tflops": round(f["fwd"] / (fwd_ms * 1e-3) / 1e12, 3),
        "fwdbwd_ms": round(fwdbwd_ms, 5),
        "fwd_grid_ms": round(fwd_grid_ms, 5),
        "fwdbwd_tflops": round(f["fwdbwd"] / (fwdbwd_ms * 1e-3) / 1e12, 3),
        "fwd_mfma_frac": round(f["fwd"] / (fwd_ms * 1e-3) / 1e12 / peak_mfma, 4),
        "fwdbwd_mfma_frac": round(f["fwdbwd"] / (fwdbwd_ms * 1e-3) / 1e12 / peak_mfma, 4),
        "stage_ms": {k_: round(v_, 5) for k_, v_ in stage_ms.items()},
        "stage_gbs": {k_: round(abytes[k_] / (stage_ms[k_] * 1e-3) / 1e9, 1)
                      for k_ in abytes if k_ in stage_ms},
        "gflop": {k_: round(v_ / 1e9, 3) for k_, v_ in f.items() if k_ != "n_kv"},
        # measured HBM bytes per launch (committed rocprofv3 FETCH_SIZE +
        # WRITE_SIZE summary of the current kernel sources), where available
        "stage_hbm_mb": {k_: round(t_ / 1e6, 1) for k_, t_ in
                         ((k_, load_traffic(k_, w) if not args.flags else None)
                          for k_ in stages) if t_ is not None},
        "roofline": roofline,
        "timing": timing,
        # each attention kernel against its own algorithmic roofline,
        # min(MFMA peak, intensity x HBM peak) with intensity = FLOP / unique bytes
        "attained_vs_roofline": {
            k_: {"tflops": round(kflops[k_] / (stage_ms[k_] * 1e-3) / 1e12, 2),
                 "tflops_incl_recompute": round(kflops_exec[k_] / (stage_ms[k_] * 1e-3) / 1e12, 2),
                 "roof_tflops": round(min(peak_mfma, kflops[k_] / abytes[k_] * HBM_PEAK_GBS / 1e3), 1),
                 "frac": round(kflops[k_] / (stage_ms[k_] * 1e-3) / 1e12 /
                               min(peak_mfma, kflops[k_] / abytes[k_] * HBM_PEAK_GBS / 1e3), 4)}
            for k_ in ("attn_fwd", "dq", "dkdv")},
        # selection: fp32 dot products (ALU) and its unique bytes (HBM)
        "select_frac": {"alu": round(f["select"] / (stage_ms["select"] * 1e-3) / 1e12 /
                                     FP32_PEAK_TFLOPS, 4),
                        "hbm": round(abytes["select"] / (stage_ms["select"] * 1e-3) / 1e9 /
                                     HBM_PEAK_GBS, 4)},
    }

    if not args.no_dense:
        print("[bench] dense SDPA reference", file=sys.stderr, flush=True)
        try:
            dense = dense_reference(w, q, k, v, do)
            res["dense_sdpa"] = dict(dense, speedup_fwd=round(dense["fwd_ms"] / fwd_ms, 2),
                                     speedup_fwdbwd=round(dense["fwdbwd_ms"] / fwdbwd_ms, 2),
                                     pages_context="28.27x inference, 6.09x training at "
                                                   "256x256 (hardware not stated)")
        except Exception as ex:  # the comparison is context, not the product
            res["dense_sdpa"] = {"error": repr(ex)[:200]}

    if args.calib_copy_mib:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = nb

    if not args.no_cpu_baseline and not args.flags:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
