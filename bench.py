#!/usr/bin/env python3
"""Benchmark of the routed-experts layer on one MI355X.

One step = the whole hot path on one batch of synthetic input already resident in HBM:
routing plan -> permute -> W13 grouped GEMM + SwiGLU -> W2 grouped GEMM -> combine, then the
backward (combine transpose + dscores -> W2 DGRAD + SwiGLU derivative -> W2 WGRAD -> W13 DGRAD ->
W13 WGRAD -> dX combine).

    python bench.py [--steps K] [--warmup W] [--workload large_hidden] [--gpus 1]

Prints one JSON line: whole-step bf16 TFLOP/s (algorithmic FLOPs 18*N*D*F per step, N = T*K
routed rows) and tokens/s, the per-stage times from HIP events recorded on the layer's stream
during the timed steps, the roofline fraction of the dominant kernel, and the CPU oracle timed on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E

METRIC = "routed-expert fwd+bwd bf16 TFLOP/s and tokens/s on 1 MI355X; % MFMA/HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.made.append(e)
        return e

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a, b):
        v = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(v), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return v.value

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(e)
        self.made = []


PLAN_STAGES = ["plan_hist", "plan_scan", "plan_scatter"]
FWD_STAGES = ["permute", "fprop_w13_swiglu", "fprop_w2", "combine"]
BWD_STAGES = ["combine_bwd_dscores", "w2_backward", "permute_bwd", "wgrad_w13", "dgrad_w13",
              "dx_combine"]
# with --recompute the backward rebuilds h13 and a first (one more gate/up GEMM)
BWD_STAGES_RECOMPUTE = BWD_STAGES[:1] + ["recompute_w13"] + BWD_STAGES[1:]


def stage_work(w):
    """Algorithmic work per launch of each stage: ('mfma', FLOPs) or ('hbm', bytes)."""
    N, T, D, F = w.N, w.T, w.D, w.F
    return {
        "permute": ("hbm", 2 * T * D + 2 * N * D),
        "permute_bwd": ("hbm", 2 * T * D + 2 * N * D),
        "fprop_w13_swiglu": ("mfma", 4 * N * D * F),
        "recompute_w13": ("mfma", 4 * N * D * F),
        "fprop_w2": ("mfma", 2 * N * D * F),
        "combine": ("hbm", 2 * N * D + 2 * T * D),
        "combine_bwd_dscores": ("hbm", 2 * T * D + 4 * N * D),
        "w2_backward": ("mfma", 4 * N * D * F),  # DGRAD W2 + SwiGLU' and WGRAD W2, one launch
        "dgrad_w13": ("mfma", 4 * N * D * F),
        "wgrad_w13": ("mfma", 4 * N * D * F),
        "dx_combine": ("hbm", 2 * N * D + 2 * T * D),
    }


def cpu_baseline(inp, n_tokens, wgrad_expert=True):
    import oracle
    import workloads as W

    w = inp.w
    toks = W.sample_tokens(w.T, n_tokens, seed=1)
    t0 = time.perf_counter()
    oracle.tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, toks, inp.dout, mode="bf16")
    dt = time.perf_counter() - t0
    flops = 12 * w.K * w.D * w.F * len(toks)  # forward 6KDF + token-local backward 6KDF per token
    res = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d seeded tokens of the %s workload: forward and the token-local backward "
                  "(out, dscores, dx; weight gradients excluded), %.1f s, %.3g tokens/s"
                  % (len(toks), w.name, dt, len(toks) / dt),
    }
    if wgrad_expert and inp.dout is not None:
        # the weight gradients of the most loaded expert, whole (the oracle's matmul form: the
        # rows' gate/up products 4DF, da 2DF, dW2 2DF and dW13 4DF per row of the expert)
        import numpy as np
        ids = np.asarray(inp.ids).reshape(-1)
        counts = np.bincount(ids[(ids >= 0) & (ids < w.E)], minlength=w.E)
        e = int(np.argmax(counts))
        t0 = time.perf_counter()
        oracle.expert_wgrad(inp.x, inp.ids, inp.scores, inp.w13, inp.w2, inp.dout, e)
        dw = time.perf_counter() - t0
        res["wgrad_sample"] = {"expert": e, "rows": int(counts[e]), "s": round(dw, 2),
                               "tflops": 12 * int(counts[e]) * w.D * w.F / dw / 1e12}
    return res


# ------------------------------------------------------------------------------------------------
# rocprofv3 summaries (profiles/) and the traffic figure read back from them

SRC_FILES = ["mixture_experts_routed_plan_amd/csrc/gemm.hip",
             "mixture_experts_routed_plan_amd/csrc/rowops.hip",
             "mixture_experts_routed_plan_amd/csrc/plan.hip",
             "mixture_experts_routed_plan_amd/csrc/router.hip",
             "mixture_experts_routed_plan_amd/csrc/abi.hip",
             "mixture_experts_routed_plan_amd/csrc/moe_internal.h"]
STAGE_KERNEL = {
    "plan_hist": "moe_plan_hist", "plan_scan": "moe_plan_scan", "plan_scatter": "moe_plan_scatter",
    "permute": "moe_permute", "permute_bwd": "moe_permute",
    "fprop_w13_swiglu": "moe_fprop_w13_swiglu",
    "fprop_w2": "moe_fprop_w2", "combine": "moe_combine<true>",
    "combine_bwd_dscores": "moe_combine_bwd_dscores", "w2_backward": "moe_w2_backward",
    "dgrad_w13": "moe_dgrad_w13", "wgrad_w13": "moe_wgrad_w13",
    "dx_combine": "moe_combine<false>", "recompute_w13": "moe_fprop_w13_swiglu",
}


def source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in SRC_FILES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _short_kernel(name):
    import re
    n = re.sub(r"^void ", "", name).replace("moe::(anonymous namespace)::", "")
    n = re.sub(r"\((?!anonymous).*$", "", n)
    return n.strip()


def _family(name):
    """Kernel name without its slot-count template argument (moe_combine<true, 8> ->
    moe_combine<true>, moe_combine_bwd_dscores<8> -> moe_combine_bwd_dscores)."""
    import re
    return re.sub(r"<\d+>$", "", re.sub(r", \d+>$", ">", name))


def _counter_means(path):
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        acc[_short_kernel(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def summarize(prof_dir, out_path, workload, cmd):
    """Write a profile summary (markdown + one machine-readable JSON line) from a rocprofv3 run
    directory holding trace/ (--kernel-trace --stats), fetch/ (FETCH_SIZE), write/ (WRITE_SIZE),
    sq/ and tcc/ counter passes."""
    import csv
    stats = {}
    for r in csv.DictReader(open(os.path.join(prof_dir, "trace", "run_kernel_stats.csv"))):
        stats[_short_kernel(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                          float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3)
    # averages over the timed steps only (the warm-up dispatches, the first warmup/(warmup+steps)
    # of each kernel's calls in start order, are left out), from the same kernel trace
    import re
    import collections
    joined = " ".join(cmd)
    m_s, m_w = re.search(r"--steps (\d+)", joined), re.search(r"--warmup (\d+)", joined)
    n_steps, n_warm = int(m_s.group(1)) if m_s else 5, int(m_w.group(1)) if m_w else 1
    disp = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(prof_dir, "trace", "run_kernel_trace.csv"))):
        disp[_short_kernel(r["Kernel_Name"])].append(
            (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    timed = {}
    for k, v in disp.items():
        v.sort()
        skip = len(v) * n_warm // (n_warm + n_steps) if len(v) % (n_warm + n_steps) == 0 else 0
        rest = [d for _, d in v[skip:]]
        timed[k] = sum(rest) / len(rest) / 1e3
    fetch = _counter_means(os.path.join(prof_dir, "fetch", "run_counter_collection.csv"))
    write = _counter_means(os.path.join(prof_dir, "write", "run_counter_collection.csv"))
    sq = _counter_means(os.path.join(prof_dir, "sq", "run_counter_collection.csv"))
    tcc = _counter_means(os.path.join(prof_dir, "tcc", "run_counter_collection.csv"))
    copy = [k for k in fetch if "copyBuffer" in k]
    if not copy:
        raise SystemExit("no copy probe kernel in the counter runs (run bench.py with --copy-probe-mib)")
    probe_kib = float(open(os.path.join(prof_dir, "probe_mib")).read()) * 1024 if os.path.exists(
        os.path.join(prof_dir, "probe_mib")) else 1024 * 1024
    f_fac = probe_kib / fetch[copy[0]]["FETCH_SIZE"]
    w_fac = probe_kib / write[copy[0]]["WRITE_SIZE"]
    copy_t = [v for k, v in stats.items() if "copyBuffer" in k]
    copy_tbs = (2 * probe_kib * 1024 / (copy_t[0][1] * 1e-6) / 1e12) if copy_t else None
    rows = []
    table = {}
    for k, (calls, avg, mn, mx) in sorted(stats.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        if not k.startswith("moe_"):
            continue
        fk = fetch.get(k, {}).get("FETCH_SIZE")
        wk = write.get(k, {}).get("WRITE_SIZE")
        tb = (fk * f_fac + wk * w_fac) * 1024 if fk is not None and wk is not None else None
        q = sq.get(k, {})
        util = (q["SQ_VALU_MFMA_BUSY_CYCLES"] / (q["GRBM_GUI_ACTIVE"] / 8 * 1024)
                if q.get("GRBM_GUI_ACTIVE") else None)
        c = tcc.get(k, {})
        hit = (c["TCC_HIT_sum"] / (c["TCC_HIT_sum"] + c["TCC_MISS_sum"])
               if c.get("TCC_HIT_sum") is not None and (c["TCC_HIT_sum"] + c["TCC_MISS_sum"]) > 0
               else None)
        table[k] = {"avg_us": round(avg, 2), "timed_avg_us": round(timed.get(k, avg), 2),
                    "calls": calls, "traffic_bytes": tb,
                    "fetch_kib_raw": fk, "write_kib_raw": wk, "mfma_busy": util, "l2_hit": hit}
        rows.append("| %s | %d | %.1f | %.1f | %.1f | %.1f | %s | %s | %s | %s |" % (
            k, calls, avg, timed.get(k, avg), mn, mx,
            "%.0f" % fk if fk is not None else "-", "%.0f" % wk if wk is not None else "-",
            "%.3f" % (tb / 1e9) if tb is not None else "-",
            ("%.2f / %.2f" % (util, hit)) if util is not None and hit is not None else "-"))
    meta = {"workload": workload, "source_digest": source_digest(), "fetch_factor": f_fac,
            "write_factor": w_fac, "kernels": table}
    lines = [
        "# Kernel profile: %s workload, plan + forward + backward" % workload, "",
        "Made with rocprofv3 on one MI355X (gfx950: 256 CUs, 1024 SIMDs, 8 XCDs, 2400 MHz max "
        "engine clock) from the repository root, five timed steps after one warm-up step:", "",
        "```",
        *cmd, "```", "",
        "and summarized with `python bench.py --summarize <run dir> <this file>`.", "",
        "Traffic calibration: the run starts with a plain 1 GiB device copy (`--copy-probe-mib "
        "1024`, runtime kernel `__amd_rocclr_copyBuffer`), which reads and writes exactly "
        "1048576 KiB. On it FETCH_SIZE reads %.0f KiB and WRITE_SIZE %.0f KiB, so HBM-side "
        "traffic = %.3f x FETCH_SIZE + %.3f x WRITE_SIZE (KiB per dispatch)."
        % (fetch[copy[0]]["FETCH_SIZE"], write[copy[0]]["WRITE_SIZE"], f_fac, w_fac)
        + (" The copy itself took %.1f us in the kernel-trace run: %.2f TB/s of reads plus "
           "writes (%.0f%% of the 8 TB/s HBM peak), the streaming rate the row kernels are "
           "measured against." % (copy_t[0][1], copy_tbs, copy_tbs / 8 * 100) if copy_tbs else ""),
        "",
        "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
        "L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS). Counter runs serialize kernels, so their "
        "durations are not used; the times come from the kernel-trace run: `avg us` is "
        "rocprofv3's average over every dispatch, `timed-step avg us` the average over the "
        "dispatches of the timed steps (the warm-up step's left out), the figure to compare with "
        "the bench line's stage times.", "",
        "| kernel | calls | avg us | timed-step avg us | min us | max us | FETCH_SIZE KiB | "
        "WRITE_SIZE KiB | traffic GB | MFMA busy / L2 hit |",
        "|---|---|---|---|---|---|---|---|---|---|",
        *rows, "",
        "Source digest of the kernels profiled (sha256 of the csrc files, first 16 hex digits): "
        "`%s`" % meta["source_digest"], "",
        "<!-- machine-readable -->",
        "    " + json.dumps(meta), ""]
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines))
    print("wrote", out_path)


def profiled_traffic(workload, kernel_short):
    """HBM bytes per launch of `kernel_short` from profiles/, or None when absent or stale."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            line = line.strip()
            if line.startswith("{") and '"source_digest"' in line:
                meta = json.loads(line)
                if meta.get("workload") != workload or meta.get("source_digest") != source_digest():
                    continue
                for k, ent in meta["kernels"].items():
                    if _family(k) == kernel_short and ent.get("traffic_bytes"):
                        return ent["traffic_bytes"]
    return None


def M_lib():
    import mixture_experts_routed_plan_amd as M
    return M


def device_info(hip):
    """The GPU's name, compute-unit count and peak engine clock as the runtime reports them."""
    import torch
    p = torch.cuda.get_device_properties(0)
    clk = ctypes.c_int()
    hip.hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                              ctypes.c_int]
    # hipDeviceAttributeClockRate (kHz)
    ok = hip.hip.hipDeviceGetAttribute(ctypes.byref(clk), 5, 0) == 0
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "max_engine_clock_mhz": round(clk.value / 1e3) if ok else None}


def spread(v):
    """median, min, max and mean of a list of durations (ms)."""
    import numpy as np
    a = np.asarray(v, np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4),
            "max": round(float(a.max()), 4), "mean": round(float(a.mean()), 4)}


def plain_copy(dst, src):
    dst.copy_(src)
    return 0


def hbm_evicted(w, M, layer, stream, hip, reps=20, evict_mib=1024):
    """The HBM-bound row kernels launched alone through the C ABI, each launch preceded by a
    read-only pass over a 1 GiB buffer (four times the 256 MB infinity cache, so no operand is
    left in any cache), timed with HIP events around the kernel alone: median, min and max over
    `reps` launches. A plain device copy of 1 GiB, also after an eviction pass, gives the
    streaming ceiling of the same run."""
    import torch
    N, T, D, K = w.N, w.T, w.D, w.K
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    rows = torch.randn(N, D, device="cuda", generator=g).to(torch.bfloat16)
    tok = torch.randn(T, D, device="cuda", generator=g).to(torch.bfloat16)
    sc = torch.rand(T, K, device="cuda", generator=g)
    big_n = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    big_t = torch.empty(T, D, dtype=torch.bfloat16, device="cuda")
    dsc = torch.empty(T, K, dtype=torch.float32, device="cuda")
    evict = torch.ones((evict_mib << 20) // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    s, plan = layer.shape, layer.plan_buf
    copy_src = torch.ones((evict_mib << 20) // 4, dtype=torch.float32, device="cuda")
    copy_dst = torch.empty_like(copy_src)
    calls = {
        "permute": (lambda: M.moe_permute(s, plan, tok, big_n, stream), 2 * T * D + 2 * N * D),
        "combine": (lambda: M.moe_combine(s, plan, rows, sc, big_t, stream), 2 * N * D + 2 * T * D),
        "dx_combine": (lambda: M.moe_combine(s, plan, rows, None, big_t, stream),
                       2 * N * D + 2 * T * D),
        "combine_bwd_dscores": (lambda: M.moe_combine_backward(s, plan, tok, rows, sc, big_n, dsc,
                                                               stream), 2 * T * D + 4 * N * D),
        "plain_copy_1gib": (lambda: plain_copy(copy_dst, copy_src), 2 * (evict_mib << 20)),
    }
    res = {}
    cur = torch.cuda.current_stream()
    for name, (fn, nbytes) in calls.items():
        times = []
        for _ in range(reps + 1):
            torch.sum(evict, dim=0, out=sink)  # read-only eviction pass
            e0, e1 = hip.create(), hip.create()
            hip.record(e0, stream)
            rc = fn()
            if rc:
                raise RuntimeError("%s: %s" % (name, M.moe_status_str(rc)))
            hip.record(e1, stream)
            cur.synchronize()
            times.append(hip.ms(e0, e1))
        sp = spread(times[1:])  # the first launch warms the code object
        res[name] = dict(sp, gbs=round(nbytes / sp["median"] / 1e6, 1),
                         frac_peak=round(nbytes / sp["median"] / 1e6 / PEAK_HBM_GBS, 4),
                         algorithmic_bytes=nbytes)
    del rows, tok, big_n, big_t, evict, copy_src, copy_dst
    return res


def extras(args, w, dv, M, x, scores, w13, w2, ids, stream, hip):
    """Forward-only timing (no saving: the permute is fused into the gate/up GEMM) and the
    router on this workload's token and expert counts."""
    import torch
    fl = dv.Layer(w.T, w.D, w.F, w.E, w.K, save_for_backward=False, alloc_grads=False)
    fl.plan(ids, stream)
    for _ in range(2):
        fl.forward(x, scores, w13, w2, stream)
    f0, f1 = hip.create(), hip.create()
    torch.cuda.synchronize()
    hip.record(f0, stream)
    for _ in range(args.steps):
        fl.forward(x, scores, w13, w2, stream)
    hip.record(f1, stream)
    torch.cuda.synchronize()
    f_ms = hip.ms(f0, f1) / args.steps
    forward_only = {"ms": round(f_ms, 4),
                    "tflops": round(6 * w.N * w.D * w.F / (f_ms / 1e3) / 1e12, 1),
                    "tokens_per_s": round(w.T / (f_ms / 1e3), 1),
                    "config": "forward without saving (permute fused into the gate/up GEMM), "
                              "plan excluded"}
    del fl

    # the router on this workload's token and expert counts (N(0,1) logits, softmax top-K,
    # renormalised): HBM-bound on logits read plus ids and weights written
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    logits = torch.randn(w.T, w.E, device="cuda", generator=g)
    r_ids = torch.empty(w.T, w.K, dtype=torch.int64, device="cuda")
    r_sc = torch.empty(w.T, w.K, dtype=torch.float32, device="cuda")
    r_shape = M.make_shape(w.T, w.D, w.F, w.E, w.K)
    r_cfg = M.make_router()
    M.check(M.moe_route(r_shape, r_cfg, logits, r_ids, r_sc, stream), "moe_route")
    r0, r1 = hip.create(), hip.create()
    torch.cuda.synchronize()
    hip.record(r0, stream)
    for _ in range(20):
        M.moe_route(r_shape, r_cfg, logits, r_ids, r_sc, stream)
    hip.record(r1, stream)
    torch.cuda.synchronize()
    r_ms = hip.ms(r0, r1) / 20
    r_bytes = 4 * w.T * w.E + 12 * w.T * w.K
    router = {"ms": round(r_ms, 4), "gbs": round(r_bytes / r_ms / 1e6, 1),
              "frac_peak": round(r_bytes / r_ms / 1e6 / PEAK_HBM_GBS, 4),
              "config": "softmax top-%d of %d, renormalised, %d tokens" % (w.K, w.E, w.T)}

    # context, not a step of the path: the vendor library's dense bf16 GEMM (torch.matmul, which
    # runs hipBLASLt) on the forward GEMMs' total work as one dense product each -- [N,D]x[D,2F]
    # and [N,F]x[F,D] -- the practical MFMA ceiling of this GPU for these shapes
    vendor = {}
    for name, (m, kd, n) in (("w13", (w.N, w.D, 2 * w.F)), ("w2", (w.N, w.F, w.D))):
        g.manual_seed(1)
        a = torch.randn(m, kd, device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn(kd, n, device="cuda", generator=g).to(torch.bfloat16).contiguous()
        for _ in range(2):
            torch.matmul(a, b)
        v0, v1 = hip.create(), hip.create()
        torch.cuda.synchronize()
        hip.record(v0, torch.cuda.current_stream().cuda_stream)
        for _ in range(5):
            torch.matmul(a, b)
        hip.record(v1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        v_ms = hip.ms(v0, v1) / 5
        vendor[name] = {"ms": round(v_ms, 4),
                        "tflops": round(2.0 * m * kd * n / (v_ms / 1e3) / 1e12, 1),
                        "shape": [m, kd, n]}
        del a, b
    vendor["note"] = ("torch.matmul (hipBLASLt) on one dense bf16 GEMM of the same FLOPs as each "
                      "forward grouped GEMM (M, K, N); no routing, gather or epilogue")

    return forward_only, router, vendor


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="large_hidden")
    ap.add_argument("--skip-extras", action="store_true",
                    help="time only the fwd+bwd step (no forward-only and router lines; for "
                         "profiling runs, so that each kernel's statistics cover the step alone)")
    ap.add_argument("--keep-xg", action="store_true",
                    help="materialize xg in the forward and save it (MOE_KEEP_XG) instead of "
                         "gathering x's token rows inside the gate/up GEMM")
    ap.add_argument("--recompute", action="store_true",
                    help="save only xg and y; the backward recomputes h13 and a")
    ap.add_argument("--wgrad", default="bf16", choices=["bf16", "bf16-accumulate", "f32", "f32-accumulate"],
                    help="weight-gradient storage: bf16 or fp32, overwritten or accumulated into")
    ap.add_argument("--cpu-baseline-tokens", type=int, default=512,
                    help="tokens in the CPU oracle sample (0: skip)")
    ap.add_argument("--summarize", nargs=2, metavar=("RUN_DIR", "OUT_MD"),
                    help="write a profile summary from a rocprofv3 run directory and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (a reference kernel of "
                         "known traffic for hardware-counter runs)")
    args = ap.parse_args()
    if args.summarize:
        cmd_file = os.path.join(args.summarize[0], "commands.txt")
        cmd = open(cmd_file).read().strip().splitlines() if os.path.exists(cmd_file) else []
        # the profiled command names its workload; it wins over --workload
        named = [m.group(1) for line in cmd for m in [re.search(r"--workload (\w+)", line)] if m]
        summarize(args.summarize[0], args.summarize[1], named[0] if named else args.workload, cmd)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this layer is one GPU's share of an "
              "expert-parallel job and this build has no multi-GPU path (asked for --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as W
    from mixture_experts_routed_plan_amd import device as dv
    from mixture_experts_routed_plan_amd import moe_trace

    w = W.WORKLOADS[args.workload]
    torch.cuda.set_device(0)

    def gpu_router(logits, K):
        # logit-routed workloads: the layer's own router on the GPU (softmax top-K, renormalised)
        import mixture_experts_routed_plan_amd as M
        T, E = logits.shape
        lg = torch.from_numpy(logits).cuda()
        ids_d = torch.empty((T, K), dtype=torch.int64, device="cuda")
        sc_d = torch.empty((T, K), dtype=torch.float32, device="cuda")
        shape = M.make_shape(T, 64, 64, E, K, ids_dtype=M.MOE_IDS_I64)
        M.check(M.moe_route(shape, M.make_router(), lg, ids_d, sc_d), "moe_route")
        torch.cuda.synchronize()
        return ids_d.cpu().numpy(), sc_d.cpu().numpy()

    t0 = time.time()
    inp = W.make_inputs(w, with_dout=True,
                        router=gpu_router if w.routing in W.LOGIT_ROUTINGS else None)
    log("bench: %s inputs drawn in %.1fs" % (w.name, time.time() - t0))

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src_buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst_buf = torch.empty_like(src_buf)
        torch.cuda.synchronize()
        dst_buf.copy_(src_buf)  # reads and writes exactly n bytes
        torch.cuda.synchronize()
        del src_buf, dst_buf
        log("bench: copy probe of %d MiB done" % args.copy_probe_mib)
    x, w13, w2, dout = (dv.to_device_bits(a) for a in (inp.x, inp.w13, inp.w2, inp.dout))
    ids = torch.from_numpy(inp.ids).cuda()
    scores = torch.from_numpy(inp.scores).cuda()
    layer = dv.Layer(w.T, w.D, w.F, w.E, w.K, save_for_backward=True,
                     wgrad_accumulate=args.wgrad.endswith("accumulate"),
                     wgrad_f32=args.wgrad.startswith("f32"), recompute=args.recompute,
                     keep_xg=args.keep_xg)
    # without MOE_KEEP_XG (and with x below 4 GiB) the forward's permute stage is empty and the
    # backward permutes xg into its workspace; with it, the other way round
    gathers = not args.keep_xg and 2 * w.T * w.D < 2 ** 32
    empty = {"permute": "fused: the gate/up GEMM gathers x's token rows, no kernel"} if gathers \
        else {"permute_bwd": "xg saved by the forward, no kernel"}
    bwd_stages = BWD_STAGES_RECOMPUTE if args.recompute else BWD_STAGES
    stream = torch.cuda.current_stream().cuda_stream
    hip = HipEvents()

    def make_trace(n):
        tr = moe_trace()
        tr.n_events = n
        evs = [hip.create() for _ in range(n)]
        for i, e in enumerate(evs):
            tr.events[i] = e.value
        return tr, evs

    def step(traces=None):
        tp, tf, tb = traces if traces else (None, None, None)
        layer.plan(ids, stream, tp)
        layer.forward(x, scores, w13, w2, stream, tf)
        layer.backward(dout, scores, w13, w2, stream, tb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("bench: %d warmup steps done" % args.warmup)

    traces = [(make_trace(4), make_trace(5), make_trace(len(bwd_stages) + 1))
              for _ in range(args.steps)]
    start, end = hip.create(), hip.create()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hip.record(start, stream)
    for k in range(args.steps):
        step(tuple(t[0] for t in traces[k]))
    hip.record(end, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = hip.ms(start, end)
    ms = total_ms / args.steps
    log("bench: %d timed steps, %.3f ms/step (wall %.3f ms/step)" %
        (args.steps, ms, 1e3 * wall / args.steps))

    names = PLAN_STAGES + FWD_STAGES + bwd_stages
    per = {n: [] for n in names}
    step_ms = []
    call_ms = {"plan": [], "forward": [], "backward": []}  # each whole ABI call
    for (tp, ep), (tf, ef), (tb, eb) in traces:
        for lst, evs in ((PLAN_STAGES, ep), (FWD_STAGES, ef), (bwd_stages, eb)):
            for i, n in enumerate(lst):
                per[n].append(hip.ms(evs[i], evs[i + 1]))
        step_ms.append(hip.ms(ep[0], eb[-1]))
        for c, evs in (("plan", ep), ("forward", ef), ("backward", eb)):
            call_ms[c].append(hip.ms(evs[0], evs[-1]))
    work = stage_work(w)
    stages = {}
    for n in names:
        avg = float(np.mean(per[n]))
        sp = spread(per[n])
        ent = {"ms": round(avg, 4), "median_ms": sp["median"], "min_ms": sp["min"],
               "max_ms": sp["max"]}
        if n in empty:
            ent["note"] = empty[n]
        elif n in work:
            kind, amount = work[n]
            if kind == "mfma":
                ent["tflops"] = round(amount / avg / 1e9, 1)
                ent["frac_peak"] = round(amount / avg / 1e9 / PEAK_BF16_TFLOPS, 4)
            else:
                ent["gbs"] = round(amount / avg / 1e6, 1)
                ent["frac_peak"] = round(amount / avg / 1e6 / PEAK_HBM_GBS, 4)
        stages[n] = ent
    dom = max((n for n in work if n in stages and n not in empty), key=lambda n: stages[n]["ms"])
    kind, amount = work[dom]
    avg_s = stages[dom]["ms"] / 1e3
    if kind == "mfma":
        roof = {"bound": "mfma", "achieved": round(amount / avg_s / 1e12, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(amount / avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = profiled_traffic(w.name, STAGE_KERNEL[dom])
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = amount

    forward_only = router = vendor = evicted = None
    if not args.skip_extras:
        forward_only, router, vendor = extras(args, w, dv, M_lib(), x, scores, w13, w2, ids, stream, hip)
        evicted = hbm_evicted(w, M_lib(), layer, stream, hip)
        for n, ent in evicted.items():
            if n in stages and "frac_peak" in stages[n]:
                ent["in_step_frac_peak"] = stages[n]["frac_peak"]

    flops = 18 * w.N * w.D * w.F
    res = {
        "metric": METRIC,
        "value": round(flops / (ms / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "tokens_per_s": round(w.T / (ms / 1e3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "step_ms": spread(step_ms),
        "call_ms": {c: spread(v) for c, v in call_ms.items()},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: T=%d D=%d F=%d E=%d K=%d, plan+forward+backward"
                               % (w.name, w.T, w.D, w.F, w.E, w.K),
                   "T": w.T, "D": w.D, "F": w.F, "E": w.E, "K": w.K,
                   "routing": w.routing, "wgrad": args.wgrad, "recompute": args.recompute,
                   "keep_xg": args.keep_xg,
                   "parallelism": "single GPU (one EP rank's share)"},
        "roofline": roof,
        "device": device_info(hip),
        "stages": stages,
        "hbm_kernels_evicted": evicted,
        "router": router,
        "forward_only": forward_only,
        "vendor_dense_gemm": vendor,
    }
    hip.close()
    if args.cpu_baseline_tokens > 0:
        log("bench: timing the CPU oracle on %d tokens" % args.cpu_baseline_tokens)
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_baseline_tokens)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
