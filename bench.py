"""Benchmark of the block-scaled GEMM hot path on one MI355X.

Default workload (one "step" = one pass of the MoE expert forward hot path):
  E = 32 experts, 16384 tokens x top-4 = 65536 routed rows; per-expert
  counts ~ Multinomial(65536, Dirichlet(1)), each group padded to a multiple
  of 128 rows (cumulative int32 ends); K = 4096, gate|up N = 2 x 1536.
    1. hq_group_wise_quant     MXFP8 quantisation of the [R, 4096] activations
    2. hq_group_contiguous_gemm_swiglu_quant  [R, 4096] x [32, 3072, 4096]^T with
       y = up * silu(gate) of the valid rows re-quantised to MXFP8 in the
       GEMM's epilogue (--workload moe_unfused: hq_group_contiguous_gemm to
       BF16 [R, 3072], then hq_fused_swiglu_quant; the per-kernel pass also
       times these two calls beside the fused one)
  Weights are quantised once before timing (they are static parameters).
  The timed loop records HIP events around every launch on the stream the
  kernels run on, so the per-kernel times (and the roofline of the dominant
  kernel) come from the timed steps themselves.

After the headline the default run times one launch configuration of each
other workload ("configs" in the JSON line; --no-configs skips them, --only
ID runs one of them alone, e.g. under a profiler):
  d0  dense MXFP8 256^3 (seed 0)
  d1  batch MXFP8 4 x 256^3 with and without bias; dense MXFP4 32 x 512 x 256
  d2  dense MXFP4 / NVFP4, N = 17408, K = 5120, M in {1, 512, 4096} (with the
      caller workspace the plan asks for: NVFP4 takes stream-K at M = 512 and
      the tail split at 4096; the MXFP4 cells run unsplit)
  d4  grouped-masked MXFP4, 64 experts x 256-row slots, K = 7168, N = 4096
  n3  the backward grouped GEMM with the dSwiGLU epilogue, MXFP8, the MoE shape
      (32 experts, 65536 routed rows, K = 4096, N = 1536, C / D [rows, 3072]);
      n3_q the same with D row-quantised (MXFP8 codes + UE8M0 scales)
  d5  quantisation bandwidth: MXFP4 [16384, 7168], NVFP4 [4096, 17408] (global
      scale supplied, and with the amax pass, whose bytes count the input's
      second read: the global scale needs all of it before the first code)
each with its time per launch (HIP events around batches of back-to-back
launches queued behind a spin kernel, so that short kernels are timed
without the host's launch latency or per-launch event markers), achieved rate, roofline fraction and, where affordable, the
oracle's time for the same work on the host cores (the d2 cells above M = 1,
d4 and n3: its rate on a sample of the rows, named in the record).

Output: one JSON line with the whole-step throughput (algorithmic GEMM FLOPs
of the valid rows per second), the per-kernel times, the roofline of the
dominant kernel (the grouped GEMM, against the dense MXFP8 matrix-core peak),
the oracle timed on a bounded sample on the host cores, and the configs.

    python bench.py [--steps K] [--warmup W] [--no-configs] [--only ID]
                    [--workload moe|moe_unfused|moe_mlp|dense_fp4|masked_fp4|permute|configs]
    python bench.py --workload sweep    # dense qualification grid + quant bandwidths,
                                        # one JSON line per case
    python bench.py --workload ab --ab-lib OTHER/libhq.so   # interleaved A/B of the
                                        # skinny cells and NVFP4 quant against another build
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"mxfp8": 5000.0, "mxfp4": 10100.0, "nvfp4_f16": 2500.0}
PEAK_HBM_GBS = 8000.0
METRIC = "MXFP8/MXFP4 grouped GEMM TFLOP/s + % MFMA peak; quant/SwiGLU GB/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class Timer:
    """Per-kernel HIP-event timing on the stream the kernels run on (the
    binding launches on torch.cuda.current_stream(), where the events are
    recorded)."""

    def __init__(self, torch):
        self.torch = torch
        self.ev = {}

    def mark(self, name, fn):
        stream = self.torch.cuda.current_stream()
        s = self.torch.cuda.Event(enable_timing=True)
        e = self.torch.cuda.Event(enable_timing=True)
        s.record(stream)
        fn()
        e.record(stream)
        self.ev.setdefault(name, []).append((s, e))

    def times_ms(self, name):
        return [s.elapsed_time(e) for s, e in self.ev[name]]

    def mean_ms(self, name):
        return float(np.mean(self.times_ms(name)))

    def median_ms(self, name):
        return float(np.median(self.times_ms(name)))


def _traffic(kernel_key):
    """HBM bytes per launch measured with counters (profiles/traffic.json), or
    None when there is no measurement or the kernel's sources changed since
    the counters were taken (their SHA-256 no longer matches)."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
        if not rec:
            return None
        h = hashlib.sha256()
        for name in rec["sources"]:
            with open(os.path.join(ROOT, "fp4_gemm_moe_amd", "csrc", name), "rb") as f:
                h.update(f.read())
        return int(rec["bytes"]) if h.hexdigest() == rec["sources_sha256"] else None
    except (OSError, ValueError, KeyError, TypeError):
        return None


# ---------------------------------------------------------------- MoE workload
def run_moe(args, torch, hq, synth, down=False, fused=False):
    """The MoE expert forward step: MXFP8 quantisation of the routed
    activations, the grouped gate|up GEMM, the fused SwiGLU + MXFP8 re-quant;
    with down=True also the down-projection grouped GEMM (K = H = 1536,
    N = hidden = 4096) on the SwiGLU codes -- the whole expert MLP; with
    fused=True the gate|up GEMM applies SwiGLU + re-quant in its epilogue
    (one call instead of two, no BF16 [rows, 3072] intermediate)."""
    dev = torch.device("cuda:0")
    log("generating MoE inputs (E=32, 65536 routed rows, K=4096, N=3072)")
    d = synth.moe_contiguous(threads=16)
    counts, ends = d["counts"], d["group_end"]
    R, K, N, H, E = int(ends[-1]), d["K"], d["N"], d["H"], len(counts)
    T = int(counts.sum())
    x = _dev_bf16(torch, d["a"], dev)
    w_bf16 = _dev_bf16(torch, d["b"].reshape(E * N, K), dev)
    wq, wsf, _ = hq.quantize(w_bf16, "mxfp8")
    del w_bf16
    wq = wq.view(E, N, K)
    wsf = wsf.view(E, N, K // 32)
    ge = torch.from_numpy(ends.astype(np.int32)).to(dev)
    valid = torch.from_numpy(counts.astype(np.int32)).to(dev)
    aq = torch.empty(R, K, dtype=torch.uint8, device=dev)
    asf = torch.empty(R, K // 32, dtype=torch.uint8, device=dev)
    out = torch.empty(R, N, dtype=torch.bfloat16, device=dev)
    yq = torch.empty(R, H, dtype=torch.uint8, device=dev)
    ysf = torch.empty(R, H // 32, dtype=torch.uint8, device=dev)
    HID = 4096
    if down:
        log("generating down-projection weights (E=32, 4096 x 1536)")
        w2 = _dev_bf16(torch, synth.moe_down_weights(E, HID, H, threads=16).reshape(E * HID, H), dev)
        w2q, w2sf, _ = hq.quantize(w2, "mxfp8")
        del w2
        w2q, w2sf = w2q.view(E, HID, H), w2sf.view(E, HID, H // 32)
        out2 = torch.empty(R, HID, dtype=torch.bfloat16, device=dev)

    timer = Timer(torch)

    def step(t=None, timed=True):
        """One step; with a timer, events around each launch.  timed=False:
        the two-call form of the fused step, timed beside it."""
        f1 = lambda: hq.hq_group_wise_quant("mxfp8", x, aq, asf)
        f2 = lambda: hq.hq_group_contiguous_gemm("mxfp8", aq, asf, wq, wsf, ge, out)
        f3 = lambda: hq.hq_fused_swiglu_quant("mxfp8", out, yq, ysf, E, ge, 0, valid)
        f4 = lambda: hq.hq_group_contiguous_gemm("mxfp8", yq, ysf, w2q, w2sf, ge, out2)
        f5 = lambda: hq.hq_group_contiguous_gemm_swiglu_quant("mxfp8", aq, asf, wq, wsf, ge, yq, ysf,
                                                              valid=valid)
        if t is None:
            if fused:
                f1(); f5()
            else:
                f1(); f2(); f3()
            if down:
                f4()
        elif not timed:
            t.mark("gemm", f2)
            t.mark("swiglu", f3)
        else:
            t.mark("quant", f1)
            if fused:
                t.mark("gemm_swiglu", f5)
            else:
                t.mark("gemm", f2)
                t.mark("swiglu", f3)
            if down:
                t.mark("down", f4)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # the timed steps: events around every launch, and around the whole run
    stream = torch.cuda.current_stream()
    t_start = torch.cuda.Event(enable_timing=True)
    t_stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step(timer, timed=True)
    t_stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the two-call form beside the fused one (not part of the step)
    if fused:
        for _ in range(args.steps):
            step(timer, timed=False)
        torch.cuda.synchronize()

    ms_step = t_start.elapsed_time(t_stop) / args.steps
    log(f"step {ms_step:.4f} ms (events), {wall * 1e3 / args.steps:.4f} ms (host clock)")
    flops = 2.0 * T * N * K
    quant_bytes = R * K * (2 + 1 + 1 / 32)     # the whole padded activation buffer
    swiglu_bytes = T * H * (4 + 1 + 1 / 32)
    quant_ms = timer.mean_ms("quant")
    sw_ms = timer.mean_ms("swiglu")
    kernels = {
        "quant_mxfp8": {"ms": quant_ms, "GB/s": quant_bytes / (quant_ms * 1e-3) / 1e9,
                        "frac_hbm": quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "traffic": _traffic("quant_mxfp8")},
    }
    gkeys = [("gemm_swiglu", "grouped_gemm_swiglu_mxfp8")] if fused else []
    gkeys.append(("gemm", "grouped_gemm_mxfp8"))
    for ev, key in gkeys:
        g_ms = timer.mean_ms(ev)
        g_tf = flops / (g_ms * 1e-3) / 1e12
        kernels[key] = {"ms": g_ms, "TFLOP/s": g_tf, "frac_mfma": g_tf / PEAK_TFLOPS["mxfp8"],
                        "traffic": _traffic(key)}
    kernels["swiglu_quant_mxfp8"] = {"ms": sw_ms, "GB/s": swiglu_bytes / (sw_ms * 1e-3) / 1e9,
                                     "frac_hbm": swiglu_bytes / (sw_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                     "traffic": _traffic("swiglu_quant_mxfp8")}
    if fused:
        kernels["grouped_gemm_mxfp8"]["note"] = "two-call form, timed beside the step"
        kernels["swiglu_quant_mxfp8"]["note"] = "two-call form, timed beside the step"
    for v in kernels.values():
        v["launches"] = args.steps
    gkey = gkeys[0][1]                  # the step's GEMM: the roofline's kernel
    gemm_ms = kernels[gkey]["ms"]
    gemm_tflops = kernels[gkey]["TFLOP/s"]
    cfg = {"workload": "moe_grouped_contiguous_mxfp8_E32_T65536_K4096_N3072_swiglu"
                       + ("_fused_epilogue" if fused else ""),
           "experts": E, "routed_rows": T, "padded_rows": R, "k": K, "n": N, "h": H,
           "group_align": 128}
    if down:
        down_ms = timer.mean_ms("down")
        down_flops = 2.0 * T * HID * H
        kernels["down_gemm_mxfp8"] = {"ms": down_ms, "TFLOP/s": down_flops / (down_ms * 1e-3) / 1e12,
                                      "frac_mfma": down_flops / (down_ms * 1e-3) / 1e12 / PEAK_TFLOPS["mxfp8"]}
        cfg = dict(cfg, workload="moe_mlp_mxfp8_E32_T65536_K4096_H1536_hidden4096", hidden=HID)
    roof = {"bound": "mfma", "achieved": gemm_tflops, "peak": PEAK_TFLOPS["mxfp8"],
            "unit": "TFLOP/s", "frac": gemm_tflops / PEAK_TFLOPS["mxfp8"],
            "traffic": _traffic(gkey),
            "kernel": gkey, "flop_per_launch": flops, "mean_launch_ms": gemm_ms,
            "median_launch_ms": timer.median_ms(gkeys[0][0]), "launches": args.steps}
    step_flops = flops + (down_flops if down else 0.0)
    value = step_flops / (ms_step * 1e-3) / 1e12
    ctx = None if down else {"counts": counts, "ends": ends, "a": d["a"], "b": d["b"], "K": K, "N": N, "H": H}
    return value, ms_step, cfg, roof, kernels, ctx


def cpu_baseline_moe(ctx, budget_s=12.0):
    """The oracle on a bounded sample of the same step: the routed rows of
    experts 0, 1, 2, ... (quantise, GEMM against the expert's weights, SwiGLU +
    re-quantise) until about budget_s seconds of CPU work.  Each expert's
    weights are quantised by the oracle before its clock starts, like the
    device path's static weights."""
    from oracle import gemm as G
    from oracle import quant as Q
    from oracle import swiglu as S
    K, N, H = ctx["K"], ctx["N"], ctx["H"]
    counts, ends = ctx["counts"], ctx["ends"]
    starts = np.concatenate([[0], ends[:-1]]).astype(np.int64)
    spent, rows_done, experts = 0.0, 0, 0
    for g in range(len(counts)):
        c = int(counts[g])
        if c == 0:
            continue
        w, wsf = Q.mx_quant_bf16(ctx["b"][g], "mxfp8")
        xa = ctx["a"][starts[g]:starts[g] + c]
        t0 = time.perf_counter()
        a, sfa = Q.mx_quant_bf16(xa, "mxfp8")
        out = G.dense_gemm("mxfp8", a, sfa, w, wsf)
        S.swiglu_quant(out, H, "mxfp8")
        spent += time.perf_counter() - t0
        rows_done += c
        experts += 1
        if spent >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    tflops = 2.0 * rows_done * N * K / spent / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"routed rows of the first {experts} non-empty experts ({rows_done} of "
                      f"{int(counts.sum())} rows): MXFP8 quant + GEMM + SwiGLU/quant, {spent:.1f} s"}


# ---------------------------------------------------------------- other workloads
def run_permute(args, torch, hq, synth):
    """Token permute into the masked layout at the shapes of the HALOps
    "GEMM" page's prefill_permute_to_masked_gemm example (1024 tokens of
    hidden 2048 in BF16, top-8 of 16 experts, max_token_num 1024, int32
    broadcast scales); --tokens scales the token count."""
    dev = torch.device("cuda:0")
    T, H, topk, E = args.tokens, 2048, 8, 16
    M = max(1024, ((T * topk // E) * 2 + 127) // 128 * 128)      # headroom for imbalance
    d = synth.permute_inputs(T, H, topk, E)
    x = _dev_bf16(torch, d["x"], dev)
    scale = torch.from_numpy(d["scale"]).to(dev)
    ids = torch.from_numpy(d["topk_ids"]).to(dev)
    px = torch.empty(E * M, H, dtype=torch.bfloat16, device=dev)
    osf = torch.empty(E, M, H // 32, dtype=torch.uint8, device=dev)
    imap = torch.empty(T, topk, dtype=torch.int32, device=dev)
    nums = torch.empty(E, dtype=torch.int32, device=dev)
    f = lambda: hq.hq_prefill_permute_to_masked_gemm(x, scale, ids, E, M, px, osf, imap, nums)
    _, us = _launch_us(torch, [f], reps=max(args.steps, 5), warm=args.warmup)
    ms = us * 1e-3
    placed = int(nums.sum().item())
    # read x, scales, ids; write the placed rows and scale rows, the map, the counts
    bytes_ = T * (2 * H + H // 128 + 8 * topk) + placed * (2 * H + H // 32) + 4 * T * topk + 4 * E
    gbs = bytes_ / (ms * 1e-3) / 1e9
    cfg = {"workload": f"prefill_permute_to_masked_T{T}_H{H}_top{topk}_E{E}_M{M}_bf16_broadcast",
           "tokens": T, "hidden": H, "topk": topk, "experts": E, "max_token_num": M}
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": _traffic("permute_bf16_T16384") if T == 16384 else None}
    return gbs, ms, cfg, roof, {"permute": {"ms": ms, "GB/s": gbs, "bytes": bytes_}}, None, "GB/s"


def run_dense_fp4(args, torch, hq, synth):
    dev = torch.device("cuda:0")
    mode = args.mode
    n, k, m = args.n, args.k, args.m
    d = synth.dense_fp4_large(n, k, m)
    x = _dev_bf16(torch, d["a"], dev)
    w = _dev_bf16(torch, d["b"], dev)
    wq, wsf, gw = hq.quantize(w, mode)
    aq, asf, ga = hq.quantize(x, mode)
    alpha = (ga * gw) if mode == "nvfp4" else None
    out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    timer = Timer(torch)
    ws = hq.gemm_workspace(mode, m, n, k, device=dev)
    f = lambda: hq.hq_dense_gemm(mode, aq, asf, wq, wsf, out, alpha=alpha, workspace=ws)
    for _ in range(args.warmup):
        f()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        timer.mark("gemm", f)
    torch.cuda.synchronize()
    ms = timer.mean_ms("gemm")
    flops = 2.0 * m * n * k
    tf = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["nvfp4_f16" if mode == "nvfp4" else mode]
    gs = 16 if mode == "nvfp4" else 32
    bytes_ = (m + n) * k * (0.5 + 1 / gs) + 2 * m * n
    cfg = {"workload": f"dense_{mode}_M{m}_N{n}_K{k}", "m": m, "n": n, "k": k}
    roof = {"bound": "mfma" if m >= 512 else "hbm", "achieved": tf if m >= 512 else bytes_ / (ms * 1e-3) / 1e9,
            "peak": peak if m >= 512 else PEAK_HBM_GBS, "unit": "TFLOP/s" if m >= 512 else "GB/s",
            "traffic": _traffic("dense_gemm_mxfp4")
            if (mode, m, n, k) == ("mxfp4", 4096, 17408, 5120) else None}
    roof["frac"] = roof["achieved"] / roof["peak"]
    return tf, ms, cfg, roof, {"dense_gemm": {"ms": ms, "TFLOP/s": tf, "GB/s": bytes_ / (ms * 1e-3) / 1e9}}, None


def run_masked_fp4(args, torch, hq, synth):
    dev = torch.device("cuda:0")
    d = synth.moe_masked(threads=16)
    E, Mmax, K, N = 64, d["max_m"], d["K"], d["N"]
    counts = d["counts"]
    T = int(counts.sum())
    x = _dev_bf16(torch, d["a"], dev)
    aq, asf, _ = hq.quantize(x, "mxfp4")
    w = _dev_bf16(torch, d["b"].reshape(E * N, K), dev)
    wq, wsf, _ = hq.quantize(w, "mxfp4")
    del w
    wq, wsf = wq.view(E, N, K // 2), wsf.view(E, N, K // 32)
    cnt = torch.from_numpy(counts.astype(np.int32)).to(dev)
    out = torch.empty(E * Mmax, N, dtype=torch.bfloat16, device=dev)
    timer = Timer(torch)
    f = lambda: hq.hq_group_masked_gemm("mxfp4", aq, asf, wq, wsf, cnt, out, Mmax)
    for _ in range(args.warmup):
        f()
    torch.cuda.synchronize()
    for _ in range(args.steps):
        timer.mark("gemm", f)
    torch.cuda.synchronize()
    ms = timer.mean_ms("gemm")
    flops = 2.0 * T * N * K
    experts = int((counts > 0).sum())
    bytes_ = T * K * (0.5 + 1 / 32) + experts * N * K * (0.5 + 1 / 32) + 2 * T * N
    gbs = bytes_ / (ms * 1e-3) / 1e9
    cfg = {"workload": "moe_grouped_masked_mxfp4_E64_Mmax256_K7168_N4096", "routed_rows": T}
    roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": gbs / PEAK_HBM_GBS, "traffic": _traffic("masked_gemm_mxfp4")}
    tf = flops / (ms * 1e-3) / 1e12
    return tf, ms, cfg, roof, {"masked_gemm_mxfp4": {"ms": ms, "TFLOP/s": tf, "GB/s": gbs}}, None


def _time_us(torch, fns, reps=15, per=20):
    """Median over `reps` batches of the mean time per launch of a batch of
    `per` launches (HIP events on the current stream); fns is cycled so that a
    ring of buffers can be rotated through (cold-cache timing).  Each batch
    queues behind a spin kernel (_hold_gpu), so the batch runs back to back on
    the GPU whatever the host's time per launch."""
    i = 0
    for _ in range(10):
        fns[i % len(fns)]()
        i += 1
    torch.cuda.synchronize()
    res = []
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        _hold_gpu(torch, 1000 + 150 * per)
        s.record()
        for _ in range(per):
            fns[i % len(fns)]()
            i += 1
        e.record()
        torch.cuda.synchronize()
        res.append(s.elapsed_time(e) * 1e3 / per)
    return float(np.median(res))


def run_sweep(args, torch, hq, synth):
    """The dense qualification grid (3 (N, K) x M in {1, 16, 512, 4096} x
    {MXFP4, NVFP4}) and the standalone quantisation bandwidths, one JSON line
    per case.  HBM-bound cases are timed warm and cold (a ring of >= 1 GB of
    buffers rotated through, larger than the 256 MB Infinity Cache)."""
    dev = torch.device("cuda:0")
    ring_bytes = 1 << 30

    def emit(rec):
        print(json.dumps(rec), flush=True)

    for (n, k) in synth.LARGE_NK:
        wbits = synth.dense_fp4_large_weights(n, k)
        w = _dev_bf16(torch, wbits, dev)
        for mode in ("mxfp4", "nvfp4"):
            wq, wsf, gw = hq.quantize(w, mode)
            wbytes = wq.numel() + wsf.numel()
            copies = max(1, -(-ring_bytes // wbytes))
            ring = [(wq.clone(), wsf.clone()) for _ in range(copies)]
            for m in synth.LARGE_M:
                x = _dev_bf16(torch, synth.dense_fp4_large_acts(n, k, m), dev)
                aq, asf, ga = hq.quantize(x, mode)
                alpha = (ga * gw) if mode == "nvfp4" else None
                out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
                ws = hq.gemm_workspace(mode, m, n, k, device=dev)
                warm = _time_us(torch, [lambda: hq.hq_dense_gemm(mode, aq, asf, wq, wsf, out, alpha=alpha,
                                                                 workspace=ws)])
                cold = None
                if m <= 16:
                    cold = _time_us(torch, [lambda q=q, s_=s_: hq.hq_dense_gemm(mode, aq, asf, q, s_, out,
                                                                                   alpha=alpha, workspace=ws)
                                            for q, s_ in ring])
                flops = 2.0 * m * n * k
                gs = 16 if mode == "nvfp4" else 32
                bytes_ = (m + n) * k * (0.5 + 1 / gs) + 2 * m * n
                peak = PEAK_TFLOPS["nvfp4_f16" if mode == "nvfp4" else mode]
                t_ideal = max(flops / (peak * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9)) * 1e6
                t = cold if cold is not None else warm
                emit({"case": "dense_gemm", "mode": mode, "m": m, "n": n, "k": k,
                      "us_warm": round(warm, 2), "us_cold": None if cold is None else round(cold, 2),
                      "TFLOP/s": round(flops / (t * 1e-6) / 1e12, 1),
                      "GB/s": round(bytes_ / (t * 1e-6) / 1e9, 1),
                      "bound": "hbm" if bytes_ / (PEAK_HBM_GBS * 1e9) > flops / (peak * 1e12) else "mfma",
                      "t_ideal_us": round(t_ideal, 2), "roofline_frac": round(t_ideal / t, 3),
                      "kernel": "direct" if m <= 16 else "tiled"})
                del x, aq, asf, out
            del ring, wq, wsf
        del w
        torch.cuda.empty_cache()

    quant_cases = [("mxfp8", 65536, 4096), ("mxfp4", 16384, 7168), ("mxfp4", 4096, 17408),
                   ("nvfp4", 4096, 17408)]
    rng = np.random.default_rng(5)
    for mode, m, k in quant_cases:
        x = _dev_bf16(torch, synth.normal_bf16(rng, (m, k)), dev)
        copies = max(1, -(-ring_bytes // (2 * m * k)))
        xs = [x] + [x.clone() for _ in range(copies - 1)]
        q, sf, g = hq.quantize(x, mode)
        gs = 16 if mode == "nvfp4" else 32
        elem = 2 + (1 if mode == "mxfp8" else 0.5) + 1 / gs
        variants = [("", None)] if mode != "nvfp4" else [(" amax", None), (" g supplied", g.clone())]
        for tag, gin in variants:
            def mk(xx, gin=gin):
                if gin is None:
                    return lambda: hq.hq_group_wise_quant(mode, xx, q, sf, g)
                return lambda: hq.hq_group_wise_quant(mode, xx, q, sf, gin, hq.HQ_GS_INPUT)
            warm = _time_us(torch, [mk(x)])
            cold = _time_us(torch, [mk(xx) for xx in xs])
            bytes_ = m * k * elem
            extra = 2 * m * k if (mode == "nvfp4" and gin is None) else 0
            emit({"case": "quant" + tag, "mode": mode, "m": m, "k": k,
                  "us_warm": round(warm, 2), "us_cold": round(cold, 2),
                  "GB/s": round(bytes_ / (cold * 1e-6) / 1e9, 1),
                  "GB/s_incl_amax_pass": round((bytes_ + extra) / (cold * 1e-6) / 1e9, 1) if extra else None,
                  "roofline_frac": round(bytes_ / (PEAK_HBM_GBS * 1e9) / (cold * 1e-6), 3)})
        del x, xs, q, sf
        torch.cuda.empty_cache()


# ---------------------------------------------------------------- per-config records
def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


_SLEEP_CYCLES_PER_US = None


def _hold_gpu(torch, us):
    """Queues a spin kernel of about `us` microseconds on the current stream,
    so that launches queued behind it start back to back: each event pair
    then brackets GPU time, not the host's time to issue the next launch."""
    global _SLEEP_CYCLES_PER_US
    if _SLEEP_CYCLES_PER_US is None:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1 << 20)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_US = (1 << 20) / max(e0.elapsed_time(e1) * 1e3, 1.0)
    torch.cuda._sleep(int(us * _SLEEP_CYCLES_PER_US))


def _launch_us(torch, fns, reps=30, warm=5, per=None):
    """Time per launch: HIP events on the current stream around batches of
    `per` back-to-back launches (about reps launches in all, at least 5
    batches) after `warm` untimed ones; fns is cycled (a ring of buffers for
    cold-cache timing).  Each batch queues behind a spin kernel that outlasts
    its issue, so the launches run back to back whatever the host's time per
    launch, and no event marker sits between two launches (a marker pair
    around every launch adds about 5 us).  Returns (median, mean) over the
    batches of the mean time per launch, in us."""
    for i in range(warm):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    if per is None:
        per = max(1, reps // 5)
    nb = max(5, reps // per)
    res = []
    i = warm
    for _ in range(nb):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        _hold_gpu(torch, 1000 + 150 * per)
        s.record()
        for _ in range(per):
            fns[i % len(fns)]()
            i += 1
        e.record()
        torch.cuda.synchronize()
        res.append(s.elapsed_time(e) * 1e3 / per)
    return float(np.median(res)), float(np.mean(res))


def _oracle_us(fn, reps=3):
    best = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        best.append(time.perf_counter() - t0)
    return float(np.median(best)) * 1e6


def _rec(cid, workload, us, flops=None, bytes_=None, bound="mfma", peak_key="mxfp8", **extra):
    """One config record: time, achieved rate against the bound's peak, and
    the call's HBM bytes measured by counters (profiles/traffic.json, key =
    the config id; None when unmeasured or the sources changed since)."""
    r = {"id": cid, "workload": workload, "us": round(us, 2), "traffic": _traffic(cid)}
    if flops is not None:
        r["TFLOP/s"] = round(flops / (us * 1e-6) / 1e12, 2)
    if bytes_ is not None:
        r["GB/s"] = round(bytes_ / (us * 1e-6) / 1e9, 1)
    if bound == "hbm":
        r.update(bound="hbm", peak=PEAK_HBM_GBS, unit="GB/s", frac=round(bytes_ / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 3))
    else:
        pk = PEAK_TFLOPS[peak_key]
        r.update(bound=bound, peak=pk, unit="TFLOP/s", frac=round(flops / (us * 1e-6) / 1e12 / pk, 4))
    r.update(extra)
    return r


CONFIG_IDS = ["d0", "d1_batch", "d1_batch_bias", "d1_mxfp4",
              "d2_mxfp4_M1", "d2_mxfp4_M512", "d2_mxfp4_M4096",
              "d2_nvfp4_M1", "d2_nvfp4_M512", "d2_nvfp4_M4096",
              "d4", "n3", "n3_q", "d5_mxfp4", "d5_nvfp4", "d5_nvfp4_amax"]


def run_configs(torch, hq, synth, only=None, oracle=True):
    """One record per config (see the module docstring).  `only`: a config id
    (or a prefix, e.g. "d2") to run alone."""
    from oracle import gemm as G
    from oracle import quant as Q
    dev = torch.device("cuda:0")
    want = lambda cid: only is None or cid.startswith(only)
    recs = []
    threads = _oracle_threads()

    def emit(r):
        log(f"config {r['id']}: {r['us']} us, frac {r['frac']}")
        recs.append(r)

    # d0: dense MXFP8 256^3, seed 0
    if want("d0"):
        d = synth.dense_mxfp8_256()
        qa, sa, _ = hq.quantize(_dev_bf16(torch, d["a"], dev), "mxfp8")
        qb, sb, _ = hq.quantize(_dev_bf16(torch, d["b"], dev), "mxfp8")
        out = torch.empty(256, 256, dtype=torch.bfloat16, device=dev)
        med, mean = _launch_us(torch, [lambda: hq.hq_dense_gemm("mxfp8", qa, sa, qb, sb, out)])
        extra = {"mean_us": round(mean, 2)}
        if oracle:
            a, sfa = Q.mx_quant_bf16(d["a"], "mxfp8")
            b, sfb = Q.mx_quant_bf16(d["b"], "mxfp8")
            extra.update(oracle_us=round(_oracle_us(lambda: G.dense_gemm("mxfp8", a, sfa, b, sfb)), 1),
                         oracle_cores=threads)
        emit(_rec("d0", "dense_mxfp8_M256_N256_K256", med, flops=2.0 * 256 ** 3, bound="latency", **extra))

    # d1: batch MXFP8 4 x 256^3 (with and without bias), dense MXFP4 32 x 512 x 256
    if want("d1_batch") or want("d1_batch_bias"):
        d = synth.batch_mxfp8()
        Bn, m, n, k = 4, 256, 256, 256
        qa, sa, _ = hq.quantize(_dev_bf16(torch, d["a"].reshape(Bn * m, k), dev), "mxfp8")
        qb, sb, _ = hq.quantize(_dev_bf16(torch, d["b"].reshape(Bn * n, k), dev), "mxfp8")
        bias = _dev_bf16(torch, d["bias"], dev)
        out = torch.empty(Bn, m, n, dtype=torch.bfloat16, device=dev)
        args = (qa.view(Bn, m, k), sa.view(Bn, m, -1), qb.view(Bn, n, k), sb.view(Bn, n, -1), out)
        for cid, bb in (("d1_batch", None), ("d1_batch_bias", bias)):
            if not want(cid):
                continue
            med, mean = _launch_us(torch, [lambda bb=bb: hq.hq_batch_gemm("mxfp8", *args, bias=bb)])
            extra = {"mean_us": round(mean, 2)}
            if oracle:
                a, sfa = Q.mx_quant_bf16(d["a"].reshape(Bn * m, k), "mxfp8")
                b, sfb = Q.mx_quant_bf16(d["b"].reshape(Bn * n, k), "mxfp8")
                ob = None if bb is None else d["bias"]
                extra.update(oracle_us=round(_oracle_us(lambda: G.batch_gemm(
                    "mxfp8", a.reshape(Bn, m, k), sfa.reshape(Bn, m, -1), b.reshape(Bn, n, k),
                    sfb.reshape(Bn, n, -1), bias=ob)), 1), oracle_cores=threads)
            emit(_rec(cid, "batch_mxfp8_B4_M256_N256_K256" + ("_bias" if bb is not None else ""), med,
                      flops=2.0 * Bn * m * n * k, bound="latency", **extra))
    if want("d1_mxfp4"):
        d = synth.dense_mxfp4_small()
        qa, sa, _ = hq.quantize(_dev_bf16(torch, d["a"], dev), "mxfp4")
        qb, sb, _ = hq.quantize(_dev_bf16(torch, d["b"], dev), "mxfp4")
        out = torch.empty(32, 512, dtype=torch.bfloat16, device=dev)
        med, mean = _launch_us(torch, [lambda: hq.hq_dense_gemm("mxfp4", qa, sa, qb, sb, out)])
        extra = {"mean_us": round(mean, 2)}
        if oracle:
            a, sfa = Q.mx_quant_bf16(d["a"], "mxfp4")
            b, sfb = Q.mx_quant_bf16(d["b"], "mxfp4")
            extra.update(oracle_us=round(_oracle_us(lambda: G.dense_gemm("mxfp4", a, sfa, b, sfb)), 1),
                         oracle_cores=threads)
        emit(_rec("d1_mxfp4", "dense_mxfp4_M32_N512_K256", med, flops=2.0 * 32 * 512 * 256, bound="latency",
                  peak_key="mxfp4", **extra))

    # d2: dense FP4 cells at (N, K) = (17408, 5120)
    n, k = 17408, 5120
    if any(want(f"d2_{md}_M{m}") for md in ("mxfp4", "nvfp4") for m in (1, 512, 4096)):
        wbits = synth.dense_fp4_large_weights(n, k)
        w = _dev_bf16(torch, wbits, dev)
        for mode in ("mxfp4", "nvfp4"):
            if not any(want(f"d2_{mode}_M{m}") for m in (1, 512, 4096)):
                continue
            wq, wsf, gw = hq.quantize(w, mode)
            gs = 16 if mode == "nvfp4" else 32
            wora = None                         # the oracle's weight codes, quantised once per mode
            for m in (1, 512, 4096):
                cid = f"d2_{mode}_M{m}"
                if not want(cid):
                    continue
                abits = synth.dense_fp4_large_acts(n, k, m)
                aq, asf, ga = hq.quantize(_dev_bf16(torch, abits, dev), mode)
                alpha = (ga * gw) if mode == "nvfp4" else None
                out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
                ws = hq.gemm_workspace(mode, m, n, k, device=dev)
                flops = 2.0 * m * n * k
                bytes_ = (m + n) * k * (0.5 + 1 / gs) + 2 * m * n
                if m == 1:
                    # weights rotated through a ring of >= 1 GB (larger than the 256 MB MALL)
                    copies = max(1, -(-(1 << 30) // (wq.numel() + wsf.numel())))
                    ring = [(wq, wsf)] + [(wq.clone(), wsf.clone()) for _ in range(copies - 1)]
                    fns = [lambda q=q, s_=s_: hq.hq_dense_gemm(mode, aq, asf, q, s_, out, alpha=alpha, workspace=ws)
                           for q, s_ in ring]
                else:
                    fns = [lambda: hq.hq_dense_gemm(mode, aq, asf, wq, wsf, out, alpha=alpha, workspace=ws)]
                med, mean = _launch_us(torch, fns, reps=30 if m < 4096 else 20)
                extra = {"mean_us": round(mean, 2), "workspace_bytes": 0 if ws is None else ws.numel()}
                if oracle:
                    # M = 1: the whole call; larger M: the oracle's time for 8 of the
                    # rows (every m/8-th), as a rate (its time grows with the rows)
                    if wora is None:
                        wora = Q.nvfp4_quant_bf16(wbits) if mode == "nvfp4" else Q.mx_quant_bf16(wbits, mode) + (None,)
                    cb, sb_, g_b = wora
                    rows = np.arange(m) if m == 1 else np.arange(0, m, m // 8)
                    if mode == "nvfp4":
                        ca, sa_, g_a = Q.nvfp4_quant_bf16(abits[rows])
                        al = np.float32(np.float32(g_a) * np.float32(g_b))
                    else:
                        (ca, sa_), al = Q.mx_quant_bf16(abits[rows], mode), None
                    ous = _oracle_us(lambda: G.dense_gemm(mode, ca, sa_, cb, sb_, alpha=al), reps=1)
                    if m == 1:
                        extra.update(oracle_us=round(ous, 1), oracle_cores=threads)
                    else:
                        extra.update(oracle_TFLOP_s=round(2.0 * len(rows) * n * k / (ous * 1e-6) / 1e12, 5),
                                     oracle_sample=f"{len(rows)} of {m} rows", oracle_cores=threads)
                if m == 1:
                    emit(_rec(cid, f"dense_{mode}_M{m}_N{n}_K{k}_cold", med, flops=flops, bytes_=bytes_,
                              bound="hbm", **extra))
                else:
                    emit(_rec(cid, f"dense_{mode}_M{m}_N{n}_K{k}", med, flops=flops, bytes_=bytes_, bound="mfma",
                              peak_key="nvfp4_f16" if mode == "nvfp4" else "mxfp4", **extra))
                del aq, asf, out, ws
                if m == 1:
                    del ring, fns
            del wq, wsf
        del w
        torch.cuda.empty_cache()

    # d4: grouped-masked MXFP4 (64 experts, 256-row slots, K = 7168, N = 4096)
    if want("d4"):
        d = synth.moe_masked(threads=16)
        E, Mmax, K, N = 64, d["max_m"], d["K"], d["N"]
        counts = d["counts"]
        T = int(counts.sum())
        aq, asf, _ = hq.quantize(_dev_bf16(torch, d["a"], dev), "mxfp4")
        w = _dev_bf16(torch, d["b"].reshape(E * N, K), dev)
        wq, wsf, _ = hq.quantize(w, "mxfp4")
        del w
        wq, wsf = wq.view(E, N, K // 2), wsf.view(E, N, K // 32)
        cnt = torch.from_numpy(counts.astype(np.int32)).to(dev)
        out = torch.empty(E * Mmax, N, dtype=torch.bfloat16, device=dev)
        med, mean = _launch_us(torch, [lambda: hq.hq_group_masked_gemm("mxfp4", aq, asf, wq, wsf, cnt, out, Mmax)],
                               reps=20)
        experts = int((counts > 0).sum())
        bytes_ = T * K * (0.5 + 1 / 32) + experts * N * K * (0.5 + 1 / 32) + 2 * T * N
        extra = {}
        if oracle:
            # the oracle's rate on the valid rows of the first expert that has any
            g = int(np.argmax(counts > 0))
            rows = int(counts[g])
            ca, sa_ = Q.mx_quant_bf16(d["a"][g * Mmax:g * Mmax + rows], "mxfp4")
            cb, sb_ = Q.mx_quant_bf16(d["b"][g], "mxfp4")
            ous = _oracle_us(lambda: G.dense_gemm("mxfp4", ca, sa_, cb, sb_), reps=1)
            extra = dict(oracle_TFLOP_s=round(2.0 * rows * N * K / (ous * 1e-6) / 1e12, 5),
                         oracle_sample=f"expert {g}: {rows} of {T} rows", oracle_cores=threads)
        emit(_rec("d4", "moe_grouped_masked_mxfp4_E64_Mmax256_K7168_N4096", med, flops=2.0 * T * N * K,
                  bytes_=bytes_, bound="hbm", mean_us=round(mean, 2), routed_rows=T,
                  mfma_frac=round(2.0 * T * N * K / (med * 1e-6) / 1e12 / PEAK_TFLOPS["mxfp4"], 4), **extra))
        del aq, asf, wq, wsf, out, d
        torch.cuda.empty_cache()

    # n3: the backward grouped GEMM with the dSwiGLU epilogue at the MoE shape
    if want("n3") or want("n3_q"):
        d = synth.moe_dglu_backward(threads=16)
        counts, ends = d["counts"], d["group_end"]
        R, K, N, E = int(ends[-1]), d["K"], d["N"], len(counts)
        T = int(counts.sum())
        qa, sa, _ = hq.quantize(_dev_bf16(torch, d["a"], dev), "mxfp8")
        w = _dev_bf16(torch, d["b"].reshape(E * N, K), dev)
        qw, sw, _ = hq.quantize(w, "mxfp8")
        del w
        qw, sw = qw.view(E, N, K), sw.view(E, N, K // 32)
        c = _dev_bf16(torch, d["c"], dev)
        ge = torch.from_numpy(ends.astype(np.int32)).to(dev)
        prob = torch.from_numpy(d["prob"]).to(dev)
        al, be = torch.from_numpy(d["alpha"]).to(dev), torch.from_numpy(d["beta"]).to(dev)
        dprob = torch.zeros(R, dtype=torch.float32, device=dev)
        dout = torch.empty(R, 2 * N, dtype=torch.bfloat16, device=dev)
        flops = 2.0 * T * N * K
        # A codes + scales and C, D of the valid rows, the experts' weights, prob and dprob
        bytes_ = T * K * (1 + 1 / 32) + E * N * K * (1 + 1 / 32) + 2 * T * 2 * N * 2 + 12 * T
        if want("n3"):
            med, mean = _launch_us(torch, [lambda: hq.hq_group_contiguous_gemm_dswiglu(
                "mxfp8", qa, sa, qw, sw, ge, c, prob, dprob, dout, alpha=al, beta=be)], reps=20)
            t_ideal = max(flops / (PEAK_TFLOPS["mxfp8"] * 1e12), bytes_ / (PEAK_HBM_GBS * 1e9))
            extra = {}
            if oracle:
                # the oracle's rate on 256 rows of the first non-empty group
                from oracle import dglu as DG
                g = int(np.argmax(counts > 0))
                r0 = int(ends[g - 1]) if g > 0 else 0
                rows = min(256, int(counts[g]))
                ca, sa_ = Q.mx_quant_bf16(d["a"][r0:r0 + rows], "mxfp8")
                cb, sb_ = Q.mx_quant_bf16(d["b"][g], "mxfp8")
                ous = _oracle_us(lambda: DG.grouped_gemm_dswiglu(
                    "mxfp8", ca, sa_, cb[None], sb_[None], np.array([rows]), d["c"][r0:r0 + rows],
                    d["prob"][r0:r0 + rows], alpha=d["alpha"][g:g + 1], beta=d["beta"][g:g + 1]), reps=1)
                extra = dict(oracle_TFLOP_s=round(2.0 * rows * N * K / (ous * 1e-6) / 1e12, 5),
                             oracle_sample=f"{rows} rows of group {g}", oracle_cores=threads)
            emit(_rec("n3", "moe_bwd_dswiglu_mxfp8_E32_T65536_K4096_N1536", med, flops=flops, bytes_=bytes_,
                      bound="mfma", mean_us=round(mean, 2), routed_rows=T,
                      hbm_frac=round(bytes_ / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 3),
                      roofline_frac=round(t_ideal / (med * 1e-6), 3), **extra))
        if want("n3_q"):
            # the same with D written row-quantised (MXFP8 codes + UE8M0 per 32)
            dq = torch.empty(R, 2 * N, dtype=torch.uint8, device=dev)
            dsf = torch.empty(R, 2 * N // 32, dtype=torch.uint8, device=dev)
            med, mean = _launch_us(torch, [lambda: hq.hq_group_contiguous_gemm_dswiglu_quant(
                "mxfp8", qa, sa, qw, sw, ge, c, prob, dprob, dq, dsf, alpha=al, beta=be)], reps=20)
            bq = bytes_ - T * 2 * N * (2 - 1 - 1 / 32)
            emit(_rec("n3_q", "moe_bwd_dswiglu_mxfp8_E32_T65536_K4096_N1536_rowquant_d", med, flops=flops,
                      bytes_=bq, bound="mfma", mean_us=round(mean, 2), routed_rows=T,
                      hbm_frac=round(bq / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)))
            del dq, dsf
        del qa, qw, c, dout, dprob, d
        torch.cuda.empty_cache()

    # d5: quantisation bandwidth (input ring of >= 1 GB: past the MALL)
    rng = np.random.default_rng(5)
    for cid, mode, m, kk, supplied in (("d5_mxfp4", "mxfp4", 16384, 7168, False),
                                       ("d5_nvfp4", "nvfp4", 4096, 17408, True),
                                       ("d5_nvfp4_amax", "nvfp4", 4096, 17408, False)):
        if not want(cid):
            continue
        xbits = synth.normal_bf16(rng, (m, kk))
        x = _dev_bf16(torch, xbits, dev)
        xs = [x] + [x.clone() for _ in range(max(1, -(-(1 << 30) // (2 * m * kk))) - 1)]
        q, sf, g = hq.quantize(x, mode)
        gin = g.clone() if supplied else None
        if gin is None:
            fns = [lambda xx=xx: hq.hq_group_wise_quant(mode, xx, q, sf, g) for xx in xs]
        else:
            fns = [lambda xx=xx: hq.hq_group_wise_quant(mode, xx, q, sf, gin, hq.HQ_GS_INPUT) for xx in xs]
        med, mean = _launch_us(torch, fns, reps=30)
        gs = 16 if mode == "nvfp4" else 32
        bytes_ = m * kk * (2 + 0.5 + 1 / gs)
        extra = {"mean_us": round(mean, 2)}
        if mode == "nvfp4" and not supplied:
            # the global scale needs the whole tensor's amax before the first
            # code, so the input is read twice: 2 more bytes per element
            extra["GB/s_single_read"] = round(bytes_ / (med * 1e-6) / 1e9, 1)
            bytes_ += 2 * m * kk
        if oracle:
            rows = 256
            sample = xbits[:rows]
            fn = (lambda: Q.mx_quant_bf16(sample, mode)) if mode != "nvfp4" else (
                lambda: Q.nvfp4_quant_bf16(sample, None if not supplied else np.float32(g.item())))
            ous = _oracle_us(fn)
            extra.update(oracle_GB_s=round(rows * kk * (2 + 0.5 + 1 / gs) / (ous * 1e-6) / 1e9, 3),
                         oracle_sample=f"{rows} rows", oracle_cores=threads)
        emit(_rec(cid, f"quant_{mode}_{m}x{kk}" + ("_g_supplied" if supplied else ("_amax" if mode == "nvfp4"
                                                                                   else "")) + "_cold",
                  med, bytes_=bytes_, bound="hbm", **extra))
        del x, xs, q, sf
        torch.cuda.empty_cache()
    return recs


def run_ab(args, torch, hq, synth):
    """Interleaved A/B of this build against another build of libhq.so
    (--ab-lib PATH, e.g. built from an earlier commit in a git worktree):
    the skinny dense cells (raw hq_dense_gemm, whose C signature both builds
    share) and NVFP4 quantisation with the amax pass.  Inputs are quantised
    by this build; per case the two builds alternate batch by batch (each
    batch queued behind a spin kernel), and their outputs are compared
    bit for bit.  One JSON line per case."""
    import ctypes
    other = ctypes.CDLL(os.path.abspath(args.ab_lib))
    for name in ("hq_dense_gemm", "hq_group_wise_quant"):
        a, r = hq._SIGS[name]
        f = getattr(other, name)
        f.argtypes, f.restype = a, r
    libs = {"this": hq.load(), "other": other}
    dev = torch.device("cuda:0")

    def ab(label, call, outs, work, unit, reps=12, per=20):
        ref = None
        same = True
        for nm in ("this", "other"):
            for o in outs:
                o.view(torch.uint8).fill_(0xA5)
            call(libs[nm])
            torch.cuda.synchronize()
            got = [o.clone() for o in outs]
            if ref is None:
                ref = got
            else:
                same = all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(ref, got))
        res = {"this": [], "other": []}
        for nm in ("this", "other"):
            for _ in range(3):
                call(libs[nm])
        torch.cuda.synchronize()
        for r in range(reps):
            for nm in (("this", "other") if r % 2 == 0 else ("other", "this")):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                _hold_gpu(torch, 1000 + 150 * per)
                e0.record()
                for _ in range(per):
                    call(libs[nm])
                e1.record()
                torch.cuda.synchronize()
                res[nm].append(e0.elapsed_time(e1) * 1e3 / per)
        ut, uo = float(np.median(res["this"])), float(np.median(res["other"]))
        line = {"workload": label, "us_this": round(ut, 2), "us_other": round(uo, 2),
                "this_over_other": round(ut / uo, 3), "same_bits": bool(same),
                unit: round(work / (ut * 1e-6) / 1e9, 1), "other_lib": args.ab_lib}
        print(json.dumps(line), flush=True)

    for mode in ("nvfp4", "mxfp4"):
        for n, k, m in ((17408, 5120, 1), (12288, 5120, 16), (5120, 17408, 1)):
            w = _dev_bf16(torch, synth.dense_fp4_large_weights(n, k), dev)
            x = _dev_bf16(torch, synth.dense_fp4_large_acts(n, k, m), dev)
            wq, wsf, gw = hq.quantize(w, mode)
            aq, asf, ga = hq.quantize(x, mode)
            al = (ga * gw) if mode == "nvfp4" else None
            out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
            st = hq._stream(aq)
            ptr = [hq._p(t) for t in (aq, asf, wq, wsf)]
            pal, po = hq._p(al), hq._p(out)

            def call(L, mc=hq.MODES[mode], st=st, ptr=ptr, pal=pal, po=po, m=m, n=n, k=k):
                rc = L.hq_dense_gemm(st, mc, ptr[0], ptr[1], ptr[2], ptr[3], None, pal, po, m, n, k, 0)
                if rc != 0:
                    raise RuntimeError(f"hq_dense_gemm returned {rc}")
            gs = 16 if mode == "nvfp4" else 32
            ab(f"dense_{mode}_M{m}_N{n}_K{k}_warm", call, [out], (m + n) * k * (0.5 + 1 / gs) + 2 * m * n, "GB/s")
            del w, x, wq, wsf, aq, asf, out
    m, k = 4096, 17408
    x = _dev_bf16(torch, synth.normal_bf16(np.random.default_rng(5), (m, k)), dev)
    q = torch.empty(m, k // 2, dtype=torch.uint8, device=dev)
    sf = torch.empty(m, k // 16, dtype=torch.uint8, device=dev)
    g = torch.empty(1, dtype=torch.float32, device=dev)
    st = hq._stream(x)
    px, pq, psf, pg = hq._p(x), hq._p(q), hq._p(sf), hq._p(g)

    def callq(L):
        rc = L.hq_group_wise_quant(st, hq.HQ_NVFP4, px, m, k, pq, psf, pg, 0)
        if rc != 0:
            raise RuntimeError(f"hq_group_wise_quant returned {rc}")
    ab(f"quant_nvfp4_{m}x{k}_amax_warm", callq, [q, sf, g], m * k * (2 + 2 + 0.5 + 1 / 16), "GB/s_incl_second_read")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="moe", choices=["moe", "moe_unfused", "moe_mlp", "dense_fp4",
                                                       "masked_fp4", "permute", "sweep", "configs", "ab"])
    ap.add_argument("--mode", default="mxfp4")
    ap.add_argument("--m", type=int, default=4096)
    ap.add_argument("--n", type=int, default=17408)
    ap.add_argument("--k", type=int, default=5120)
    ap.add_argument("--tokens", type=int, default=1024, help="--workload permute: token count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config records")
    ap.add_argument("--only", default=None, help="run one config record alone (--workload configs)")
    ap.add_argument("--ab-lib", default=None, help="--workload ab: another build of libhq.so to time against")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run one plain device copy of this many MiB (calibrates "
                         "the FETCH_SIZE / WRITE_SIZE counters against a known byte count)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp4_gemm_moe_amd as hq
    import synth
    hq.load()
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    if args.copy_probe_mb > 0:
        nbytes = args.copy_probe_mb << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {nbytes} bytes read and written once")
        del src, dst
    if args.workload == "sweep":
        run_sweep(args, torch, hq, synth)
        return
    if args.workload == "ab":
        if not args.ab_lib:
            raise SystemExit("--workload ab needs --ab-lib PATH (another build of libhq.so)")
        run_ab(args, torch, hq, synth)
        return
    if args.workload == "configs":
        recs = run_configs(torch, hq, synth, only=args.only, oracle=not args.no_cpu_baseline)
        print(json.dumps({"configs": recs, "device": {"name": props.name,
                                                       "cus": props.multi_processor_count}}), flush=True)
        return
    runner = {"moe": lambda *a: run_moe(*a, fused=True), "moe_unfused": run_moe,
              "dense_fp4": run_dense_fp4, "masked_fp4": run_masked_fp4, "permute": run_permute,
              "moe_mlp": lambda *a: run_moe(*a, down=True, fused=True)}[args.workload]
    res = runner(args, torch, hq, synth)
    value, ms_step, cfg, roof, kernels, ctx = res[:6]
    unit = res[6] if len(res) > 6 else "TFLOP/s"
    cpu = None
    if ctx is not None and not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample (cpu_baseline)")
        cpu = cpu_baseline_moe(ctx)
    recs = None
    if args.workload == "moe" and not args.no_configs:
        del ctx
        torch.cuda.empty_cache()
        recs = run_configs(torch, hq, synth, oracle=not args.no_cpu_baseline)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"moe": "mxfp8", "moe_mlp": "mxfp8", "moe_unfused": "mxfp8",
                  "permute": "bf16"}.get(args.workload, args.mode),
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "configs": recs,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
