#!/usr/bin/env python3
"""Throughput of the draft step (hidden states of a packed block -> drafted
tokens) on one MI355X, on synthetic inputs of the Qwen3-4B batch shape
(32 requests x 7 rows, hidden 2560, vocabulary 151936, K = 64, rank 256).

A step is one dflash_draft_block call over the whole batch: lm_head GEMM with
the LSE epilogue, Top-K with d2t and unary, pairwise scores, walk.  Inputs
are resident in HBM before the timed region.  Prints ONE JSON line on stdout
(progress goes to stderr).

The headline `value` times exactly --steps steps between two events after
--warmup untimed ones.  Beside it:
  * per-iteration events over --iters steps, warm (back to back) and cold (a
    1 GiB read-modify-write of a scratch buffer before every iteration, outside
    the events, which evicts the 256 MB Infinity Cache): median, p10, p90;
  * every stage entry point alone (the lm_head launch gives the roofline);
  * the other workloads of the draft step (one request at the Qwen3-4B shape,
    the gated 27B shape, the pruned vocabulary) with blocks/s, rows/s and the
    step's fraction of its HBM roofline;
  * the CPU oracle on the same host: the baseline rate, a one-thread rate on
    the tiny and single-request workloads, and the parity of the GPU's tokens
    with the oracle's on every request of every workload.

    python bench.py [--steps K] [--warmup W] [--iters N] [--workload NAME] [--walk viterbi|greedy]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "drafted blocks/sec (1 GPU) at Qwen3-4B shape; MFMA util + HBM GB/s vs peak"
EXTRA_WORKLOADS = ("qwen3_4b_1", "dflash2_27b", "pruned_ocr")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": usable, "os_cpu_count": os.cpu_count()}


def step_bytes(s):
    """Bytes of one step of workload shape s.

    floor: W + hidden + the table rows the scorer gathers, (1 + (L-1)K + LK) rows of r fp32
    per request; as_architected: the floor plus one fp32 write and one read of all logits
    (the kernel split lm_head -> Top-K with the logits in HBM between them)."""
    w = s.Vd * s.H * 2
    h = s.M * s.H * 2
    gather = s.R * (1 + (s.L - 1) * s.K + s.L * s.K) * s.r * 4
    logits = s.M * s.Vd * 4
    floor = w + h + gather
    return {"floor": floor, "as_architected": floor + 2 * logits, "lm_head": w + h + logits}


def stats(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "mean_us": round(float(a.mean()), 2),
            "iters": int(a.size)}


class Timer:
    """HIP-event timing on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.flush_buf = None

    def flush(self):
        # 1 GiB read-modify-write: evicts the Infinity Cache and the L2s
        if self.flush_buf is None:
            self.flush_buf = self.torch.zeros(1 << 30, dtype=self.torch.uint8, device="cuda")
        self.flush_buf.add_(1)

    def prime(self, cycles):
        """Queue a bounded GPU spin so that the host can queue work ahead of the GPU."""
        try:
            self.torch.cuda._sleep(int(cycles))
        except (AttributeError, RuntimeError):
            pass

    def region(self, fn, n, warm):
        """Mean ms per call of n calls between two events, after `warm` untimed calls."""
        torch = self.torch
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(n):
            fn()
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def per_iter(self, fn, n, warm=3, cold=False):
        """ms of every one of n calls, each between its own pair of events.

        A bounded spin kernel (torch.cuda._sleep) is queued first, so that the host has queued
        the calls before the GPU reaches them: the events then time the GPU work of a call, not
        the host's launch overhead (which matters for the short kernels)."""
        torch = self.torch
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        self.prime(n * 100_000)
        for a, b in ev:
            if cold:
                self.flush()
            a.record(self.stream)
            fn()
            b.record(self.stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]


class Workload:
    """One synthetic workload resident on the GPU, with its step closures."""

    def __init__(self, name, torch, api, di, walk):
        import numpy as np
        self.torch, self.api = torch, api
        self.shape = s = di.SHAPES[name]
        log(f"workload {s.name}: R={s.R} L={s.L} M={s.M} H={s.H} V_d={s.Vd} V_t={s.Vt} K={s.K} r={s.r}; "
            "drawing inputs")
        t0 = time.time()
        self.inp = inp = di.make_inputs(s)
        log(f"  inputs drawn in {time.time() - t0:.1f} s; uploading")

        def dev(x):
            return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()

        self.hidden = torch.from_numpy(np.ascontiguousarray(inp.hidden).view(np.int16)).cuda()
        self.W = torch.from_numpy(np.ascontiguousarray(inp.lm_head).view(np.int16)).cuda()
        self.tables, self.last_tok = dev(inp.tables), dev(inp.last_tok)
        self.d2t, self.gate_w = dev(inp.d2t), dev(inp.gate_w)
        self.tokens = torch.empty(s.M, dtype=torch.int64, device="cuda")
        self.scores = torch.empty(s.R, dtype=torch.float32, device="cuda")
        self.ws = api.Workspace("cuda:0")
        self.walk = walk
        torch.cuda.synchronize()

    def step(self):
        s = self.shape
        self.api.draft_block(self.hidden, self.W, self.tables, self.last_tok, top_k=s.K, d2t=self.d2t,
                             gate_w=self.gate_w, block_len=s.L, walk=self.walk, workspace=self.ws,
                             out=(self.tokens, self.scores))

    def step_filtered(self):
        """The step with the opt-in logits filter (DFLASH_OPT_FILTER_LOGITS)."""
        s = self.shape
        self.api.draft_block(self.hidden, self.W, self.tables, self.last_tok, top_k=s.K, d2t=self.d2t,
                             gate_w=self.gate_w, block_len=s.L, walk=self.walk, workspace=self.ws,
                             out=(self.tokens, self.scores), filter_logits=True)

    def lm_head(self, zbuf):
        return lambda: self.api.lm_head(self.hidden, self.W, workspace=self.ws, with_lse=False, out=zbuf)

    def candidates(self):
        """The GPU's slots (draft ids) of every row, from the stage entry points (the same kernels
        as the fused step's; a GPU test checks that both give identical tokens)."""
        z, lse = self.api.lm_head(self.hidden, self.W, workspace=self.ws)
        idx, _, _ = self.api.topk(z, lse, self.shape.K, d2t=self.d2t, target_vocab=self.shape.Vt, workspace=self.ws)
        return idx.cpu().numpy()

    def gpu_tokens(self):
        self.step()
        self.torch.cuda.synchronize()
        return self.tokens.cpu().numpy().copy()


def workload_entry(w, timer, args):
    """blocks/s and rows/s of one workload: warm and cold per-iteration events, the lm_head alone."""
    s = w.shape
    warm = stats(timer.per_iter(w.step, args.iters, warm=5))
    cold = stats(timer.per_iter(w.step, args.iters, warm=2, cold=True))
    zbuf = w.torch.empty((s.M, w.api.logits_stride(s.Vd)), dtype=w.torch.float32, device="cuda")
    lm = stats(timer.per_iter(w.lm_head(zbuf), args.iters, warm=3))
    filt = stats(timer.per_iter(w.step_filtered, args.iters, warm=3))
    del zbuf
    b = step_bytes(s)
    t = warm["median_us"] * 1e-6
    floor_s = b["floor"] / (HBM_PEAK_GBS * 1e9)
    arch_s = b["as_architected"] / (HBM_PEAK_GBS * 1e9)
    return {
        "blocks_per_s": round(s.R / t, 1), "rows_per_s": round(s.M / t, 1),
        "blocks_per_s_cold": round(s.R / (cold["median_us"] * 1e-6), 1),
        "step_warm": warm, "step_cold": cold,
        "roofline": {"bound": "hbm", "peak_gbs": HBM_PEAK_GBS,
                     "floor_bytes": b["floor"], "floor_us": round(floor_s * 1e6, 2),
                     "frac_of_floor": round(floor_s / t, 4),
                     "as_architected_bytes": b["as_architected"], "as_architected_us": round(arch_s * 1e6, 2),
                     "frac_of_as_architected": round(arch_s / t, 4)},
        "lm_head_alone": lm,
        "step_with_logits_filter": {**filt, "note": "opt-in DFLASH_OPT_FILTER_LOGITS: sample GEMM + bound + "
                                    "filtered lm_head; same tokens"},
        "lm_head_gbs": round(b["lm_head"] / (lm["mean_us"] * 1e-6) / 1e9, 1),
        "lm_head_mfma_tflops": round(2.0 * s.M * s.H * s.Vd / (lm["mean_us"] * 1e-6) / 1e12, 1),
    }


def parity_block(w, gpu_tokens, gpu_idx, res):
    """The GPU's tokens against the oracle's on every request.  A request is compared bit for
    bit unless one of its rows has a GPU Top-K set other than the oracle's (the boundary
    exemption) or its oracle runner-up margin is below 1e-5 * max(|S|, 1)."""
    import numpy as np
    s = w.shape
    rows_differ = np.array([set(gpu_idx[m].tolist()) != set(res.cand.idx[m].tolist()) for m in range(s.M)])
    out = {"requests": s.R, "compared": 0, "tokens_equal": 0, "topk_set_differs_rows": int(rows_differ.sum()),
           "topk_exempt_requests": 0, "margin_exempt_requests": 0}
    for r in range(s.R):
        a, b = r * s.L, (r + 1) * s.L
        if rows_differ[a:b].any():
            out["topk_exempt_requests"] += 1
            continue
        if res.margins[r] < 1e-5 * max(1.0, abs(res.scores[r])):
            out["margin_exempt_requests"] += 1
            continue
        out["compared"] += 1
        out["tokens_equal"] += int(np.array_equal(gpu_tokens[a:b], res.tokens[a:b]))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--iters", type=int, default=200, help="per-iteration events of the warm and cold timings")
    ap.add_argument("--workload", default="qwen3_4b_32")
    ap.add_argument("--walk", default="viterbi", choices=["viterbi", "greedy"])
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle (baseline and parity)")
    ap.add_argument("--no-extra-workloads", action="store_true", help="time the main workload only")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.copy_probe:
        import torch
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 5}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log(f"bench.py measures the draft step on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
            "the draft step runs on one GPU and is not sharded across GPUs.")
        sys.exit(2)

    import numpy as np
    import torch

    import draft_inputs as di
    from block_draft_markov_amd import api

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    torch.cuda.set_device(0)
    timer = Timer(torch)
    w = Workload(args.workload, torch, api, di, args.walk)
    shape = w.shape
    R, L, M, H, Vd, Vt, K, r = shape.R, shape.L, shape.M, shape.H, shape.Vd, shape.Vt, shape.K, shape.r

    # ---- per-iteration distributions, warm and cold
    main_entry = workload_entry(w, timer, args)
    log(f"per-iteration: warm {main_entry['step_warm']}, cold {main_entry['step_cold']}")
    # host time to enqueue one step (binding + C ABI + four launches), GPU not awaited
    torch.cuda.synchronize()
    timer.prime(50 * 2_000_000)
    t0 = time.perf_counter()
    for _ in range(50):
        w.step()
    host_us = (time.perf_counter() - t0) / 50 * 1e6
    torch.cuda.synchronize()
    log(f"host enqueue time per step: {host_us:.1f} us")

    # ---- every stage entry point alone (per-iteration events, warm unless stated)
    zbuf = torch.empty((M, api.logits_stride(Vd)), dtype=torch.float32, device="cuda")
    k1 = main_entry["lm_head_alone"]
    z, lse = api.lm_head(w.hidden, w.W, workspace=w.ws)
    topk_fn = lambda: api.topk(z, lse, K, d2t=w.d2t, target_vocab=Vt, workspace=w.ws)
    k2 = stats(timer.per_iter(topk_fn, args.iters))
    k2c = stats(timer.per_iter(topk_fn, args.iters, cold=True))
    idx, ctok, un = topk_fn()
    k3 = stats(timer.per_iter(lambda: api.pair_scores(ctok, w.tables, w.last_tok, gate_w=w.gate_w, hidden=w.hidden,
                                                      block_len=L), args.iters))
    pair = api.pair_scores(ctok, w.tables, w.last_tok, gate_w=w.gate_w, hidden=w.hidden, block_len=L)
    k4 = stats(timer.per_iter(lambda: api.walk(ctok, un, pair, R, block_len=L, walk=args.walk), args.iters))
    k34 = stats(timer.per_iter(lambda: api.lattice(ctok, un, w.tables, w.last_tok, gate_w=w.gate_w, hidden=w.hidden,
                                                   block_len=L, walk=args.walk, workspace=w.ws), args.iters))
    log(f"stages (median us): lm_head {k1['median_us']}, top-k {k2['median_us']} (cold {k2c['median_us']}), "
        f"pair {k3['median_us']}, walk {k4['median_us']}, lattice {k34['median_us']}")
    # ---- the other head modes on the same rows
    nh_tok = torch.empty(M, dtype=torch.int64, device="cuda")
    nh = stats(timer.per_iter(lambda: api.draft_argmax(w.hidden, w.W, d2t=w.d2t, target_vocab=Vt, out_scale=1.0,
                                                       soft_cap=30.0, workspace=w.ws, with_values=False,
                                                       out=(nh_tok, None)), args.iters))
    dn = stats(timer.per_iter(lambda: api.draft_dense(w.hidden, w.W, w.tables, w.last_tok, d2t=w.d2t, block_len=L,
                                                      out_scale=1.0, soft_cap=30.0, workspace=w.ws,
                                                      with_values=False, out=(nh_tok, None)), args.iters))
    uni = torch.rand(M, dtype=torch.float64, device="cuda", generator=torch.Generator("cuda").manual_seed(11))
    sp = stats(timer.per_iter(lambda: api.draft_block_sampled(w.hidden, w.W, w.tables, w.last_tok, uni, top_k=K,
                                                              temperature=1.0, d2t=w.d2t, gate_w=w.gate_w,
                                                              block_len=L, workspace=w.ws), args.iters))
    log(f"head-less {nh['median_us']} us, dense {dn['median_us']} us, sampled {sp['median_us']} us")

    # ---- attainable peaks on this GPU, from vendor-library probes (torch): a 2 GiB fp32 sum
    # (HBM read) and an 8192^3 bf16 product (hipBLASLt)
    big = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    rd = stats(timer.per_iter(lambda: big.sum(), 20, cold=True))
    del big
    a16 = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b16 = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    mm = stats(timer.per_iter(lambda: torch.mm(a16, b16), 20))
    del a16, b16
    attain = {"hbm_read_gbs": round((1 << 31) / (rd["median_us"] * 1e-6) / 1e9, 1),
              "bf16_mm_tflops": round(2 * 8192 ** 3 / (mm["median_us"] * 1e-6) / 1e12, 1),
              "probes": "torch fp32 sum over 2 GiB (cold), torch.mm 8192^3 bf16"}
    log(f"attainable: {attain}")

    # ---- the timed region: exactly --steps whole steps after --warmup untimed ones (run after
    # the measurements above, so that the GPU is at its working clocks)
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    ms = timer.region(w.step, args.steps, args.warmup)
    blocks_per_s = R / (ms / 1e3)
    rows_per_s = M / (ms / 1e3)
    log(f"{ms * 1e3:.1f} us/step -> {blocks_per_s:.0f} blocks/s, {rows_per_s:.0f} rows/s")

    # ---- roofline of the dominant kernel (the lm_head GEMM with its LSE epilogue), launched alone
    b = step_bytes(shape)
    k1_bytes = b["lm_head"]
    k1_s = k1["mean_us"] * 1e-6
    k1_gbs = k1_bytes / k1_s / 1e9
    k1_tflops = 2.0 * M * H * Vd / k1_s / 1e12
    # Top-K pass graded cold: the stand-alone dflash_topk reads every logit once
    k2_bytes = M * Vd * 4 + M * 4 + M * K * (4 + 8 + 4)
    k2_gbs = k2_bytes / (k2c["median_us"] * 1e-6) / 1e9

    # HBM traffic of the dominant kernel, from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    # record of this workload, valid only while the kernel sources are those it was taken on
    traffic = None
    rec_path = os.path.join(ROOT, "profiles", f"lmhead_dma_kernel__{shape.name}.traffic.json")
    if os.path.exists(rec_path):
        import hashlib
        rec = json.load(open(rec_path))
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])).hexdigest()
        if h == rec["sources_sha256"]:
            traffic = int(rec["traffic_bytes"])
        else:
            log("kernel sources changed since the traffic counters were taken: traffic = null")

    out = {
        "metric": METRIC,
        "value": round(blocks_per_s, 1),
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random weights and hidden states of the workload's shapes)",
        "config": {"workload": shape.name, "requests": R, "block_len": L, "rows": M, "hidden": H,
                   "draft_vocab": Vd, "target_vocab": Vt, "top_k": K, "rank": r, "gated": shape.gated,
                   "pruned": shape.pruned, "walk": args.walk, "parallelism": "single GPU"},
        "rows_per_s": round(rows_per_s, 1),
        "roofline": {"kernel": "lmhead_dma_kernel", "bound": "hbm",
                     "achieved": round(k1_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": k1_bytes, "avg_launch_us": k1["mean_us"],
                     "median_launch_us": k1["median_us"],
                     "mfma_tflops": round(k1_tflops, 1), "mfma_peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                     "mfma_frac": round(k1_tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
        "timing": {"warm": main_entry["step_warm"], "cold": main_entry["step_cold"],
                   "host_enqueue_us_per_step": round(host_us, 1),
                   "cold_flush": "1 GiB read-modify-write before every iteration, outside the events"},
        "step_roofline": main_entry["roofline"],
        "step_with_logits_filter": main_entry["step_with_logits_filter"],
        "standalone_topk_pass": {"achieved_gbs": round(k2_gbs, 1), "frac": round(k2_gbs / HBM_PEAK_GBS, 4),
                                 "bytes_per_launch": k2_bytes, "cold": k2c, "warm": k2,
                                 "graded_on": "cold median"},
        "standalone_stages": {"lm_head": k1, "topk": k2, "topk_cold": k2c, "pair_scores": k3, "walk": k4,
                              "lattice": k34},
        "headless_step": {**nh, "blocks_per_s": round(R / (nh["median_us"] * 1e-6), 1), "out_scale": 1.0,
                          "soft_cap": 30.0},
        "dense_step": {**dn, "blocks_per_s": round(R / (dn["median_us"] * 1e-6), 1), "out_scale": 1.0,
                       "soft_cap": 30.0,
                       # per position: the gathered B rows of every draft id and the rows' logits
                       "bytes_per_position": Vd * r * 4 + R * Vd * 4},
        "sampled_step": {**sp, "blocks_per_s": round(R / (sp["median_us"] * 1e-6), 1), "temperature": 1.0},
        "attainable": attain,
        "host": host_info(),
    }

    # ---- the other workloads (timed here; their oracle parity below)
    extras = {}
    if not args.no_extra_workloads:
        for name in EXTRA_WORKLOADS:
            if name == shape.name:
                continue
            x = Workload(name, torch, api, di, args.walk)
            e = workload_entry(x, timer, args)
            log(f"{name}: {e['blocks_per_s']} blocks/s warm, {e['blocks_per_s_cold']} cold; "
                f"lm_head {e['lm_head_alone']['median_us']} us")
            # the GPU's tokens and slots for the oracle's parity check; then free the device copies
            x.gpu_tok, x.gpu_idx = x.gpu_tokens(), x.candidates()
            x.W = x.tables = x.hidden = x.ws = None
            torch.cuda.empty_cache()
            extras[name] = (x, e)
        out["workloads"] = {name: e for name, (x, e) in extras.items()}

    # ---- the CPU oracle: baseline rate and parity (test infrastructure; not the product path)
    if not args.no_cpu_baseline:
        from oracle import draft_step as O
        owalk = O.WALK_VITERBI if args.walk == "viterbi" else O.WALK_GREEDY
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        except Exception:
            threadpool_limits, cores = None, 1
        inp = w.inp
        log(f"CPU oracle on all {R} requests ({M} rows) of {shape.name}")
        times = []
        while True:
            t0 = time.perf_counter()
            res = O.draft_block(inp.hidden, inp.lm_head, inp.d2t, inp.tables, inp.gate_w, inp.last_tok, K,
                                walk=owalk)
            times.append(time.perf_counter() - t0)
            if sum(times) >= 10.0 or len(times) >= 20:
                break
        dt = float(np.median(times))
        gpu_tok = w.gpu_tokens()
        parity = {shape.name: parity_block(w, gpu_tok, w.candidates(), res)}
        out["cpu_baseline"] = {"value": round(R / dt, 3), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
                               "sample": f"all {R} requests ({M} rows) of {shape.name}, fp64 numpy oracle, "
                                         f"median of {len(times)} runs of {dt:.2f} s; the fp64 products run on "
                                         f"{cores} BLAS threads, the rest of the oracle on one",
                               "gpu_tokens_equal_requests": int(sum(
                                   np.array_equal(res.tokens[i * L:(i + 1) * L], gpu_tok[i * L:(i + 1) * L])
                                   for i in range(R))),
                               **host_info()}
        log(f"oracle: {dt:.2f} s for {R} blocks -> {R / dt:.3f} blocks/s on {cores} threads")
        # one thread: the tiny workload and one Qwen3-4B request
        if threadpool_limits is not None:
            one = {}
            with threadpool_limits(1):
                for name in ("tiny", "qwen3_4b_1"):
                    xs = di.SHAPES[name]
                    xi = inp if name == shape.name else di.make_inputs(xs)
                    reps, tt = 0, []
                    while reps < 50 and sum(tt) < 3.0:
                        t0 = time.perf_counter()
                        O.draft_block(xi.hidden, xi.lm_head, xi.d2t, xi.tables, xi.gate_w, xi.last_tok, xs.K,
                                      walk=owalk)
                        tt.append(time.perf_counter() - t0)
                        reps += 1
                    one[name] = {"blocks_per_s": round(xs.R / float(np.median(tt)), 3), "runs": reps}
            out["cpu_baseline"]["one_thread"] = one
            log(f"oracle on one thread: {one}")
        # parity of every other workload, every request
        for name, (x, e) in extras.items():
            xs = x.shape
            log(f"oracle parity: {name}")
            xr = O.draft_block(x.inp.hidden, x.inp.lm_head, x.inp.d2t, x.inp.tables, x.inp.gate_w, x.inp.last_tok,
                               xs.K, walk=owalk)
            parity[name] = parity_block(x, x.gpu_tok, x.gpu_idx, xr)
        out["parity"] = parity
        log(f"parity: {parity}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
