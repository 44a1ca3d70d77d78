#!/usr/bin/env python3
"""Throughput of the draft step (hidden states of a packed block -> drafted
tokens) on one MI355X, on synthetic inputs of the Qwen3-4B batch shape
(32 requests x 7 rows, hidden 2560, vocabulary 151936, K = 64, rank 256).

A step is one dflash_draft_block call over the whole batch: lm_head GEMM with
the LSE epilogue, Top-K with d2t and unary, pairwise scores, walk.  Inputs
are resident in HBM before the timed region.  Prints ONE JSON line on stdout
(progress goes to stderr).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--walk viterbi|greedy]
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_4b_32")
    ap.add_argument("--walk", default="viterbi", choices=["viterbi", "greedy"])
    ap.add_argument("--cpu-sample-requests", type=int, default=32,
                    help="requests of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    shape = di.SHAPES[args.workload]
    R, L, M, H, Vd, Vt, K, r = shape.R, shape.L, shape.M, shape.H, shape.Vd, shape.Vt, shape.K, shape.r
    log(f"workload {shape.name}: R={R} L={L} M={M} H={H} V_d={Vd} V_t={Vt} K={K} r={r}; drawing inputs")
    t0 = time.time()
    inp = di.make_inputs(shape)
    log(f"inputs drawn in {time.time() - t0:.1f} s; uploading")

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()

    def dev(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()

    hidden, W = dev_bf16(inp.hidden), dev_bf16(inp.lm_head)
    tables, last_tok, d2t, gate_w = dev(inp.tables), dev(inp.last_tok), dev(inp.d2t), dev(inp.gate_w)
    tokens = torch.empty(M, dtype=torch.int64, device="cuda")
    scores = torch.empty(R, dtype=torch.float32, device="cuda")
    ws = api.Workspace("cuda:0")
    torch.cuda.synchronize()

    def step():
        api.draft_block(hidden, W, tables, last_tok, top_k=K, d2t=d2t, gate_w=gate_w, block_len=L, walk=args.walk,
                        workspace=ws, out=(tokens, scores))

    stream = torch.cuda.current_stream()

    def timed(fn, n, warm):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n  # ms per call

    # ---- the timed region: K whole steps
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    ms = timed(step, args.steps, args.warmup)
    blocks_per_s = R / (ms / 1e3)
    rows_per_s = M / (ms / 1e3)
    log(f"{ms * 1e3:.1f} us/step -> {blocks_per_s:.0f} blocks/s, {rows_per_s:.0f} rows/s")

    # ---- per-stage durations of the stand-alone entry points, each alone on the same stream
    # (HIP events).  The fused step runs the same lm_head kernel; its Top-K reads only the
    # tiles the lm_head tile maxima keep, so it is faster than the stand-alone Top-K below,
    # which reads every logit.
    zbuf = torch.empty((M, api.logits_stride(Vd)), dtype=torch.float32, device="cuda")
    k1_ms = timed(lambda: api.lm_head(hidden, W, workspace=ws, with_lse=False, out=zbuf), args.steps, 3)
    z, lse = api.lm_head(hidden, W, workspace=ws)
    k2_ms = timed(lambda: api.topk(z, lse, K, d2t=d2t, target_vocab=Vt, workspace=ws), args.steps, 3)
    idx, ctok, un = api.topk(z, lse, K, d2t=d2t, target_vocab=Vt, workspace=ws)
    k3_ms = timed(lambda: api.pair_scores(ctok, tables, last_tok, gate_w=gate_w, hidden=hidden, block_len=L),
                  args.steps, 3)
    pair = api.pair_scores(ctok, tables, last_tok, gate_w=gate_w, hidden=hidden, block_len=L)
    k4_ms = timed(lambda: api.walk(ctok, un, pair, R, block_len=L, walk=args.walk), args.steps, 3)
    # ---- the head-less draft step on the same rows (scaled, soft-capped argmax), timed alone
    nh_tok = torch.empty(M, dtype=torch.int64, device="cuda")
    nh_ms = timed(lambda: api.draft_argmax(hidden, W, d2t=d2t, target_vocab=Vt, out_scale=1.0, soft_cap=30.0,
                                           workspace=ws, with_values=False, out=(nh_tok, None)), args.steps, 3)
    log(f"head-less step (scale 1, soft cap 30, argmax): {nh_ms * 1e3:.1f} us")
    # ---- the dense Markov walk on the same rows and tables (no gate), timed alone
    dn_ms = timed(lambda: api.draft_dense(hidden, W, tables, last_tok, d2t=d2t, block_len=L, out_scale=1.0,
                                          soft_cap=30.0, workspace=ws, with_values=False, out=(nh_tok, None)),
                  args.steps, 3)
    log(f"dense walk step (scale 1, soft cap 30): {dn_ms * 1e3:.1f} us")
    # ---- the whole step with the sampled walk (one seeded double uniform per row), timed alone
    uni = torch.rand(M, dtype=torch.float64, device="cuda", generator=torch.Generator("cuda").manual_seed(11))
    sp_ms = timed(lambda: api.draft_block_sampled(hidden, W, tables, last_tok, uni, top_k=K, temperature=1.0, d2t=d2t,
                                                  gate_w=gate_w, block_len=L, workspace=ws), args.steps, 3)
    log(f"sampled-walk step (temperature 1): {sp_ms * 1e3:.1f} us")
    # ---- one request of the same workload alone (its first block: L rows, the same weights)
    h1, lt1 = hidden[:L].contiguous(), last_tok[:1].contiguous()
    one_ms = timed(lambda: api.draft_block(h1, W, tables, lt1, top_k=K, d2t=d2t, gate_w=gate_w, block_len=L,
                                           walk=args.walk, workspace=ws), args.steps, 3)
    log(f"single request ({L} rows): {one_ms * 1e3:.1f} us")
    log(f"stages: lm_head {k1_ms * 1e3:.1f} us, top-k {k2_ms * 1e3:.1f} us, pair {k3_ms * 1e3:.1f} us, "
        f"walk {k4_ms * 1e3:.1f} us")

    # ---- roofline of the dominant kernel (the lm_head GEMM with its LSE epilogue)
    # algorithmic bytes of one launch: read W and the hidden states once, write the fp32 logits once
    w_bytes = Vd * H * 2
    h_bytes = M * H * 2
    z_bytes = M * Vd * 4
    k1_bytes = w_bytes + h_bytes + z_bytes
    k1_gbs = k1_bytes / (k1_ms * 1e-3) / 1e9
    k1_flops = 2.0 * M * H * Vd
    k1_tflops = k1_flops / (k1_ms * 1e-3) / 1e12
    # Top-K pass: reads the logits once, writes K candidates per row
    k2_bytes = z_bytes + M * 4 + M * K * (4 + 8 + 4)
    k2_gbs = k2_bytes / (k2_ms * 1e-3) / 1e9

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
                     "traffic": traffic, "bytes_per_launch": k1_bytes, "avg_launch_us": round(k1_ms * 1e3, 2),
                     "mfma_tflops": round(k1_tflops, 1), "mfma_peak_tflops": BF16_MFMA_PEAK_TFLOPS,
                     "mfma_frac": round(k1_tflops / BF16_MFMA_PEAK_TFLOPS, 4)},
        "standalone_topk_pass": {"achieved_gbs": round(k2_gbs, 1), "frac": round(k2_gbs / HBM_PEAK_GBS, 4),
                      "bytes_per_launch": k2_bytes, "avg_launch_us": round(k2_ms * 1e3, 2)},
        "headless_step": {"us": round(nh_ms * 1e3, 2), "blocks_per_s": round(R / (nh_ms * 1e-3), 1),
                          "out_scale": 1.0, "soft_cap": 30.0},
        "dense_step": {"us": round(dn_ms * 1e3, 2), "blocks_per_s": round(R / (dn_ms * 1e-3), 1),
                       "out_scale": 1.0, "soft_cap": 30.0,
                       # per position: the gathered B rows of every draft id and the rows' logits
                       "bytes_per_position": Vd * r * 4 + R * Vd * 4},
        "single_request_step": {"us": round(one_ms * 1e3, 2), "blocks_per_s": round(1 / (one_ms * 1e-3), 1),
                                "rows": L},
        "sampled_step": {"us": round(sp_ms * 1e3, 2), "blocks_per_s": round(R / (sp_ms * 1e-3), 1),
                         "temperature": 1.0},
        "standalone_stages_us": {"lm_head": round(k1_ms * 1e3, 2), "topk": round(k2_ms * 1e3, 2),
                      "pair_scores": round(k3_ms * 1e3, 2), "walk": round(k4_ms * 1e3, 2)},
    }

    # ---- the CPU oracle on a bounded sample of the same workload (baseline, not the target)
    if not args.no_cpu_baseline:
        from oracle import draft_step as O
        S = max(1, min(args.cpu_sample_requests, R))
        rows = S * L
        log(f"CPU oracle on {S} of {R} requests ({rows} rows)")
        try:
            from threadpoolctl import threadpool_info
            cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        except Exception:
            cores = 1
        # repeat the sample until about 10 s of CPU work; report the median rate
        times = []
        while True:
            t0 = time.perf_counter()
            res = O.draft_block(inp.hidden[:rows], inp.lm_head, inp.d2t, inp.tables, inp.gate_w, inp.last_tok[:S],
                                K, walk=O.WALK_VITERBI if args.walk == "viterbi" else O.WALK_GREEDY)
            times.append(time.perf_counter() - t0)
            if sum(times) >= 10.0 or len(times) >= 20:
                break
        dt = float(np.median(times))
        step()
        torch.cuda.synchronize()
        same = int(sum(np.array_equal(res.tokens[i * L:(i + 1) * L], tokens[i * L:(i + 1) * L].cpu().numpy())
                       for i in range(S)))
        out["cpu_baseline"] = {"value": round(S / dt, 3), "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
                               "sample": f"{S} of {R} requests ({rows} rows) of {shape.name}, fp64 numpy oracle, "
                                         f"median of {len(times)} runs of {dt:.2f} s",
                               "gpu_tokens_equal_requests": same}
        log(f"oracle: {dt:.1f} s for {S} blocks -> {S / dt:.3f} blocks/s on {cores} threads; "
            f"{same}/{S} requests drafted the same tokens as the GPU")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
