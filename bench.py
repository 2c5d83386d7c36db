"""Benchmark of the SeerAttention-R decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole decode hot path over one batch: K
Compression Cache update, gate scores, block selection and block-sparse
decode with its split merge, through the fused seer_decode_step call.  The
default workload is the Qwen3-14B-shaped batch (16 sequences, 40 query / 8 KV heads, d = 128, 32k context, 64-token
blocks, top-k 52 of 512 blocks = 90% sparsity).  Inputs are synthetic and
already resident in HBM.  To keep the 256 MB Infinity Cache from serving
repeated reads, the timed loop cycles through 24 independent replicas of
the inputs (each step touches a different one).  The V rows are read with
non-temporal loads and pass the Infinity Cache by; the rest (the selected K
rows, compressed cache, W_q, q, split partials: about 130 MB per replica)
does stay there, so the replicas together must hold well over 256 MB of it.
Even the 21 MB that is not K needs more than 16 replicas: with only that
kept, 16 replicas measured 0.5 us per step faster, 24 and 32 the same.

Prints one JSON line: µs per step (lower is better), achieved HBM bandwidth
of the decode kernel on its algorithmic bytes against the 8 TB/s peak, the
speedup over the library's own dense decode at equal shape, and the float64
oracle's whole step timed on the host cores.  Its "extra" object holds the
other configurations (step, decode and dense µs, GB/s, fraction of peak and
speedup each): the Qwen3-8B-shaped layer at batch 1, the 64-sequence
threshold batch, the 256-step 128k pipeline, the benchmarked batch over a
paged cache and with top-p 0.9 and 0.99 (--no-extra leaves it out).  The line also carries
the training-side call, seer_prefill_attention (causal prefill forward with
the gate's ground truth) on a 32k-token Qwen3-14B-shaped layer, against the
2.5 PFLOP/s dense bf16 MFMA peak ("prefill_gt"; --prefill-only runs just
that leg, for profiling).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("sparse decode µs/step + achieved HBM GB/s (% peak); "
          "speedup vs dense @90% sparsity")
PEAK_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 MFMA, MI355X
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SRCS = [os.path.join(ROOT, "block_sparse_attention_seer_amd", "csrc", f)
               for f in ("decode.hip", "seer_device.hpp")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_src_hash() -> str:
    """Hash of the decode kernel's sources (the kernel file and its device
    helpers): stored counter figures apply only to the kernel they measured."""
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter runs,
    or None if they are absent or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_src_sha256_16") != decode_src_hash():
        return None
    return t


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3_14b_b16")
    ap.add_argument("--replicas", type=int, default=24)
    ap.add_argument("--dense-steps", type=int, default=20)
    ap.add_argument("--num-split", type=int, default=0)
    ap.add_argument("--select", choices=("workload", "topk", "threshold", "topp"),
                    default="workload",
                    help="selection rule of the timed steps (default: the workload's own)")
    ap.add_argument("--mass", type=float, default=0.9,
                    help="threshold tau or top-p mass p when --select overrides the rule")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="budget of the oracle CPU baseline (the whole step when it fits)")
    ap.add_argument("--flushed-iters", type=int, default=100,
                    help="iterations of the per-iteration timing with a 1 GiB cache flush "
                         "(0 skips it)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only seer_prefill_attention and print its object")
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true",
                    help="leave the other configurations out of the headline line")
    ap.add_argument("--extra", action="store_true",
                    help="instead of the headline line: one JSON line each for the Qwen3-8B-shaped "
                         "layer, the 64-sequence threshold batch, the 256-step 128k pipeline, "
                         "the benchmarked batch over a paged cache and with top-p, and the pages' "
                         "microbenchmark grid (64/8 heads, batch 1/4/16, 8k/32k/128k, "
                         "50%%/90%% sparsity)")
    ap.add_argument("--counter-pass", "--traffic-pass", dest="counter_pass", action="store_true",
                    help="for rocprofv3 --pmc runs: launches of every kernel of the path with "
                         "their algorithmic bytes, and a plain copy of known size (the counters' "
                         "scale); prints one JSON line describing them, then exits")
    ap.add_argument("--counter-summary", nargs=3, metavar=("PASS_JSON", "FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: HBM bytes per kernel from the counter pass's JSON line and "
                         "the FETCH_SIZE and WRITE_SIZE counter_collection CSVs of two "
                         "--counter-pass runs; writes profiles/decode_traffic.json and prints "
                         "a markdown table")
    args = ap.parse_args()
    if args.counter_summary:
        return counter_summary(*args.counter_summary)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decode path of one layer is measured on a "
              "single MI355X (no multi-GPU path is built); use --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import block_sparse_attention_seer_amd as S
    from workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    S.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.counter_pass:
        return counter_pass(S, torch, np, dev)
    if args.prefill_only:
        print(json.dumps({"prefill_gt": prefill_leg(S, torch, dev, args.prefill_steps)}),
              flush=True)
        return 0
    if args.extra:
        return extra_lines(S, torch, np, dev)
    w = WORKLOADS[args.workload]
    if args.select != "workload":
        w = w.replace(mode=args.select, tau=args.mass)
    if w.seq_len is None:
        print("bench.py times single-length workloads (qwen3_8b_layer, qwen3_14b_b16, tiny)",
              file=sys.stderr)
        return 2
    B, Hq, Hkv, d, dg, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate, w.block_size
    g = w.group
    L = w.seq_len
    dims = S.make_dims(B, Hq, Hkv, d, dg, bs, w.max_seq_len)
    mode = {"topk": S.SELECT_TOPK, "threshold": S.SELECT_THRESHOLD, "topp": S.SELECT_TOPP}[w.mode]

    # ---- replicas of the inputs, each with its own cache and step buffers
    R = max(1, args.replicas)
    reps = []
    for r in range(R):
        log(f"generating replica {r + 1}/{R}")
        inp = make_inputs(w.replace(seed=w.seed + 7919 * r), device=str(dev))
        st = S.DecodeStep(dims, mode=mode, topk_blocks=w.topk_blocks, threshold=w.tau,
                          num_split=args.num_split, device=dev)
        seq = inp["seq_lens"]
        st.build_cache(inp["k"], inp["w_k"], seq)
        reps.append((inp, st))
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(d)

    # the whole decode step (cache update, gate, selection, sparse decode) as
    # one seer_decode_step call per replica; the binding checks the tensors
    # once (bind_step) so that its per-call Python checks stay out of the loop
    bound = [st.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                          inp["w_k"], inp["seq_lens"], scale, 1, False) for inp, st in reps]

    def step(r):
        bound[r]()

    def decode_only(r):
        inp, st = reps[r]
        S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], st.block_idx,
                             st.num_selected, st.max_selected, scale, st.num_split, st.decode_ws,
                             st.out, st.lse)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g0.record()
    for i in range(args.steps):
        step(i % R)
    g1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    step_gpu_us = 1e3 * g0.elapsed_time(g1) / args.steps

    # the same step replayed from HIP graphs (one per replica), for the
    # launch overhead the eager loop above pays on the host
    graphs = []
    for inp, st in reps:
        graphs.append(st.capture_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                                      inp["w_k"], inp["seq_lens"], scale, 1, False))
    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / args.steps

    # eight steps (eight replicas, as the layers of one token would be) in
    # one graph: the replay's fixed cost is paid once per eight steps
    G8 = 8
    multi = []
    for r0 in range(0, R - R % G8, G8):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph):
            for r in range(r0, r0 + G8):
                step(r)
        multi.append(gph)
    graph8_us = None
    if multi:
        for i in range(max(2, args.warmup // G8)):
            multi[i % len(multi)].replay()
        torch.cuda.synchronize()
        n8 = max(1, args.steps // G8)
        t0 = time.perf_counter()
        for i in range(n8):
            multi[i % len(multi)].replay()
        torch.cuda.synchronize()
        graph8_us = (time.perf_counter() - t0) * 1e6 / (n8 * G8)
    del multi

    # the dominant kernel alone, event-timed on the stream it runs on, on the
    # same replicas and the selections the steps just made
    # (the binding launches on torch's current stream, which these events see)
    log(f"timing {args.steps} decode launches")
    for i in range(3):  # the standalone decode kernel's first launches (code loading) untimed
        decode_only(i % R)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        decode_only(i % R)
    e1.record()
    torch.cuda.synchronize()
    dec_us = 1e3 * e0.elapsed_time(e1) / args.steps

    # ---- algorithmic bytes (per step, from the actual selections)
    nb = L // bs
    sel_tokens = float(np.mean([selected_tokens(st, L, bs) for _, st in reps]))
    qo_bytes = 2 * B * Hq * d * 2
    kv_bytes = sel_tokens * 2 * d * 2
    idx_bytes = B * Hkv * (reps[0][1].max_selected + 1) * 4
    decode_alg = kv_bytes + qo_bytes + idx_bytes
    step_alg = decode_alg + B * Hkv * nb * dg * 2 + Hkv * dg * g * d * 2
    achieved = decode_alg / (dec_us * 1e-6) / 1e9
    step_gbps = step_alg / (ms_per_step * 1e-3) / 1e9

    # ---- dense baseline at equal shape
    log(f"dense baseline {args.dense_steps} steps")
    ns_dense = S.seer_decode_num_split(dims, dims.nb_max, 0)
    dws = torch.zeros(max(S.seer_decode_workspace_bytes(dims, dims.nb_max, ns_dense), 256) // 4 + 64,
                      dtype=torch.float32, device=dev)
    dout = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    dlse = torch.empty((B, Hq), dtype=torch.float32, device=dev)

    def dense(r):
        inp, _ = reps[r]
        S.seer_dense_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale, ns_dense,
                            dws, dout, dlse)

    for i in range(3):
        dense(i % R)
    torch.cuda.synchronize()
    dev_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.dense_steps)]
    for i in range(args.dense_steps):
        dev_evs[i][0].record()
        dense(i % R)
        dev_evs[i][1].record()
    torch.cuda.synchronize()
    dense_us = 1e3 * float(np.mean([a.elapsed_time(b) for a, b in dev_evs]))
    dense_bytes = B * Hkv * L * 2 * d * 2 + qo_bytes
    dense_gbps = dense_bytes / (dense_us * 1e-6) / 1e9

    # ---- per-iteration timing with the caches flushed: before each timed
    # iteration 1 GiB goes through the memory system outside the timed region,
    # so the 256 MB Infinity Cache and the L2s hold nothing of the step's data;
    # each iteration is event-timed on its own (median, p10, p90).  Two
    # flushes: writing 1 GiB, which leaves the Infinity Cache full of dirty
    # lines whose write-back then shares HBM with the timed reads, and reading
    # 1 GiB, which evicts as thoroughly without that write-back.
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def flushed(fn, iters, warm, how):
        times = []
        for i in range(warm + iters):
            if how == "write":
                flush.fill_(float(i))
            else:
                flush.sum()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            fn(i % R)
            b_.record()
            torch.cuda.synchronize()
            if i >= warm:
                times.append(a_.elapsed_time(b_) * 1e3)
        q = np.percentile(times, [10, 50, 90])
        return {"p10": round(float(q[0]), 2), "median": round(float(q[1]), 2),
                "p90": round(float(q[2]), 2)}

    flushed_step = flushed_decode = flushed_dense = None
    if args.flushed_iters > 0:  # 0: skipped (profiler runs)
        log("flushed per-iteration timing")
        flushed_step = {how + "_flush": flushed(step, args.flushed_iters, 10, how)
                        for how in ("read", "write")}
        flushed_decode = {how + "_flush": flushed(decode_only, args.flushed_iters, 10, how)
                          for how in ("read", "write")}
        flushed_dense = {"read_flush": flushed(dense, max(10, args.flushed_iters // 5), 3,
                                               "read")}
    del flush

    # ---- amortised cost of a real cache update (one block per (b, h))
    inp0, st0 = reps[0]
    kupd = []
    for i in range(5):
        st0.kcomp_lens.fill_(nb - 1)
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        S.seer_kcomp_update(dims, inp0["k"], inp0["w_k"], inp0["seq_lens"], st0.kcomp_lens,
                            st0.kcomp, 1, w.theta)
        b_.record()
        torch.cuda.synchronize()
        kupd.append(a_.elapsed_time(b_) * 1e3)
    kcomp_us = float(np.median(kupd))

    # ---- the bulk build of a prompt's whole cache (every complete block of
    # every pair), once per replica in turn: each build reads keys that no
    # recent call has touched (cold caches); the entries are rebuilt as they
    # were, so the replicas' state is unchanged
    bulk = []
    for r in range(R):
        inp_r, st_r = reps[r]
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st_r.kcomp_lens.zero_()
        a_.record()
        S.seer_kcomp_update(dims, inp_r["k"], inp_r["w_k"], inp_r["seq_lens"], st_r.kcomp_lens,
                            st_r.kcomp, dims.nb_max, w.theta)
        b_.record()
        torch.cuda.synchronize()
        bulk.append(a_.elapsed_time(b_) * 1e3)
    bulk_us = float(np.median(bulk))
    bulk_bytes = B * Hkv * nb * (bs * d * 2 + dg * 2) + Hkv * dg * 3 * d * 2

    # ---- float64 oracle on the host cores, bounded sample
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(reps[0][0], w, args.cpu_seconds)

    log("prefill with ground truth")
    prefill = prefill_leg(S, torch, dev, args.prefill_steps)

    traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
                   "d_gate": dg, "block_size": bs, "seq_len": L, "mode": w.mode,
                   **({"topk_blocks": w.topk_blocks} if w.mode == "topk" else {"mass": w.tau}),
                   "num_split": reps[0][1].num_split,
                   "replicas": R},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel (block-sparse split decode + LSE merge)",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "algorithmic_bytes": int(decode_alg),
            "avg_launch_us": round(dec_us, 3),
            "timing": "one HIP event pair on the launch stream around K back-to-back decode "
                      "launches (same replicas and selections as the timed steps); avg = "
                      "elapsed / K",
        },
        "step_us_events": round(step_gpu_us, 3),
        "step_us_flushed": flushed_step,
        "decode_us_flushed": flushed_decode,
        "dense_us_flushed": flushed_dense,
        "speedup_vs_dense_step_read_flush": (
            round(flushed_dense["read_flush"]["median"] / flushed_step["read_flush"]["median"], 3)
            if flushed_step is not None else None),
        "step_us_graph_replay": round(graph_us, 3),
        "step_us_graph_replay_8_steps_per_graph": (round(graph8_us, 3) if graph8_us is not None
                                                   else None),
        "step_algorithmic_bytes": int(step_alg),
        "step_GBps": round(step_gbps, 1),
        "step_frac_of_peak": round(step_gbps / PEAK_GBPS, 4),
        "dense_us": round(dense_us, 2),
        "dense_GBps": round(dense_gbps, 1),
        "speedup_vs_dense_step": round(dense_us / (ms_per_step * 1e3), 3),
        "speedup_vs_dense_kernel": round(dense_us / dec_us, 3),
        "kcomp_update_us_per_completion": round(kcomp_us, 2),
        "kcomp_update_us_amortised": round(kcomp_us / bs, 3),
        "kcomp_bulk_build": {"us_median": round(bulk_us, 1), "builds": R,
                             "entries": B * Hkv * nb, "algorithmic_bytes": int(bulk_bytes),
                             "GBps": round(bulk_bytes / (bulk_us * 1e-6) / 1e9, 1),
                             "timing": "event pair around one seer_kcomp_update of the whole "
                                       "cache per replica in turn (cold), median"},
        "selected_fraction": round(sel_tokens / (B * Hkv * L), 4),
        "cpu_baseline": cpu,
        "prefill_gt": prefill,
    }
    if not args.no_extra:
        # the other configurations, after the headline's replicas are freed
        del reps, bound, graphs, inp0, st0, dws, dout, dlse
        import gc
        gc.collect()
        torch.cuda.empty_cache()
        t_extra = time.perf_counter()
        line["extra"] = {}
        for key, obj in extra_measurements(S, torch, np, dev, grid=False):
            line["extra"][key] = obj
        log(f"extra configurations took {time.perf_counter() - t_extra:.1f} s")
    print(json.dumps(line), flush=True)
    return 0


def prefill_leg(S, torch, dev, steps):
    """seer_prefill_attention on the 32k-token Qwen3-14B-shaped layer: the
    call with the ground truth and the attention-only call, each event-timed
    over `steps` back-to-back calls on the launch stream.  `achieved` is the
    algorithmic MFMA work (4 d flops per query-key pair the causal mask keeps:
    2d for q.k, 2d for p.v) over the whole call, so the small V-transpose
    and ground-truth kernels count against it."""
    from workloads import PREFILL_WORKLOADS, make_prefill_inputs
    w = PREFILL_WORKLOADS["qwen3_14b_prefill_32k"]
    B, Hq, Hkv, d, L = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.max_seq_len
    inp = make_prefill_inputs(w, device=str(dev))
    dims = S.make_dims(B, Hq, Hkv, d, d, w.block_size, L)
    ws = torch.empty(S.seer_prefill_workspace_bytes(dims) // 4 + 64, dtype=torch.float32,
                     device=dev)
    out = torch.empty((B, Hq, L, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    gt = torch.empty((B, Hkv, L, dims.nb_max), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    flops = sum(2.0 * d * n * (n + 1) for n in w.seq_lens) * Hq
    us = {}
    for label, g in (("gt", gt), ("attn", None)):
        for _ in range(2):
            S.seer_prefill_attention(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale,
                                     ws, out, lse, g)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            S.seer_prefill_attention(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale,
                                     ws, out, lse, g)
        e1.record()
        torch.cuda.synchronize()
        us[label] = 1e3 * e0.elapsed_time(e1) / steps
    achieved = flops / (us["gt"] * 1e-6) / 1e12
    return {
        "workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "head_dim": d,
        "block_size": w.block_size, "seq_len": L, "calls": steps,
        "us_per_call": round(us["gt"], 1),
        "attention_only_us": round(us["attn"], 1),
        "ground_truth_overhead": round(us["gt"] / us["attn"] - 1, 4),
        "algorithmic_tflop": round(flops / 1e12, 3),
        "roofline": {"bound": "mfma", "kernel": "seer_prefill_attention (vt_kernel + "
                     "fa_fwd_kernel + gt_kernel)", "achieved": round(achieved, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "attention_only_achieved": round(flops / (us["attn"] * 1e-6) / 1e12, 1)},
    }


def selected_tokens(st, L, bs):
    ns = st.num_selected.cpu().numpy()
    idx = st.block_idx.cpu().numpy()
    tot = 0
    for b_ in range(ns.shape[0]):
        for h_ in range(ns.shape[1]):
            for j in idx[b_, h_, :ns[b_, h_]]:
                tot += min(bs, L - int(j) * bs)
    return tot


def _alg_decode(st, lens, B, Hq, Hkv, d, bs):
    """Algorithmic bytes of one sparse decode launch: the selected K and V
    rows, q, out, the index rows and counts."""
    return (_selected_tokens(st, lens, bs) * 2 * d * 2 + 2 * B * Hq * d * 2
            + B * Hkv * (st.max_selected + 1) * 4)


def _alg_gate(lens, B, Hq, Hkv, d, dg, bs, max_sel):
    """Algorithmic bytes of one selecting gate launch: the group's pre-RoPE
    queries, the cached entries of every complete block, W_q once, the
    index rows and counts written (no logits written)."""
    g = Hq // Hkv
    nc = int((np_floor_div(lens, bs)).sum())
    return B * Hq * d * 2 + nc * Hkv * dg * 2 + Hkv * dg * g * d * 2 + B * Hkv * (max_sel + 1) * 4


def np_floor_div(lens, bs):
    import numpy as np
    return np.asarray(lens, dtype=np.int64) // bs


def counter_pass(S, torch, np, dev):
    """--counter-pass: for rocprofv3 --pmc runs, one pass over every kernel
    of the path on the benchmarked batch (and the 64-sequence threshold
    batch), each group with its algorithmic bytes per launch, then three
    torch.neg copies of 256 MiB (read 256 MiB, write 256 MiB each) whose
    counts give the counters' scale.  Prints one JSON line that
    --counter-summary reads."""
    from workloads import WORKLOADS, make_inputs
    groups = []

    def group(label, kernel, workgroups, alg, launches):
        groups.append({"label": label, "kernel": kernel, "workgroups": workgroups,
                       "algorithmic_bytes_per_launch": int(alg), "launches": launches})

    # ---- the benchmarked batch: cache build, fused steps, decode alone,
    # dense decode, then the stream-K decode of a top-p 0.9 step
    w = WORKLOADS["qwen3_14b_b16"]
    B, Hq, Hkv, d, dg, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate, w.block_size
    dims = S.make_dims(B, Hq, Hkv, d, dg, bs, w.max_seq_len)
    scale = 1.0 / math.sqrt(d)
    log("counter pass: qwen3_14b_b16")
    inp = make_inputs(w, device=str(dev))
    lens = inp["seq_lens"].cpu().numpy()
    st = S.DecodeStep(dims, mode=S.SELECT_TOPK, topk_blocks=w.topk_blocks, device=dev)
    for _ in range(3):
        st.build_cache(inp["k"], inp["w_k"], inp["seq_lens"])
    nbm = dims.nb_max
    group("cache build (bulk, every complete block)", "prep_bulk_kernel<128, 128>",
          B * Hkv * -(-nbm // 16),
          int(np_floor_div(lens, bs).sum()) * Hkv * (bs * d * 2 + dg * 2) + Hkv * dg * 3 * d * 2, 3)
    run = st.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"], inp["w_k"],
                       inp["seq_lens"], scale, 1, False)
    for _ in range(10):
        run()
    torch.cuda.synchronize()
    group("gate, top-k 52 (128 pairs)", "gate_kernel<128, 128>", B * Hkv,
          _alg_gate(lens, B, Hq, Hkv, d, dg, bs, st.max_selected), 10)
    for _ in range(10):
        S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], st.block_idx,
                             st.num_selected, st.max_selected, scale, st.num_split, st.decode_ws,
                             st.out, st.lse)
    torch.cuda.synchronize()
    group("sparse decode, top-k 52, fixed splits", "decode_kernel<128, 64, false, 8, false, false>",
          B * Hkv * st.num_split, _alg_decode(st, lens, B, Hq, Hkv, d, bs), 20)
    dn = _dense_buffers(S, torch, dims, dev)
    for _ in range(3):
        S.seer_dense_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale, *dn)
    torch.cuda.synchronize()
    group("dense decode (baseline)", "decode_kernel<128, 64, true, 8, false, false>",
          B * Hkv * dn[0], int(lens.sum()) * Hkv * 2 * d * 2 + 2 * B * Hq * d * 2, 3)
    stp = S.DecodeStep(dims, mode=S.SELECT_TOPP, threshold=0.9, device=dev)
    stp.kcomp.copy_(st.kcomp)
    stp.kcomp_lens.copy_(st.kcomp_lens)
    run_p = stp.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                          inp["w_k"], inp["seq_lens"], scale, 1, False)
    for _ in range(10):
        run_p()
    torch.cuda.synchronize()
    group("sparse decode, top-p 0.9, stream-K (fused step)",
          "decode_kernel<128, 64, false, 8, false, true>", None,
          _alg_decode(stp, lens, B, Hq, Hkv, d, bs), 10)
    del inp, st, stp, run, run_p, dn
    torch.cuda.empty_cache()

    # ---- the 64-sequence threshold batch (b = 128, fixed splits)
    w = WORKLOADS["threshold_b128"]
    B, Hq, Hkv, d, dg, bs = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate, w.block_size
    dims = S.make_dims(B, Hq, Hkv, d, dg, bs, w.max_seq_len)
    scale = 1.0 / math.sqrt(d)
    log("counter pass: threshold_b128")
    inp = make_inputs(w, device=str(dev))
    lens = inp["seq_lens"].cpu().numpy()
    st = S.DecodeStep(dims, mode=S.SELECT_THRESHOLD, threshold=w.tau, device=dev)
    st.build_cache(inp["k"], inp["w_k"], inp["seq_lens"])
    run = st.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"], inp["w_k"],
                       inp["seq_lens"], scale, 1, False)
    for _ in range(5):
        run()
    torch.cuda.synchronize()
    group(f"gate, threshold 0.01 ({B * Hkv} pairs, b = 128)", "gate_kernel<128, 128>", B * Hkv,
          _alg_gate(lens, B, Hq, Hkv, d, dg, bs, st.max_selected), 5)
    group("sparse decode, threshold 0.01, b = 128, fixed splits",
          "decode_kernel<128, 128, false", B * Hkv * st.num_split,
          _alg_decode(st, lens, B, Hq, Hkv, d, bs), 5)
    del inp, st, run
    torch.cuda.empty_cache()

    copy_bytes = 256 << 20
    src = torch.ones(copy_bytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"counter_pass": True, "groups": groups, "copy_kernel": "neg_kernel",
                      "copy_bytes_each_way": copy_bytes, "copies": 3,
                      "decode_src_sha256_16": decode_src_hash()}), flush=True)
    return 0


def _read_counters(path):
    """{(kernel name, workgroups): [value per dispatch, in dispatch order]}
    for the one counter of a rocprofv3 --pmc counter_collection CSV."""
    import csv
    import re
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            name = re.sub(r"^void ", "", row["Kernel_Name"])
            name = re.sub(r"seer::\(anonymous namespace\)::|seer::", "", name)
            wg = int(row["Grid_Size"]) // max(1, int(row["Workgroup_Size"]))
            out.setdefault((name, wg), []).append((int(row.get("Dispatch_Id", 0) or 0),
                                                   float(row["Counter_Value"])))
    return {k: [v for _, v in sorted(vals)] for k, vals in out.items()}


def counter_summary(pass_json, fetch_csv, write_csv):
    """--counter-summary: scaled HBM bytes per launch of each group of the
    counter pass (the mean over the group's last `launches` dispatches), the
    counters' scale from the copy, and profiles/decode_traffic.json for the
    benchmarked decode."""
    with open(pass_json) as f:
        info = next(json.loads(line) for line in f if line.startswith("{"))
    fetch, write = _read_counters(fetch_csv), _read_counters(write_csv)

    def pick(table, kernel, wg, n):
        keys = [k for k in table if k[0].startswith(kernel) and (wg is None or k[1] == wg)]
        if len(keys) != 1:
            raise SystemExit(f"counter summary: {len(keys)} kernel groups match {kernel!r} "
                             f"with {wg} workgroups: {keys}")
        vals = table[keys[0]][-n:]
        return sum(vals) / len(vals), keys[0]

    n_copy = info["copies"]
    copy_f = [v for k, vals in fetch.items() if info["copy_kernel"] in k[0] for v in vals][-n_copy:]
    copy_w = [v for k, vals in write.items() if info["copy_kernel"] in k[0] for v in vals][-n_copy:]
    cf, cw = sum(copy_f) / len(copy_f), sum(copy_w) / len(copy_w)
    known_kib = info["copy_bytes_each_way"] / 1024
    fs, ws_ = known_kib / cf, known_kib / cw
    rows = []
    for g in info["groups"]:
        f_raw, key = pick(fetch, g["kernel"], g["workgroups"], g["launches"])
        w_raw, _ = pick(write, g["kernel"], g["workgroups"], g["launches"])
        fb, wb = f_raw * fs * 1024, w_raw * ws_ * 1024
        rows.append({"label": g["label"], "kernel": key[0], "workgroups": key[1],
                     "fetch_kib_raw": round(f_raw, 1), "write_kib_raw": round(w_raw, 1),
                     "fetch_bytes": int(fb), "write_bytes": int(wb),
                     "algorithmic_bytes": g["algorithmic_bytes_per_launch"],
                     "traffic_over_algorithmic": round((fb + wb) / g["algorithmic_bytes_per_launch"],
                                                       4)})
    dec = next(r for r in rows if r["label"].startswith("sparse decode, top-k 52"))
    traffic = {
        "kernel": "decode_kernel", "workload": "qwen3_14b_b16",
        "decode_src_sha256_16": info["decode_src_sha256_16"],
        "fetch_kib_per_launch_raw": dec["fetch_kib_raw"],
        "write_kib_per_launch_raw": dec["write_kib_raw"],
        "copy_fetch_kib_raw": round(cf, 1), "copy_write_kib_raw": round(cw, 1),
        "copy_bytes_each_way": info["copy_bytes_each_way"],
        "fetch_scale": round(known_kib / round(cf, 1), 5),
        "write_scale": round(known_kib / round(cw, 1), 5),
    }
    # the same bytes as the table row (unrounded scales)
    traffic["fetch_bytes_per_launch"] = dec["fetch_bytes"]
    traffic["write_bytes_per_launch"] = dec["write_bytes"]
    traffic["bytes_per_launch"] = traffic["fetch_bytes_per_launch"] + traffic["write_bytes_per_launch"]
    traffic["algorithmic_bytes_per_launch"] = dec["algorithmic_bytes"]
    traffic["traffic_over_algorithmic"] = round(traffic["bytes_per_launch"] /
                                                dec["algorithmic_bytes"], 4)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    print(f"| kernel group | kernel | workgroups | FETCH_SIZE KiB | WRITE_SIZE KiB | "
          f"HBM bytes (scaled) | algorithmic bytes | ratio |")
    print("|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['label']} | `{r['kernel']}` | {r['workgroups']} | {r['fetch_kib_raw']} | "
              f"{r['write_kib_raw']} | {r['fetch_bytes'] + r['write_bytes']:,} | "
              f"{r['algorithmic_bytes']:,} | {r['traffic_over_algorithmic']} |")
    print(f"\ncopy `{info['copy_kernel']}` of {info['copy_bytes_each_way']:,} B each way: "
          f"FETCH_SIZE {cf:.1f} KiB (scale {fs:.5f}), WRITE_SIZE {cw:.1f} KiB (scale {ws_:.5f})")
    return 0


def blas_threads():
    """Threads of the BLAS library NumPy calls (None if it cannot be asked)."""
    try:
        from threadpoolctl import threadpool_info
    except ImportError:
        return None
    n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
    return max(n) if n else None


def cpu_baseline(inp, w, budget_s, repeats=3):
    """The float64 oracle's decode step (gate query, logits, selection,
    attention) over every (b, h) pair of the batch: each pair's cache is built
    untimed, then its decode is timed `repeats` times and the median kept; the
    step is the sum of the pairs' medians.  Pairs go in a seeded random order;
    if the budget runs out first, the mean of the timed pairs is scaled to the
    whole batch (the line says how many pairs were timed)."""
    import numpy as np

    import oracle as O

    f = lambda t: t.detach().double().cpu().numpy()  # noqa: E731
    L = w.seq_len
    g = w.group
    pairs = [(b, h) for b in range(w.batch) for h in range(w.num_kv_heads)]
    order = np.random.default_rng(0).permutation(len(pairs))
    log(f"cpu baseline: {len(pairs)} pairs, budget {budget_s:.0f} s")
    medians = []
    t_start = time.perf_counter()
    for i in order:
        b, h = pairs[i]
        q = f(inp["q"][b, h * g:(h + 1) * g])
        k, v = f(inp["k"][b, h, :L]), f(inp["v"][b, h, :L])
        kc = O.build_kcomp(k, f(inp["w_k"][h]), L, w.block_size, w.theta)
        wq = f(inp["w_q"][h])
        times = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            O.decode_pair(q, q, k, k, v, wq, kc, L, w.block_size, mode=w.mode, topk=w.topk_blocks,
                          tau=w.tau, scale=1.0 / math.sqrt(w.head_dim), theta=w.theta)
            times.append(time.perf_counter() - t0)
        medians.append(float(np.median(times)))
        if time.perf_counter() - t_start > budget_s:
            break
    full = len(medians) == len(pairs)
    value = sum(medians) if full else float(np.mean(medians)) * len(pairs)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    threads = blas_threads()
    return {"value": round(value * 1e6, 1), "unit": "us/step",
            "cores": threads if threads is not None else affinity, "kind": "oracle",
            "os_cpu_count": os.cpu_count(), "affinity_cpus": affinity, "blas_threads": threads,
            "pairs_timed": len(medians), "pairs": len(pairs),
            "sample": (f"the whole step: all {len(pairs)} (b, h) pairs, each pair's decode "
                       f"timed {repeats} times (median), summed" if full else
                       f"{len(medians)} of {len(pairs)} (b, h) pairs in a seeded random order, "
                       f"each timed {repeats} times (median); mean pair time x {len(pairs)}")
            + "; caches built untimed; NumPy float64, BLAS threads at default"}


# ----------------------------------------------------------------- --extra


def _events_us(torch, fn, n):
    """Average µs of n back-to-back calls fn(i), one event pair around them."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / n


def _flushed_median_us(torch, fn, n, flush):
    """Median µs of n calls, each event-timed on its own after 1 GiB has been
    read outside the timed region (cold Infinity Cache and L2)."""
    times = []
    for i in range(n + 3):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        torch.cuda.synchronize()
        if i >= 3:
            times.append(1e3 * a.elapsed_time(b))
    times.sort()
    return times[len(times) // 2]


def _dense_buffers(S, torch, dims, dev):
    """Split count, zeroed workspace and outputs of a dense decode call."""
    ns = S.seer_decode_num_split(dims, dims.nb_max, 0)
    ws = torch.zeros(max(S.seer_decode_workspace_bytes(dims, dims.nb_max, ns), 256) // 4 + 64,
                     dtype=torch.float32, device=dev)
    out = torch.empty((dims.batch, dims.num_q_heads, dims.head_dim), dtype=torch.bfloat16,
                      device=dev)
    lse = torch.empty((dims.batch, dims.num_q_heads), dtype=torch.float32, device=dev)
    return ns, ws, out, lse


def _selected_tokens(st, lens, bs):
    ns = st.num_selected.cpu().numpy()
    idx = st.block_idx.cpu().numpy()
    tot = 0
    for b_ in range(ns.shape[0]):
        L = int(lens[b_])
        for h_ in range(ns.shape[1]):
            for j in idx[b_, h_, :ns[b_, h_]]:
                tot += max(0, min(bs, L - int(j) * bs))
    return tot


def extra_measurements(S, torch, np, dev, grid=False):
    """Measurements beyond the headline configuration: yields (key, object)
    for the Qwen3-8B-shaped layer, the 64-sequence threshold batch, the
    256-step 128k pipeline, the benchmarked batch over a paged cache and with
    top-p 0.9 / 0.99, and (grid=True) the pages' microbenchmark grid."""
    from workloads import WORKLOADS, make_inputs
    modes = {"topk": S.SELECT_TOPK, "threshold": S.SELECT_THRESHOLD}
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    # ---- single steps of the Qwen3-8B-shaped layer and the threshold batch
    for name in ("qwen3_8b_layer", "threshold_b128"):
        w = WORKLOADS[name]
        log(f"extra: {name}")
        B, Hq, Hkv, d, dg, bs = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate,
                                 w.block_size)
        dims = S.make_dims(B, Hq, Hkv, d, dg, bs, w.max_seq_len)
        scale = 1.0 / math.sqrt(d)
        reps = []
        for r in range(2):
            inp = make_inputs(w.replace(seed=w.seed + 7919 * r), device=str(dev))
            st = S.DecodeStep(dims, mode=modes[w.mode], topk_blocks=w.topk_blocks,
                              threshold=w.tau, device=dev)
            st.build_cache(inp["k"], inp["w_k"], inp["seq_lens"])
            run = st.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                               inp["w_k"], inp["seq_lens"], scale, 1, False)
            reps.append((inp, st, run))
        for i in range(10):
            reps[i % 2][2]()
        step_us = _events_us(torch, lambda i: reps[i % 2][2](), 100)
        # the same step replayed from one HIP graph per replica
        graphs = [st.capture_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                                  inp["w_k"], inp["seq_lens"], scale, 1, False)
                  for inp, st, _ in reps]
        for i in range(10):
            graphs[i % 2].replay()
        graph_us = _events_us(torch, lambda i: graphs[i % 2].replay(), 100)
        del graphs
        # eight steps (the two replicas alternating) in one graph
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8):
            for i in range(8):
                reps[i % 2][2]()
        for _ in range(3):
            g8.replay()
        graph8_us = _events_us(torch, lambda i: g8.replay(), 20) / 8
        del g8

        def dec(i):
            inp, st, _ = reps[i % 2]
            S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                 st.block_idx, st.num_selected, st.max_selected, scale,
                                 st.num_split, st.decode_ws, st.out, st.lse)

        dn = _dense_buffers(S, torch, dims, dev)

        def dense(i):
            inp = reps[i % 2][0]
            S.seer_dense_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale, *dn)

        dec_us = _events_us(torch, dec, 100)
        dense_us = _events_us(torch, dense, 10)
        lens = reps[0][0]["seq_lens"].cpu().numpy()
        sel = float(np.mean([_selected_tokens(st, inp["seq_lens"].cpu().numpy(), bs)
                             for inp, st, _ in reps]))
        qo = 2 * B * Hq * d * 2
        idx_bytes = B * Hkv * (reps[0][1].max_selected + 1) * 4
        dec_alg = sel * 2 * d * 2 + qo + idx_bytes
        step_alg = dec_alg + sum(int(L) // bs for L in lens) * Hkv * dg * 2 + Hkv * dg * (Hq // Hkv) * d * 2
        dense_bytes = int(lens.sum()) * Hkv * 2 * d * 2 + qo
        yield name, {
            "kind": "config", "workload": name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
            "head_dim": d, "block_size": bs, "mode": w.mode,
            "seq_len": int(lens[0]) if w.seq_len else [int(lens.min()), int(lens.max())],
            "step_us": round(step_us, 2), "step_us_graph_replay": round(graph_us, 2),
            "step_us_graph_replay_8_steps_per_graph": round(graph8_us, 2),
            "decode_us": round(dec_us, 2),
            "decode_GBps": round(dec_alg / (dec_us * 1e-6) / 1e9, 1),
            "decode_frac_of_peak": round(dec_alg / (dec_us * 1e-6) / 1e9 / PEAK_GBPS, 4),
            "step_GBps": round(step_alg / (step_us * 1e-6) / 1e9, 1),
            "dense_us": round(dense_us, 2),
            "dense_GBps": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
            "speedup_vs_dense_step": round(dense_us / step_us, 3),
            "speedup_vs_dense_kernel": round(dense_us / dec_us, 3),
            "selected_fraction": round(sel / float(lens.sum() * Hkv), 4),
            "timing": "event pair around back-to-back launches, two input replicas alternating",
        }
        del reps
        torch.cuda.empty_cache()

    # ---- the 256-step pipeline: appends, block completions, fused steps
    w = WORKLOADS["pipeline_128k"]
    log("extra: pipeline_128k")
    B, Hq, Hkv, d, dg, bs = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate,
                             w.block_size)
    dims = S.make_dims(B, Hq, Hkv, d, dg, bs, w.max_seq_len)
    scale = 1.0 / math.sqrt(d)
    inp = make_inputs(w, device=str(dev))  # the appended tokens' K/V are drawn up front
    st = S.DecodeStep(dims, mode=S.SELECT_TOPK, topk_blocks=w.topk_blocks, device=dev)
    L0 = inp["seq_lens"].clone()
    lens = [(L0 + s + 1).to(torch.int32) for s in range(w.steps)]
    runs = [st.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                         inp["w_k"], lens[s], scale, 1, False) for s in range(w.steps)]
    times = []
    for rep in range(2):  # the first pass warms up; the second is timed
        st.build_cache(inp["k"], inp["w_k"], L0)
        torch.cuda.synchronize()
        times.append(_events_us(torch, lambda i: runs[i](), w.steps))
    l0 = L0.cpu().numpy().astype(np.int64)
    completions = int(((l0 + w.steps) // bs - l0 // bs).sum())
    # algorithmic bytes of the last step (its selections are still in st)
    l_last = lens[-1].cpu().numpy().astype(np.int64)
    g_ = Hq // Hkv
    last_alg = (_selected_tokens(st, l_last, bs) * 2 * d * 2 + 2 * B * Hq * d * 2
                + B * Hkv * (st.max_selected + 1) * 4 + int((l_last // bs).sum()) * Hkv * dg * 2
                + Hkv * dg * g_ * d * 2)
    dn = _dense_buffers(S, torch, dims, dev)
    dense_last = _events_us(torch, lambda i: S.seer_dense_decode(
        dims, inp["q"], inp["k"], inp["v"], lens[-1], scale, *dn), 5)
    yield "pipeline_128k", {
        "kind": "pipeline", "workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
        "head_dim": d, "block_size": bs, "topk_blocks": w.topk_blocks, "steps": w.steps,
        "start_len": [int(l0.min()), int(l0.max())],
        "us_per_step": round(times[1], 2), "block_completions": completions,
        "step_GBps_last_step_bytes": round(last_alg / (times[1] * 1e-6) / 1e9, 1),
        "step_frac_of_peak_last_step_bytes": round(last_alg / (times[1] * 1e-6) / 1e9 / PEAK_GBPS,
                                                   4),
        "dense_us_at_last_length": round(dense_last, 2),
        "speedup_vs_dense_step": round(dense_last / times[1], 3),
        "timing": "event pair around the 256 fused steps (cache update, gate, selection, "
                  "decode), after one untimed pass from the same start",
    }
    del inp, st, runs
    torch.cuda.empty_cache()

    # ---- the benchmarked workload over a paged KV cache, and with top-p
    w = WORKLOADS["qwen3_14b_b16"]
    log("extra: paged cache and top-p on qwen3_14b_b16")
    B, Hq, Hkv, d, dg, bs = (w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.d_gate,
                             w.block_size)
    dims = S.make_dims(B, Hq, Hkv, d, dg, bs, w.max_seq_len)
    scale = 1.0 / math.sqrt(d)
    inp = make_inputs(w, device=str(dev))
    lens = inp["seq_lens"].cpu().numpy()
    st = S.DecodeStep(dims, mode=S.SELECT_TOPK, topk_blocks=w.topk_blocks, device=dev)
    st.build_cache(inp["k"], inp["w_k"], inp["seq_lens"])
    run_topk = st.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                            inp["w_k"], inp["seq_lens"], scale, 1, False)
    run_topk()
    # one page per gate block of every KV head, scattered over the pool in a
    # seeded random order
    nbm = w.max_seq_len // bs
    perm = torch.randperm(B * nbm, generator=torch.Generator().manual_seed(w.seed + 17))
    perm_d = perm.to(dev)

    def to_pool(x):
        pool = torch.empty((B * nbm, Hkv, bs, d), dtype=x.dtype, device=dev)
        pool[perm_d] = x.view(B, Hkv, nbm, bs, d).transpose(1, 2).reshape(B * nbm, Hkv, bs, d)
        return pool

    kp, vp = to_pool(inp["k"]), to_pool(inp["v"])
    table = perm.view(B, nbm).to(torch.int32).to(dev)
    dn = _dense_buffers(S, torch, dims, dev)

    def dec(i):
        S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], st.block_idx,
                             st.num_selected, st.max_selected, scale, st.num_split,
                             st.decode_ws, st.out, st.lse)

    def dec_paged(i):
        S.seer_sparse_decode_paged(dims, inp["q"], kp, vp, table, inp["seq_lens"], st.block_idx,
                                   st.num_selected, st.max_selected, scale, st.num_split,
                                   st.decode_ws, st.out, st.lse)

    def dense(i):
        S.seer_dense_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"], scale, *dn)

    def dense_paged(i):
        S.seer_dense_decode_paged(dims, inp["q"], kp, vp, table, inp["seq_lens"], scale, *dn)

    dec(0)
    ref = st.out.clone()
    dec_paged(0)
    same = bool(torch.equal(ref, st.out))
    dense(0)
    ref = dn[2].clone()
    dense_paged(0)
    same_dense = bool(torch.equal(ref, dn[2]))
    t = {f.__name__: _flushed_median_us(torch, f, 30 if f.__name__.startswith("dec") else 10,
                                        flush)
         for f in (dec, dec_paged, dense, dense_paged)}
    sel = _selected_tokens(st, lens, bs)
    blocks = int(st.num_selected.sum().item())
    qo = 2 * B * Hq * d * 2
    alg = sel * 2 * d * 2 + qo + B * Hkv * (st.max_selected + 1) * 4
    yield "qwen3_14b_b16_paged", {
        "kind": "paged", "workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
        "head_dim": d, "block_size": bs, "seq_len": int(lens[0]), "pages": B * nbm,
        "sparse_decode_us": round(t["dec"], 2), "sparse_decode_paged_us": round(t["dec_paged"], 2),
        "sparse_paged_GBps": round((alg + 4 * blocks) / (t["dec_paged"] * 1e-6) / 1e9, 1),
        "sparse_paged_frac_of_peak": round((alg + 4 * blocks) / (t["dec_paged"] * 1e-6) / 1e9
                                           / PEAK_GBPS, 4),
        "dense_decode_us": round(t["dense"], 2), "dense_decode_paged_us": round(t["dense_paged"], 2),
        "speedup_vs_dense_kernel_paged": round(t["dense_paged"] / t["dec_paged"], 3),
        "paged_equals_contiguous": same and same_dense,
        "timing": "median of per-launch event pairs, 1 GiB read before each",
    }
    del kp, vp, table, perm_d

    # top-p over the same inputs: the fused step (whose decode divides the
    # uneven selections evenly over the grid when there are fewer pairs than
    # compute units), then the standalone decode call with fixed splits and
    # with the balanced division (SEER_SPLIT_BALANCED)
    for p_mass in (0.9, 0.99):
        stp = S.DecodeStep(dims, mode=S.SELECT_TOPP, threshold=p_mass, device=dev)
        stp.build_cache(inp["k"], inp["w_k"], inp["seq_lens"])
        run = stp.bind_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                            inp["w_k"], inp["seq_lens"], scale, 1, False)
        run()

        def dec_p(i):
            S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                 stp.block_idx, stp.num_selected, stp.max_selected, scale,
                                 stp.num_split, stp.decode_ws, stp.out, stp.lse)

        def dec_bal(i):
            S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                 stp.block_idx, stp.num_selected, stp.max_selected, scale,
                                 S.SPLIT_BALANCED, stp.decode_ws, stp.out, stp.lse)

        step_us = _flushed_median_us(torch, lambda i: run(), 30, flush)
        dec_us = _flushed_median_us(torch, dec_p, 30, flush)
        bal_us = _flushed_median_us(torch, dec_bal, 30, flush)
        sel_p = _selected_tokens(stp, lens, bs)
        alg_p = sel_p * 2 * d * 2 + qo + B * Hkv * (stp.max_selected + 1) * 4
        yield f"qwen3_14b_b16_topp_{p_mass}", {
            "kind": "topp", "workload": w.name, "p": p_mass, "batch": B, "q_heads": Hq,
            "kv_heads": Hkv, "seq_len": int(lens[0]),
            "step_us": round(step_us, 2), "decode_fixed_splits_us": round(dec_us, 2),
            "decode_fixed_splits_GBps": round(alg_p / (dec_us * 1e-6) / 1e9, 1),
            "decode_fixed_splits_frac_of_peak": round(alg_p / (dec_us * 1e-6) / 1e9 / PEAK_GBPS,
                                                      4),
            "decode_balanced_us": round(bal_us, 2),
            "decode_balanced_frac_of_peak": round(alg_p / (bal_us * 1e-6) / 1e9 / PEAK_GBPS, 4),
            "selected_fraction": round(sel_p / float(lens.sum() * Hkv), 4),
            "dense_decode_us": round(t["dense"], 2),
            "speedup_vs_dense_step": round(t["dense"] / step_us, 3),
            "timing": "median of per-launch event pairs, 1 GiB read before each",
        }
        del stp
    del inp, st, run_topk, dn
    torch.cuda.empty_cache()

    if not grid:
        del flush
        return
    # ---- the pages' microbenchmark grid: kernel-level sparse vs dense
    base = WORKLOADS["qwen3_8b_layer"]
    for B in (1, 4, 16):
        for L in (8192, 32768, 131072):
            wgrid = base.replace(name="grid", batch=B, num_q_heads=64, num_kv_heads=8,
                                 seq_len=L, max_seq_len=L, seed=3000 + B + L)
            log(f"extra: grid batch {B} length {L}")
            inp = make_inputs(wgrid, device=str(dev))
            dims = S.make_dims(B, 64, 8, 128, 128, 64, L)
            nb = L // 64
            for sp in (0.5, 0.9):
                k = math.ceil((1 - sp) * nb)
                st = S.DecodeStep(dims, mode=S.SELECT_TOPK, topk_blocks=k, device=dev)
                st.build_cache(inp["k"], inp["w_k"], inp["seq_lens"])
                st.fused_step(inp["q"], inp["q"], inp["k"], inp["k"], inp["v"], inp["w_q"],
                              inp["w_k"], inp["seq_lens"], keep_logits=False)
                dn = _dense_buffers(S, torch, dims, dev)
                torch.cuda.synchronize()
                scale = 1.0 / math.sqrt(128)

                def dec(i):
                    S.seer_sparse_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                         st.block_idx, st.num_selected, st.max_selected, scale,
                                         st.num_split, st.decode_ws, st.out, st.lse)

                def dense(i):
                    S.seer_dense_decode(dims, inp["q"], inp["k"], inp["v"], inp["seq_lens"],
                                        scale, *dn)

                sp_us = _flushed_median_us(torch, dec, 30, flush)
                de_us = _flushed_median_us(torch, dense, 10, flush)
                sel = _selected_tokens(st, inp["seq_lens"].cpu().numpy(), 64)
                alg = sel * 2 * 128 * 2 + 2 * B * 64 * 128 * 2 + B * 8 * (st.max_selected + 1) * 4
                yield f"grid_b{B}_l{L}_s{sp}", {
                    "kind": "grid", "batch": B, "q_heads": 64, "kv_heads": 8, "head_dim": 128,
                    "block_size": 64, "seq_len": L, "sparsity": sp, "topk_blocks": k,
                    "sparse_decode_us": round(sp_us, 2), "dense_decode_us": round(de_us, 2),
                    "speedup_kernel": round(de_us / sp_us, 3),
                    "sparse_GBps": round(alg / (sp_us * 1e-6) / 1e9, 1),
                    "timing": "median of per-launch event pairs, 1 GiB read before each",
                }
                del st
            del inp
            torch.cuda.empty_cache()
    del flush


def extra_lines(S, torch, np, dev):
    """--extra: every extra measurement, the grid included, one JSON line each."""
    for _, obj in extra_measurements(S, torch, np, dev, grid=True):
        print(json.dumps(obj), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
