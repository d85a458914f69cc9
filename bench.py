#!/usr/bin/env python3
"""Benchmark: one step = the whole hot path on one batch of synthetic input.

Step = lp_score on the Qwen3-8B-shaped scoring batch (T = 8192 rows =
16 sequences x 512 response tokens, H = 4096, V = 151 936, bf16 inputs, fp32
accumulation, temperature 1.0) followed by lp_compare of generation (A),
the replay scores just produced (B) and trainer scores (C) over those
16 x 512 tokens. Inputs are resident in HBM before timing starts.

Prints ONE JSON line on stdout; progress goes to stderr.
    python bench.py [--steps K] [--warmup W] [--gpus 1]
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

METRIC = "scored tokens/s + % bf16 MFMA peak, H=4096 V=151936; batch-invariance bit-exact"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_qwen8b_traffic.json")
SCORE_SRC = os.path.join(ROOT, "rollout_logprob_consistency_amd", "csrc", "score.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def score_source_hash() -> str:
    return hashlib.sha256(open(SCORE_SRC, "rb").read()).hexdigest()


def measured_traffic():
    """Per-launch HBM bytes from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("score_hip_sha256") != score_source_hash():
        return None
    return t.get("bytes_per_launch")


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The clock settles over the first ~6 calls (traced: 8.3, 8.2, 7.5, 7.0, 6.9, 6.8 ms, then
    # 6.7): ten untimed calls keep that ramp out of the timed steps.
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="rows of the batch the fp64 oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-qwen17b", action="store_true",
                    help="skip the Qwen3-1.7B-shaped (H=2048) scoring record")
    ap.add_argument("--sweep-n", type=str, default="512,4096,32768",
                    help="sequence counts of the comparison bandwidth probe (L = 2304); the "
                         "tail statistics and the correction are timed at N = 4096 when listed")
    ap.add_argument("--compare-n", type=int, default=4096,
                    help="sequences (L = 2304) of the compare / tails / quantiles profiler modes")
    ap.add_argument("--small-batches", type=str, default="1,7,64",
                    help="row counts at which lp_score is timed as a stream over W")
    ap.add_argument("--mode", choices=("bench", "score", "stats", "small", "compare", "tails",
                                       "quantiles", "copy"),
                    default="bench",
                    help="score: only `steps` lp_score calls on the benchmark batch; stats: "
                         "the same with lp_score_stats (entropy and argmax too); small: "
                         "`steps` lp_score calls on its first row; compare: `steps` lp_compare "
                         "calls at N=--compare-n, L=2304; tails / quantiles: `steps` lp_compare_tails / "
                         "lp_compare_quantiles calls on the same arrays (these for profilers); "
                         "copy: one plain "
                         "1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scoring path has no cross-GPU "
              "exchange, and the library and its benchmark run on a single MI355X "
              "(use --gpus 1).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import rollout_logprob_consistency_amd as lp
    from workloads import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, H, V, NSEQ, LSEQ = 8192, 4096, 151936, 16, 512

    if args.mode == "copy":
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(7)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copied 1 GiB device to device")
        return 0

    t0 = time.time()
    log("bench: generating Qwen3-8B-shaped inputs (seeded, host) ...")
    w_bits = synth.qwen_weight(H, V)
    case = synth.qwen_case(T=T, H=H, V=V, w_bits=w_bits)
    log(f"bench: inputs ready in {time.time() - t0:.1f} s; uploading")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    x, w = bf16(case.x_bits), bf16(w_bits)
    ids = torch.from_numpy(case.ids).to(dev)
    out = torch.empty(T, dtype=torch.float32, device=dev)
    ws = torch.empty(lp.score_workspace_bytes(T, H, V), dtype=torch.uint8, device=dev)

    # Comparison inputs: trainer C = a replay of the same rows (bitwise equal
    # when the scorer is deterministic), generation A = C + N(0, 1e-3).
    lp.score(x, w, ids, out=out, workspace=ws, check=True)
    torch.cuda.synchronize()
    C = out.view(NSEQ, LSEQ).clone()
    gen = torch.Generator(device=dev).manual_seed(synth.BASE_SEED)
    A = (C.double() + 1e-3 * torch.randn(C.shape, generator=gen, device=dev,
                                          dtype=torch.float64)).float()
    mask = torch.ones((NSEQ, LSEQ), dtype=torch.uint8, device=dev)
    B = out.view(NSEQ, LSEQ)
    stats_buf = torch.empty(3 * NSEQ * lp.SEQ_STATS_DTYPE.itemsize, dtype=torch.uint8, device=dev)

    if args.mode == "score":
        for _ in range(args.steps):
            lp.score(x, w, ids, out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"bench: {args.steps} lp_score calls done")
        return 0
    ent = torch.empty(T, dtype=torch.float32, device=dev)
    amax = torch.empty(T, dtype=torch.int64, device=dev)
    ws_stats = torch.empty(lp.score_stats_workspace_bytes(T, H, V), dtype=torch.uint8, device=dev)
    out_stats = torch.empty(T, dtype=torch.float32, device=dev)
    stats_args = (x.data_ptr(), H, w.data_ptr(), ids.data_ptr(), T, H, V, V, 1.0,
                  out_stats.data_ptr(), None, ent.data_ptr(), amax.data_ptr(), None,
                  ws_stats.data_ptr(), ws_stats.numel(), torch.cuda.current_stream().cuda_stream)
    c_stats = lp._lib.lib().lp_score_stats

    def score_stats_call():
        st_ = c_stats(*stats_args)
        if st_ != 0:
            raise lp.LpError(st_, "lp_score_stats")

    if args.mode == "stats":
        for _ in range(args.steps):
            score_stats_call()
        torch.cuda.synchronize()
        log(f"bench: {args.steps} lp_score_stats calls done")
        return 0
    if args.mode == "small":
        for _ in range(args.steps):
            lp.score(x[:1], w, ids[:1], out=out[:1], workspace=ws)
        torch.cuda.synchronize()
        log(f"bench: {args.steps} one-row lp_score calls done")
        return 0
    if args.mode in ("compare", "tails", "quantiles"):
        sc = synth.compare_sweep_case(N=args.compare_n)
        tA, tB, tC, tM = (torch.from_numpy(a).to(dev) for a in (sc.A, sc.B, sc.C, sc.mask))
        if args.mode == "compare":
            sbuf = torch.empty(3 * sc.N * lp.SEQ_STATS_DTYPE.itemsize, dtype=torch.uint8,
                               device=dev)
            for _ in range(args.steps):
                lp.compare_raw(tA, tB, tC, tM, out=sbuf)
        elif args.mode == "tails":
            for _ in range(args.steps):
                lp.compare_tails(tA, tB, tC, tM, positions=True)
        else:
            qout = torch.empty((sc.N, 3, 3), dtype=torch.float64, device=dev)
            for _ in range(args.steps):
                lp.compare_quantiles(tA, tB, tC, tM, out=qout, sync=False)
        torch.cuda.synchronize()
        log(f"bench: {args.steps} {args.mode} calls (N={sc.N}, L={sc.L}) done")
        return 0

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        lp.score(x, w, ids, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()
        lp.compare_raw(A, B, C, mask, out=stats_buf)
        if ev is not None:
            ev[2].record()

    log(f"bench: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    score_ms = [e[0].elapsed_time(e[1]) for e in events]
    cmp_ms = [e[1].elapsed_time(e[2]) for e in events]
    score_avg = float(np.mean(score_ms)) / 1e3
    cmp_avg = float(np.mean(cmp_ms)) / 1e3

    st = lp.stats_from_bytes(stats_buf, NSEQ)
    assert (st["BC"]["mismatch"] == 0).all(), "replay differs from an identical earlier scoring"

    flops = 2.0 * T * H * V
    achieved = flops / score_avg / 1e12
    log(f"bench: lp_score {score_avg * 1e3:.3f} ms avg (min {min(score_ms):.3f}, max "
        f"{max(score_ms):.3f}) = {achieved:.1f} TFLOP/s = {100 * achieved / PEAK_BF16_TFLOPS:.1f}% "
        f"of bf16 peak; lp_compare {cmp_avg * 1e6:.1f} us")

    def median_us(fn, calls=20, reps=7):
        """Per-call duration of fn() in microseconds: `calls` back-to-back
        calls between two HIP events on the current stream, repeated `reps`
        times; returns the median, min and max of the per-call averages (3
        untimed calls first). Back-to-back calls keep short kernels from being
        timed together with the host's launch gaps."""
        for _ in range(3):
            fn()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in evs:
            e[0].record()
            for _ in range(calls):
                fn()
            e[1].record()
        torch.cuda.synchronize()
        t = sorted(e[0].elapsed_time(e[1]) * 1e3 / calls for e in evs)
        return t[len(t) // 2], t[0], t[-1]

    # The same scoring with the row entropy and argmax (lp_score_stats).
    st_med, st_lo, st_hi = median_us(score_stats_call, calls=3, reps=5)
    score_stats_call()
    torch.cuda.synchronize()
    assert torch.equal(out_stats.view(torch.int32), out.view(torch.int32)), \
        "lp_score_stats logprob bits differ from lp_score"
    stats_rec = {"ms": round(st_med / 1e3, 4), "min_ms": round(st_lo / 1e3, 4),
                 "max_ms": round(st_hi / 1e3, 4),
                 "TFLOPs": round(flops / st_med / 1e6, 2),
                 "frac": round(flops / st_med / 1e6 / PEAK_BF16_TFLOPS, 4)}
    log(f"bench: lp_score_stats {st_med / 1e3:.3f} ms = {flops / st_med / 1e6:.1f} TFLOP/s")

    # The bf16-logit mode (lp_score_ex): one conversion per logit in the epilogue.
    out_bf = torch.empty(T, dtype=torch.float32, device=dev)
    c_ex = lp._lib.lib().lp_score_ex
    ex_args = (x.data_ptr(), H, w.data_ptr(), ids.data_ptr(), T, H, V, V, 1.0,
               lp.SCORE_BF16_LOGITS, out_bf.data_ptr(), None, None, None, None, ws.data_ptr(),
               ws.numel(), torch.cuda.current_stream().cuda_stream)

    def score_bf16_call():
        st_ = c_ex(*ex_args)
        if st_ != lp.LP_OK:
            raise lp.LpError(st_, "lp_score_ex")

    bf_med, bf_lo, bf_hi = median_us(score_bf16_call, calls=3, reps=5)
    bf16_rec = {"ms": round(bf_med / 1e3, 4), "min_ms": round(bf_lo / 1e3, 4),
                "max_ms": round(bf_hi / 1e3, 4),
                "TFLOPs": round(flops / bf_med / 1e6, 2),
                "frac": round(flops / bf_med / 1e6 / PEAK_BF16_TFLOPS, 4)}
    log(f"bench: lp_score_ex bf16 logits {bf_med / 1e3:.3f} ms = {flops / bf_med / 1e6:.1f} TFLOP/s")

    # Vocabulary-parallel scoring at its per-GPU shape: rank 0 of 8 canonical
    # shards scores its rows of W; the merge folds the 16 gathered segment
    # records. All 8 shards, scored here one after another into one exchange
    # buffer, must merge to lp_score's bits.
    n_sh = 8
    parts = lp.shard_partials(T, False, dev)
    shards = []
    for r in range(n_sh):
        sh = lp.vocab_shard(V, n_sh, r)
        rows = sh["row_end"] - sh["row_begin"]
        wsh = torch.empty(lp._lib.lib().lp_score_shard_workspace_bytes(T, V, n_sh, r, 0),
                          dtype=torch.uint8, device=dev)
        shards.append((r, rows, w[sh["row_begin"]:sh["row_end"]], wsh))

    def shard_call(k):
        r, _, w_own, wsh = shards[k]
        lp.score_shard(x, w_own, ids, V, n_sh, r, parts, workspace=wsh)

    for k in range(n_sh):
        shard_call(k)
    merged = lp.merge_shards(parts, ids, V)
    torch.cuda.synchronize()
    assert torch.equal(merged.view(torch.int32), out.view(torch.int32)), \
        "merged vocabulary shards differ from lp_score"
    sh_med, sh_lo, sh_hi = median_us(lambda: shard_call(0), calls=5, reps=5)
    all_med, _, _ = median_us(lambda: [shard_call(k) for k in range(n_sh)], calls=2, reps=3)
    mg_med, _, _ = median_us(lambda: lp.merge_shards(parts, ids, V))
    sh_flops = 2.0 * T * H * shards[0][1]
    shard_rec = {"shards": n_sh, "rank": 0, "rows": shards[0][1],
                 "ms": round(sh_med / 1e3, 4), "min_ms": round(sh_lo / 1e3, 4),
                 "max_ms": round(sh_hi / 1e3, 4),
                 "TFLOPs": round(sh_flops / sh_med / 1e6, 2),
                 "frac": round(sh_flops / sh_med / 1e6 / PEAK_BF16_TFLOPS, 4),
                 "all_shards_one_gpu_ms": round(all_med / 1e3, 4),
                 "merge_us": round(mg_med, 2),
                 "exchange_bytes_per_row_per_rank": 16 * 3 * 4 // n_sh,
                 "bitwise_equal_lp_score": True}
    log(f"bench: vocab shard 0/{n_sh} ({shards[0][1]} rows) {sh_med / 1e3:.3f} ms = "
        f"{sh_flops / sh_med / 1e6:.1f} TFLOP/s; all {n_sh} shards {all_med / 1e3:.3f} ms; "
        f"merge {mg_med:.1f} us; bitwise equal to lp_score")
    del parts, shards

    # Qwen3-1.7B-shaped scoring: T = 4096 (8 x 512), H = 2048, V = 151 936, at
    # temperatures 1.0 and 0.7; fp64 oracle parity on every row (outside the
    # timed region, the logits formed once per 512-row block for both
    # temperatures).
    q17 = None
    if not args.no_qwen17b:
        T2, H2 = 4096, 2048
        w2_bits = synth.qwen_weight(H2, V)
        c2 = synth.qwen_case(T=T2, H=H2, V=V, w_bits=w2_bits)
        x2, w2 = bf16(c2.x_bits), bf16(w2_bits)
        ids2 = torch.from_numpy(c2.ids).to(dev)
        ws2 = torch.empty(lp.score_workspace_bytes(T2, H2, V), dtype=torch.uint8, device=dev)
        flops2 = 2.0 * T2 * H2 * V
        q17 = {"T": T2, "H": H2, "V": V, "runs": []}
        outs2 = {}
        for temp in (1.0, 0.7):
            o2 = torch.empty(T2, dtype=torch.float32, device=dev)
            med, lo, hi = median_us(lambda: lp.score(x2, w2, ids2, temp, out=o2, workspace=ws2),
                                    calls=5, reps=5)
            torch.cuda.synchronize()
            outs2[temp] = o2.cpu().numpy().astype(np.float64)
            q17["runs"].append({"temperature": temp, "ms": round(med / 1e3, 4),
                                "min_ms": round(lo / 1e3, 4), "max_ms": round(hi / 1e3, 4),
                                "tokens_per_s": round(T2 / (med / 1e6), 1),
                                "TFLOPs": round(flops2 / med / 1e6, 2),
                                "frac": round(flops2 / med / 1e6 / PEAK_BF16_TFLOPS, 4)})
            log(f"bench: Qwen3-1.7B shape T={T2} H={H2} temperature {temp}: {med / 1e3:.3f} ms = "
                f"{flops2 / med / 1e6:.1f} TFLOP/s")
        if not args.no_cpu_baseline:
            import oracle
            errs = {t: 0.0 for t in outs2}
            for r0 in range(0, T2, 512):
                z = oracle.logits(c2.x_bits[r0:r0 + 512], w2_bits)
                for temp in outs2:
                    ref2, _ = oracle.log_softmax_at(z, c2.ids[r0:r0 + 512], temp)
                    errs[temp] = max(errs[temp],
                                     float(np.max(np.abs(outs2[temp][r0:r0 + 512] - ref2))))
                del z
            for run in q17["runs"]:
                e = errs[run["temperature"]]
                run["parity"] = {"rows": T2, "max_abs_diff_nats": e, "within_tolerance": e <= 1e-3}
                log(f"bench: Qwen3-1.7B shape temperature {run['temperature']}: max |lp_score - "
                    f"fp64 oracle| over {T2} rows = {e:.3e} nats")
                assert e <= 1e-3, "Qwen3-1.7B-shaped parity outside 1e-3 nats"
        del x2, w2, ids2, ws2

    # Small batches: the product is a stream over W (HBM-bound); report the
    # algorithmic bytes (W, the rows, ids and outputs) per second.
    small = []
    for b in (int(v) for v in args.small_batches.split(",") if v):
        xs, ids_s = x[:b].contiguous(), ids[:b].contiguous()
        out_s = torch.empty(b, dtype=torch.float32, device=dev)
        ws_s = torch.empty(lp.score_workspace_bytes(b, H, V), dtype=torch.uint8, device=dev)
        med, lo, hi = median_us(lambda: lp.score(xs, w, ids_s, out=out_s, workspace=ws_s))
        nbytes = 2.0 * V * H + 2.0 * b * H + 16.0 * b
        small.append({"rows": b, "us": round(med, 2), "min_us": round(lo, 2), "max_us": round(hi, 2),
                      "GBps": round(nbytes / med / 1e3, 1),
                      "frac_hbm": round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4)})
        log(f"bench: lp_score {b} rows: {med:.1f} us = {nbytes / med / 1e3:.1f} GB/s")

    # Comparison bandwidth probe at sizes that are not launch-latency bound.
    sweep = []
    tails_rec = None
    corr_rec = None
    for n_seq in (int(v) for v in args.sweep_n.split(",") if v):
        sc = synth.compare_sweep_case(N=n_seq)
        tA, tB, tC, tM = (torch.from_numpy(a).to(dev) for a in (sc.A, sc.B, sc.C, sc.mask))
        sbuf = torch.empty(3 * sc.N * lp.SEQ_STATS_DTYPE.itemsize, dtype=torch.uint8, device=dev)
        lp.compare_raw(tA, tB, tC, tM, out=sbuf)  # argument checks once, then the bare C call
        cargs = (tA.data_ptr(), tB.data_ptr(), tC.data_ptr(), tM.data_ptr(), sc.N, sc.L, sc.L,
                 2.0, -1.0, sbuf.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
        c_compare = lp._lib.lib().lp_compare
        med, lo, hi = median_us(lambda: c_compare(*cargs))
        nbytes = 13.0 * sc.N * sc.L
        sweep.append({"N": sc.N, "L": sc.L, "us": round(med, 2), "min_us": round(lo, 2),
                      "max_us": round(hi, 2), "GBps": round(nbytes / med / 1e3, 1),
                      "frac_hbm": round(nbytes / med / 1e3 / PEAK_HBM_GBPS, 4),
                      "bytes_per_token": 13})
        log(f"bench: lp_compare N={sc.N} L={sc.L}: {med:.1f} us = {nbytes / med / 1e3:.1f} GB/s")
        if sc.N == 4096:
            # Batch tail statistics on the same arrays: selection passes 0
            # and 1 and the position profile each read the 13 bytes of every
            # position; the later passes read only the candidate lists.
            tw = torch.empty(lp._lib.lib().lp_compare_tails_workspace_bytes(sc.N, sc.L),
                             dtype=torch.uint8, device=dev)
            tout = torch.empty(3 * lp.TAIL_STATS_DTYPE.itemsize, dtype=torch.uint8, device=dev)
            tps = torch.empty((3, sc.L), dtype=torch.float64, device=dev)
            tpc = torch.empty((3, sc.L), dtype=torch.int32, device=dev)
            targs = (tA.data_ptr(), tB.data_ptr(), tC.data_ptr(), tM.data_ptr(), sc.N, sc.L,
                     sc.L, tout.data_ptr(), tps.data_ptr(), tpc.data_ptr(), tw.data_ptr(),
                     tw.numel(), torch.cuda.current_stream().cuda_stream)
            c_tails = lp._lib.lib().lp_compare_tails
            tmed, tlo, thi = median_us(lambda: c_tails(*targs), calls=5, reps=5)
            tbytes = 3 * 13.0 * sc.N * sc.L
            tails_rec = {"N": sc.N, "L": sc.L, "us": round(tmed, 2), "min_us": round(tlo, 2),
                         "max_us": round(thi, 2), "passes": 3,
                         "GBps": round(tbytes / tmed / 1e3, 1),
                         "frac_hbm": round(tbytes / tmed / 1e3 / PEAK_HBM_GBPS, 4)}
            log(f"bench: lp_compare_tails N={sc.N} L={sc.L}: {tmed:.1f} us "
                f"({tbytes / tmed / 1e3:.1f} GB/s over 3 reads of the batch)")
            # The same call with the 16 worst tokens of each pair
            # (lp_compare_tails_ex): a fourth selection target per pair, a
            # counting pass, a writing pass and a 16-row sort.
            kw = 16
            tw2 = torch.empty(lp._lib.lib().lp_compare_tails_ex_workspace_bytes(sc.N, sc.L, kw),
                              dtype=torch.uint8, device=dev)
            twr = torch.empty(3 * kw * lp.WORST_DTYPE.itemsize, dtype=torch.uint8, device=dev)
            targs2 = (tA.data_ptr(), tB.data_ptr(), tC.data_ptr(), tM.data_ptr(), sc.N, sc.L,
                      sc.L, kw, tout.data_ptr(), twr.data_ptr(), tps.data_ptr(), tpc.data_ptr(),
                      tw2.data_ptr(), tw2.numel(), torch.cuda.current_stream().cuda_stream)
            c_tails_ex = lp._lib.lib().lp_compare_tails_ex
            wmed, _, _ = median_us(lambda: c_tails_ex(*targs2), calls=5, reps=5)
            tails_rec["worst_k"] = kw
            tails_rec["with_worst_us"] = round(wmed, 2)
            log(f"bench: lp_compare_tails_ex (16 worst tokens per pair): {wmed:.1f} us")
            # Per-sequence p50 / p95 / p99 (lp_compare_quantiles): one read of
            # the 13 bytes of every position, selection in LDS.
            qout = torch.empty((sc.N, 3, 3), dtype=torch.float64, device=dev)
            qargs = (tA.data_ptr(), tB.data_ptr(), tC.data_ptr(), tM.data_ptr(), sc.N, sc.L,
                     sc.L, qout.data_ptr(), torch.cuda.current_stream().cuda_stream)
            c_quant = lp._lib.lib().lp_compare_quantiles
            qmed, qlo, qhi = median_us(lambda: c_quant(*qargs), calls=5, reps=5)
            qbytes = 13.0 * sc.N * sc.L
            tails_rec["seq_quantiles_us"] = round(qmed, 2)
            tails_rec["seq_quantiles_GBps"] = round(qbytes / qmed / 1e3, 1)
            log(f"bench: lp_compare_quantiles N={sc.N} L={sc.L}: {qmed:.1f} us "
                f"({qbytes / qmed / 1e3:.1f} GB/s over one read)")
            del qout
            # Correction consumer on the same arrays: rollout = A, trainer = C;
            # TIS cap, MIS interval and K3 rejection, weights written. Bytes:
            # 2 x fp32 + mask read, fp32 weight written per position.
            cw = torch.empty((sc.N, sc.L), dtype=torch.float32, device=dev)
            cout = torch.empty(sc.N * lp.CORR_SEQ_DTYPE.itemsize, dtype=torch.uint8, device=dev)
            cargs2 = (tA.data_ptr(), tC.data_ptr(), tM.data_ptr(), sc.N, sc.L, sc.L, 1.001,
                      -0.003, 0.003, lp.REJECT_K3, float("-inf"), 2e-4, cw.data_ptr(),
                      cout.data_ptr(), torch.cuda.current_stream().cuda_stream)
            c_corr = lp._lib.lib().lp_correct
            cmed, clo, chi = median_us(lambda: c_corr(*cargs2))
            cbytes = 13.0 * sc.N * sc.L
            corr_rec = {"N": sc.N, "L": sc.L, "us": round(cmed, 2), "min_us": round(clo, 2),
                        "max_us": round(chi, 2), "bytes_per_token": 13,
                        "GBps": round(cbytes / cmed / 1e3, 1),
                        "frac_hbm": round(cbytes / cmed / 1e3 / PEAK_HBM_GBPS, 4)}
            log(f"bench: lp_correct N={sc.N} L={sc.L}: {cmed:.1f} us = "
                f"{cbytes / cmed / 1e3:.1f} GB/s")
            del cw, cout
        del tA, tB, tC, tM

    # Batch invariance at the headline shape (outside the timed region): the
    # first 64 rows of the batch scored alone (the streaming kernel), each at
    # a random position of a 7-row batch of other rows, and inside the whole
    # batch rolled by 1000 rows (the tile kernel, other tile slots); every
    # result must equal the timed run's bits.
    n_probe = 64
    ref_bits = out[:n_probe].clone().view(torch.int32)
    alone = lp.score(x[:n_probe], w, ids[:n_probe])
    rng = np.random.default_rng(synth.BASE_SEED)
    in7 = torch.empty(n_probe, dtype=torch.float32, device=dev)
    for j in range(n_probe):
        rows = torch.from_numpy(rng.choice(np.arange(n_probe, T), 7, replace=False)).to(dev)
        slot = int(rng.integers(7))
        rows[slot] = j
        in7[j] = lp.score(x[rows], w, ids[rows])[slot]
    rolled = lp.score(torch.roll(x, 1000, 0), w, torch.roll(ids, 1000, 0))[1000:1000 + n_probe]
    torch.cuda.synchronize()
    inv_ok = all(torch.equal(t.view(torch.int32), ref_bits) for t in (alone, in7, rolled))
    assert inv_ok, "batch invariance broken at the headline shape"
    invariance = {"probe_rows": n_probe, "batches": [n_probe, 7, T], "bitwise_equal": inv_ok}
    log(f"bench: batch invariance (64 probe rows alone, in 7-row batches, rolled in {T}): "
        f"{'bitwise equal' if inv_ok else 'DIFFERENT'}")

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        n = min(args.cpu_rows, T)
        log(f"bench: timing the fp64 oracle on {n} rows ...")
        tc = time.perf_counter()
        ref_lp, _ = oracle.score(case.x_bits[:n], w_bits, case.ids[:n], 1.0)
        dt = time.perf_counter() - tc
        # The same rows of the timed run against the fp64 oracle (the
        # tolerance is 1e-3 nats).
        err = float(np.max(np.abs(out[:n].double().cpu().numpy() - ref_lp)))
        parity = {"rows": n, "max_abs_diff_nats": err, "tolerance_nats": 1e-3,
                  "within_tolerance": err <= 1e-3}
        log(f"bench: max |lp_score - fp64 oracle| over {n} rows = {err:.3e} nats")
        cpu = {"value": round(n / dt, 3), "unit": "tokens/s", "cores": blas_threads(),
               "kind": "oracle",
               "sample": f"first {n} of the {T} rows (H={H}, V={V}), fp64 numpy/OpenBLAS, "
                         f"{dt:.1f} s"}
        log(f"bench: oracle {n / dt:.2f} tokens/s ({dt:.1f} s, {cpu['cores']} threads)")

    traffic = measured_traffic()
    rec = {
        "metric": METRIC,
        "value": round(T * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3-8B-shaped selected-token logprob T=8192 (16x512) "
                               "H=4096 V=151936 temperature 1.0, then three-way compare "
                               "of the 16x512 scores",
                   "T": T, "H": H, "V": V, "temperature": 1.0, "accumulate": "fp32",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "parity": parity,
        "batch_invariance": invariance,
        "kernels": {"lp_score_ms": round(score_avg * 1e3, 4),
                    "lp_score_ms_median": round(float(np.median(score_ms)), 4),
                    "lp_score_ms_min": round(min(score_ms), 4),
                    "lp_score_ms_max": round(max(score_ms), 4),
                    "lp_compare_us": round(cmp_avg * 1e6, 2)},
        "score_stats": stats_rec,
        "score_bf16_logits": bf16_rec,
        "vocab_parallel": shard_rec,
        "qwen3_1_7b_shape": q17,
        "small_batch": small,
        "compare_sweep": sweep,
        "compare_tails": tails_rec,
        "correct": corr_rec,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
