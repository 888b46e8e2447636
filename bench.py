#!/usr/bin/env python3
"""Benchmark of the packed lookahead + verification round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full round (pool lookup, row manifest, target forward over the
packed rows, LM head on the required rows, verification, K/V commit, pool
upsert, window advance) through the C ABI's la_step.  Default workload: a
Llama-2-7B-shaped random-init bf16 decoder (32 layers, d 4096, 32 heads,
MLP 11008, vocab 32000), 512-token prompt from the seeded order-2 Markov
chain, greedy lookahead with W=7, N=5, G=7, 256 new tokens.  Weights and
prompt are resident in HBM before timing; prefill is outside the timed
region.  value = emitted tokens / wall time of the K timed rounds.

Also reported on the same line:
  * roofline: the dominant kernel of the step (the batch-invariant GEMM that
    streams the weights), algorithmic bytes per launch over its average
    launch time from HIP events on the library's stream;
  * lookahead_attn: the isolated lookahead-mask attention op (bf16, 32 heads
    x 128, committed prefix 1024, 121 query rows: W=15, N=5, G=15 with the
    rectangular window), timed with HIP events over rotating input sets that
    exceed the 256 MB Infinity Cache;
  * lookahead_attn_8192: the same op over 8192 committed keys (the
    long-prefix workload's per-layer shape, 134 MB of K/V per call);
  * lookahead_attn_34b_gqa: the op at the 34B-shaped round's per-layer shape
    (64 query heads on 8 KV heads, N=7: 180 rows, 2048 committed keys);
  * step_roofline: the round against the HBM bound (streamed weight bytes
    plus the committed K/V read at the mean committed length, over 8 TB/s);
  * init_prefill_ms: context set-up and prompt prefill (wall clock, untimed
    in value);
  * ar_tokens_per_s: plain autoregressive decoding with the same kernels;
  * cpu_baseline: the CPU oracle on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "accepted tokens/sec per sequence + lookahead-attn HBM GB/s (% of peak), 1 GPU"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    "llama7b_w7n5g7": dict(model="llama7b", W=7, N=5, G=7, prompt=512, max_new=256, desc=(
        "Llama-2-7B-shaped bf16 decoder, 512-token Markov prompt, greedy lookahead W=7 N=5 G=7, 256 new tokens")),
    "llama7b_long_w15n5g15": dict(model="llama7b", W=15, N=5, G=15, prompt=8192, max_new=256, desc=(
        "Llama-2-7B-shaped bf16 decoder, 8192-token Markov prompt, greedy lookahead W=15 N=5 G=15")),
    "codellama34b_w15n7g15": dict(model="codellama34b", W=15, N=7, G=15, prompt=2048, max_new=256, copyspan=True, desc=(
        "CodeLlama-34B-shaped bf16 decoder (GQA 64/8 heads), 2048-token Markov prompt with 30% copied spans, "
        "greedy lookahead W=15 N=7 G=15, 256 new tokens")),
    "tiny_w5n3g5": dict(model="tiny", W=5, N=3, G=5, prompt=32, max_new=64, desc=(
        "tiny fp32 decoder (2 layers, d 64), 32-token Markov prompt, greedy lookahead W=5 N=3 G=5, 64 new tokens")),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_roofline(model, dims, wl, tokens, steps, secs):
    """The round against the HBM bound: every streamed weight byte (all layers
    and the LM head; the embedding is gathered, not streamed) plus the committed
    K/V the attention reads, at the mean committed length of the timed rounds
    (prompt + half the tokens they emitted), over 8 TB/s."""
    streamed = model.weight_bytes - model.embed.numel() * model.embed.element_size()
    esize = 2 if dims.dtype == "bf16" else 4
    kv = 2 * dims.n_layers * dims.n_kv_heads * dims.head_dim * esize * (wl["prompt"] + tokens / 2)
    at_peak_ms = (streamed + kv) / (HBM_PEAK_GBS * 1e9) * 1e3
    ms = secs * 1e3 / steps
    return {"bytes_per_round": streamed + kv, "weight_bytes": streamed, "kv_bytes": kv,
            "ms_at_peak": at_peak_ms, "ms_per_round": ms, "frac": at_peak_ms / ms}


def run_steps(make_session, sess, steps):
    """Time exactly `steps` rounds (steps > 0; a finished generation is restarted
    outside the clock) or, for steps == 0, every round of one fresh generation."""
    import torch
    tokens = 0
    elapsed = 0.0
    done = 0
    if steps == 0:
        sess = make_session()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while True:
            out = sess.la_step()
            if not out:
                break
            tokens += len(out)
            done += 1
        torch.cuda.synchronize()
        return tokens, time.perf_counter() - t0, sess, done
    while done < steps:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n_here = 0
        while done < steps:
            out = sess.la_step()
            if not out:
                break
            tokens += len(out)
            done += 1
            n_here += 1
        torch.cuda.synchronize()
        elapsed += time.perf_counter() - t0
        if done < steps:
            sess = make_session()
    return tokens, elapsed, sess, done


def attention_op(reps=200, sets=16, p=1024, H=32, Hkv=32, N=5):
    """Isolated lookahead-mask attention (W=15, G=15, bf16, head dim 128) over a committed prefix
    of p keys, rotating input sets (more bytes than the 256 MB Infinity Cache).  N=5, 32 heads:
    the rectangular window of the config, 121 rows; N=7 with 64 query heads on 8 KV heads: the
    34B-shaped round's pinned layout ([14, 15, 15, 15, 15, 15] + 15 x 6 candidate rows = 180)."""
    import numpy as np
    import torch
    import exact_lookahead_decoding_amd.la as la
    dh, S, R = 128, N - 1, N - 1
    if N == 5:
        levels, starts = [list(range(100, 115))] * 4, [1, 1, 1, 1]
    else:
        levels, starts = [list(range(100, 114))] + [list(range(100, 115))] * (R - 1), [1] + [0] * (R - 1)
    desc = la.rows_desc(p, levels, S, 15, 7, 16, starts=starts)
    win = torch.zeros((R, 16), dtype=torch.int32, device="cuda")
    win[:, :15] = torch.arange(100, 115, dtype=torch.int32, device="cuda")
    cand = torch.arange(15 * S, dtype=torch.int32, device="cuda")
    rows, info = la.la_build_rows(desc, win, cand)
    Q = info.Q
    g = torch.Generator(device="cuda").manual_seed(0)
    mk = lambda *s: torch.randn(*s, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    bufs = [(mk(Q, H, dh), mk(Hkv, p + 8, dh), mk(Hkv, p + 8, dh), mk(Hkv, Q, dh), mk(Hkv, Q, dh))
            for _ in range(sets)]
    ws = torch.empty(la.load().la_attention_workspace(Q, H, dh, p + 1 + info.maxp, p + 8), dtype=torch.uint8,
                     device="cuda")
    outs = [torch.empty(Q, H, dh, dtype=torch.bfloat16, device="cuda") for _ in range(sets)]
    for i in range(sets):
        la.la_attention(*bufs[i], rows, info, p + 1, out=outs[i], workspace=ws)
    torch.cuda.synchronize()
    # one HIP graph holds a launch per rotating input set, so that host-side
    # launch overhead stays out of the event-timed region
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(sets):
            la.la_attention(*bufs[i], rows, info, p + 1, out=outs[i], workspace=ws)
    graph.replay()
    torch.cuda.synchronize()
    n_rep = max(1, reps // sets)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_rep)]
    for r in range(n_rep):
        ev[r][0].record()
        graph.replay()
        ev[r][1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev])) / sets
    reps = n_rep * sets
    alg = 2 * Hkv * p * dh * 2 + Q * Hkv * dh * 2 * 2 + 2 * Q * H * dh * 2
    gbs = alg / (ms * 1e-3) / 1e9
    kv_gbs = (2 * Hkv * p * dh * 2) / (ms * 1e-3) / 1e9
    heads = f"{H} heads" if H == Hkv else f"{H} query heads on {Hkv} KV heads"
    return {"workload": f"lookahead-mask attention, bf16, {heads} x 128, prefix {p}, {Q} rows (W=15 N={N} G=15)",
            "avg_us": ms * 1e3, "algorithmic_bytes": alg, "achieved_GBps": gbs, "kv_stream_GBps": kv_gbs,
            "peak_GBps": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS, "reps": reps, "input_sets": sets}


TRAFFIC_MD = os.path.join(ROOT, "profiles", "la_gemm_kernel_llama7b_w7n5g7_hbm_traffic.md")
GEMM_SRC = os.path.join(ROOT, "exact_lookahead_decoding_amd", "csrc", "la_gemm.hip")
COPY_BYTES = 1 << 30


def _sha256(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def gemm_traffic():
    """HBM bytes per round GEMM launch from the committed counter summary, or
    None when the GEMM source changed since the counters were taken."""
    try:
        txt = open(TRAFFIC_MD).read()
    except OSError:
        return None
    vals = dict(l.split(":", 1) for l in txt.splitlines() if l.startswith(("traffic_bytes_per_launch:",
                                                                               "la_gemm.hip sha256:")))
    if vals.get("la_gemm.hip sha256", "").strip() != _sha256(GEMM_SRC):
        return None
    return float(vals["traffic_bytes_per_launch"])


def pmc_sample(rounds=16):
    """The workload rounds whose GEMM dispatches the counter runs read, then a
    plain copy of COPY_BYTES that calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch
    import synthetic
    import exact_lookahead_decoding_amd.la as la
    la.load()
    torch.cuda.set_device(0)
    wl = WORKLOADS["llama7b_w7n5g7"]
    dims = synthetic.PRESETS[wl["model"]]
    model = la.DeviceModel(dims, seed=0)
    prompt = synthetic.markov_prompt(dims.vocab, wl["prompt"], 0)
    sess = la.Session(model, prompt, W=wl["W"], N=wl["N"], G=wl["G"], max_new=wl["max_new"])
    sess.la_profile(True)
    for _ in range(rounds):
        sess.la_step()
    torch.cuda.synchronize()
    pr = sess.la_profile_read()
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"rounds": rounds, "gemm_launches": pr["gemm_launches"],
                      "gemm_alg_bytes_per_launch": pr["gemm_bytes"] / max(1, pr["gemm_launches"]),
                      "copy_bytes": COPY_BYTES}), flush=True)


def pmc_summary(fetch_db, write_db, sample_json):
    """Per-launch HBM traffic of the round GEMMs (la_gemm_kernel with at most 4
    row tiles: the prefill chunks use 8) from a FETCH_SIZE and a WRITE_SIZE
    run of --pmc-sample, each scaled by what the counter reads for the copy."""
    import collections
    import re
    import sqlite3

    def per_dispatch(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select dispatch_id, kernel_name, value from counters_collection where counter_name = ?",
                           (counter,)).fetchall()
        agg = collections.defaultdict(float)
        names = {}
        for d, k, v in rows:
            agg[d] += v
            names[d] = k
        return agg, names

    out = {}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        agg, names = per_dispatch(db, counter)
        gemm = [agg[d] for d, k in names.items()
                if (m := re.search(r"la_gemm_kernel<[^,]+, (\d+),", k)) and int(m.group(1)) <= 4]
        copy = [agg[d] for d, k in names.items() if "copy" in k.lower()]
        out[counter] = (gemm, max(copy) if copy else 0.0)
    sample = json.loads(open(sample_json).read().strip().splitlines()[-1])
    f_gemm, f_copy = out["FETCH_SIZE"]
    w_gemm, w_copy = out["WRITE_SIZE"]
    ff = sample["copy_bytes"] / (f_copy * 1024.0)
    fw = sample["copy_bytes"] / (w_copy * 1024.0)
    fetch = sum(f_gemm) / len(f_gemm) * 1024.0 * ff
    write = sum(w_gemm) / len(w_gemm) * 1024.0 * fw
    alg = sample["gemm_alg_bytes_per_launch"]
    return "\n".join([
        "# HBM traffic of the round GEMM: 7B-shaped lookahead rounds (W=7, N=5, G=7, 512-token prompt)",
        "",
        "Commands (run from /tmp with TMPDIR=/tmp on one MI355X; each counter in a run of its own):",
        "",
        "```",
        "python3 bench.py --pmc-sample > out/pmc_sample.json",
        "rocprofv3 --pmc FETCH_SIZE -d out/pmc_fetch -o f -- python3 bench.py --pmc-sample",
        "rocprofv3 --pmc WRITE_SIZE -d out/pmc_write -o w -- python3 bench.py --pmc-sample",
        "python3 bench.py --pmc-summary out/pmc_fetch/f_results.db out/pmc_write/w_results.db out/pmc_sample.json",
        "```",
        "",
        f"The sample runs {sample['rounds']} lookahead rounds after prefill, then copies a "
        f"{sample['copy_bytes'] >> 20} MiB buffer three times.  Round GEMM dispatches: la_gemm_kernel with at "
        f"most 4 row tiles ({len(f_gemm)} dispatches; prefill chunks use 8).",
        "",
        "| quantity | value |",
        "|---|---:|",
        f"| copy: FETCH_SIZE (KiB) | {f_copy:.0f} |",
        f"| copy: WRITE_SIZE (KiB) | {w_copy:.0f} |",
        f"| FETCH_SIZE scale (copy bytes / counter bytes) | {ff:.3f} |",
        f"| WRITE_SIZE scale | {fw:.3f} |",
        f"| round GEMM: mean FETCH_SIZE per dispatch (KiB) | {sum(f_gemm) / len(f_gemm):.0f} |",
        f"| round GEMM: mean WRITE_SIZE per dispatch (KiB) | {sum(w_gemm) / len(w_gemm):.0f} |",
        f"| HBM read per launch, scaled (MB) | {fetch / 1e6:.2f} |",
        f"| HBM write per launch, scaled (MB) | {write / 1e6:.2f} |",
        f"| algorithmic bytes per launch (MB) | {alg / 1e6:.2f} |",
        f"| traffic / algorithmic | {(fetch + write) / alg:.3f} |",
        "",
        f"traffic_bytes_per_launch: {fetch + write:.0f}",
        f"la_gemm.hip sha256: {_sha256(GEMM_SRC)}",
        "",
    ])


def cpu_baseline(wl, budget_rounds=2, prefix=32):
    """The oracle as it stands, on host cores: a `prefix`-token prompt, then `budget_rounds` rounds."""
    import synthetic
    from oracle.decode import lookahead_generate
    from oracle.model import OracleModel
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    dims = synthetic.PRESETS[wl["model"]]
    w = synthetic.model_weights(dims, 0)
    prompt = synthetic.markov_prompt(dims.vocab, wl["prompt"], 0)[:prefix]
    om = OracleModel(dims, w)
    times = []
    res = lookahead_generate(om, prompt, wl["W"], wl["N"], wl["G"], 1 + budget_rounds, round_times=times)
    toks = len(res["tokens"]) - 1
    secs = sum(times)
    return {"value": toks / secs, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"numpy fp64 oracle, same model and W/N/G, prompt truncated to its first {prefix} tokens, "
                      f"prefill untimed, then {budget_rounds} rounds ({toks} tokens) in {secs:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="rounds to time; 0 (default) times one complete generation of the workload")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama7b_w7n5g7", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-attn", action="store_true")
    ap.add_argument("--pool-from-prompt", action="store_true",
                    help="seed the n-gram pool with the prompt's n-grams (lookahead sessions)")
    ap.add_argument("--pmc-sample", action="store_true", help="run the GEMM counter sample (see profiles/)")
    ap.add_argument("--attention-op-only", action="store_true", help="time only the isolated attention op")
    ap.add_argument("--pmc-summary", nargs=3, metavar=("FETCH_DB", "WRITE_DB", "SAMPLE_JSON"),
                    help="write the GEMM traffic summary under profiles/ from two counter runs")
    args = ap.parse_args()
    if args.pmc_summary:
        md = pmc_summary(*args.pmc_summary)
        open(TRAFFIC_MD, "w").write(md)
        print(md)
        return
    if args.pmc_sample:
        pmc_sample()
        return
    if args.attention_op_only:
        import torch
        torch.cuda.set_device(0)
        print(json.dumps(attention_op()), flush=True)
        print(json.dumps(attention_op(reps=24, sets=4, p=8192)), flush=True)
        print(json.dumps(attention_op(reps=64, sets=32, p=2048, H=64, Hkv=8, N=7)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the lookahead round runs on a single MI355X (got --gpus {args.gpus}); "
              f"lookahead parallelism across GPUs is not implemented: the library runs on one device", file=sys.stderr)
        sys.exit(2)
    import torch
    import synthetic
    import exact_lookahead_decoding_amd.la as la
    la.load()
    torch.cuda.set_device(0)
    wl = WORKLOADS[args.workload]
    dims = synthetic.PRESETS[wl["model"]]
    t = time.time()
    model = la.DeviceModel(dims, seed=0)
    log(f"weights on device: {model.weight_bytes / 1e9:.2f} GB in {time.time() - t:.1f} s")
    if wl.get("copyspan"):
        prompt, copied = synthetic.copyspan_prompt(dims.vocab, wl["prompt"], 0)
        log(f"prompt: {len(prompt)} tokens, {copied * 100:.1f}% copied spans")
    else:
        prompt = synthetic.markov_prompt(dims.vocab, wl["prompt"], 0)

    def make(ar=False, profile=False):
        s = la.Session(model, prompt, W=wl["W"], N=wl["N"], G=wl["G"], max_new=wl["max_new"], ar_only=ar,
                       pool_from_prompt=args.pool_from_prompt and not ar)
        if profile:
            s.la_profile(True)
        return s

    sess = make()
    for _ in range(args.warmup):
        sess.la_step()
    tokens, secs, sess, steps = run_steps(make, sess, args.steps)
    value = tokens / secs
    log(f"lookahead: {tokens} tokens in {steps} rounds, {secs * 1e3 / steps:.3f} ms/round, {value:.1f} tokens/s")
    # autoregressive decoding with the same kernels
    ar = make(ar=True)
    for _ in range(args.warmup):
        ar.la_step()
    ar_tokens, ar_secs, _, ar_steps = run_steps(lambda: make(ar=True), ar, args.steps)
    ar_tps = ar_tokens / ar_secs
    log(f"autoregressive: {ar_tokens} tokens in {ar_steps} rounds, {ar_tps:.1f} tokens/s")
    # dominant kernel: GEMM weight stream, events around each launch
    # a second pass with HIP events around every GEMM / attention launch (one
    # context's totals; with --steps K the first context's rounds are the ones read)
    torch.cuda.synchronize()
    t = time.perf_counter()
    prof = make(profile=True)           # context set-up and prompt prefill, outside every timed region
    torch.cuda.synchronize()
    init_prefill_ms = (time.perf_counter() - t) * 1e3
    sr = step_roofline(model, dims, wl, tokens, steps, secs)
    log(f"round vs HBM bound: {sr['bytes_per_round'] / 1e9:.2f} GB per round, {sr['ms_at_peak']:.2f} ms at 8 TB/s, "
        f"{sr['frac'] * 100:.1f}% of it; set-up + prefill {init_prefill_ms:.0f} ms")
    for _ in range(args.warmup):
        prof.la_step()
    prof.la_profile(True)
    _, prof_secs, prof_end, _ = run_steps(lambda: make(profile=True), prof, args.steps)
    pr = (prof_end if args.steps == 0 else prof).la_profile_read()
    gemm_avg_ms = pr["gemm_ms"] / max(1, pr["gemm_launches"])
    gemm_bytes = pr["gemm_bytes"] / max(1, pr["gemm_launches"])
    achieved = pr["gemm_bytes"] / (pr["gemm_ms"] * 1e-3) / 1e9 if pr["gemm_ms"] > 0 else 0.0
    attn_in_step = pr["attn_bytes"] / (pr["attn_ms"] * 1e-3) / 1e9 if pr["attn_ms"] > 0 else 0.0
    log(f"gemm: {pr['gemm_launches']} launches, avg {gemm_avg_ms * 1e3:.1f} us, {achieved:.0f} GB/s; "
        f"attention in step: {pr['attn_launches']} launches, avg {pr['attn_ms'] / max(1, pr['attn_launches']) * 1e3:.1f} us, "
        f"{attn_in_step:.0f} GB/s; share of step: gemm {pr['gemm_ms'] / (secs * 1e3) * 100:.0f}%")
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": secs * 1e3 / steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if dims.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": wl["desc"], "W": wl["W"], "N": wl["N"], "G": wl["G"], "prompt_tokens": wl["prompt"],
                   "max_new": wl["max_new"], "verify": "greedy", "batch": 1,
                   "pool_from_prompt": bool(args.pool_from_prompt)},
        "tokens_per_round": tokens / steps,
        "ar_tokens_per_s": ar_tps,
        "speedup_vs_ar": value / ar_tps,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": gemm_traffic(),
                     "kernel": "la_gemm_kernel (+ split reduction), all projections, MLP and LM head of a round",
                     "avg_launch_us": gemm_avg_ms * 1e3, "algorithmic_bytes_per_launch": gemm_bytes,
                     "launches": pr["gemm_launches"]},
        "step_roofline": sr,
        "init_prefill_ms": init_prefill_ms,
        "attention_in_step": {"achieved_GBps": attn_in_step, "avg_launch_us":
                              pr["attn_ms"] / max(1, pr["attn_launches"]) * 1e3, "launches": pr["attn_launches"]},
    }
    if not args.no_attn:
        a = attention_op()
        log(f"lookahead attention op: {a['avg_us']:.2f} us, {a['achieved_GBps']:.0f} GB/s ({a['frac'] * 100:.1f}%)")
        line["lookahead_attn"] = a
        # the same op over the long-prefix workload's 8192 committed keys (134 MB of K/V per call)
        a = attention_op(reps=24, sets=4, p=8192)
        log(f"lookahead attention op, prefix 8192: {a['avg_us']:.2f} us, {a['achieved_GBps']:.0f} GB/s "
            f"({a['frac'] * 100:.1f}%)")
        line["lookahead_attn_8192"] = a
        # the 34B-shaped round's attention: 64 query heads on 8 KV heads, 180 rows, 2048 keys
        a = attention_op(reps=64, sets=32, p=2048, H=64, Hkv=8, N=7)
        log(f"lookahead attention op, 34B GQA shape: {a['avg_us']:.2f} us, {a['achieved_GBps']:.0f} GB/s "
            f"({a['frac'] * 100:.1f}%)")
        line["lookahead_attn_34b_gqa"] = a
    if not args.no_cpu_baseline and wl["model"] == "codellama34b":
        log("cpu baseline skipped: the oracle would hold the 34B-shaped weights in host memory")
    elif not args.no_cpu_baseline:
        t = time.time()
        line["cpu_baseline"] = cpu_baseline(wl)
        log(f"cpu baseline: {line['cpu_baseline']['value']:.4f} tokens/s ({time.time() - t:.0f} s)")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
